"""Low-bit (W4/W2) mixture-of-experts FFN layer for AMD MI355X (gfx950).

The compute lives in libmoe_w4.so (hand-written HIP kernels behind the C
ABI of include/moe_w4.h); this package is its Python binding (`_lib`), the
device-resident layer driver (`layer`) and the build script (`build`).
"""
from . import _lib  # noqa: F401
from ._lib import (MOE_A16, MOE_A8, MOE_PATH_AUTO, MOE_PATH_GEMV,  # noqa: F401
                   MOE_PATH_MFMA, MoeError)
