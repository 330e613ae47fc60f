"""The C-ABI library without a GPU: it loads, exports every function the
header declares, reports its ABI version, sizes buffers, and rejects bad
arguments on the host before touching any device (no compute here)."""
import os
import re

import pytest

from packed_bit_grouped_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4.h")

lib = pytest.importorskip("ctypes")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(
        r"^\s*(?:moe_status|int|size_t|const char\s*\*)\s+(moe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_function():
    lib = L.load()
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.EXPORTED, n


def test_abi_version_matches_header():
    text = open(HEADER).read()
    v = int(re.search(r"#define MOE_W4_ABI_VERSION (\d+)", text).group(1))
    assert L.moe_abi_version() == v == L.ABI_VERSION


def test_status_strings():
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(L.status_str(s), str) and L.status_str(s)


def test_max_tiles_bound():
    # min(P, floor(P / tile_m) + min(E, P))
    assert L.moe_permute_max_tiles(1, 8, 128, 16) == 8
    assert L.moe_permute_max_tiles(12, 8, 128, 16) == 96
    assert L.moe_permute_max_tiles(4096, 8, 256, 64) == 512 + 256
    assert L.moe_permute_max_tiles(0, 8, 256, 64) == 0


def up256(n):
    return (n + 255) // 256 * 256


def test_workspace_sizes():
    # header (error word, then the one-launch layer's 1024 barrier flags) +
    # fp32 y rows (+ int8 x and fp32 scales for A8) (+ per-workgroup counts
    # of the multi-workgroup sort from 8192 pairs) (+ for the A16 matrix
    # core path when H, I, I_shared are multiples of 128: one fp16 copy of
    # x or h, and the fp16 h rows the gate/up epilogue writes), each region
    # 256-byte aligned
    HDR = 256 + 1024 * 4
    a16 = up256(max(1 * 2048 * 2, 9 * 768 * 2)) + up256(9 * 768 * 2)
    assert L.moe_workspace_bytes(0, 1, 2048, 768, 128, 8, 1, 768) == \
        HDR + 9 * 2048 * 4 + a16
    # the prefill chunk: 32768 pairs over 16 sort workgroups of 2048
    pre = L.moe_workspace_bytes(0, 4096, 4096, 1536, 256, 8, 0, 0)
    assert pre == HDR + 32768 * 4096 * 4 + 16 * 256 * 4 + up256(max(4096 * 4096 * 2,
                                                                    32768 * 1536 * 2)) \
        + 32768 * 1536 * 2
    # A8: int8 x + scales, then int8 h rows (stride max(I, I_shared)) + scales
    a8 = L.moe_workspace_bytes(1, 64, 2048, 768, 128, 8, 0, 0)
    assert a8 == HDR + 64 * 2048 + 256 + 512 * 768 + 512 * 4 + 512 * 2048 * 4
    a8 = L.moe_workspace_bytes(1, 3, 512, 256, 8, 2, 1, 384)
    assert a8 == HDR + up256(3 * 512) + 256 + up256(9 * 384) + 256 + up256(9 * 512 * 4)
    assert L.moe_workspace_bytes(0, 0, 2048, 768, 128, 8, 0, 0) == HDR
    # no matrix-core copies when a dimension is not a multiple of 128
    assert L.moe_workspace_bytes(0, 4, 256, 96, 8, 2, 0, 0) == HDR + up256(8 * 256 * 4)
    # shared expert wider than the routed ones sets the h stride
    a16 = up256(max(3 * 512 * 2, 3 * (2 + 1) * 384 * 2)) + up256(3 * (2 + 1) * 384 * 2)
    assert L.moe_workspace_bytes(0, 3, 512, 256, 8, 2, 1, 384) == \
        HDR + up256(3 * 3 * 512 * 4) + a16


FAKE = 1 << 20   # a non-null pointer value; never dereferenced on the host


@pytest.mark.parametrize("args,code", [
    ((FAKE, 4, 0, 1, 1, FAKE, FAKE), L.MOE_E_INVAL),       # E = 0
    ((FAKE, 4, 8, 9, 1, FAKE, FAKE), L.MOE_E_INVAL),       # k > E
    ((FAKE, 4, 8, 0, 1, FAKE, FAKE), L.MOE_E_INVAL),       # k = 0
    ((FAKE, 4, 8, 2, 2, FAKE, FAKE), L.MOE_E_INVAL),       # renormalize not 0/1
    ((FAKE, -1, 8, 2, 1, FAKE, FAKE), L.MOE_E_INVAL),      # T < 0
    ((None, 4, 8, 2, 1, FAKE, FAKE), L.MOE_E_INVAL),       # null logits
    ((FAKE, 4, 2000, 2, 1, FAKE, FAKE), L.MOE_E_UNSUPPORTED),  # E > 1024
    ((None, 0, 8, 2, 1, None, None), L.MOE_OK),            # T = 0: nothing to do
])
def test_route_validation(args, code):
    assert L.moe_route_topk(*args, stream=0, check=False) == code


def test_permute_validation():
    ok = dict(topk_ids=FAKE, T=4, k=2, E=8, tile_m=16, counts=FAKE, offsets=FAKE,
              sorted_pair=FAKE, pair_pos=FAKE, tiles=FAKE, n_tiles=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_permute(*a.values(), stream=0, check=False)
    assert call(E=600) == L.MOE_E_UNSUPPORTED
    assert call(tile_m=0) == L.MOE_E_INVAL
    assert call(counts=None) == L.MOE_E_INVAL
    assert call(tiles=FAKE + 4) == L.MOE_E_INVAL      # tiles must be 16-byte aligned
    assert call(T=1 << 22, k=8) == L.MOE_E_UNSUPPORTED


def _gateup(**kw):
    a = dict(act=0, x=FAKE, T=4, H=256, I=128, E=8, k=2, w13=FAKE, w13_shared=None,
             n_shared=0, I_shared=0, offsets=FAKE, sorted_pair=FAKE, tiles=FAKE,
             n_tiles=FAKE, tile_m=16, h=FAKE, workspace=FAKE, ws_bytes=1 << 30, flags=0)
    a.update(kw)
    return L.moe_w4_gateup_silu(*a.values(), stream=0, check=False)


def test_gateup_validation():
    assert _gateup(act=2) == L.MOE_E_INVAL
    assert _gateup(k=9) == L.MOE_E_INVAL
    assert _gateup(H=250) == L.MOE_E_UNSUPPORTED         # K % 32
    assert _gateup(I=100) == L.MOE_E_UNSUPPORTED
    assert _gateup(n_shared=1, I_shared=0) == L.MOE_E_INVAL
    assert _gateup(n_shared=1, I_shared=128, w13_shared=None) == L.MOE_E_INVAL
    assert _gateup(x=None) == L.MOE_E_INVAL
    assert _gateup(x=FAKE + 2) == L.MOE_E_INVAL          # 16-byte alignment
    assert _gateup(ws_bytes=16) == L.MOE_E_WORKSPACE
    assert _gateup(workspace=None) == L.MOE_E_WORKSPACE
    assert _gateup(workspace=FAKE + 64) == L.MOE_E_WORKSPACE  # 256-byte alignment
    assert _gateup(flags=8) == L.MOE_E_INVAL
    assert _gateup(flags=128) == L.MOE_E_INVAL
    assert _gateup(flags=L.MOE_X_PREPARED, act=1) == L.MOE_E_DEVICE
    assert _gateup(flags=L.MOE_QUANT_SEPARATE | L.MOE_PATH_MFMA16, act=1) == L.MOE_E_DEVICE
    # forced 16-row MFMA tiles: tiles of at most 16 rows, activations in LDS
    assert _gateup(flags=L.MOE_PATH_MFMA16, tile_m=32) == L.MOE_E_UNSUPPORTED
    assert _gateup(flags=L.MOE_PATH_MFMA16, T=16, H=8192) == L.MOE_E_UNSUPPORTED
    assert _gateup(flags=L.MOE_PATH_MFMA16) == L.MOE_E_DEVICE
    # forced MFMA grouped GEMM on a shape it does not cover
    assert _gateup(flags=L.MOE_PATH_MFMA, I=96) == L.MOE_E_UNSUPPORTED
    assert _gateup(flags=L.MOE_PATH_MFMA, act=1) == L.MOE_E_UNSUPPORTED
    assert _gateup(E=600, k=2) == L.MOE_E_UNSUPPORTED
    assert _gateup(T=0, x=None) == L.MOE_OK               # empty batch
    # everything valid: only the device check remains, and there is no GPU here
    assert _gateup() == L.MOE_E_DEVICE


def test_down_validation():
    a = dict(act=0, h=FAKE, T=4, H=256, I=128, E=8, k=2, w2=FAKE, w2_shared=None,
             n_shared=0, I_shared=0, topk_w=FAKE, offsets=FAKE, sorted_pair=FAKE,
             pair_pos=FAKE, tiles=FAKE, n_tiles=FAKE, tile_m=16, out=FAKE,
             workspace=FAKE, ws_bytes=1 << 30, flags=0)

    def call(**kw):
        b = dict(a, **kw)
        return L.moe_w4_down_combine(*b.values(), stream=0, check=False)
    assert call(topk_w=None) == L.MOE_E_INVAL
    assert call(pair_pos=None) == L.MOE_E_INVAL
    assert call(out=FAKE + 2) == L.MOE_E_INVAL
    assert call(out=FAKE + 8, flags=L.MOE_OUT_F32) == L.MOE_E_INVAL   # fp32 out: 16 bytes
    assert call(out=FAKE + 8) == L.MOE_E_DEVICE
    assert call(flags=L.MOE_OUT_F32) == L.MOE_E_DEVICE
    assert call(ws_bytes=100) == L.MOE_E_WORKSPACE
    assert call(T=0, h=None) == L.MOE_OK
    assert call(flags=L.MOE_PATH_MFMA16, tile_m=17) == L.MOE_E_UNSUPPORTED
    assert call(flags=L.MOE_PATH_MFMA16) == L.MOE_E_DEVICE
    assert call() == L.MOE_E_DEVICE


def test_stamps_hook_is_inert_in_the_regular_library():
    """moe_dbg_dec_stamps only works in the MOE_DEC_STAMPS build; the
    regular library reports it unsupported and touches nothing."""
    assert L.moe_dbg_dec_stamps(FAKE, check=False) == L.MOE_E_UNSUPPORTED
    assert L.moe_dbg_dec_stamps(None, check=False) == L.MOE_E_UNSUPPORTED


def test_quant_validation():
    assert L.moe_quant_a8_rows(FAKE, 2, 4, 8, 8, FAKE, FAKE, stream=0, check=False) == L.MOE_E_INVAL
    assert L.moe_quant_a8_rows(FAKE, 0, 4, 8, 4, FAKE, FAKE, stream=0, check=False) == L.MOE_E_INVAL
    assert L.moe_quant_a8_rows(None, 0, 0, 8, 8, None, None, stream=0, check=False) == L.MOE_OK


def test_debug_hooks_need_partials():
    assert L.moe_dbg_w4a8_gateup_partials(
        FAKE, 4, 256, 128, 8, 2, FAKE, None, 0, 0, FAKE, FAKE, FAKE, FAKE, 16,
        FAKE, FAKE, 1 << 30, None, 8, stream=0, check=False) == L.MOE_E_INVAL
    # the hooks take the product's path choice; the matrix-core prefill path is A16 only
    for flags, want in ((L.MOE_PATH_MFMA, L.MOE_E_UNSUPPORTED), (L.MOE_PATH_AUTO, L.MOE_E_DEVICE),
                        (L.MOE_PATH_GEMV, L.MOE_E_DEVICE), (L.MOE_PATH_MFMA16, L.MOE_E_DEVICE)):
        assert L.moe_dbg_w4a8_gateup_partials(
            FAKE, 4, 256, 128, 8, 2, FAKE, None, 0, 0, FAKE, FAKE, FAKE, FAKE, 16,
            FAKE, FAKE, 1 << 30, FAKE, 8, flags=flags, stream=0, check=False) == want
        assert L.moe_dbg_w4a8_down_partials(
            FAKE, 4, 256, 128, 8, 2, FAKE, None, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE,
            FAKE, 16, FAKE, FAKE, 1 << 30, FAKE, 8, flags=flags, stream=0,
            check=False) == want


def test_route_permute_validation():
    ok = dict(logits=FAKE, T=4, E=8, k=2, renormalize=1, tile_m=16, topk_ids=FAKE,
              topk_w=FAKE, counts=FAKE, offsets=FAKE, sorted_pair=FAKE, pair_pos=FAKE,
              tiles=FAKE, n_tiles=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_route_permute(*a.values(), stream=0, check=False)
    assert call(T=65) == L.MOE_E_UNSUPPORTED             # fused only for small batches
    assert call(T=64, k=65, E=512) == L.MOE_E_UNSUPPORTED   # T*k > 4096
    assert call(E=513, k=2) == L.MOE_E_UNSUPPORTED
    assert call(k=9) == L.MOE_E_INVAL
    assert call(tile_m=0) == L.MOE_E_INVAL
    assert call(topk_w=None) == L.MOE_E_INVAL
    assert call() == L.MOE_E_DEVICE


def test_layer_validation():
    """moe_w4_layer checks its arguments on the host: the one-launch shape
    (bf16 decode batch) and a shape that takes the two-call form."""
    ok = dict(act=0, logits=FAKE, x=FAKE, T=1, H=2048, I=768, E=128, k=8, renormalize=1,
              w13=FAKE, w2=FAKE, w13_shared=FAKE, w2_shared=FAKE, n_shared=1,
              I_shared=768, tile_m=16, topk_ids=FAKE, topk_w=FAKE, counts=FAKE,
              offsets=FAKE, sorted_pair=FAKE, pair_pos=FAKE, tiles=FAKE, n_tiles=FAKE,
              h=FAKE, out=FAKE, workspace=FAKE, ws_bytes=1 << 30, flags=0)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_w4_layer(*a.values(), stream=0, check=False)
    assert call(renormalize=2) == L.MOE_E_INVAL
    assert call(act=2) == L.MOE_E_INVAL
    assert call(k=129) == L.MOE_E_INVAL
    assert call(flags=128) == L.MOE_E_INVAL
    assert call(out=None) == L.MOE_E_INVAL
    assert call(w2_shared=None) == L.MOE_E_INVAL
    assert call(workspace=None) == L.MOE_E_WORKSPACE
    assert call(ws_bytes=64) == L.MOE_E_WORKSPACE
    assert call(H=2047) == L.MOE_E_UNSUPPORTED
    # valid arguments reach the device check (no GPU here), for the two-call
    # form and the one-launch form alike
    assert call() == L.MOE_E_DEVICE
    assert call(flags=L.MOE_LAYER_ONE_LAUNCH) == L.MOE_E_DEVICE
    assert call(T=64, act=1, n_shared=0) == L.MOE_E_DEVICE
    q = L.moe_w4_layer_one_launch
    one = L.MOE_LAYER_ONE_LAUNCH
    assert q(0, 1, 2048, 768, 128, 8, 1, 768, 16, one) == L.MOE_E_DEVICE   # needs the device
    assert q(0, 1, 2048, 768, 128, 8, 1, 768, 16, 0) == 0                  # default: two calls
    assert q(1, 64, 2048, 768, 128, 8, 0, 0, 16, one) == 0                 # A8: two calls
    assert q(0, 1, 2048, 768, 256, 8, 1, 768, 16, one) == 0                # E > 128
    assert q(2, 1, 2048, 768, 128, 8, 1, 768, 16, 0) == L.MOE_E_INVAL


def test_router_validation_and_workspace():
    """moe_router_topk checks its arguments on the host; small batches
    split H over chunks and need a workspace for the partial sums."""
    # one token, 2 expert tiles: H = 2048 in 64 chunks of 32 -> 64 * 1 * 128 partials
    assert L.moe_router_workspace_bytes(1, 2048, 128) == 64 * 128 * 4
    assert L.moe_router_workspace_bytes(4096, 4096, 256) == 0   # one chunk
    assert L.moe_router_workspace_bytes(0, 2048, 128) == 0
    ok = dict(x=FAKE, T=1, H=2048, router_w=FAKE, prior=None, E=128, k=8, renormalize=1,
              logits=FAKE, topk_ids=FAKE, topk_w=FAKE, workspace=FAKE, ws_bytes=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_router_topk(*a.values(), stream=0, check=False)
    assert call(k=0) == L.MOE_E_INVAL
    assert call(k=129) == L.MOE_E_INVAL
    assert call(renormalize=3) == L.MOE_E_INVAL
    assert call(H=0) == L.MOE_E_INVAL
    assert call(E=1025, k=2) == L.MOE_E_UNSUPPORTED
    assert call(logits=None) == L.MOE_E_INVAL
    assert call(workspace=None) == L.MOE_E_WORKSPACE
    assert call(ws_bytes=16) == L.MOE_E_WORKSPACE
    assert call(T=0, x=None) == L.MOE_OK
    assert call() == L.MOE_E_DEVICE
    assert call(T=4096, H=4096, E=256, workspace=None, ws_bytes=0) == L.MOE_E_DEVICE


def test_noalloc_validation():
    """moe_w4_layer_noalloc checks the shape and that its workspace fits the
    library's static scratch array on the host, before touching a device."""
    ok = dict(act=0, logits=FAKE, x=FAKE, T=1, H=2048, I=768, E=128, k=8, renormalize=1,
              w13=FAKE, w2=FAKE, w13_shared=FAKE, w2_shared=FAKE, n_shared=1,
              I_shared=768, tile_m=16, topk_ids=FAKE, topk_w=FAKE, counts=FAKE,
              offsets=FAKE, sorted_pair=FAKE, pair_pos=FAKE, tiles=FAKE, n_tiles=FAKE,
              h=FAKE, out=FAKE, err_out=None, flags=0)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_w4_layer_noalloc(*a.values(), stream=0, check=False)
    assert call(act=3) == L.MOE_E_INVAL
    assert call(T=-1) == L.MOE_E_INVAL
    # a 4096-token prefill chunk needs far more than the 32 MiB array
    assert L.moe_workspace_bytes(0, 4096, 4096, 1536, 256, 8) > L.MOE_NOALLOC_SCRATCH_BYTES
    assert call(T=4096, H=4096, I=1536, E=256, n_shared=0, I_shared=0,
                tile_m=160) == L.MOE_E_WORKSPACE
    # decode shapes fit (the 64-token W4A8 layer included) and reach the device check
    assert L.moe_workspace_bytes(1, 64, 2048, 768, 128, 8) <= L.MOE_NOALLOC_SCRATCH_BYTES
    assert call(act=1, T=64, n_shared=0, I_shared=0) == L.MOE_E_DEVICE
    assert call() == L.MOE_E_DEVICE


def test_prepack_validation():
    ok = dict(codes=FAKE, bits=4, N=256, K=512, gate_up=1, dst=FAKE + 4096)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_w4_prepack(*a.values(), stream=0, check=False)
    assert call(bits=3) == L.MOE_E_UNSUPPORTED
    assert call(N=48) == L.MOE_E_UNSUPPORTED       # blocks of 32 rows
    assert call(N=96) == L.MOE_E_UNSUPPORTED       # gate/up: blocks of 32 units
    assert call(N=96, gate_up=0) == L.MOE_E_DEVICE
    assert call(K=64) == L.MOE_E_UNSUPPORTED       # K % 128
    assert call(gate_up=2) == L.MOE_E_INVAL
    assert call(dst=FAKE) == L.MOE_E_INVAL         # in place
    assert call(dst=None) == L.MOE_E_INVAL
    assert call(codes=FAKE + 8) == L.MOE_E_INVAL   # 16-byte aligned
    assert call() == L.MOE_E_DEVICE


def test_prepack_scales_validation():
    ok = dict(scales=FAKE, N=256, K=512, group=128, gate_up=1, dst=FAKE + 4096)

    def call(**kw):
        a = dict(ok, **kw)
        return L.moe_w4_prepack_scales(*a.values(), stream=0, check=False)
    assert call(group=16) == L.MOE_E_UNSUPPORTED
    assert call(K=448) == L.MOE_E_UNSUPPORTED      # K % group
    assert call(N=96) == L.MOE_E_UNSUPPORTED       # pairs of 32-row blocks
    assert call(N=96, gate_up=0) == L.MOE_E_UNSUPPORTED
    assert call(gate_up=2) == L.MOE_E_INVAL
    assert call(N=0) == L.MOE_E_INVAL
    assert call(dst=FAKE) == L.MOE_E_INVAL         # in place
    assert call(dst=None) == L.MOE_E_INVAL
    assert call(scales=FAKE + 2) == L.MOE_E_INVAL  # 4-byte aligned
    assert call(dst=FAKE + 4104) == L.MOE_E_INVAL  # 16-byte aligned
    assert call(K=8192, group=64) == L.MOE_E_UNSUPPORTED   # more than 64 groups
    assert call() == L.MOE_E_DEVICE
    assert call(gate_up=0, group=32) == L.MOE_E_DEVICE
