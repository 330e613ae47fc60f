"""ctypes binding of libmoe_w4.so (the C ABI in include/moe_w4.h).

Argument marshalling only: every function below converts torch tensors to
device pointers, picks the current HIP stream when none is given, calls
the C function of the same name and turns a non-zero status into a
MoeError.  No computation happens here, and there is no fallback: if the
library is not built the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_w4.so")
ABI_VERSION = 4

MOE_OK, MOE_E_INVAL, MOE_E_UNSUPPORTED, MOE_E_DEVICE, MOE_E_WORKSPACE = 0, -1, -2, -3, -4
MOE_A16, MOE_A8 = 0, 1
MOE_PATH_AUTO, MOE_PATH_GEMV, MOE_PATH_MFMA, MOE_PATH_MFMA16 = 0, 1, 2, 3
MOE_QUANT_SEPARATE = 4
MOE_X_PREPARED = 64
MOE_LAYER_ONE_LAUNCH = 8
MOE_OUT_F32 = 16
MOE_W_PREPACKED = 32
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20

c_int, c_size_t, c_void_p = ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p

# name -> (restype, argtypes), mirroring include/moe_w4.h
_SIGS = {
    "moe_abi_version": (c_int, []),
    "moe_status_str": (ctypes.c_char_p, [c_int]),
    "moe_route_topk": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p,
                               c_void_p, c_void_p]),
    "moe_router_workspace_bytes": (c_size_t, [c_int, c_int, c_int]),
    "moe_router_topk": (c_int, [c_void_p, c_int, c_int, c_void_p, c_void_p, c_int, c_int,
                                c_int, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                c_void_p]),
    "moe_permute": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p,
                            c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                            c_void_p]),
    "moe_permute_max_tiles": (c_int, [c_int, c_int, c_int, c_int]),
    "moe_route_permute": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_int,
                                  c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p]),
    "moe_quant_a8_rows": (c_int, [c_void_p, c_int, c_int, c_int, c_int,
                                  c_void_p, c_void_p, c_void_p]),
    "moe_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int,
                                       c_int, c_int, c_int]),
    "moe_preferred_tile_m": (c_int, [c_int, c_int, c_int, c_int]),
    "moe_w4_gateup_silu": (c_int, [c_int, c_void_p, c_int, c_int, c_int,
                                   c_int, c_int, c_void_p, c_void_p, c_int,
                                   c_int, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_int, c_void_p, c_void_p,
                                   c_size_t, c_int, c_void_p]),
    "moe_w4_route_gateup_silu": (c_int, [c_int, c_void_p, c_void_p, c_int, c_int,
                                         c_int, c_int, c_int, c_int, c_void_p,
                                         c_void_p, c_int, c_int, c_int, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_size_t, c_int, c_void_p]),
    "moe_w4_down_combine": (c_int, [c_int, c_void_p, c_int, c_int, c_int,
                                    c_int, c_int, c_void_p, c_void_p, c_int,
                                    c_int, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_void_p, c_void_p, c_void_p, c_int,
                                    c_void_p, c_void_p, c_size_t, c_int,
                                    c_void_p]),
    "moe_w4_layer": (c_int, [c_int, c_void_p, c_void_p, c_int, c_int, c_int,
                             c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_int, c_int, c_void_p, c_int, c_void_p, c_void_p,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                             c_int, c_void_p]),
    "moe_read_stream": (c_int, [c_void_p, c_size_t, c_void_p, c_int, c_void_p]),
    "moe_w4_prepack": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p, c_void_p]),
    "moe_w4_prepack_scales": (c_int, [c_void_p, c_int, c_int, c_int, c_int, c_void_p,
                                      c_void_p]),
    "moe_w4_layer_noalloc": (c_int, [c_int, c_void_p, c_void_p, c_int, c_int, c_int,
                                     c_int, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_int, c_int, c_void_p, c_int, c_void_p,
                                     c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                     c_void_p]),
    "moe_w4_layer_one_launch": (c_int, [c_int, c_int, c_int, c_int, c_int, c_int,
                                        c_int, c_int, c_int, c_int]),
    "moe_dbg_w4a8_gateup_partials": (c_int, [c_void_p, c_int, c_int, c_int,
                                             c_int, c_int, c_void_p, c_void_p,
                                             c_int, c_int, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_int,
                                             c_void_p, c_void_p, c_size_t, c_int,
                                             c_void_p, c_int, c_void_p]),
    "moe_dbg_w4a8_down_partials": (c_int, [c_void_p, c_int, c_int, c_int,
                                           c_int, c_int, c_void_p, c_void_p,
                                           c_int, c_int, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_int, c_void_p,
                                           c_void_p, c_size_t, c_int, c_void_p,
                                           c_int, c_void_p]),
    "moe_dbg_dec_stamps": (c_int, [c_void_p]),
}

EXPORTED = tuple(_SIGS)


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


class QMatDesc(ctypes.Structure):
    """struct moe_qmat (32 bytes)."""
    _fields_ = [("codes", c_void_p), ("scales", c_void_p),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32),
                ("N", ctypes.c_int32), ("K", ctypes.c_int32)]


assert ctypes.sizeof(QMatDesc) == 32

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once and check its ABI version."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m packed_bit_grouped_amd.build` "
            "(there is no fallback path)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    v = lib.moe_abi_version()
    if v != ABI_VERSION:
        raise RuntimeError(f"libmoe_w4.so ABI {v} != binding ABI {ABI_VERSION}; rebuild")
    _lib = lib
    return lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    raise TypeError(f"cannot pass {type(t)} as a device pointer")


def _stream(stream):
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def status_str(status: int) -> str:
    return load().moe_status_str(status).decode()


def _call(name, *args, check=True):
    st = getattr(load(), name)(*args)
    if check and st != MOE_OK:
        raise MoeError(name, st, status_str(st))
    return st


def moe_abi_version() -> int:
    return load().moe_abi_version()


def moe_permute_max_tiles(T, k, E, tile_m) -> int:
    return load().moe_permute_max_tiles(T, k, E, tile_m)


def moe_workspace_bytes(act, T, H, I, E, k, n_shared=0, I_shared=0) -> int:
    return load().moe_workspace_bytes(act, T, H, I, E, k, n_shared, I_shared)


def moe_preferred_tile_m(act, T, E, k) -> int:
    return load().moe_preferred_tile_m(act, T, E, k)


def moe_route_topk(logits, T, E, k, renormalize, topk_ids, topk_w,
                   stream=None, check=True):
    return _call("moe_route_topk", _ptr(logits), T, E, k, renormalize,
                 _ptr(topk_ids), _ptr(topk_w), _stream(stream), check=check)


def moe_router_workspace_bytes(T, H, E) -> int:
    return load().moe_router_workspace_bytes(T, H, E)


def moe_router_topk(x, T, H, router_w, prior, E, k, renormalize, logits, topk_ids,
                    topk_w, workspace, ws_bytes, stream=None, check=True):
    return _call("moe_router_topk", _ptr(x), T, H, _ptr(router_w), _ptr(prior), E, k,
                 renormalize, _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(workspace),
                 ws_bytes, _stream(stream), check=check)


def moe_permute(topk_ids, T, k, E, tile_m, counts, offsets, sorted_pair,
                pair_pos, tiles, n_tiles, stream=None, check=True):
    return _call("moe_permute", _ptr(topk_ids), T, k, E, tile_m, _ptr(counts),
                 _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos), _ptr(tiles),
                 _ptr(n_tiles), _stream(stream), check=check)


def moe_route_permute(logits, T, E, k, renormalize, tile_m, topk_ids, topk_w,
                      counts, offsets, sorted_pair, pair_pos, tiles, n_tiles,
                      stream=None, check=True):
    return _call("moe_route_permute", _ptr(logits), T, E, k, renormalize, tile_m,
                 _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                 _ptr(sorted_pair), _ptr(pair_pos), _ptr(tiles), _ptr(n_tiles),
                 _stream(stream), check=check)


FUSED_ROUTE_MAX_T, FUSED_ROUTE_MAX_P, PERMUTE_MAX_E = 64, 4096, 512


def moe_quant_a8_rows(src, src_is_f32, R, C, ld, q, s, stream=None, check=True):
    return _call("moe_quant_a8_rows", _ptr(src), src_is_f32, R, C, ld, _ptr(q),
                 _ptr(s), _stream(stream), check=check)


def moe_w4_gateup_silu(act, x, T, H, I, E, k, w13, w13_shared, n_shared,
                       I_shared, offsets, sorted_pair, tiles, n_tiles, tile_m,
                       h, workspace, ws_bytes, flags=0, stream=None, check=True):
    return _call("moe_w4_gateup_silu", act, _ptr(x), T, H, I, E, k, _ptr(w13),
                 _ptr(w13_shared), n_shared, I_shared, _ptr(offsets),
                 _ptr(sorted_pair), _ptr(tiles), _ptr(n_tiles), tile_m, _ptr(h),
                 _ptr(workspace), ws_bytes, flags, _stream(stream), check=check)


def moe_w4_route_gateup_silu(act, logits, x, T, H, I, E, k, renormalize, w13,
                             w13_shared, n_shared, I_shared, tile_m, topk_ids,
                             topk_w, counts, offsets, sorted_pair, pair_pos, tiles,
                             n_tiles, h, workspace, ws_bytes, flags=0, stream=None,
                             check=True):
    return _call("moe_w4_route_gateup_silu", act, _ptr(logits), _ptr(x), T, H, I, E,
                 k, renormalize, _ptr(w13), _ptr(w13_shared), n_shared, I_shared,
                 tile_m, _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets),
                 _ptr(sorted_pair), _ptr(pair_pos), _ptr(tiles), _ptr(n_tiles),
                 _ptr(h), _ptr(workspace), ws_bytes, flags, _stream(stream),
                 check=check)


def moe_w4_down_combine(act, h, T, H, I, E, k, w2, w2_shared, n_shared,
                        I_shared, topk_w, offsets, sorted_pair, pair_pos, tiles,
                        n_tiles, tile_m, out, workspace, ws_bytes, flags=0,
                        stream=None, check=True, shared_gate=None):
    return _call("moe_w4_down_combine", act, _ptr(h), T, H, I, E, k, _ptr(w2),
                 _ptr(w2_shared), n_shared, I_shared, _ptr(shared_gate), _ptr(topk_w),
                 _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos), _ptr(tiles),
                 _ptr(n_tiles), tile_m, _ptr(out), _ptr(workspace), ws_bytes,
                 flags, _stream(stream), check=check)


def moe_w4_layer(act, logits, x, T, H, I, E, k, renormalize, w13, w2, w13_shared,
                 w2_shared, n_shared, I_shared, tile_m, topk_ids, topk_w, counts,
                 offsets, sorted_pair, pair_pos, tiles, n_tiles, h, out, workspace,
                 ws_bytes, flags=0, stream=None, check=True, shared_gate=None):
    return _call("moe_w4_layer", act, _ptr(logits), _ptr(x), T, H, I, E, k,
                 renormalize, _ptr(w13), _ptr(w2), _ptr(w13_shared), _ptr(w2_shared),
                 n_shared, I_shared, _ptr(shared_gate), tile_m, _ptr(topk_ids), _ptr(topk_w),
                 _ptr(counts), _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos),
                 _ptr(tiles), _ptr(n_tiles), _ptr(h), _ptr(out), _ptr(workspace),
                 ws_bytes, flags, _stream(stream), check=check)


def moe_w4_prepack(codes, bits, N, K, gate_up, dst, stream=None, check=True):
    return _call("moe_w4_prepack", _ptr(codes), bits, N, K, gate_up, _ptr(dst),
                 _stream(stream), check=check)


def moe_w4_prepack_scales(scales, N, K, group, gate_up, dst, stream=None, check=True):
    return _call("moe_w4_prepack_scales", _ptr(scales), N, K, group, gate_up, _ptr(dst),
                 _stream(stream), check=check)


def moe_read_stream(src, nbytes, sink, n_blocks, stream=None, check=True):
    return _call("moe_read_stream", _ptr(src), nbytes, _ptr(sink), n_blocks,
                 _stream(stream), check=check)


def moe_w4_layer_noalloc(act, logits, x, T, H, I, E, k, renormalize, w13, w2, w13_shared,
                         w2_shared, n_shared, I_shared, tile_m, topk_ids, topk_w, counts,
                         offsets, sorted_pair, pair_pos, tiles, n_tiles, h, out, err_out=None,
                         flags=0, stream=None, check=True, shared_gate=None):
    return _call("moe_w4_layer_noalloc", act, _ptr(logits), _ptr(x), T, H, I, E, k,
                 renormalize, _ptr(w13), _ptr(w2), _ptr(w13_shared), _ptr(w2_shared),
                 n_shared, I_shared, _ptr(shared_gate), tile_m, _ptr(topk_ids), _ptr(topk_w),
                 _ptr(counts), _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos),
                 _ptr(tiles), _ptr(n_tiles), _ptr(h), _ptr(out), _ptr(err_out),
                 flags, _stream(stream), check=check)


def moe_w4_layer_one_launch(act, T, H, I, E, k, n_shared=0, I_shared=0, tile_m=16,
                            flags=0) -> int:
    return load().moe_w4_layer_one_launch(act, T, H, I, E, k, n_shared, I_shared,
                                          tile_m, flags)


def moe_dbg_w4a8_gateup_partials(x, T, H, I, E, k, w13, w13_shared, n_shared,
                                 I_shared, offsets, sorted_pair, tiles, n_tiles,
                                 tile_m, h, workspace, ws_bytes, partials, ng_ld,
                                 flags=0, stream=None, check=True):
    return _call("moe_dbg_w4a8_gateup_partials", _ptr(x), T, H, I, E, k,
                 _ptr(w13), _ptr(w13_shared), n_shared, I_shared, _ptr(offsets),
                 _ptr(sorted_pair), _ptr(tiles), _ptr(n_tiles), tile_m, _ptr(h),
                 _ptr(workspace), ws_bytes, flags, _ptr(partials), ng_ld,
                 _stream(stream), check=check)


def moe_dbg_w4a8_down_partials(h, T, H, I, E, k, w2, w2_shared, n_shared,
                               I_shared, topk_w, offsets, sorted_pair, pair_pos,
                               tiles, n_tiles, tile_m, out, workspace, ws_bytes,
                               partials, ng_ld, flags=0, stream=None, check=True,
                               shared_gate=None):
    return _call("moe_dbg_w4a8_down_partials", _ptr(h), T, H, I, E, k,
                 _ptr(w2), _ptr(w2_shared), n_shared, I_shared, _ptr(shared_gate),
                 _ptr(topk_w),
                 _ptr(offsets), _ptr(sorted_pair), _ptr(pair_pos), _ptr(tiles),
                 _ptr(n_tiles), tile_m, _ptr(out), _ptr(workspace), ws_bytes,
                 flags, _ptr(partials), ng_ld, _stream(stream), check=check)


def moe_dbg_dec_stamps(stamps, check=True):
    """The decode kernels' phase-stamp buffer (a MOE_DEC_STAMPS build only)."""
    return _call("moe_dbg_dec_stamps", _ptr(stamps), check=check)
