"""Device-resident MoE W4 FFN layer: buffers plus the four C-ABI calls.

PyTorch serves here only as the device allocator and stream provider;
every step of the layer runs in the HIP kernels behind the C ABI.

* ``upload_bank`` packs the quantized expert matrices of a layer into one
  device buffer (each array 256-byte aligned) and builds the device
  descriptor tables (struct moe_qmat) the kernels read.
* ``LayerBuffers`` preallocates every per-step buffer once; a step reuses
  them and never reads device memory back (no host sync in the path).
* ``run_layer`` issues route -> permute -> gate/up -> down+combine.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

from . import _lib as L


def _torch():
    import torch
    return torch


def _align(n: int, a: int = 256) -> int:
    return (n + a - 1) // a * a


@dataclass
class Bank:
    """Packed matrices of one layer in one device buffer + descriptor tables."""
    buf: "object"            # torch uint8 [bytes]
    w13: "object"            # torch uint8 [E * 32] (device moe_qmat table)
    w2: "object"
    w13_sh: Optional[object]
    w2_sh: Optional[object]
    layout: list             # (matrix tag, offset codes, offset scales, meta)
    nbytes_by_expert: np.ndarray   # packed bytes (codes + scales) per routed expert
    nbytes_shared: int

    prepacked: bool = False  # codes in the matrix-core layout (MOE_W_PREPACKED)

    def rebased(self, buf) -> "Bank":
        """Same layout on another buffer (a device copy of ``buf``)."""
        t13, t2, s13, s2 = _tables(self.layout, buf)
        return Bank(buf, t13, t2, s13, s2, self.layout, self.nbytes_by_expert,
                    self.nbytes_shared, self.prepacked)

    def prepack(self) -> "Bank":
        """A copy of the bank with every code matrix re-tiled by
        moe_w4_prepack and its scales by moe_w4_prepack_scales; calls on it
        need MOE_W_PREPACKED (run_layer adds it)."""
        buf = self.buf.clone()
        base, dst = self.buf.data_ptr(), buf.data_ptr()
        for tag, oc, os_, (bits, group, N, K) in self.layout:
            gu = 1 if tag in ("w13", "w13_sh") else 0
            L.moe_w4_prepack(base + oc, bits, N, K, gu, dst + oc)
            L.moe_w4_prepack_scales(base + os_, N, K, group, gu, dst + os_)
        b = self.rebased(buf)
        b.prepacked = True
        return b


def _qmat_bytes(qm) -> int:
    return int(qm.codes.nbytes + qm.scales.nbytes)


def _tables(layout, buf):
    torch = _torch()
    base = buf.data_ptr()
    groups = {"w13": [], "w2": [], "w13_sh": [], "w2_sh": []}
    for tag, oc, os_, (bits, group, N, K) in layout:
        d = L.QMatDesc(base + oc, base + os_, bits, group, N, K)
        groups[tag].append(bytes(d))
    out = []
    for tag in ("w13", "w2", "w13_sh", "w2_sh"):
        if not groups[tag]:
            out.append(None)
            continue
        raw = np.frombuffer(b"".join(groups[tag]), dtype=np.uint8).copy()
        out.append(torch.from_numpy(raw).to(buf.device))
    return tuple(out)


def upload_bank(experts: Sequence, shared: Sequence, device) -> Bank:
    """Copy every expert's codes and scales into one device buffer."""
    torch = _torch()
    entries = []
    off = 0
    for tag, lst, mats in (("w13", experts, "w13"), ("w2", experts, "w2"),
                           ("w13_sh", shared, "w13"), ("w2_sh", shared, "w2")):
        for ex in lst:
            qm = getattr(ex, mats)
            oc = off
            off = _align(off + qm.codes.nbytes)
            os_ = off
            off = _align(off + qm.scales.nbytes)
            entries.append((tag, oc, os_, qm))
    host = np.zeros(off, dtype=np.uint8)
    layout = []
    for tag, oc, os_, qm in entries:
        host[oc:oc + qm.codes.nbytes] = np.ascontiguousarray(qm.codes).view(np.uint8).ravel()
        host[os_:os_ + qm.scales.nbytes] = np.ascontiguousarray(qm.scales).view(np.uint8).ravel()
        layout.append((tag, oc, os_, (qm.bits, qm.group, qm.N, qm.K)))
    buf = torch.from_numpy(host).to(device)
    del host
    t13, t2, s13, s2 = _tables(layout, buf)
    per = np.array([_qmat_bytes(e.w13) + _qmat_bytes(e.w2) for e in experts], dtype=np.int64)
    nsh = sum(_qmat_bytes(e.w13) + _qmat_bytes(e.w2) for e in shared)
    return Bank(buf, t13, t2, s13, s2, layout, per, nsh)


class LayerBuffers:
    """Every per-step buffer of one layer shape, allocated once."""

    def __init__(self, T, H, I, E, k, n_shared=0, I_shared=0, act=L.MOE_A16,
                 tile_m=None, device="cuda", out_f32=False):
        torch = _torch()
        self.T, self.H, self.I, self.E, self.k = T, H, I, E, k
        self.n_shared, self.I_shared, self.act = n_shared, I_shared, act
        self.tile_m = tile_m or L.moe_preferred_tile_m(act, T, E, k)
        P = T * k
        self.P = P
        self.R = P + n_shared * T
        self.ld_h = max(I, I_shared if n_shared else 0)
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        self.ids = torch.empty((max(T, 1), k), **i32)
        self.w = torch.empty((max(T, 1), k), dtype=torch.float32, device=dev)
        self.counts = torch.empty(E, **i32)
        self.offsets = torch.empty(E + 1, **i32)
        self.sorted_pair = torch.empty(max(P, 1), **i32)
        self.pair_pos = torch.empty(max(P, 1), **i32)
        self.max_tiles = max(L.moe_permute_max_tiles(T, k, E, self.tile_m), 1)
        self.tiles = torch.empty((self.max_tiles, 4), **i32)
        self.n_tiles = torch.zeros(1, **i32)
        hdt = torch.int16 if act == L.MOE_A16 else torch.float32
        # zeroed once: the columns past a shorter expert's I are never written
        self.h = torch.zeros((max(self.R, 1), self.ld_h), dtype=hdt, device=dev)
        self.ws_bytes = L.moe_workspace_bytes(act, T, H, I, E, k, n_shared, I_shared)
        self.ws = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)
        # bf16 bit patterns, or fp32 (the unrounded sum, MOE_OUT_F32)
        self.out_flags = L.MOE_OUT_F32 if out_f32 else 0
        self.out = torch.empty((max(T, 1), H), dtype=torch.float32 if out_f32 else torch.int16,
                               device=dev)

    def error_word(self) -> int:
        return int(self.ws[:4].view(_torch().int32).item())


def fused_routing_ok(T, E, k) -> bool:
    """Route and permute in one launch when the batch is small."""
    return (0 < T <= L.FUSED_ROUTE_MAX_T and T * k <= L.FUSED_ROUTE_MAX_P
            and E <= L.PERMUTE_MAX_E)


def run_layer(bank: Bank, x, logits, B: LayerBuffers, renormalize: int = 1,
              flags: int = 0, stream=None, fused: bool = True,
              one_call: bool = True, shared_gate=None) -> None:
    """One layer step: route, permute, gate/up + SiLU*mul, down + combine.
    With ``fused`` and ``one_call`` the whole step is moe_w4_layer (with
    MOE_LAYER_ONE_LAUNCH in ``flags``: one launch for small bf16 decode
    batches); with ``fused`` alone the first three go through
    moe_w4_route_gateup_silu and the rest through moe_w4_down_combine;
    otherwise every call is issued separately.  ``shared_gate``: fp32
    [T][n_shared] gate logits of the shared experts (sigmoid gate), or
    None (weight 1.0)."""
    T, H, I, E, k = B.T, B.H, B.I, B.E, B.k
    flags |= B.out_flags
    if bank.prepacked:
        flags |= L.MOE_W_PREPACKED
    if not (fused and one_call):
        flags &= ~L.MOE_LAYER_ONE_LAUNCH   # only moe_w4_layer takes it
    if fused and one_call:
        L.moe_w4_layer(B.act, logits, x, T, H, I, E, k, renormalize, bank.w13,
                       bank.w2, bank.w13_sh, bank.w2_sh, B.n_shared, B.I_shared,
                       B.tile_m, B.ids, B.w, B.counts, B.offsets, B.sorted_pair,
                       B.pair_pos, B.tiles, B.n_tiles, B.h, B.out, B.ws,
                       B.ws_bytes, flags, stream, shared_gate=shared_gate)
        return
    if fused:
        L.moe_w4_route_gateup_silu(B.act, logits, x, T, H, I, E, k, renormalize,
                                   bank.w13, bank.w13_sh, B.n_shared, B.I_shared,
                                   B.tile_m, B.ids, B.w, B.counts, B.offsets,
                                   B.sorted_pair, B.pair_pos, B.tiles, B.n_tiles,
                                   B.h, B.ws, B.ws_bytes, flags, stream)
    elif fused_routing_ok(T, E, k):
        L.moe_route_permute(logits, T, E, k, renormalize, B.tile_m, B.ids, B.w,
                            B.counts, B.offsets, B.sorted_pair, B.pair_pos,
                            B.tiles, B.n_tiles, stream)
    else:
        L.moe_route_topk(logits, T, E, k, renormalize, B.ids, B.w, stream)
        L.moe_permute(B.ids, T, k, E, B.tile_m, B.counts, B.offsets,
                      B.sorted_pair, B.pair_pos, B.tiles, B.n_tiles, stream)
    if not fused:
        L.moe_w4_gateup_silu(B.act, x, T, H, I, E, k, bank.w13, bank.w13_sh,
                             B.n_shared, B.I_shared, B.offsets, B.sorted_pair,
                             B.tiles, B.n_tiles, B.tile_m, B.h, B.ws, B.ws_bytes,
                             flags, stream)
    L.moe_w4_down_combine(B.act, B.h, T, H, I, E, k, bank.w2, bank.w2_sh,
                          B.n_shared, B.I_shared, B.w, B.offsets,
                          B.sorted_pair, B.pair_pos, B.tiles, B.n_tiles,
                          B.tile_m, B.out, B.ws, B.ws_bytes, flags, stream,
                          shared_gate=shared_gate)


def bf16_to_float(t):
    """int16 tensor of bf16 bit patterns -> float32 tensor (exact)."""
    torch = _torch()
    return (t.to(torch.int32) << 16).view(torch.float32)


@dataclass
class DeviceLayer:
    """A synthetic layer resident on the device."""
    cfg: object
    x: object          # int16 [T][H] (bf16 bits)
    logits: object     # float32 [T][E]
    bank: Bank
    shared_gate: Optional[object] = None   # float32 [T][n_shared] gate logits, or None

    @classmethod
    def from_synth(cls, layer, device="cuda") -> "DeviceLayer":
        torch = _torch()
        dev = torch.device(device)
        x = torch.from_numpy(layer.x_bf16.view(np.int16).copy()).to(dev)
        logits = torch.from_numpy(np.ascontiguousarray(layer.logits)).to(dev)
        bank = upload_bank(layer.experts, layer.shared, dev)
        sg = getattr(layer, "shared_gate_logits", None)
        sg = None if sg is None else torch.from_numpy(np.ascontiguousarray(sg)).to(dev)
        return cls(layer.cfg, x, logits, bank, sg)

    def buffers(self, act=None, tile_m=None, out_f32=False) -> LayerBuffers:
        c = self.cfg
        a = {"a16": L.MOE_A16, "a8": L.MOE_A8}[act or c.act]
        return LayerBuffers(c.T, c.H, c.I, c.E, c.k, c.n_shared, c.I_shared, a,
                            tile_m, self.x.device, out_f32)

    def run(self, B: LayerBuffers, flags: int = 0, stream=None, fused: bool = True,
            one_call: bool = True) -> None:
        run_layer(self.bank, self.x, self.logits, B, self.cfg.renormalize,
                  flags, stream, fused, one_call, self.shared_gate)
