"""Helpers of the GPU parity tests: run the layer through the C ABI and
bring every intermediate back to the host (the host copies happen here,
in the test, never inside the layer)."""
import numpy as np

ACTS = {"a16": 0, "a8": 1}


def torch_mod():
    import torch
    return torch


def to_np(t):
    return t.detach().cpu().numpy()


def bf16_bits_to_f64(u16):
    u = np.asarray(u16).astype(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def run_layer_gpu(dl, act=None, tile_m=None, flags=0, stream=None, fused=True,
                  one_call=True, out_f32=False):
    """Run one layer step on the device; returns host copies of everything
    (out as float64 values: of the bf16 output, or with out_f32 of the fp32
    output the library writes under MOE_OUT_F32)."""
    torch = torch_mod()
    B = dl.buffers(act, tile_m, out_f32)
    dl.run(B, flags, stream, fused, one_call)
    torch.cuda.synchronize()
    return collect(B), B


def collect(B):
    torch = torch_mod()
    nt = int(B.n_tiles.item())
    res = {
        "ids": to_np(B.ids)[:B.T], "w": to_np(B.w)[:B.T].astype(np.float64),
        "counts": to_np(B.counts), "offsets": to_np(B.offsets),
        "sorted_pair": to_np(B.sorted_pair)[:B.P], "pair_pos": to_np(B.pair_pos)[:B.P],
        "tiles": to_np(B.tiles)[:nt], "n_tiles": nt,
        "out": (to_np(B.out)[:B.T].astype(np.float64) if B.out_flags else
                bf16_bits_to_f64(to_np(B.out)[:B.T])),
        "out_bits": None if B.out_flags else to_np(B.out)[:B.T].astype(np.uint16),
        "err": int(B.ws[:4].view(torch.int32).item()),
    }
    if B.act == 0:
        res["h"] = bf16_bits_to_f64(to_np(B.h)[:B.R])
    else:
        res["h32"] = to_np(B.h)[:B.R].astype(np.float32)
    return res


def float_gate(got, ref, rel_l2=5e-3, max_abs_frac=2e-2):
    """rel-L2 <= 5e-3 and max-abs <= 2e-2 * rms(ref).  Returns the errors."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = got - ref
    nref = np.linalg.norm(ref)
    rl2 = np.linalg.norm(d) / nref if nref > 0 else np.linalg.norm(d)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    mabs = np.abs(d).max() if d.size else 0.0
    ok = rl2 <= rel_l2 and mabs <= max_abs_frac * rms if rms > 0 else mabs == 0
    return ok, rl2, mabs, rms


def h_gate(got, ref, act):
    """Check of the intermediate h.  A16: both sides round h to bf16, so an
    element may differ by one bf16 unit in the last place (2^-7 of its
    magnitude at most) where the two unrounded values straddle a rounding
    boundary; otherwise max-abs <= 2e-2 * rms.  rel-L2 <= 5e-3 always.
    A8: fp32 h, the plain float gate.  Returns (ok, rel-L2, worst ratio)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    nref = np.linalg.norm(ref)
    rl2 = np.linalg.norm(got - ref) / nref if nref > 0 else np.linalg.norm(got - ref)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    bound = np.full(ref.shape, 2e-2 * rms)
    if act == "a16":
        bound = np.maximum(bound, 2.0 ** -7 * np.abs(ref))
    worst = float((d / np.maximum(bound, 1e-300)).max()) if d.size else 0.0
    return (rl2 <= 5e-3 and worst <= 1.0), rl2, worst


def bf16_rne_bits(f32):
    """fp32 values -> bf16 bit patterns, round to nearest even (finite input)."""
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def worst_error(got, ref):
    """(flat index, ref value, got value) of the largest absolute error."""
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    i = int(np.argmax(np.abs(got - ref))) if ref.size else 0
    return i, float(ref[i]) if ref.size else 0.0, float(got[i]) if ref.size else 0.0


def check_out(g_bf16, g_f32, ref, tag=""):
    """The output gate, on the computation and on the stored result:
    the fp32 output (the combined sum before rounding) meets rel-L2 <=
    5e-3 and max-abs <= 2e-2 * rms(ref), and the bf16 output is exactly
    its round-to-nearest-even.  (The bf16 rounding itself can exceed
    2e-2 * rms: its half-unit is 2^-9..2^-8 of |out|, e.g. 2^-7 = 0.0078
    for |out| in [2, 4), so it is checked as this identity instead.)"""
    ok, rl2, mabs, rms = float_gate(g_f32["out"], ref)
    i, rv, gv = worst_error(g_f32["out"], ref)
    print(f"[parity] {tag} out fp32 rel-L2 {rl2:.2e} max-abs {mabs:.2e} (gate {2e-2 * rms:.2e}) "
          f"worst at {i}: ref {rv:.6g} got {gv:.6g}", flush=True)
    assert ok, ("out", rl2, mabs, rms, i, rv, gv)
    want = bf16_rne_bits(g_f32["out"].astype(np.float32))
    assert np.array_equal(g_bf16["out_bits"], want), "bf16 output is not the RNE of the fp32 output"
    ok2, rl2b, mabsb, _ = float_gate(g_bf16["out"], ref)
    print(f"[parity] {tag} out bf16 rel-L2 {rl2b:.2e} max-abs {mabsb:.2e}", flush=True)
    assert rl2b <= 5e-3
