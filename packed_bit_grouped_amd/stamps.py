"""Phase timeline of a decode step from the kernels' clock stamps.

Usage (repo root, one GPU), with the stamped library built first:
    python -m packed_bit_grouped_amd.build --stamps packed_bit_grouped_amd/libmoe_w4_stamps.so
    python -m packed_bit_grouped_amd.stamps [--config 1] [--reps 60] [--out FILE.md]

The step's two launches (fused route + sort + gate/up, then down + combine)
run one at a time on weight copies rotated over at least 1.5 GB (every
weight read comes from HBM, as in the benchmark), each launch with the stamp
buffer named just before it.  Workgroups stamp the 100 MHz realtime counter
(10 ns ticks) at each phase end (moe_dbg_dec_stamps in include/moe_w4.h
names the phases).  Reported per phase: the median over launches of the
median workgroup's and of the last workgroup's time since the launch's
first workgroup started.  Eager launches: each starts from an idle GPU.
"""
from __future__ import annotations

import argparse
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
STAMPS_LIB = os.path.join(HERE, "libmoe_w4_stamps.so")

GU_PHASES = ["entry", "routed (logits, descriptors, top-k)", "sorted (tile list)",
             "weight loads issued", "activations staged", "products + h stored"]
DN_PHASES = ["entry", "tables in", "weight loads issued", "h rows staged", "products done",
             "outputs stored"]


def _timeline(st):
    """st: [grid][8] ticks of one launch -> (per-slot median, per-slot max)
    in us after the first workgroup's entry, and the workgroup count."""
    live = st[:, 0] > 0
    s = st[live].astype(np.int64)
    t0 = s[:, 0].min()
    med, last = [], []
    for i in range(6):
        v = s[:, i]
        v = v[v > 0]
        med.append(np.median(v - t0) / 100.0 if len(v) else np.nan)
        last.append((v.max() - t0) / 100.0 if len(v) else np.nan)
    return np.array(med), np.array(last), int(live.sum()), int((s[:, 5] > 0).sum())


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--reps", type=int, default=60)
    ap.add_argument("--lib", default=STAMPS_LIB)
    ap.add_argument("--rotate-bytes", type=float, default=1.5e9)
    ap.add_argument("--out", default=None)
    args = ap.parse_args(argv)

    import torch  # first: the library binds to the HIP runtime torch loads

    sys.path.insert(0, ROOT)
    from packed_bit_grouped_amd import _lib as L
    L.load(args.lib)
    from packed_bit_grouped_amd.layer import DeviceLayer
    from synth import CONFIGS, make_layer

    cfg = CONFIGS[args.config]
    if cfg.act != "a16" or cfg.T * cfg.k > 64:
        raise SystemExit("the stamped kernels are the bf16 decode kernels of up to 64 pairs")
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    dl = DeviceLayer.from_synth(make_layer(cfg), "cuda:0")
    B = dl.buffers("a16")
    dl.run(B, 0)
    torch.cuda.synchronize()
    counts = B.counts.cpu().numpy()
    # packed bytes (codes + scales) of the touched routed experts and the
    # shared ones: what a step reads
    step_bytes = int(dl.bank.nbytes_by_expert[counts > 0].sum()) + int(dl.bank.nbytes_shared)
    R = max(2, math.ceil(args.rotate_bytes / step_bytes))
    banks = [dl.bank] + [dl.bank.rebased(dl.bank.buf.clone()) for _ in range(R - 1)]

    # one row of 8 stamps per workgroup: bounded by one workgroup per unit
    # of every possible tile (gate/up) and by H / 4 column blocks (down)
    slots = max((T * k + E + cfg.n_shared * T) * max(I, cfg.I_shared), H // 4)
    if slots > 1 << 22:
        raise SystemExit("layer too large for the stamp buffer bound")
    sg = torch.zeros(slots * 8, dtype=torch.int64, device="cuda")
    sd = torch.zeros(slots * 8, dtype=torch.int64, device="cuda")

    def gateup(bk):
        L.moe_w4_route_gateup_silu(B.act, dl.logits, dl.x, T, H, I, E, k, cfg.renormalize,
                                   bk.w13, bk.w13_sh, cfg.n_shared, cfg.I_shared, B.tile_m,
                                   B.ids, B.w, B.counts, B.offsets, B.sorted_pair,
                                   B.pair_pos, B.tiles, B.n_tiles, B.h, B.ws, B.ws_bytes, 0)

    def down(bk):
        L.moe_w4_down_combine(B.act, B.h, T, H, I, E, k, bk.w2, bk.w2_sh, cfg.n_shared,
                              cfg.I_shared, B.w, B.offsets, B.sorted_pair, B.pair_pos,
                              B.tiles, B.n_tiles, B.tile_m, B.out, B.ws, B.ws_bytes)

    res = {"gu": [], "dn": []}
    n_wg = {}
    for rep in range(args.reps + 2):
        bk = banks[rep % R]
        for key, buf, fn in (("gu", sg, gateup), ("dn", sd, down)):
            buf.zero_()
            torch.cuda.synchronize()
            L.moe_dbg_dec_stamps(buf)
            fn(bk)
            torch.cuda.synchronize()
            L.moe_dbg_dec_stamps(None)
            if rep >= 2:   # two warm-up steps
                med, last, n_all, n_work = _timeline(buf.view(slots, 8).cpu().numpy())
                res[key].append((med, last))
                n_wg[key] = (n_all, n_work)
        if rep == 0:
            print(f"[stamps] {cfg.name}: {R} weight copies, {step_bytes / 1e6:.1f} MB per step",
                  flush=True)

    lines = [f"# Phase timeline: {cfg.name} (T={T}, H={H}, E={E}, top-{k}, I={I}, "
             f"{cfg.n_shared} shared expert(s), bf16 activations)", "",
             "Command (repo root, one MI355X):", "",
             "    python -m packed_bit_grouped_amd.build --stamps "
             "packed_bit_grouped_amd/libmoe_w4_stamps.so",
             f"    python -m packed_bit_grouped_amd.stamps --config {args.config} "
             f"--reps {args.reps} --out <this file>", "",
             f"Each of the step's two launches run {args.reps} times on weight copies rotated "
             f"over {R * step_bytes / 1e9:.2f} GB ({R} copies of the {step_bytes / 1e6:.1f} MB "
             "a step reads), one launch at a time from an idle GPU, in the library built with "
             "MOE_DEC_STAMPS.  Thread 0 of every workgroup stamps the 100 MHz realtime counter "
             "(10 ns ticks) at each phase end; times are us after the launch's first workgroup "
             "entered, the median over launches of the median workgroup and of the last one.",
             ""]
    for key, title, phases in (("gu", "dec_route_gateup_kernel (route + sort + gate/up + "
                                      "SiLU*mul)", GU_PHASES),
                               ("dn", "dec_down_combine_kernel (down + weighted combine)",
                                DN_PHASES)):
        med = np.nanmedian(np.stack([m for m, _ in res[key]]), axis=0)
        last = np.nanmedian(np.stack([l for _, l in res[key]]), axis=0)
        n_all, n_work = n_wg[key]
        did = (f"all of them did products" if n_work == n_all else
               f"{n_work} of them did products (the rest exit after the tile lookup)")
        lines += [f"## {title}", "", f"{n_all} workgroups entered, {did}.", "",
                  "| phase end | median workgroup (us) | last workgroup (us) |",
                  "|---|---|---|"]
        lines += [f"| {p} | {m:.2f} | {l:.2f} |" for p, m, l in zip(phases, med, last)]
        lines.append("")
    text = "\n".join(lines)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text, flush=True)


if __name__ == "__main__":
    main()
