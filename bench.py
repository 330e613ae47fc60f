#!/usr/bin/env python3
"""Benchmark of the low-bit MoE FFN layer on one MI355X.

A step is one pass of the whole layer (route -> permute -> gate/up+SiLU*mul
-> down+combine) over one batch of synthetic input resident in HBM.
Default workload: the single-token decode layer (T=1, H=2048, E=128, top-8,
I=768, int4 G128 experts, one always-on shared expert).  Decode throughput
is packed-weight GB/s over the experts a step touches (codes + fp16
scales, each touched expert counted once); prefill (--config 4) is TFLOP/s
over 6*P*H*I useful flops.

So that repeated steps measure HBM rather than the 256 MB Infinity Cache,
decode steps rotate over R device copies of the weight bank (same routing,
distinct addresses) with R * touched bytes >= --rotate-bytes.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE W4 FFN layer: packed-weight GB/s (decode) and TFLOP/s (prefill)"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def touched_bytes(dl, counts, which=("w13", "w2")):
    """Packed bytes (codes + fp16 scales) of the routed experts with at
    least one pair, plus every shared expert, for the given matrices."""
    per = {"w13": [], "w2": [], "w13_sh": [], "w2_sh": []}
    for tag, oc, os_, (bits, group, N, K) in dl.bank.layout:
        per[tag].append(N * K * bits // 8 + N * (K // group) * 2)
    tot = 0
    for m in which:
        tot += sum(b for b, c in zip(per[m], counts) if c > 0)
        tot += sum(per[m + "_sh"])
    return tot


def measured_traffic(key):
    """HBM bytes per launch from the byte-counter profiles (profiles/
    traffic.json), or None when they are absent or were taken on other
    kernel sources."""
    import hashlib
    try:
        with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
            t = json.load(f)[key]
        h = hashlib.sha256()
        for src in t["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        return t["bytes_per_launch"] if h.hexdigest() == t["source_sha256"] else None
    except (OSError, KeyError, ValueError):
        return None


def cpu_baseline(layer, seconds, unit_amount, unit, sample_note):
    import numpy as np  # noqa: F401
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.oracle_layer(layer)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    return {"value": unit_amount / per, "unit": unit, "cores": cores,
            "kind": "oracle",
            "sample": f"{sample_note}; {n} full oracle layer passes in {el:.1f} s "
                      f"({per * 1e3:.1f} ms each); cores = BLAS threads"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=1)
    ap.add_argument("--rotate-bytes", type=float, default=1.5e9)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=["auto", "gemv", "mfma"], default="auto")
    ap.add_argument("--one-launch", action="store_true",
                    help="run small bf16 decode layers as one launch (moe_w4_layer's "
                         "opt-in single-launch form)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MB",
                    help="after the run, one device copy of MB MiB (a plain copy kernel of "
                         "known size, the scale for hardware byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this layer runs on one GPU; multi-GPU runs are "
                          "not part of this benchmark (use --gpus 1)"}))
        log("bench.py: --gpus N with N > 1 is not supported: the layer is a "
            "single-GPU kernel library (expert-parallel sharding is design only)")
        sys.exit(2)

    import numpy as np
    import torch

    from packed_bit_grouped_amd import _lib as L
    from packed_bit_grouped_amd.layer import DeviceLayer, run_layer
    from synth import CONFIGS, make_layer

    cfg = CONFIGS[args.config]
    flags = {"auto": 0, "gemv": 1, "mfma": 2}[args.path]
    layer_flags = flags | (L.MOE_LAYER_ONE_LAUNCH if args.one_launch else 0)
    torch.cuda.set_device(0)
    t0 = time.time()
    log(f"[bench] generating {cfg.name} ...")
    layer = make_layer(cfg)
    log(f"[bench] generated in {time.time() - t0:.1f} s; uploading")
    dl = DeviceLayer.from_synth(layer, "cuda:0")
    act = cfg.act
    B = dl.buffers(act)

    # routing is identical on every step: learn the touched experts once
    dl.run(B, layer_flags)
    torch.cuda.synchronize()
    counts = B.counts.cpu().numpy()
    n_touched = int((counts > 0).sum())
    decode = args.config != 4
    bytes_all = touched_bytes(dl, counts)
    bytes_w13 = touched_bytes(dl, counts, ("w13",))
    P = cfg.T * cfg.k
    flops = 6.0 * P * cfg.H * cfg.I + 6.0 * cfg.n_shared * cfg.T * cfg.H * cfg.I_shared
    flops_gateup = 4.0 * P * cfg.H * cfg.I + 4.0 * cfg.n_shared * cfg.T * cfg.H * cfg.I_shared

    banks = [dl.bank]
    if decode:
        R = max(1, math.ceil(args.rotate_bytes / bytes_all))
        R = min(R, 128)
        free, _ = torch.cuda.mem_get_info()
        R = max(1, min(R, int(0.5 * free // dl.bank.buf.numel())))
        for _ in range(R - 1):
            banks.append(dl.bank.rebased(dl.bank.buf.clone()))
        log(f"[bench] {n_touched} routed experts touched, {bytes_all / 1e6:.3f} MB/step; "
            f"rotating over {R} bank copies ({R * bytes_all / 1e9:.2f} GB touched per cycle)")

    def step(i):
        run_layer(banks[i % len(banks)], dl.x, dl.logits, B, cfg.renormalize, layer_flags)

    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k

    # bf16 decode batches of at most 64 pairs route, sort and run gate/up in
    # one launch (the library's rule for moe_w4_route_gateup_silu); other
    # shapes time the gate/up call alone (A8: with its int8 x quantizer)
    fused = (decode and act == "a16" and cfg.T * cfg.k <= 64 and cfg.E <= 512
             and B.tile_m <= 16 and cfg.H <= 2048)

    # with --one-launch, small bf16 decode batches run the whole layer as one
    # launch when the device holds every workgroup of its grid at once (the
    # library's rule for moe_w4_layer); that launch is then the dominant kernel
    one = decode and L.moe_w4_layer_one_launch(B.act, T, H, I, E, k, cfg.n_shared,
                                               cfg.I_shared, B.tile_m, layer_flags) == 1

    def gateup(bk):
        if one:
            run_layer(bk, dl.x, dl.logits, B, cfg.renormalize, layer_flags)
        elif fused:
            L.moe_w4_route_gateup_silu(B.act, dl.logits, dl.x, T, H, I, E, k,
                                       cfg.renormalize, bk.w13, bk.w13_sh, cfg.n_shared,
                                       cfg.I_shared, B.tile_m, B.ids, B.w, B.counts,
                                       B.offsets, B.sorted_pair, B.pair_pos, B.tiles,
                                       B.n_tiles, B.h, B.ws, B.ws_bytes, flags)
        else:
            L.moe_w4_gateup_silu(B.act, dl.x, T, H, I, E, k, bk.w13, bk.w13_sh,
                                 cfg.n_shared, cfg.I_shared, B.offsets, B.sorted_pair,
                                 B.tiles, B.n_tiles, B.tile_m, B.h, B.ws, B.ws_bytes, flags)

    def timed(fn, n):
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(torch.cuda.current_stream())
        for i in range(n):
            fn(i)
        e1.record(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        step(i)
    # eager issue from Python (secondary number: includes host launch cost)
    ms_eager = timed(step, args.steps)
    log(f"[bench] eager: {ms_eager * 1e3:.2f} us/step")

    # the served form: HIP graphs of G consecutive steps over G distinct
    # weight-bank copies (as a model's decode graph holds its layers, each
    # with its own weights), replayed back to back
    G = next(g for g in (16, 8, 4, 2, 1) if g <= len(banks) and args.steps % g == 0)
    n_graphs = len(banks) // G
    graphs = []
    for gi in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(G):
                run_layer(banks[gi * G + i], dl.x, dl.logits, B, cfg.renormalize,
                          layer_flags)
        graphs.append(g)
    reps = args.steps // G
    for i in range(max(1, args.warmup // G)):
        graphs[i % n_graphs].replay()
    ms = timed(lambda i: graphs[i % n_graphs].replay(), reps) / G
    log(f"[bench] graph replay: {reps * G} steps ({G} per graph): {ms * 1e3:.2f} us/step")
    # check the replayed steps against an eager one (same inputs, same bank)
    out_g = B.out.clone()
    step((reps - 1) % n_graphs * G + G - 1)
    torch.cuda.synchronize()
    if not torch.equal(out_g, B.out):
        log("[bench] graph replay output differs from the eager step")
        sys.exit(3)

    # the dominant kernel (gate/up + SiLU*mul) alone: a graph of back-to-back
    # launches over distinct bank copies, timed with events on the stream
    # the graph runs on
    n_k = min(len(banks), 32) if decode else 4
    if one:
        kname = "dec_layer_kernel (route + sort + gate/up + SiLU*mul + down + combine)"
    elif fused:
        kname = "dec_route_gateup_kernel (route + sort + gate/up + SiLU*mul)"
    elif decode:
        kname = ("proj_m16_kernel<0> (gate/up + SiLU*mul)" if act == "a16" else
                 "proj_m16_kernel<0> (int8 x rows made in the kernel, gate/up + SiLU*mul)")
    else:
        kname = "proj_mfma_kernel<0> + convert_x_kernel (gate/up + SiLU*mul)"
    gk = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gk):
        for i in range(n_k):
            gateup(banks[i % len(banks)])
    gk.replay()
    reps = max(1, args.steps // n_k)
    gu_ms = timed(lambda i: gk.replay(), reps) / n_k
    log(f"[bench] {'layer' if one else 'gate/up'} kernel: {gu_ms * 1e3:.2f} us/launch")

    if decode:
        value = bytes_all / (ms * 1e-3) / 1e9
        unit = "GB/s"
        alg = bytes_all if one else bytes_w13
        ach = alg / (gu_ms * 1e-3) / 1e9
        key = ("dec_layer_kernel@" if one else
               "dec_route_gateup_kernel@" if fused else "gateup_call@") + cfg.name
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS,
                "traffic": measured_traffic(key),
                "kernel": kname,
                "algorithmic_bytes": alg}
    else:
        value = flops / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
        ach = flops_gateup / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                "traffic": measured_traffic(f"gateup_call@{cfg.name}"),
                "kernel": kname, "algorithmic_flops": flops_gateup}

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the CPU oracle for ~{args.cpu_seconds:.0f} s")
        if decode:
            cpu = cpu_baseline(layer, args.cpu_seconds, bytes_all / 1e9, "GB/s",
                               f"{cfg.name}, same seeded layer")
        else:
            cpu = {"value": None, "unit": "TFLOP/s", "cores": None, "kind": "oracle",
                   "sample": "prefill oracle not timed by default"}

    line = {
        "metric": METRIC, "value": value, "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if act == "a16" else "int8",
        "data": "synthetic (seeded; int4/int2 experts quantized from N(0, 0.02))",
        "config": {"workload": cfg.name, "T": cfg.T, "H": cfg.H, "E": cfg.E, "k": cfg.k,
                   "I": cfg.I, "n_shared": cfg.n_shared, "act": act,
                   "experts_touched": n_touched,
                   "bytes_per_step": bytes_all, "flops_per_step": flops,
                   "bank_copies_rotated": len(banks), "path": args.path,
                   "layer_form": "one launch" if one else "separate calls",
                   "timing": f"HIP graphs of {G} steps over {G} weight copies, replayed back to back",
                   "ms_per_step_eager": ms_eager},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    if args.copy_probe > 0:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {n} bytes read and written")


if __name__ == "__main__":
    main()
