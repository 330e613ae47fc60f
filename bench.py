#!/usr/bin/env python3
"""Benchmark of the low-bit MoE FFN layer on one MI355X.

A step is one pass of the whole layer (route -> permute -> gate/up+SiLU*mul
-> down+combine) over one batch of synthetic input resident in HBM.

Default run: every benchmark layer, one JSON line.  The headline is the
prefill chunk (T=4096, H=4096, E=256, top-8, I=1536, 192 int4/G128 + 64
int2/G64 experts): TFLOP/s over 6*P*H*I useful flops (P = T*k pairs).  The
three decode layers (T=1 with a shared expert, T=12 Zipf-skewed with a
shared expert, T=64 W4A8) follow as sub-records: packed-weight GB/s over the
experts a step touches (codes + fp16 scales, each touched expert counted
once).  Every record carries the roofline of its dominant kernel (timed live
with HIP events on the stream it runs on) and the CPU oracle timed on a
bounded sample.  --config N runs one layer alone.

Decode steps rotate over R device copies of the weight bank (same routing,
distinct addresses, R * touched bytes >= --rotate-bytes) and every timed step
continues the cycle where the previous step left it, so each step reads
weights last touched R steps (>= 1.5 GB) earlier: the 256 MB Infinity Cache
cannot serve them.

Prints ONE JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE W4 FFN layer: packed-weight GB/s (decode) and TFLOP/s (prefill)"
HBM_PEAK_GBS = 8000.0
F16_PEAK_TFLOPS = 2500.0      # dense fp16 / bf16 MFMA
HEADLINE = 4                  # the prefill chunk
SUBS = (1, 2, 3)              # decode layers


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


def host_info():
    """CPU model, affinity and BLAS threads of the host the oracle runs on."""
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = os.cpu_count() or 1
    blas, threads = "unknown", 1
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = max(i.get("num_threads", 1) for i in info)
    except Exception:  # pragma: no cover
        pass
    return {"cpu_model": model, "cpu_affinity": affinity, "blas": blas,
            "blas_threads": threads}


def timed_loop(fn, n, torch):
    """Average ms of fn(i), i < n, between HIP events on the current stream
    (the stream every call here is issued on)."""
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(torch.cuda.current_stream())
    for i in range(n):
        fn(i)
    e1.record(torch.cuda.current_stream())
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def cpu_oracle_decode(layer, seconds, gbytes, hi):
    """Full oracle layer passes on the host for about `seconds` (at least
    one), as GB/s of the step's packed bytes."""
    import oracle
    t0 = time.perf_counter()
    n = 0
    while True:
        oracle.oracle_layer(layer)
        n += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    per = el / n
    return {"value": gbytes / per, "unit": "GB/s", "cores": hi["blas_threads"],
            "kind": "oracle",
            "sample": f"{layer.cfg.name}: {n} full fp64 oracle layer passes in {el:.1f} s "
                      f"({per * 1e3:.1f} ms each)",
            **hi}


def cpu_oracle_prefill(layer, n_experts, hi):
    """The oracle on a bounded sample of the prefill layer: routing and the
    stable grouping of all 4096 tokens, then gate/up + SiLU*mul and down
    for every pair routed to the first n_experts experts (int4 and int2 as
    in the layer); TFLOP/s over those pairs' 6*H*I flops each."""
    import numpy as np
    import oracle
    cfg = layer.cfg
    t0 = time.perf_counter()
    ids, w = oracle.route_topk(layer.logits, cfg.k, cfg.renormalize)
    perm = oracle.permute(ids, cfg.E, 16)
    off = perm["offsets"]
    keep = np.arange(cfg.E) < n_experts
    counts = np.where(keep, np.diff(off), 0)
    sub = {"offsets": np.concatenate([[0], np.cumsum(counts)]).astype(np.int64),
           "sorted_pair": perm["sorted_pair"][:int(off[n_experts])]}
    sub_layer = type(layer)(**{**layer.__dict__,
                               "cfg": cfg.replace(n_shared=0, I_shared=0), "shared": []})
    h, _ = oracle.gateup_a16(sub_layer, sub)
    oracle.down_a16(sub_layer, sub, h)
    el = time.perf_counter() - t0
    pairs = int(counts.sum())
    flops = 6.0 * pairs * cfg.H * cfg.I
    n2 = int(sum(1 for e in range(n_experts) if layer.experts[e].w13.bits == 2))
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": hi["blas_threads"],
            "kind": "oracle",
            "sample": f"{cfg.name}: fp64 oracle routing + grouping of all {cfg.T} tokens, then "
                      f"gate/up + down of the {pairs} pairs routed to experts 0..{n_experts - 1} "
                      f"({n2} of them int2) in {el:.1f} s",
            **hi}


READ_GRIDS = (256, 512, 1024, 2048, 4096)


def read_ceiling(torch, L, nbytes):
    """Measured HBM read-stream ceiling: GB/s of one plain streaming read of
    nbytes (rotating over two buffers so no read is served by the cache),
    the best of several grid sizes."""
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(2)]
    for b in bufs:
        b.fill_(1)
    best = None
    for n_blocks in READ_GRIDS:
        sink = torch.zeros(n_blocks, dtype=torch.int32, device="cuda")
        for b in bufs:
            L.moe_read_stream(b, nbytes, sink, n_blocks)
        ms = timed_loop(lambda i: L.moe_read_stream(bufs[i % 2], nbytes, sink, n_blocks), 10,
                        torch)
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["achieved"]:
            best = {"achieved": gbs, "unit": "GB/s", "bytes": nbytes,
                    "kernel": f"read_stream_kernel (16-byte loads, {n_blocks} workgroups of 256)"}
    del bufs
    torch.cuda.empty_cache()
    return best


def read_ceiling_at(torch, L, nbytes, total):
    """The same plain streaming read at one decode size: back-to-back reads
    of nbytes in a HIP graph, each from its own slot of a buffer of at least
    `total` bytes (the bytes the decode step graphs cycle through: several
    times the 256 MB Infinity Cache, so reads come from HBM under the same
    conditions as the rotated weight copies); the best of several grid
    sizes, GB/s per read."""
    nbytes = nbytes // 16 * 16          # the read's granularity
    stride = -(-nbytes // 256) * 256
    n = max(2, int(-(-total // stride)))
    buf = torch.ones(n * stride, dtype=torch.uint8, device="cuda")
    best = None
    for n_blocks in READ_GRIDS:
        sink = torch.zeros(n_blocks, dtype=torch.int32, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                L.moe_read_stream(buf[i * stride:], nbytes, sink, n_blocks)
        g.replay()
        ms = timed_loop(lambda i: g.replay(), 3, torch) / n
        gbs = nbytes / (ms * 1e-3) / 1e9
        if best is None or gbs > best["achieved"]:
            best = {"achieved": gbs, "unit": "GB/s", "bytes": nbytes, "ms_per_read": ms,
                    "kernel": f"read_stream_kernel (16-byte loads, {n_blocks} workgroups of "
                              f"256), {n} distinct slots per graph"}
        del g
    del buf
    torch.cuda.empty_cache()
    return best


def run_config(cid, args, torch, L, hi, ceiling):
    from packed_bit_grouped_amd.layer import DeviceLayer, run_layer
    from synth import CONFIGS, make_layer

    cfg = CONFIGS[cid]
    decode = cid != 4
    flags = {"auto": 0, "gemv": 1, "mfma": 2}[args.path]
    t0 = time.time()
    log(f"[bench] generating {cfg.name} ...")
    layer = make_layer(cfg)
    log(f"[bench] generated in {time.time() - t0:.1f} s; uploading")
    dl = DeviceLayer.from_synth(layer, "cuda:0")
    if not args.canonical_weights and not decode and args.path != "gemv":
        # the served form of the prefill bank: codes re-tiled once, at load
        # time, into the matrix-core layout (moe_w4_prepack)
        dl.bank = dl.bank.prepack()
        torch.cuda.synchronize()
    act = cfg.act
    B = dl.buffers(act)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k

    # routing is identical on every step: learn the touched experts once
    dl.run(B, flags)
    torch.cuda.synchronize()
    counts = B.counts.cpu().numpy()
    n_touched = int((counts > 0).sum())
    bytes_all = touched_bytes(dl, counts)
    bytes_w13 = touched_bytes(dl, counts, ("w13",))
    P = T * k
    flops = 6.0 * P * H * I + 6.0 * cfg.n_shared * T * H * cfg.I_shared
    flops_gateup = 4.0 * P * H * I + 4.0 * cfg.n_shared * T * H * cfg.I_shared

    # steps per graph: a divisor of --steps (the timed region is exactly K steps)
    G = next(g for g in (16, 8, 4, 2, 1) if args.steps % g == 0)
    banks = [dl.bank]
    if decode:
        R = max(G, math.ceil(args.rotate_bytes / bytes_all))
        R = min(-(-R // G) * G, 128 // G * G)
        free, _ = torch.cuda.mem_get_info()
        R = max(G, min(R, int(0.5 * free // dl.bank.buf.numel()) // G * G))
        for _ in range(R - 1):
            banks.append(dl.bank.rebased(dl.bank.buf.clone()))
        log(f"[bench] {n_touched} routed experts touched, {bytes_all / 1e6:.3f} MB/step; "
            f"{R} bank copies ({R * bytes_all / 1e9:.2f} GB per cycle)")
    else:
        G = 1

    def step_on(bk):
        run_layer(bk, dl.x, dl.logits, B, cfg.renormalize, flags)

    # the served form: HIP graphs of G consecutive steps over G distinct bank
    # copies, replayed in cycle order; warm-up replays come first and the
    # timed replays continue the cycle
    n_graphs = len(banks) // G
    graphs = []
    for gi in range(n_graphs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(G):
                step_on(banks[gi * G + i])
        graphs.append(g)
    w_reps = max(1, -(-args.warmup // G))
    for i in range(w_reps):
        graphs[i % n_graphs].replay()
    reps = args.steps // G
    ms = timed_loop(lambda i: graphs[(w_reps + i) % n_graphs].replay(), reps, torch) / G
    log(f"[bench] {cfg.name}: graph replay, {reps * G} steps ({G} per graph): "
        f"{ms * 1e3:.2f} us/step")
    # the replayed steps against an eager one (same inputs, same bank)
    last = (w_reps + reps - 1) % n_graphs
    out_g = B.out.clone()
    step_on(banks[last * G + G - 1])
    torch.cuda.synchronize()
    if not torch.equal(out_g, B.out):
        log("[bench] graph replay output differs from the eager step")
        sys.exit(3)
    # eager issue from Python (secondary: includes host launch cost)
    ms_eager = timed_loop(lambda i: step_on(banks[i % len(banks)]), args.steps, torch)
    log(f"[bench] {cfg.name}: eager {ms_eager * 1e3:.2f} us/step")

    # the dominant kernel (gate/up + SiLU*mul) alone: a graph of back-to-back
    # launches over every bank copy, timed with events on the stream it runs on
    fused = (decode and act == "a16" and P <= 64 and E <= 512 and B.tile_m <= 16 and H <= 2048)

    def gateup(bk):
        gflags = flags | (L.MOE_W_PREPACKED if bk.prepacked else 0)
        if (decode and act == "a8") or not decode:
            # the step's gate/up reads the copy of x its routing launch made
            # (int8 rows / the fp16 copy; still in the workspace from the
            # steps above)
            gflags |= L.MOE_X_PREPARED
        if fused:
            L.moe_w4_route_gateup_silu(B.act, dl.logits, dl.x, T, H, I, E, k,
                                       cfg.renormalize, bk.w13, bk.w13_sh, cfg.n_shared,
                                       cfg.I_shared, B.tile_m, B.ids, B.w, B.counts,
                                       B.offsets, B.sorted_pair, B.pair_pos, B.tiles,
                                       B.n_tiles, B.h, B.ws, B.ws_bytes, flags)
        else:
            L.moe_w4_gateup_silu(B.act, dl.x, T, H, I, E, k, bk.w13, bk.w13_sh,
                                 cfg.n_shared, cfg.I_shared, B.offsets, B.sorted_pair,
                                 B.tiles, B.n_tiles, B.tile_m, B.h, B.ws, B.ws_bytes, gflags)

    if fused:
        kname = "dec_route_gateup_kernel (route + sort + gate/up + SiLU*mul)"
    elif decode:
        kname = ("proj_m16_kernel<0> (gate/up + SiLU*mul)" if act == "a16" else
                 "proj_m16_kernel<0> (gate/up + SiLU*mul on the int8 x rows of the routing launch)")
    else:
        kname = ("proj_mfma8_kernel<0> (gate/up + SiLU*mul on the fp16 x copy of the routing launch)"
                 + (", prepacked weights" if dl.bank.prepacked else ""))
    n_k = len(banks) if decode else 4
    gk = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gk):
        for i in range(n_k):
            gateup(banks[i % len(banks)])
    gk.replay()
    k_reps = max(1, -(-args.steps // n_k))
    gu_ms = timed_loop(lambda i: gk.replay(), k_reps, torch) / n_k
    log(f"[bench] {cfg.name}: gate/up call {gu_ms * 1e3:.2f} us/launch")

    if decode:
        value = bytes_all / (ms * 1e-3) / 1e9
        unit = "GB/s"
        ach = bytes_w13 / (gu_ms * 1e-3) / 1e9
        # what one plain read of the same bytes reaches from HBM: the
        # gate/up call's bytes, and the step's bytes in a single read
        cyc = len(banks) * bytes_all
        c_gu = read_ceiling_at(torch, L, bytes_w13, cyc)
        c_step = read_ceiling_at(torch, L, bytes_all, cyc)
        log(f"[bench] {cfg.name}: plain read of {bytes_w13 / 1e6:.1f} MB {c_gu['achieved']:.0f} "
            f"GB/s, of {bytes_all / 1e6:.1f} MB {c_step['achieved']:.0f} GB/s")
        key = ("dec_route_gateup_kernel@" if fused else "gateup_call@") + cfg.name
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": measured_traffic(key),
                "kernel": kname, "algorithmic_bytes": bytes_w13,
                "ms_per_launch": gu_ms,
                "frac_of_measured_read_ceiling": ach / ceiling["achieved"] if ceiling else None,
                "read_ceiling_at_size": c_gu,
                "frac_of_read_ceiling_at_size": ach / c_gu["achieved"]}
        dtype = "bf16" if act == "a16" else "int8"
    else:
        value = flops / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
        ach = flops_gateup / (gu_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": F16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / F16_PEAK_TFLOPS,
                "traffic": measured_traffic(f"gateup_call@{cfg.name}"),
                "kernel": kname, "algorithmic_flops": flops_gateup,
                "ms_per_launch": gu_ms}
        dtype = "fp16"   # x and the dequantized weights enter the MFMAs as fp16

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] {cfg.name}: timing the CPU oracle")
        if decode:
            cpu = cpu_oracle_decode(layer, args.cpu_seconds, bytes_all / 1e9, hi)
        else:
            cpu = cpu_oracle_prefill(layer, args.cpu_prefill_experts, hi)
        log(f"[bench] {cfg.name}: CPU oracle {cpu['value']:.4g} {cpu['unit']}")

    rec = {
        "metric": METRIC, "value": value, "unit": unit, "ms_per_step": ms,
        "dtype": dtype,
        "config": {"workload": cfg.name, "T": T, "H": H, "E": E, "k": k, "I": I,
                   "n_shared": cfg.n_shared, "act": act, "experts_touched": n_touched,
                   "bytes_per_step": bytes_all, "flops_per_step": flops,
                   "bank_copies_rotated": len(banks), "path": args.path,
                   "weights": "prepacked" if dl.bank.prepacked else "canonical",
                   "timing": (f"HIP graphs of {G} steps over {G} weight copies, replayed in "
                              f"cycle order after {w_reps} warm-up replays"),
                   "ms_per_step_eager": ms_eager},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if decode:
        rec["step_read_ceiling"] = c_step
        rec["frac_of_step_read_ceiling"] = value / c_step["achieved"]
    del graphs, gk, banks, dl, B, layer
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=None,
                    help="one benchmark layer (0-4); default: the prefill headline "
                         "plus the three decode layers")
    ap.add_argument("--rotate-bytes", type=float, default=1.5e9)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="CPU oracle time per decode layer")
    ap.add_argument("--cpu-prefill-experts", type=int, default=12,
                    help="experts of the prefill layer in the CPU oracle's sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--canonical-weights", action="store_true",
                    help="prefill: run on the canonical code layout instead of the bank "
                         "re-tiled by moe_w4_prepack")
    ap.add_argument("--path", choices=["auto", "gemv", "mfma"], default="auto")
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

    import torch

    from packed_bit_grouped_amd import _lib as L

    torch.cuda.set_device(0)
    hi = host_info()
    ceiling = read_ceiling(torch, L, 2 << 30)
    log(f"[bench] HBM read ceiling: {ceiling['achieved']:.0f} GB/s over "
        f"{ceiling['bytes'] / 2**30:.0f} GiB")

    cids = [args.config] if args.config is not None else [HEADLINE, *SUBS]
    recs = [run_config(c, args, torch, L, hi, ceiling) for c in cids]
    head, subs = recs[0], recs[1:]
    line = {
        "metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded; int4/int2 experts quantized from N(0, 0.02))",
        "config": head["config"], "roofline": head["roofline"],
        "cpu_baseline": head["cpu_baseline"],
        "hbm_read_ceiling": ceiling,
    }
    for key in ("step_read_ceiling", "frac_of_step_read_ceiling"):
        if key in head:
            line[key] = head[key]
    if subs:
        line["sub_records"] = subs
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
