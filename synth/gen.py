"""Seeded synthetic MoE FFN layers.

Every array is drawn from its own counter-free numpy stream keyed by
``SeedSequence([seed, config key, stream, expert, matrix])`` so that an
expert can be regenerated alone and in any process.

Workload recipe (the five layer shapes, activation and weight
distributions, per-group fp16 scales, nibble order) is the one the
low-bit MoE FFN benchmark describes; where it leaves a detail open the
reading taken here is stated next to the code.

Stored format produced here (consumed by both the oracle and the GPU
library):

* activations ``x``: bf16 bit patterns, uint16 [T][H], row-major;
* router logits: float32 [T][E];
* a quantized matrix W [N][K] (K contiguous): ``codes`` uint8
  [N][K*bits/8] (int4: two codes per byte, the even-K code in the low
  nibble; int2: four codes per byte, the lowest K index in the lowest
  two bits; two's complement) and ``scales`` uint16 [N][K/group]
  holding fp16 bit patterns;
* each expert: ``w13`` = gate rows (0..I-1) then up rows (I..2I-1),
  shape [2I][H]; ``w2`` = down, shape [H][I].
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ProcessPoolExecutor
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

import multiprocessing as mp
import numpy as np

# stream ids of SeedSequence([seed, key, stream, expert, matrix])
_S_X, _S_ROUTER, _S_ZIPF, _S_INT2, _S_EXPERT, _S_SHGATE = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class LayerConfig:
    name: str
    key: int                 # seeds the streams; distinct per config
    T: int                   # tokens
    H: int                   # hidden size (K of gate/up, N of down)
    E: int                   # routed experts
    k: int                   # experts per token
    I: int                   # expert intermediate size
    act: str = "a16"         # "a16": bf16 activations; "a8": dynamic int8
    bits: int = 4            # bits of the regular experts
    group: int = 128         # K-group of the regular experts
    n_int2: int = 0          # experts stored as int2 instead (chosen by seed)
    group_int2: int = 64
    n_shared: int = 0        # always-on shared experts (weight 1.0)
    I_shared: int = 0
    zipf_s: float = 0.0      # 0: no router bias; else Zipf(s) log-prior bias
    shared_gate: bool = False   # shared experts gated by sigmoid(x . w_gate)
    renormalize: int = 1
    x_std: float = 1.0
    w_std: float = 0.02
    router_std: float = 0.02
    description: str = ""

    @property
    def P(self) -> int:
        return self.T * self.k

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five benchmark layers.  Readings: "N(0,0.02)" is a standard deviation
# of 0.02; the shared expert uses the routed experts' int4/G128 format; no
# seed is stated for the larger layers, so all use seed 0.
CONFIGS: Dict[int, LayerConfig] = {
    0: LayerConfig("tiny_w4a16", 0, T=16, H=256, E=8, k=2, I=128, group=32,
                   description="tiny W4A16 layer, group 32, oracle-sized"),
    1: LayerConfig("decode_w4a16_t1", 1, T=1, H=2048, E=128, k=8, I=768,
                   group=128, n_shared=1, I_shared=768,
                   description="single-token decode, 8 routed + 1 shared"),
    2: LayerConfig("specdecode_w4a16_t12", 2, T=12, H=2048, E=128, k=8, I=768,
                   group=128, n_shared=1, I_shared=768, zipf_s=1.1,
                   description="4 requests x 3 draft positions, Zipf-skewed"),
    3: LayerConfig("decode_w4a8_t64", 3, T=64, H=2048, E=128, k=8, I=768,
                   group=128, act="a8",
                   description="batched decode, int8 activations"),
    4: LayerConfig("prefill_mixed_t4096", 4, T=4096, H=4096, E=256, k=8,
                   I=1536, group=128, n_int2=64, group_int2=64,
                   description="prefill chunk, 192 int4/G128 + 64 int2/G64"),
}


# The same layers by name.
LAYERS: Dict[str, LayerConfig] = {c.name: c for c in CONFIGS.values()}


def config_by_id(cid: int) -> LayerConfig:
    return CONFIGS[cid]


def _rng(seed: int, key: int, stream: int, expert: int = 0,
         matrix: int = 0) -> np.random.Generator:
    return np.random.default_rng(
        np.random.SeedSequence([seed, key, stream, expert, matrix]))


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def quantize_matrix(w: np.ndarray, bits: int, group: int):
    """Symmetric per-group quantization of a float32 [N][K] matrix along K.

    scale = fp16(fp32(max|w_g|) / qmax) with qmax = 7 (int4) or 1 (int2),
    code = clamp(rint(w / fp32(scale)), -2^(bits-1), 2^(bits-1)-1), fp32
    division, round half to even; an all-zero group gets scale 0, codes 0.
    The int2 rule mirrors the int4 one (qmax = 2^(bits-1)-1) so that no code
    is ever clipped.
    Returns (codes int8 [N][K], scales fp16 [N][K/group]).
    """
    assert bits in (2, 4)
    N, K = w.shape
    assert K % group == 0
    qmax = np.float32(7.0 if bits == 4 else 1.0)
    lo, hi = (-8, 7) if bits == 4 else (-2, 1)
    g = np.ascontiguousarray(w, dtype=np.float32).reshape(N, K // group, group)
    amax = np.abs(g).max(axis=2)
    s16 = (amax / qmax).astype(np.float16)
    s32 = s16.astype(np.float32)
    safe = np.where(s32 == 0, np.float32(1.0), s32)
    q = np.rint(g / safe[:, :, None])
    q[s32 == 0] = 0
    np.clip(q, lo, hi, out=q)
    return q.astype(np.int8).reshape(N, K), s16


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """int8 codes [N][K] -> packed uint8 [N][K*bits/8] (see module doc)."""
    N, K = codes.shape
    u = (codes.astype(np.int16) & ((1 << bits) - 1)).astype(np.uint8)
    per = 8 // bits
    assert K % per == 0
    u = u.reshape(N, K // per, per)
    out = np.zeros((N, K // per), dtype=np.uint8)
    for j in range(per):
        out |= (u[:, :, j] << np.uint8(bits * j)).astype(np.uint8)
    return out


@dataclass
class QMat:
    """One quantized [N][K] matrix in the stored format."""
    codes: np.ndarray     # uint8 [N][K*bits/8]
    scales: np.ndarray    # uint16 [N][K/group] (fp16 bit patterns)
    bits: int
    group: int
    N: int
    K: int


@dataclass
class Expert:
    w13: QMat             # [2I][H]
    w2: QMat              # [H][I]


@dataclass
class Layer:
    cfg: LayerConfig
    seed: int
    x_bf16: np.ndarray           # uint16 [T][H]
    router_w: np.ndarray         # float32 [H][E]
    bias: Optional[np.ndarray]   # float64 [E] or None
    logits: np.ndarray           # float32 [T][E]
    experts: List[Expert]        # E routed experts
    shared: List[Expert]         # n_shared shared experts
    int2_experts: np.ndarray     # int64 sorted ids of the int2 experts
    # sigmoid-gated shared experts: gate weights fp32 [n_shared][H] and the
    # gate logits fp32 [T][n_shared] = fp32(x . w in fp64); None otherwise
    shared_gate_w: Optional[np.ndarray] = None
    shared_gate_logits: Optional[np.ndarray] = None

    def expert_bits(self) -> np.ndarray:
        return np.array([e.w13.bits for e in self.experts], dtype=np.int32)


def _quant_pack(w: np.ndarray, bits: int, group: int) -> QMat:
    N, K = w.shape
    codes, s16 = quantize_matrix(w, bits, group)
    return QMat(pack_codes(codes, bits), s16.view(np.uint16), bits, group, N, K)


def gen_expert(seed: int, key: int, e: int, H: int, I: int, bits: int,
               group: int, w_std: float, keep_float: bool = False):
    """Draw expert e's fp32 weights N(0, w_std) and quantize/pack them.

    Returns Expert (and, with keep_float, the fp32 matrices as well)."""
    sd = np.float32(w_std)
    w13 = _rng(seed, key, _S_EXPERT, e, 0).standard_normal(
        (2 * I, H), dtype=np.float32)
    w13 *= sd
    w2 = _rng(seed, key, _S_EXPERT, e, 1).standard_normal(
        (H, I), dtype=np.float32)
    w2 *= sd
    ex = Expert(_quant_pack(w13, bits, group), _quant_pack(w2, bits, group))
    if keep_float:
        return ex, w13, w2
    return ex


def _gen_expert_job(args):
    return gen_expert(*args)


def zipf_bias(E: int, s: float, rng: np.random.Generator) -> np.ndarray:
    """Zipf(s) log-prior per expert: bias_e = log(r_e^-s / sum_r r^-s).

    r_e is a seeded random permutation of the ranks 1..E.  Reading of "a
    Zipf(s)-distributed per-expert bias": the expert of rank r gets prior
    probability proportional to r^-s; its log is added to the logits."""
    ranks = rng.permutation(E) + 1
    r = np.arange(1, E + 1, dtype=np.float64)
    logz = math.log(float(np.sum(r ** (-s))))
    return -s * np.log(ranks.astype(np.float64)) - logz


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_layer(cfg: LayerConfig, seed: int = 0, workers: Optional[int] = None,
               experts_only: Optional[Sequence[int]] = None,
               cache_dir: Optional[str] = None) -> Layer:
    """Build the seeded synthetic layer for ``cfg``.

    experts_only: regenerate only these routed experts (others are None);
    used where a test needs a few experts of a large bank.
    cache_dir (or $MOE_SYNTH_CACHE): store/load the layer as an .npz so
    that several processes of one run share one generation.
    """
    cache_dir = cache_dir or os.environ.get("MOE_SYNTH_CACHE")
    if cache_dir and experts_only is None:
        path = os.path.join(cache_dir, f"{cfg.name}_key{cfg.key}_seed{seed}"
                            f"_{_cfg_hash(cfg)}.npz")
        if os.path.exists(path):
            return _load_layer(cfg, seed, path)
    T, H, E, k, I = cfg.T, cfg.H, cfg.E, cfg.k, cfg.I
    x32 = _rng(seed, cfg.key, _S_X).standard_normal((T, H), dtype=np.float32)
    x32 *= np.float32(cfg.x_std)
    x_bf16 = bf16_bits_from_f32(x32)
    x64 = (x_bf16.astype(np.uint32) << np.uint32(16)).view(np.float32)
    x64 = x64.astype(np.float64)
    router_w = _rng(seed, cfg.key, _S_ROUTER).standard_normal(
        (H, E), dtype=np.float32) * np.float32(cfg.router_std)
    bias = None
    acc = x64 @ router_w.astype(np.float64)
    if cfg.zipf_s:
        bias = zipf_bias(E, cfg.zipf_s, _rng(seed, cfg.key, _S_ZIPF))
        acc = acc + bias[None, :]
    logits = acc.astype(np.float32)

    if cfg.n_int2:
        int2 = np.sort(_rng(seed, cfg.key, _S_INT2).choice(
            E, cfg.n_int2, replace=False))
    else:
        int2 = np.zeros(0, dtype=np.int64)
    int2_set = set(int(i) for i in int2)

    wanted = range(E) if experts_only is None else sorted(set(experts_only))
    jobs = []
    for e in wanted:
        if e in int2_set:
            jobs.append((seed, cfg.key, e, H, I, 2, cfg.group_int2, cfg.w_std))
        else:
            jobs.append((seed, cfg.key, e, H, I, cfg.bits, cfg.group, cfg.w_std))
    for s in range(cfg.n_shared):
        jobs.append((seed, cfg.key, E + s, H, cfg.I_shared, cfg.bits,
                     cfg.group, cfg.w_std))
    total = sum(3 * j[3] * j[4] for j in jobs)
    nw = workers if workers is not None else _workers()
    if nw > 1 and total > 32_000_000 and len(jobs) > 1:
        ctx = mp.get_context("spawn")   # never fork a process that may hold GPU state
        with ProcessPoolExecutor(max_workers=min(nw, len(jobs)),
                                 mp_context=ctx) as ex:
            made = list(ex.map(_gen_expert_job, jobs, chunksize=1))
    else:
        made = [_gen_expert_job(j) for j in jobs]
    experts: List[Optional[Expert]] = [None] * E
    for e, ex in zip(wanted, made[:len(wanted)]):
        experts[e] = ex
    shared = made[len(wanted):]
    sg_w = sg_logits = None
    if cfg.shared_gate and cfg.n_shared:
        # one gate vector per shared expert, drawn like the router weights;
        # its logits are computed once here, as the router logits are
        sg_w = _rng(seed, cfg.key, _S_SHGATE).standard_normal(
            (cfg.n_shared, H), dtype=np.float32) * np.float32(cfg.router_std)
        sg_logits = (x64 @ sg_w.astype(np.float64).T).astype(np.float32)
    layer = Layer(cfg, seed, x_bf16, router_w, bias, logits, experts, shared,
                  int2, sg_w, sg_logits)
    if cache_dir and experts_only is None:
        os.makedirs(cache_dir, exist_ok=True)
        _save_layer(layer, path)
    return layer


def with_random_codes(layer: Layer, seed: int = 0) -> Layer:
    """The same layer with every packed code byte (routed and shared
    experts, both matrices) replaced by uniformly random bytes, scales
    kept.  Every bit pattern then occurs, including the codes the
    quantizer never emits (int4 -8, int2 -2)."""
    def rnd(qm: QMat, tag: int, i: int, m: int) -> QMat:
        rng = _rng(seed, layer.cfg.key, 100 + tag, i, m)
        codes = rng.integers(0, 256, size=qm.codes.shape, dtype=np.uint8)
        return QMat(codes, qm.scales.copy(), qm.bits, qm.group, qm.N, qm.K)

    experts = [Expert(rnd(ex.w13, 0, i, 0), rnd(ex.w2, 0, i, 1))
               for i, ex in enumerate(layer.experts)]
    shared = [Expert(rnd(ex.w13, 1, i, 0), rnd(ex.w2, 1, i, 1))
              for i, ex in enumerate(layer.shared)]
    return dataclasses.replace(layer, experts=experts, shared=shared)


def with_x_rows(layer: Layer, rows: Dict[int, np.ndarray]) -> Layer:
    """The same layer with token rows of x replaced: rows maps a token to
    float32 values [H] (stored as bf16, round to nearest even).  The router
    logits are kept as they are (they are an input of the layer)."""
    x = layer.x_bf16.copy()
    for t, v in rows.items():
        x[t] = bf16_bits_from_f32(np.asarray(v, dtype=np.float32).reshape(1, -1))[0]
    return dataclasses.replace(layer, x_bf16=x)


def _cfg_hash(cfg: LayerConfig) -> str:
    import hashlib
    return hashlib.sha1(repr(dataclasses.astuple(cfg)).encode()).hexdigest()[:10]


def _save_layer(layer: Layer, path: str) -> None:
    arrs = {"x_bf16": layer.x_bf16, "router_w": layer.router_w,
            "logits": layer.logits, "int2": layer.int2_experts}
    if layer.bias is not None:
        arrs["bias"] = layer.bias
    if layer.shared_gate_w is not None:
        arrs["shared_gate_w"] = layer.shared_gate_w
        arrs["shared_gate_logits"] = layer.shared_gate_logits
    for tag, lst in (("e", layer.experts), ("s", layer.shared)):
        for i, ex in enumerate(lst):
            for m in ("w13", "w2"):
                q = getattr(ex, m)
                arrs[f"{tag}{i}_{m}_codes"] = q.codes
                arrs[f"{tag}{i}_{m}_scales"] = q.scales
                arrs[f"{tag}{i}_{m}_meta"] = np.array([q.bits, q.group, q.N, q.K])
    tmp = path + ".tmp.npz"
    np.savez(tmp, **arrs)
    os.replace(tmp, path)


def _load_layer(cfg: LayerConfig, seed: int, path: str) -> Layer:
    z = np.load(path, allow_pickle=False)

    def qm(tag, i, m):
        b, g, n, kk = (int(v) for v in z[f"{tag}{i}_{m}_meta"])
        return QMat(z[f"{tag}{i}_{m}_codes"], z[f"{tag}{i}_{m}_scales"], b, g, n, kk)

    experts = [Expert(qm("e", i, "w13"), qm("e", i, "w2")) for i in range(cfg.E)]
    shared = [Expert(qm("s", i, "w13"), qm("s", i, "w2"))
              for i in range(cfg.n_shared)]
    bias = z["bias"] if "bias" in z.files else None
    sg = (z["shared_gate_w"], z["shared_gate_logits"]) if "shared_gate_w" in z.files else (None, None)
    return Layer(cfg, seed, z["x_bf16"], z["router_w"], bias, z["logits"],
                 experts, shared, z["int2"], *sg)
