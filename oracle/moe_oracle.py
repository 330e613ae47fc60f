"""Plain fp64 CPU oracle of the low-bit MoE FFN layer (test infrastructure).

Source of the method: the build log "Two 96 GB Ascend cards run Qwen3.8
Flash-Next" (ai-pulse-lab), section "Keep low-bit weights packed, do the
work on the NPU": the first working W4 path dequantized the packed expert
weights eagerly and then ran an ordinary matmul; the production path routes
tokens to experts on the device and runs grouped expert projections with
fused gate/up handling straight from packed weights.  This module is that
eager form written out in fp64: decode every stored value exactly, route,
group, then dot products.  The layer format it decodes (softmax top-k
gating renormalised over the chosen experts, symmetric int4 codes in
[-8, 7] with one fp16 scale per K-group, two codes per byte with the even
K index in the low nibble, int2 in [-2, 1] four per byte, SiLU(gate)*up,
weighted combine of the k expert outputs) is the layer definition of the
benchmark these pages motivate; where that definition is silent the
reading used is stated in the function that applies it.

Nothing here is shared with the GPU library.  Only tests, the smoke check
and the CPU-baseline leg of the benchmark may import it.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

__all__ = [
    "decode_bf16", "decode_fp16", "unpack_codes", "dequantize",
    "router_logits", "route_topk", "permute", "quant_rows_a8", "silu", "round_to_bf16",
    "x_float", "expert_rows", "gateup_a16", "gateup_a8", "down_a16",
    "down_a8", "a8_group_partials", "shared_weights", "combine", "oracle_layer",
    "oracle_token_outputs", "touched_experts",
]


# --------------------------------------------------------------------------
# exact decoding of the stored formats
# --------------------------------------------------------------------------

def decode_bf16(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values.

    bf16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits; the
    value is (-1)^s * 2^(e-127) * (1 + f/128) for 0 < e < 255 and
    (-1)^s * 2^-126 * f/128 for e = 0.  Inf/NaN are rejected."""
    b = np.asarray(bits, dtype=np.int64)
    s = (b >> 15) & 1
    e = (b >> 7) & 0xFF
    f = b & 0x7F
    if np.any(e == 0xFF):
        raise ValueError("bf16 input holds inf or NaN")
    mag = np.where(e == 0, np.ldexp(f / 128.0, -126),
                   np.ldexp(1.0 + f / 128.0, (e - 127).astype(np.int64)))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def decode_fp16(bits) -> np.ndarray:
    """IEEE binary16 bit patterns (uint16) -> exact float64 values.

    1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; subnormals
    are 2^-14 * f/1024.  Inf/NaN are rejected."""
    b = np.asarray(bits, dtype=np.int64)
    s = (b >> 15) & 1
    e = (b >> 10) & 0x1F
    f = b & 0x3FF
    if np.any(e == 0x1F):
        raise ValueError("fp16 input holds inf or NaN")
    mag = np.where(e == 0, np.ldexp(f / 1024.0, -14),
                   np.ldexp(1.0 + f / 1024.0, (e - 15).astype(np.int64)))
    return np.where(s == 1, -mag, mag).astype(np.float64)


def unpack_codes(packed, bits: int, K: int) -> np.ndarray:
    """Packed uint8 [N][K*bits/8] -> signed integer codes int64 [N][K].

    int4: byte j of a row holds K index 2j in its low nibble and 2j+1 in
    its high nibble.  int2: byte j holds K indices 4j..4j+3, the lowest
    index in the lowest two bits.  Codes are two's complement: a nibble
    n >= 8 means n - 16; a 2-bit code c >= 2 means c - 4."""
    p = np.asarray(packed, dtype=np.int64)
    if p.ndim == 1:
        p = p[None, :]
    N = p.shape[0]
    per = 8 // bits
    if p.shape[1] * per != K:
        raise ValueError("packed width does not match K")
    base = 1 << bits
    fields = []
    rest = p.copy()
    for _ in range(per):             # peel fields from the least significant bits
        fields.append(rest % base)
        rest = rest // base
    u = np.stack(fields, axis=2).reshape(N, K)
    return np.where(u >= base // 2, u - base, u)


def dequantize(qm) -> np.ndarray:
    """Quantized matrix -> float64 [N][K] with w[n][k] = code[n][k] * scale[n][k // G].

    Exact in fp64 (a small integer times an fp16 value)."""
    codes = unpack_codes(qm.codes, qm.bits, qm.K).astype(np.float64)
    if qm.scales.shape != (qm.N, qm.K // qm.group):
        raise ValueError("scale table shape does not match N, K / group")
    s = decode_fp16(qm.scales)
    return codes * np.repeat(s, qm.group, axis=1)


def x_float(x_bf16) -> np.ndarray:
    """Token activations as exact float64."""
    return decode_bf16(x_bf16)


# --------------------------------------------------------------------------
# routing (pages: tokens are routed to experts on the device; routing was
# moved out of Python -- sections "Keep low-bit weights packed ..." and
# "Remove sync and launch overhead from the token loop")
# --------------------------------------------------------------------------

def router_logits(x_bf16, router_w, bias=None) -> np.ndarray:
    """Router logits of every token: the dot product of the token's
    activations with each expert's router column, plus an optional
    per-expert additive prior, in float64 (pages: tokens are scored and
    routed on the device -- section "Keep low-bit weights packed, do the
    work on the NPU").

    x_bf16 uint16 [T][H] (bf16 bit patterns), router_w float32 [H][E],
    bias float [E] or None.  Every input value is decoded exactly; the
    result is the exact sum up to float64 rounding.  Returns float64 [T][E].
    """
    x = decode_bf16(x_bf16)
    w = np.asarray(router_w, dtype=np.float32).astype(np.float64)
    if x.ndim != 2 or w.ndim != 2 or x.shape[1] != w.shape[0]:
        raise ValueError("need x [T][H] and router_w [H][E]")
    lg = x @ w
    if bias is not None:
        lg = lg + np.asarray(bias, dtype=np.float64)[None, :]
    return lg


def route_topk(logits, k: int, renormalize: int = 1):
    """Top-k softmax gating.

    For each token the k experts with the largest logits, in descending
    logit order, ties broken towards the lower expert index (the pages do
    not fix the order; this reading makes the result unique).  Weights are
    the softmax over all E logits restricted to the chosen k and, with
    renormalize=1, divided by their sum -- equal to a softmax over the k
    chosen logits.  With renormalize=0 they are the plain softmax values.
    Computed in float64 with the maximum subtracted.

    Returns ids int32 [T][k], w float64 [T][k]."""
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-lg[t, e], e))[:k]
        ids[t] = order
        m = lg[t, order[0]]
        ex = np.exp(lg[t, order] - m)
        denom = ex.sum() if renormalize else np.exp(lg[t] - m).sum()
        w[t] = ex / denom
    return ids, w


def permute(ids, E: int, tile_m: int):
    """Group the (token, expert) pairs by expert.

    Pair p = t*k + j is routed to expert ids[t][j].  counts[e] is the
    number of pairs routed to e; offsets is its exclusive prefix sum
    (length E+1); sorted_pair lists, for e = 0, 1, ..., E-1 in turn, the
    pairs routed to e in increasing p (a stable grouping: token-major
    within an expert); pair_pos is the inverse (pair_pos[sorted_pair[r]]
    = r).  tiles lists, per expert in order, consecutive row ranges of at
    most tile_m sorted rows: (expert, first row, end row).

    Returns a dict of int32 arrays."""
    flat = np.asarray(ids, dtype=np.int64).ravel()
    P = flat.size
    if np.any((flat < 0) | (flat >= E)):
        raise ValueError("expert id out of range")
    groups = [np.nonzero(flat == e)[0] for e in range(E)]
    counts = np.array([g.size for g in groups], dtype=np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    run = 0
    for e in range(E):
        offsets[e] = run
        run += counts[e]
    offsets[E] = run
    sorted_pair = (np.concatenate(groups) if P else np.zeros(0)).astype(np.int32)
    pair_pos = np.empty(P, dtype=np.int32)
    pair_pos[sorted_pair] = np.arange(P, dtype=np.int32)
    tiles = []
    for e in range(E):
        for r0 in range(0, int(counts[e]), tile_m):
            tiles.append((e, offsets[e] + r0,
                          offsets[e] + min(r0 + tile_m, int(counts[e]))))
    tiles = np.array(tiles, dtype=np.int32).reshape(-1, 3)
    return {"counts": counts, "offsets": offsets, "sorted_pair": sorted_pair,
            "pair_pos": pair_pos, "tiles": tiles}


# --------------------------------------------------------------------------
# dynamic int8 row quantization (the dedicated W4A8 execution of section
# "Keep low-bit weights packed ..."; rule: scale = max|row| / 127)
# --------------------------------------------------------------------------

def quant_rows_a8(rows):
    """Per-row symmetric int8 quantization, fixed bit-for-bit in IEEE fp32.

    a = max|row| (exact); s = fp32(a) / 127 (one correctly rounded fp32
    division); q = clamp(rint(row / s), -127, 127) with the division in
    fp32 and rint rounding half to even.  A zero row gets s = 0, q = 0.
    Returns q int8 [R][C], s float32 [R]."""
    r = np.asarray(rows, dtype=np.float32)
    if r.ndim == 1:
        r = r[None, :]
    a = np.abs(r).max(axis=1) if r.shape[1] else np.zeros(r.shape[0], np.float32)
    s = (a.astype(np.float32) / np.float32(127.0)).astype(np.float32)
    q = np.zeros(r.shape, dtype=np.int8)
    nz = a > 0
    if np.any(nz):
        quot = (r[nz] / s[nz, None]).astype(np.float32)
        q[nz] = np.clip(np.rint(quot), -127, 127).astype(np.int8)
    s = np.where(nz, s, np.float32(0.0)).astype(np.float32)
    return q, s


# --------------------------------------------------------------------------
# expert projections
# --------------------------------------------------------------------------

def silu(g):
    """SiLU(g) = g / (1 + exp(-g)), float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def round_to_bf16(v) -> np.ndarray:
    """float64 -> nearest bf16 value, ties to even, returned as float64.

    bf16 keeps 8 significant bits for normal values (|v| >= 2^-126), so the
    spacing of representable values around v = m * 2^e (0.5 <= |m| < 1) is
    2^(e - 8); below 2^-126 the subnormals are spaced 2^-133 apart.  v is
    divided by that spacing (exact: a power of two), rounded half to even
    and scaled back; a result of magnitude 2^128 or more is infinite.
    Used for the A16 intermediate h: with 16-bit activations the down
    projection consumes h in bf16 (a reading; the unrounded variant is
    available as h_exact)."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                     # v = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e, -125) - 8            # log2 of the spacing at v
    r = np.ldexp(np.rint(np.ldexp(v, -q)), q)
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)


def expert_rows(perm, E: int, T: int, n_shared: int):
    """Row bookkeeping shared by the projections.

    Rows 0..P-1 of h / y are the sorted pairs (row r belongs to expert e
    when offsets[e] <= r < offsets[e+1] and to token sorted_pair[r] // k).
    Rows P + s*T + t belong to shared expert s and token t.
    Yields (expert index e, rows array, shared index s or None, tokens
    array); routed experts yield the sorted pair ids in place of tokens."""
    off = perm["offsets"]
    sp = perm["sorted_pair"]
    P = int(off[E])
    for e in range(E):
        r = np.arange(off[e], off[e + 1])
        if r.size:
            yield e, r, None, sp[r]
    for s in range(n_shared):
        yield E + s, P + s * T + np.arange(T), s, np.arange(T)


def gateup_a16(layer, perm, tokens_of_rows=None):
    """A16 gate/up with fused SiLU*mul.

    For row r (expert e, token t): g_i = x_t . deq(W13_e)[i],
    u_i = x_t . deq(W13_e)[I + i], h = SiLU(g) * u, all in float64, then
    h rounded to bf16 (the down projection's 16-bit input).
    Returns (h_bf16_values, h_exact) float64 [R][I]."""
    cfg = layer.cfg
    k, E, T = cfg.k, cfg.E, cfg.T
    x = x_float(layer.x_bf16)
    P = int(perm["offsets"][E])
    R = P + cfg.n_shared * T
    I_max = max([cfg.I] + [cfg.I_shared] * (cfg.n_shared > 0))
    h = np.zeros((R, I_max))
    sp = perm["sorted_pair"]
    for e, rows, s, toks in expert_rows(perm, E, T, cfg.n_shared):
        ex = layer.experts[e] if s is None else layer.shared[s]
        toks = sp[rows] // k if s is None else toks
        W = dequantize(ex.w13)
        I = W.shape[0] // 2
        X = x[toks]
        g = X @ W[:I].T
        u = X @ W[I:].T
        h[rows, :I] = silu(g) * u
    return round_to_bf16(h), h


def a8_group_partials(q_rows, w_codes, group: int) -> np.ndarray:
    """Per-group integer partial sums of an int8 x int-code product.

    q_rows int [R][K], w_codes int [N][K] -> int64 [R][N][K/group] with
    P[r][n][c] = sum over K in group c of q_rows[r][K] * w_codes[n][K].
    Each product is an integer with |P| <= 127*8*group < 2^53, so the
    float64 matmul used for the sum is exact in any summation order."""
    q = np.asarray(q_rows, dtype=np.float64)
    w = np.asarray(w_codes, dtype=np.float64)
    R, K = q.shape
    N = w.shape[0]
    out = np.empty((R, N, K // group), dtype=np.int64)
    for c in range(K // group):
        sl = slice(c * group, (c + 1) * group)
        out[:, :, c] = np.rint(q[:, sl] @ w[:, sl].T).astype(np.int64)
    return out


def _a8_project(q_rows, s_rows, qm):
    """y[r][n] = s_row[r] * sum_c scale[n][c] * P[r][n][c], float64."""
    codes = unpack_codes(qm.codes, qm.bits, qm.K)
    Pg = a8_group_partials(q_rows, codes, qm.group)
    sw = decode_fp16(qm.scales)                      # [N][K/G]
    acc = np.einsum("rnc,nc->rn", Pg.astype(np.float64), sw)
    return acc * np.asarray(s_rows, dtype=np.float64)[:, None], Pg


def gateup_a8(layer, perm, want_partials: bool = False):
    """A8 gate/up.

    x_t is quantized per token with quant_rows_a8 (x is bf16, exact in
    fp32).  Per row r (expert e, token t) and output i: integer per-group
    partials P = sum_{K in group} qx[t][K] * code[i][K]; then
    g = s_x[t] * sum_groups scale[i][group] * P in float64 (same for u),
    h = SiLU(g) * u in float64.  h is handed to the down projection as
    fp32 and quantized per row (the int8 activation of the second GEMM).
    Returns dict: qx, sx, h (float64), h32, qh, sh and optionally the
    partials per expert."""
    cfg = layer.cfg
    k, E, T = cfg.k, cfg.E, cfg.T
    x32 = x_float(layer.x_bf16).astype(np.float32)
    qx, sx = quant_rows_a8(x32)
    P = int(perm["offsets"][E])
    R = P + cfg.n_shared * T
    I_max = max([cfg.I] + [cfg.I_shared] * (cfg.n_shared > 0))
    h = np.zeros((R, I_max))
    parts = {}
    sp = perm["sorted_pair"]
    for e, rows, s, toks in expert_rows(perm, E, T, cfg.n_shared):
        ex = layer.experts[e] if s is None else layer.shared[s]
        toks = sp[rows] // k if s is None else toks
        gu, Pg = _a8_project(qx[toks], sx[toks], ex.w13)
        I = gu.shape[1] // 2
        h[rows, :I] = silu(gu[:, :I]) * gu[:, I:]
        if want_partials:
            parts[(e, s)] = (rows, Pg)
    h32 = h.astype(np.float32)
    qh, sh = quant_rows_a8(h32)
    out = {"qx": qx, "sx": sx, "h": h, "h32": h32, "qh": qh, "sh": sh}
    if want_partials:
        out["partials"] = parts
    return out


def down_a16(layer, perm, h_vals):
    """y[r][n] = h[r] . deq(W2_e)[n] in float64 (h as given, e.g. bf16 values)."""
    cfg = layer.cfg
    E, T = cfg.E, cfg.T
    R = h_vals.shape[0]
    y = np.zeros((R, cfg.H))
    for e, rows, s, toks in expert_rows(perm, E, T, cfg.n_shared):
        ex = layer.experts[e] if s is None else layer.shared[s]
        W = dequantize(ex.w2)
        I = W.shape[1]
        y[rows] = h_vals[rows, :I] @ W.T
    return y


def down_a8(layer, perm, qh, sh, want_partials: bool = False):
    """A8 down projection from given int8 h codes and fp32 row scales:
    y[r][n] = s_h[r] * sum_groups scale[n][group] * P, P the integer
    per-group partials of qh[r] with W2_e's codes."""
    cfg = layer.cfg
    E, T = cfg.E, cfg.T
    R = qh.shape[0]
    y = np.zeros((R, cfg.H))
    parts = {}
    for e, rows, s, toks in expert_rows(perm, E, T, cfg.n_shared):
        ex = layer.experts[e] if s is None else layer.shared[s]
        I = ex.w2.K
        yy, Pg = _a8_project(qh[rows, :I], sh[rows], ex.w2)
        y[rows] = yy
        if want_partials:
            parts[(e, s)] = (rows, Pg)
    return (y, parts) if want_partials else y


def shared_weights(layer) -> np.ndarray:
    """Weight of shared expert s for token t, float64 [T][n_shared].

    A shared expert is always on and sits outside the renormalised top-k
    gate.  Without gate logits it joins with weight 1.0 (a reading: nothing
    fixes a shared-expert gate); with per-token gate logits l (the layer's
    sigmoid-gated variant) its weight is sigmoid(l) = 1 / (1 + exp(-l))."""
    cfg = layer.cfg
    lg = getattr(layer, "shared_gate_logits", None)
    if lg is None:
        return np.ones((cfg.T, cfg.n_shared))
    lg = np.asarray(lg, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-lg))


def combine(layer, perm, w, y):
    """out[t] = sum_j w[t][j] * y[row of pair t*k+j] + sum_s g[t][s] * y[P + s*T + t]
    with g the shared-expert weights (shared_weights).  float64, unrounded."""
    cfg = layer.cfg
    T, k, E = cfg.T, cfg.k, cfg.E
    P = int(perm["offsets"][E])
    out = np.zeros((T, cfg.H))
    pos = perm["pair_pos"]
    g = shared_weights(layer)
    for t in range(T):
        for j in range(k):
            out[t] += w[t, j] * y[pos[t * k + j]]
        for s in range(cfg.n_shared):
            out[t] += g[t, s] * y[P + s * T + t]
    return out


def oracle_layer(layer, act: Optional[str] = None, tile_m: int = 16,
                 want_partials: bool = False) -> Dict[str, np.ndarray]:
    """The whole layer: route -> permute -> gate/up (+SiLU*mul) -> down ->
    combine, for the activation mode ``act`` ("a16" or "a8", default the
    layer's own)."""
    cfg = layer.cfg
    act = act or cfg.act
    ids, w = route_topk(layer.logits, cfg.k, cfg.renormalize)
    perm = permute(ids, cfg.E, tile_m)
    res = {"ids": ids, "w": w, **perm}
    if act == "a16":
        h, h_exact = gateup_a16(layer, perm)
        y = down_a16(layer, perm, h)
        res.update(h=h, h_exact=h_exact, y=y)
    elif act == "a8":
        g = gateup_a8(layer, perm, want_partials)
        if want_partials:
            y, p2 = down_a8(layer, perm, g["qh"], g["sh"], True)
            res["partials2"] = p2
        else:
            y = down_a8(layer, perm, g["qh"], g["sh"])
        res.update({kk: v for kk, v in g.items() if kk != "partials"})
        if want_partials:
            res["partials1"] = g["partials"]
        res["y"] = y
    else:
        raise ValueError(act)
    res["out"] = combine(layer, perm, w, y)
    return res


def touched_experts(ids) -> np.ndarray:
    """Distinct routed experts that receive at least one token."""
    return np.unique(np.asarray(ids).ravel())


def oracle_token_outputs(layer, tokens: Sequence[int], act: Optional[str] = None,
                         deq_cache: Optional[dict] = None):
    """Layer outputs of selected tokens only (each token's output depends on
    that token alone), for checking large layers on a sample.  Same
    definitions as oracle_layer; A8 rows are quantized from this token's
    own h, as in the full layer.
    Returns dict: ids [n][k], w [n][k], h rows per (token, slot), out [n][H]."""
    cfg = layer.cfg
    act = act or cfg.act
    tokens = list(tokens)
    ids_all, w_all = route_topk(layer.logits[tokens], cfg.k, cfg.renormalize)
    x = x_float(layer.x_bf16)
    gsh = shared_weights(layer)
    cache = {} if deq_cache is None else deq_cache

    def deq(key, qm):
        if key not in cache:
            cache[key] = dequantize(qm)
        return cache[key]

    out = np.zeros((len(tokens), cfg.H))
    hs = {}
    for n, t in enumerate(tokens):
        plan = [(int(ids_all[n, j]), None, w_all[n, j]) for j in range(cfg.k)]
        plan += [(cfg.E + s, s, gsh[t, s]) for s in range(cfg.n_shared)]
        for slot, (e, s, wt) in enumerate(plan):
            ex = layer.experts[e] if s is None else layer.shared[s]
            if act == "a16":
                W13 = deq(("w13", e), ex.w13)
                I = W13.shape[0] // 2
                g = W13[:I] @ x[t]
                u = W13[I:] @ x[t]
                hv = round_to_bf16(silu(g) * u)
                y = deq(("w2", e), ex.w2) @ hv
            else:
                qx, sx = quant_rows_a8(x[t][None, :].astype(np.float32))
                gu, _ = _a8_project(qx, sx, ex.w13)
                I = gu.shape[1] // 2
                hv = silu(gu[0, :I]) * gu[0, I:]
                qh, sh = quant_rows_a8(hv.astype(np.float32)[None, :])
                y, _ = _a8_project(qh, sh, ex.w2)
                y = y[0]
            hs[(t, slot)] = hv
            out[n] += wt * y
    return {"ids": ids_all, "w": w_all, "h": hs, "out": out}
