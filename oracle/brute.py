"""Pure-Python brute force of the MoE FFN layer, for tiny inputs only.

Test infrastructure that pins the numpy oracle: per-token, per-expert
loops over Python ints and floats, its own bit decoding (integer
arithmetic on the stored patterns), its own selection (a linear scan), its
own grouping (nested loops) and its own fp32 emulation (an fp64 quotient
rounded once to fp32, which equals the correctly rounded fp32 quotient
because 53 >= 2*24 + 2).  It shares no helper with moe_oracle.
"""
from __future__ import annotations

import math
import struct


def _bits_to_float(u: int, exp_bits: int, frac_bits: int) -> float:
    bias = (1 << (exp_bits - 1)) - 1
    sign = -1.0 if (u >> (exp_bits + frac_bits)) & 1 else 1.0
    e = (u >> frac_bits) & ((1 << exp_bits) - 1)
    f = u & ((1 << frac_bits) - 1)
    if e == (1 << exp_bits) - 1:
        raise ValueError("inf/nan")
    if e == 0:
        return sign * f * 2.0 ** (1 - bias - frac_bits)
    return sign * ((1 << frac_bits) + f) * 2.0 ** (e - bias - frac_bits)


def bf16(u: int) -> float:
    return _bits_to_float(int(u), 8, 7)


def fp16(u: int) -> float:
    return _bits_to_float(int(u), 5, 10)


def f32(v: float) -> float:
    """Round a Python float to the nearest IEEE fp32 value (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", v))[0]


def code_at(row_bytes, bits: int, kk: int) -> int:
    per = 8 // bits
    byte = int(row_bytes[kk // per])
    c = (byte >> (bits * (kk % per))) & ((1 << bits) - 1)
    return c - (1 << bits) if c & (1 << (bits - 1)) else c


def bf16_round(v: float) -> float:
    if v == 0.0:
        return 0.0
    m, e = math.frexp(v)
    return math.ldexp(round(m * 256.0), e - 8)   # round(): half to even


def silu(g: float) -> float:
    if g < -700:
        return 0.0 * g
    return g / (1.0 + math.exp(-g))


def topk(logits_row, k: int, renormalize: int = 1):
    remaining = list(range(len(logits_row)))
    chosen = []
    for _ in range(k):
        best = remaining[0]
        for e in remaining[1:]:
            if logits_row[e] > logits_row[best]:
                best = e                   # strict: earlier index wins ties
        chosen.append(best)
        remaining.remove(best)
    top = float(logits_row[chosen[0]])
    ex = [math.exp(float(logits_row[e]) - top) for e in chosen]
    if renormalize:
        den = math.fsum(ex)
    else:
        den = math.fsum(math.exp(float(v) - top) for v in logits_row)
    return chosen, [v / den for v in ex]


def group_pairs(ids, E: int):
    flat = [int(e) for row in ids for e in row]
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    sorted_pair = []
    for e in range(E):
        for p, pe in enumerate(flat):
            if pe == e:
                sorted_pair.append(p)
    pair_pos = [0] * len(flat)
    for r, p in enumerate(sorted_pair):
        pair_pos[p] = r
    return counts, offsets, sorted_pair, pair_pos


def quant_row(vals):
    """Per-row int8 quantization with fp32 semantics (see module doc)."""
    vals = [f32(v) for v in vals]
    a = max((abs(v) for v in vals), default=0.0)
    if a == 0.0:
        return [0] * len(vals), 0.0
    s = f32(a / 127.0)
    q = []
    for v in vals:
        r = round(f32(v / s))          # half to even
        q.append(max(-127, min(127, r)))
    return q, s


def _expert_list(layer):
    return list(layer.experts) + list(layer.shared)


def layer_brute(layer, act=None):
    """Whole layer by loops.  Returns a dict like the oracle's (lists)."""
    cfg = layer.cfg
    act = act or cfg.act
    T, H, E, k = cfg.T, cfg.H, cfg.E, cfg.k
    x = [[bf16(layer.x_bf16[t][c]) for c in range(H)] for t in range(T)]
    ids, ws = [], []
    for t in range(T):
        c, w = topk([float(v) for v in layer.logits[t]], k, cfg.renormalize)
        ids.append(c)
        ws.append(w)
    counts, offsets, sorted_pair, pair_pos = group_pairs(ids, E)
    P = T * k
    experts = _expert_list(layer)
    # (row, expert index, token) for every h / y row
    plan = [(r, ids[p // k][p % k], p // k) for r, p in enumerate(sorted_pair)]
    plan += [(P + s * T + t, E + s, t) for s in range(cfg.n_shared) for t in range(T)]
    h, y = {}, {}
    qx = sx = None
    if act == "a8":
        qx, sx = zip(*[quant_row(x[t]) for t in range(T)])
    hq = {}
    mats = {}

    def mat(e):
        """Expert e decoded once: per matrix its codes, scales and values."""
        if e not in mats:
            ex = experts[e]
            d = {}
            for name in ("w13", "w2"):
                qm = getattr(ex, name)
                codes = [[code_at(qm.codes[n], qm.bits, c) for c in range(qm.K)]
                         for n in range(qm.N)]
                scl = [[fp16(v) for v in qm.scales[n]] for n in range(qm.N)]
                vals = [[codes[n][c] * scl[n][c // qm.group] for c in range(qm.K)]
                        for n in range(qm.N)]
                d[name] = (codes, scl, vals, qm.group)
            mats[e] = d
        return mats[e]

    def a8_dot(qrow, s_row, codes, scl, group, n):
        tot = 0.0
        for c0 in range(0, len(qrow), group):
            part = 0
            for c in range(c0, c0 + group):
                part += qrow[c] * codes[n][c]
            tot += scl[n][c0 // group] * part
        return s_row * tot

    for r, e, t in plan:
        m = mat(e)
        c13, s13, v13, g13 = m["w13"]
        c2, s2, v2, g2 = m["w2"]
        I = len(v13) // 2
        hrow = []
        for i in range(I):
            if act == "a16":
                g = math.fsum(x[t][c] * v13[i][c] for c in range(H))
                u = math.fsum(x[t][c] * v13[I + i][c] for c in range(H))
            else:
                g = a8_dot(qx[t], sx[t], c13, s13, g13, i)
                u = a8_dot(qx[t], sx[t], c13, s13, g13, I + i)
            hrow.append(silu(g) * u)
        hv = [bf16_round(v) for v in hrow] if act == "a16" else hrow
        h[r] = hv
        if act == "a8":
            hq[r] = quant_row(hv)
        yrow = []
        for n in range(H):
            if act == "a16":
                yrow.append(math.fsum(hv[i] * v2[n][i] for i in range(I)))
            else:
                q, s = hq[r]
                yrow.append(a8_dot(q, s, c2, s2, g2, n))
        y[r] = yrow
    # shared experts: weight 1, or sigmoid of the token's gate logit
    sgl = getattr(layer, "shared_gate_logits", None)
    gate = [[1.0 if sgl is None else 1.0 / (1.0 + math.exp(-float(sgl[t][s])))
             for s in range(cfg.n_shared)] for t in range(T)]
    out = []
    for t in range(T):
        row = []
        for n in range(H):
            terms = [ws[t][j] * y[pair_pos[t * k + j]][n] for j in range(k)]
            terms += [gate[t][s] * y[P + s * T + t][n] for s in range(cfg.n_shared)]
            row.append(math.fsum(terms))
        out.append(row)
    return {"ids": ids, "w": ws, "counts": counts, "offsets": offsets,
            "sorted_pair": sorted_pair, "pair_pos": pair_pos, "h": h, "y": y,
            "out": out, "qx": qx, "sx": sx, "hq": hq}
