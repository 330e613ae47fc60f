"""Pins of the CPU oracle against things other than itself (no GPU).

Hand-worked values of the formats (tests/golden), textbook routines
(numpy's stable argsort / bincount / cumsum, scipy's softmax), invariants,
a pure-Python brute force, a dense dequantize-then-matmul SwiGLU FFN for
E = k = 1, closed forms for layers with a single non-zero code, and exact
scaling laws.  Each is chosen so that a plausible slip in the oracle (a
swapped nibble, gate/up swapped, a transposed weight, a dropped shared
term, a wrong tie-break, a non-stable grouping, truncation instead of
round-half-even) fails at least one test."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import brute
from synth import LAYERS, LayerConfig, make_layer, pack_codes, quantize_matrix
from synth.gen import Expert, Layer, QMat, bf16_bits_from_f32
from tests.minis import MINIS

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                   "format_handworked.json")))


# ------------------------------------------------------------ formats ----

def test_golden_int4_nibble_order():
    g = GOLD["int4_bytes"]
    codes = oracle.unpack_codes(np.array([g["bytes"]], np.uint8), 4, len(g["codes"]))
    assert codes[0].tolist() == g["codes"]


def test_golden_int2_order():
    g = GOLD["int2_bytes"]
    codes = oracle.unpack_codes(np.array([g["bytes"]], np.uint8), 2, len(g["codes"]))
    assert codes[0].tolist() == g["codes"]


def test_golden_bit_patterns():
    g = GOLD["bf16_bits"]
    v = oracle.decode_bf16(np.array(g["bits"], np.uint16))
    assert v.tolist() == g["values"]
    assert math.copysign(1.0, v[3]) == -1.0
    g = GOLD["fp16_bits"]
    assert oracle.decode_fp16(np.array(g["bits"], np.uint16)).tolist() == g["values"]


BF16_ROUND = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                         "bf16_rounding.json")))


def test_golden_bf16_rounding():
    """round_to_bf16 on hand-worked cases: ties to even (down and up), the
    carry into the exponent, sign symmetry, the smallest normal, subnormal
    ties, and the overflow of the halfway point above the largest finite
    value.  Each fixture input is checked to equal its stated sum of powers
    of two, and each expected value to equal its stated bit pattern."""
    from fractions import Fraction
    cases = BF16_ROUND["cases"]
    for c in cases:
        expr = c["in"].replace("^", "**").replace("2**", "Fraction(2)**")
        assert Fraction(c["v"]) == eval(expr, {"Fraction": Fraction}), c["in"]
        out = math.inf if c["out"] == "inf" else c["out"]
        b = c["bits"]
        e, f = (b >> 7) & 0xFF, b & 0x7F
        dec = (math.inf if e == 0xFF else
               math.ldexp(f, -133) if e == 0 else math.ldexp(128 + f, e - 134))
        assert math.copysign(dec, -1.0 if b >> 15 else 1.0) == out, c["in"]
    v = np.array([c["v"] for c in cases])
    want = np.array([math.inf if c["out"] == "inf" else c["out"] for c in cases])
    got = oracle.round_to_bf16(v)
    assert np.array_equal(got, want), [(c["in"], g) for c, g, w in zip(cases, got, want) if g != w]
    assert np.array_equal(oracle.round_to_bf16(-v), -want)


def test_decoders_match_hardware_conversions():
    # every fp16 pattern against numpy's own binary16, every bf16 pattern
    # against the float32 whose top half it is
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    fin16 = ((allb >> 10) & 0x1F) != 0x1F
    ref16 = allb[fin16].view(np.float16).astype(np.float64)
    assert np.array_equal(oracle.decode_fp16(allb[fin16]), ref16)
    finb = ((allb >> 7) & 0xFF) != 0xFF
    refb = (allb[finb].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(oracle.decode_bf16(allb[finb]), refb)


@pytest.mark.parametrize("bits", [4, 2])
def test_pack_unpack_round_trip_all_codes(bits):
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    rng = np.random.default_rng(7)
    codes = rng.integers(lo, hi + 1, size=(5, 64)).astype(np.int8)
    codes[0, : hi - lo + 1] = np.arange(lo, hi + 1)        # every code once
    got = oracle.unpack_codes(pack_codes(codes, bits), bits, 64)
    assert np.array_equal(got, codes)
    # and brute force's independent bit reader agrees
    packed = pack_codes(codes, bits)
    for n in range(5):
        assert [brute.code_at(packed[n], bits, c) for c in range(64)] == codes[n].tolist()


@pytest.mark.parametrize("bits,group", [(4, 32), (4, 128), (2, 64)])
def test_generator_quantization_error_bound(bits, group):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    w[3, :group] = 0.0
    codes, s16 = quantize_matrix(w, bits, group)
    qm = QMat(pack_codes(codes, bits), s16.view(np.uint16), bits, group, 16, 256)
    deq = oracle.dequantize(qm)
    s = np.repeat(s16.astype(np.float64), group, axis=1)
    err = np.abs(w.astype(np.float64) - deq)
    assert np.all(err <= s / 2 * (1 + 2.0 ** -10) + 1e-30)
    assert np.all(deq[3, :group] == 0)
    assert codes.min() >= -(1 << (bits - 1)) and codes.max() <= (1 << (bits - 1)) - 1


# ------------------------------------------------------------ routing ----

def test_golden_route():
    for case in GOLD["route"]:
        ids, w = oracle.route_topk(np.array([case["logits"]], np.float32), case["k"])
        assert ids[0].tolist() == case["ids"]
        assert np.allclose(w[0], case["w"], atol=1e-7, rtol=0)


def test_route_matches_stable_argsort_and_softmax():
    rng = np.random.default_rng(11)
    lg = rng.standard_normal((200, 37)).astype(np.float32)
    lg[:, 5] = lg[:, 9]                       # exact ties
    lg[::3, 20] = lg[::3, 2]
    lg[7, :] = 0.25
    for k in (1, 3, 8, 37):
        ids, w = oracle.route_topk(lg, k)
        ref = np.argsort(-lg.astype(np.float64), axis=1, kind="stable")[:, :k]
        assert np.array_equal(ids, ref)
        sel = np.take_along_axis(lg.astype(np.float64), ref, axis=1)
        assert np.allclose(w, softmax(sel, axis=1), rtol=1e-13, atol=0)
        assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-15 * k)


def test_route_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(12)
    lg = (rng.standard_normal((9, 6)) * 3).astype(np.float32)
    ids, w = oracle.route_topk(lg, 6)
    full = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(np.take_along_axis(full, ids, 1), w, rtol=1e-13)


def test_route_without_renormalisation():
    rng = np.random.default_rng(13)
    lg = rng.standard_normal((5, 10)).astype(np.float32)
    ids, w = oracle.route_topk(lg, 3, renormalize=0)
    full = softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(np.take_along_axis(full, ids, 1), w, rtol=1e-13)
    assert np.all(w.sum(1) < 1.0)


# ------------------------------------------------------------ grouping ---

def test_golden_permute():
    g = GOLD["permute"]
    p = oracle.permute(np.array(g["ids"]), g["E"], g["tile_m"])
    for key in ("counts", "offsets", "sorted_pair", "pair_pos", "tiles"):
        assert p[key].tolist() == g[key], key


@pytest.mark.parametrize("T,E,k,tile_m", [(1, 128, 8, 16), (12, 128, 8, 4),
                                          (333, 16, 4, 32), (4096, 256, 8, 64)])
def test_permute_matches_textbook_routines(T, E, k, tile_m):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    p = oracle.permute(ids, E, tile_m)
    flat = ids.ravel()
    assert np.array_equal(p["counts"], np.bincount(flat, minlength=E))
    assert np.array_equal(p["offsets"], np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(p["sorted_pair"], np.argsort(flat, kind="stable"))
    assert np.array_equal(p["sorted_pair"][p["pair_pos"]], np.arange(T * k))
    assert np.array_equal(p["pair_pos"][p["sorted_pair"]], np.arange(T * k))
    assert p["counts"].sum() == T * k
    assert np.all(np.diff(flat[p["sorted_pair"]]) >= 0)
    # tiles cover each sorted row once, never straddle an expert, <= tile_m rows
    cover = np.zeros(T * k, np.int64)
    for e, a, b in p["tiles"]:
        assert 0 < b - a <= tile_m
        assert p["offsets"][e] <= a and b <= p["offsets"][e + 1]
        cover[a:b] += 1
    assert np.all(cover == 1)
    assert len(p["tiles"]) == sum(-(-c // tile_m) for c in p["counts"])


# ------------------------------------------------------- A8 quantizer ----

def test_golden_a8_rows():
    for case in GOLD["a8_rows"]:
        q, s = oracle.quant_rows_a8(np.array([case["row"]], np.float32))
        assert q[0].tolist() == case["codes"]
        assert float(s[0]) == case["scale"]


def test_a8_quantizer_matches_brute_force():
    rng = np.random.default_rng(21)
    rows = (rng.standard_normal((40, 300)) * rng.uniform(0.01, 50, (40, 1))).astype(np.float32)
    rows[3] = 0
    rows[4, ::2] = 0
    q, s = oracle.quant_rows_a8(rows)
    for r in range(rows.shape[0]):
        bq, bs = brute.quant_row([float(v) for v in rows[r]])
        assert q[r].tolist() == bq
        assert float(s[r]) == bs


# ------------------------------------------------- whole layer vs loops ---

def _close(a, b, rel=1e-12):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() <= rel * scale


@pytest.mark.parametrize("name", list(MINIS))
def test_oracle_matches_brute_force(name):
    cfg = MINIS[name]
    layer = make_layer(cfg, seed=0)
    o = oracle.oracle_layer(layer)
    b = brute.layer_brute(layer)
    assert o["ids"].tolist() == b["ids"]
    assert np.allclose(o["w"], b["w"], rtol=1e-14, atol=0)
    for key in ("counts", "offsets", "sorted_pair", "pair_pos"):
        assert list(o[key]) == b[key], key
    if cfg.act == "a8":
        assert o["qx"].tolist() == [list(r) for r in b["qx"]]
        assert o["sx"].tolist() == list(b["sx"])
        for r, (q, s) in b["hq"].items():
            I = len(q)
            assert o["qh"][r, :I].tolist() == q
            assert float(o["sh"][r]) == s
    for r, hv in b["h"].items():
        assert _close(o["h"][r, :len(hv)], hv), r
    assert _close(o["out"], b["out"])


def test_config0_layer_shape_and_scale():
    layer = make_layer(LAYERS["tiny_w4a16"])
    o = oracle.oracle_layer(layer)
    assert o["out"].shape == (16, 256)
    assert o["ids"].shape == (16, 2)
    rms = np.sqrt(np.mean(o["out"] ** 2))
    assert 1e-3 < rms < 1.0


# --------------------------------------------------------- reductions ---

def _dense_swiglu(x, W13, W2):
    """An independent dense FFN: out = (silu(x W_g^T) * (x W_u^T)) W2^T."""
    I = W13.shape[0] // 2
    g = np.einsum("th,ih->ti", x, W13[:I])
    u = np.einsum("th,ih->ti", x, W13[I:])
    a = g / (1 + np.exp(-g)) * u
    return a, np.einsum("ti,hi->th", a, W2)


def test_single_expert_is_dense_w4_swiglu():
    cfg = MINIS["e1"]
    layer = make_layer(cfg)
    o = oracle.oracle_layer(layer)
    x = (layer.x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ex = layer.experts[0]

    def deq(qm):
        per = 8 // qm.bits
        raw = np.unpackbits(qm.codes[:, :, None], axis=2, bitorder="little")
        raw = raw.reshape(qm.N, qm.K // per, per, qm.bits)
        u = (raw * (1 << np.arange(qm.bits))).sum(-1).reshape(qm.N, qm.K)
        c = u - (u >= (1 << (qm.bits - 1))) * (1 << qm.bits)
        return c * np.repeat(qm.scales.view(np.float16).astype(np.float64), qm.group, 1)

    a, ref = _dense_swiglu(x, deq(ex.w13), deq(ex.w2))
    # the oracle rounds h to bf16 between the projections; compare the
    # intermediate before rounding exactly and the output within that rounding
    assert np.allclose(o["h_exact"][:, :cfg.I], a, rtol=1e-12, atol=1e-15)
    assert np.allclose(o["out"], ref, rtol=2 ** -7, atol=2 ** -8 * np.abs(ref).max())
    assert np.all(o["w"] == 1.0)


def _manual_layer(T, H, E, k, I, group, x, logits, experts, shared=(), act="a16"):
    cfg = LayerConfig("manual", 999, T=T, H=H, E=E, k=k, I=I, group=group,
                      act=act, n_shared=len(shared),
                      I_shared=(shared[0].w13.N // 2 if shared else 0))
    return Layer(cfg, 0, bf16_bits_from_f32(np.asarray(x, np.float32)),
                 np.zeros((H, E), np.float32), None,
                 np.asarray(logits, np.float32), list(experts), list(shared),
                 np.zeros(0, np.int64))


def _qmat(codes, scales, bits, group):
    codes = np.asarray(codes, np.int8)
    N, K = codes.shape
    s = np.asarray(scales, np.float16).reshape(N, K // group)
    return QMat(pack_codes(codes, bits), s.view(np.uint16), bits, group, N, K)


def test_single_nonzero_codes_closed_form():
    """Expert 1 of 2 is chosen; W13 has one gate code and one up code in
    row i0, W2 one code in column i0.  Only out[:, n0] is non-zero and it
    equals w * s2 * c2 * bf16(SiLU(s_g c_g x[kg]) * s_u c_u x[ku])."""
    T, H, I, G = 3, 64, 32, 32
    i0, kg, ku, n0 = 5, 40, 3, 17
    rng = np.random.default_rng(5)
    x = rng.standard_normal((T, H)).astype(np.float32)
    c13 = np.zeros((2 * I, H), np.int8)
    c13[i0, kg] = 3
    c13[I + i0, ku] = -2
    s13 = np.full((2 * I, H // G), 0.5)
    s13[i0, kg // G] = 0.25
    c2 = np.zeros((H, I), np.int8)
    c2[n0, i0] = 7
    s2 = np.full((H, I // G), 0.125)
    ex1 = Expert(_qmat(c13, s13, 4, G), _qmat(c2, s2, 4, G))
    ex0 = Expert(_qmat(np.zeros((2 * I, H)), np.ones((2 * I, H // G)), 4, G),
                 _qmat(np.zeros((H, I)), np.ones((H, I // G)), 4, G))
    logits = np.tile([0.0, 1.0], (T, 1))
    layer = _manual_layer(T, H, 2, 1, I, G, x, logits, [ex0, ex1])
    o = oracle.oracle_layer(layer)
    xb = (layer.x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for t in range(T):
        g = 0.25 * 3 * xb[t, kg]
        u = 0.5 * -2 * xb[t, ku]
        hv = brute.bf16_round(g / (1 + math.exp(-g)) * u)
        expect = np.zeros(H)
        expect[n0] = 0.125 * 7 * hv
        assert np.array_equal(o["out"][t], expect)


def test_zero_activations_give_zero_output():
    for name in ("c0", "c0_a8", "mixed_shared"):
        layer = make_layer(MINIS[name])
        layer.x_bf16[:] = 0
        o = oracle.oracle_layer(layer)
        assert np.all(o["out"] == 0)


def test_up_scales_times_power_of_two_scale_output_exactly():
    """Multiplying every up-row scale by 2 multiplies u, h (also after bf16
    rounding) and the output by exactly 2; multiplying the gate-row scales
    does not (SiLU is not homogeneous).  Fails if gate and up are swapped."""
    layer = make_layer(MINIS["c0"])
    base = oracle.oracle_layer(layer)["out"]
    I = layer.cfg.I
    for ex in layer.experts:
        s = ex.w13.scales.view(np.float16).copy()
        s[I:] *= np.float16(2)
        ex.w13.scales = s.view(np.uint16)
    assert np.array_equal(oracle.oracle_layer(layer)["out"], 2 * base)
    layer2 = make_layer(MINIS["c0"])
    for ex in layer2.experts:
        s = ex.w13.scales.view(np.float16).copy()
        s[:I] *= np.float16(2)
        ex.w13.scales = s.view(np.uint16)
    assert not np.allclose(oracle.oracle_layer(layer2)["out"], 2 * base)


def test_a8_codes_invariant_under_power_of_two_input_scaling():
    layer = make_layer(MINIS["c0_a8"])
    a = oracle.oracle_layer(layer, want_partials=True)
    x = (layer.x_bf16.astype(np.uint32) << 16).view(np.float32) * np.float32(4.0)
    layer.x_bf16 = bf16_bits_from_f32(x)
    b = oracle.oracle_layer(layer, want_partials=True)
    assert np.array_equal(a["qx"], b["qx"])
    assert np.array_equal(a["sx"] * 4, b["sx"])
    for key in a["partials1"]:
        assert np.array_equal(a["partials1"][key][1], b["partials1"][key][1])


def test_shared_expert_joins_with_weight_one():
    """The layer with a shared expert equals the routed-only layer plus the
    shared expert's own dense FFN output (weight 1.0, a reading)."""
    layer = make_layer(MINIS["mixed_shared"])
    full = oracle.oracle_layer(layer)["out"]
    routed = Layer(layer.cfg.replace(n_shared=0, I_shared=0), 0, layer.x_bf16,
                   layer.router_w, layer.bias, layer.logits, layer.experts, [],
                   layer.int2_experts)
    r_out = oracle.oracle_layer(routed)["out"]
    x = (layer.x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    sh = layer.shared[0]
    W13 = oracle.dequantize(sh.w13)
    W2 = oracle.dequantize(sh.w2)
    a, _ = _dense_swiglu(x, W13, W2)
    ref = r_out + oracle.round_to_bf16(a) @ W2.T
    assert np.allclose(full, ref, rtol=1e-12, atol=1e-15)


def test_shared_gate_is_the_sigmoid_of_the_gate_logit():
    """Sigmoid-gated shared experts: with every gate logit set to l the
    layer equals the routed-only layer (built without shared experts) plus
    sigmoid(l) times the shared experts' ungated contribution; sigmoid(0) =
    1/2, sigmoid(ln 3) = 3/4 and sigmoid(-ln 3) = 1/4 exactly, so a gate
    applied to the wrong terms or with the wrong sign fails."""
    import dataclasses
    layer = make_layer(MINIS["gated_shared"])
    cfg = layer.cfg
    assert layer.shared_gate_logits.shape == (cfg.T, cfg.n_shared)
    routed = Layer(cfg.replace(n_shared=0, I_shared=0, shared_gate=False), 0, layer.x_bf16,
                   layer.router_w, layer.bias, layer.logits, layer.experts, [],
                   layer.int2_experts)
    r_out = oracle.oracle_layer(routed)["out"]
    u_out = oracle.oracle_layer(dataclasses.replace(layer, shared_gate_logits=None))["out"]
    for lv, sig in ((0.0, 0.5), (math.log(3.0), 0.75), (-math.log(3.0), 0.25),
                    (2.5, 1.0 / (1.0 + math.exp(-2.5)))):
        gl = np.full((cfg.T, cfg.n_shared), lv)
        o = oracle.oracle_layer(dataclasses.replace(layer, shared_gate_logits=gl))["out"]
        assert np.allclose(o, r_out + sig * (u_out - r_out), rtol=1e-12, atol=1e-14), lv
    # the gate logits are the generator's fp32(x . w_gate), one per token and shared expert
    x = (layer.x_bf16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    want = np.array([[sum(x[t, h] * float(layer.shared_gate_w[s, h]) for h in range(cfg.H))
                      for s in range(cfg.n_shared)] for t in range(cfg.T)])
    assert np.allclose(layer.shared_gate_logits, want, rtol=1e-6, atol=1e-7)


def test_token_sample_path_matches_full_layer():
    for name in ("mixed_shared", "mixed_shared_a8", "c0"):
        layer = make_layer(MINIS[name])
        full = oracle.oracle_layer(layer)
        toks = [0, layer.cfg.T - 1, layer.cfg.T // 2]
        s = oracle.oracle_token_outputs(layer, toks)
        assert np.array_equal(s["ids"], full["ids"][toks])
        assert np.allclose(s["out"], full["out"][toks], rtol=1e-12, atol=1e-15)


def test_zipf_prior_skews_routing():
    """12 tokens with the Zipf(1.1) log-prior: a few experts take several
    tokens and most take none (the skew that layer is meant to have)."""
    layer = make_layer(LAYERS["specdecode_w4a16_t12"].replace(H=256), experts_only=[])
    ids, _ = oracle.route_topk(layer.logits, 8)
    counts = np.bincount(ids.ravel(), minlength=128)
    assert 12 <= (counts > 0).sum() <= 48
    assert counts.max() >= 6


# ---------------------------------------------------------------------------
# router logits (on-device scoring of the tokens)
# ---------------------------------------------------------------------------

def _bf16(a):
    return bf16_bits_from_f32(np.asarray(a, dtype=np.float32))


def test_router_logits_match_python_sums():
    rng = np.random.default_rng(11)
    T, H, E = 3, 37, 5
    xb = _bf16(rng.standard_normal((T, H)))
    w = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    bias = rng.standard_normal(E)
    lg = oracle.router_logits(xb, w, bias)
    xs = [[float(v) for v in row] for row in
          ((xb.astype(np.uint32) << 16).view(np.float32))]
    for t in range(T):
        for e in range(E):
            ref = math.fsum(xs[t][h] * float(w[h, e]) for h in range(H)) + float(bias[e])
            assert abs(lg[t, e] - ref) <= 1e-15 * (1 + abs(ref))


def test_router_logits_one_hot_token_gives_router_row():
    rng = np.random.default_rng(12)
    H, E = 64, 9
    w = (rng.standard_normal((H, E)) * 0.02).astype(np.float32)
    x = np.zeros((H, H), dtype=np.float32)
    x[np.arange(H), np.arange(H)] = 1.0
    lg = oracle.router_logits(_bf16(x), w)
    assert np.array_equal(lg, w.astype(np.float64))
    # a transposed operand or a dropped row would break this
    x2 = np.zeros((1, H), dtype=np.float32)
    x2[0, 5], x2[0, 40] = 2.0, -0.5
    assert np.array_equal(oracle.router_logits(_bf16(x2), w)[0],
                          2.0 * w[5].astype(np.float64) - 0.5 * w[40].astype(np.float64))


def test_router_logits_scale_exactly_with_the_input():
    rng = np.random.default_rng(13)
    xb = _bf16(rng.standard_normal((4, 128)))
    w = (rng.standard_normal((128, 16)) * 0.02).astype(np.float32)
    x2 = ((xb.astype(np.uint32) << 16).view(np.float32) * np.float32(4.0))
    assert np.array_equal(oracle.router_logits(_bf16(x2), w), 4.0 * oracle.router_logits(xb, w))


def test_router_logits_reproduce_the_benchmark_logits():
    """The generator stores fp32(x . W_r + prior) for every layer; the
    oracle's logits round to the same fp32 values."""
    for cfg in (LAYERS["tiny_w4a16"], LAYERS["specdecode_w4a16_t12"]):
        layer = make_layer(cfg)
        lg = oracle.router_logits(layer.x_bf16, layer.router_w, layer.bias)
        assert np.array_equal(lg.astype(np.float32), layer.logits)
