"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer stages (routing ids, counts, offsets, permutation, tiles, A8 codes
and int32 per-group partials) must match bit for bit; float outputs must
have rel-L2 <= 5e-3 and max-abs <= 2e-2 * rms(oracle).  Sizes: the small
layers the oracle finishes in seconds (several tiles, ragged tails, int2
and int4 experts, shared experts), the decode layers at full size, and the
prefill layer at full size on a sample of tokens.
"""
import os
import sys

import numpy as np
import pytest

import oracle
from synth import LAYERS, LayerConfig, make_layer
from tests.gpu_util import (bf16_bits_to_f64, check_out, collect, float_gate, h_gate,
                            run_layer_gpu, to_np, torch_mod)
from tests.minis import MINIS

pytestmark = pytest.mark.gpu

MID = {
    # several tiles per expert, ragged tails, mixed int2/int4, shared expert
    "mid_mixed": LayerConfig("mid_mixed", 200, T=100, H=512, E=16, k=4, I=256,
                             group=64, n_int2=5, group_int2=64, n_shared=1,
                             I_shared=192),
    "mid_mixed_a8": LayerConfig("mid_mixed_a8", 201, T=70, H=512, E=12, k=3,
                                I=320, group=32, n_int2=4, group_int2=32,
                                act="a8"),
    "mid_g128_a8_shared": LayerConfig("mid_g128_a8_shared", 202, T=33, H=1024,
                                      E=20, k=6, I=384, group=128, n_int2=3,
                                      group_int2=128, n_shared=2, I_shared=256,
                                      act="a8"),
    "mid_g256": LayerConfig("mid_g256", 203, T=9, H=768, E=10, k=2, I=512,
                            group=256, n_int2=2, group_int2=256),
}

# MFMA-path layers: H, I multiple of 128; some experts over 128 rows
MFMA = {
    "mfma_mixed": LayerConfig("mfma_mixed", 210, T=600, H=512, E=16, k=4, I=256,
                              group=128, n_int2=4, group_int2=64, n_shared=1,
                              I_shared=384),
    "mfma_g32_int2": LayerConfig("mfma_g32_int2", 211, T=257, H=384, E=6, k=2,
                                 I=128, group=64, n_int2=3, group_int2=32),
    "mfma_g256": LayerConfig("mfma_g256", 212, T=130, H=1024, E=8, k=3, I=512,
                             group=256, n_int2=2, group_int2=128),
    # 8800 pairs: the sort over five workgroups of 2048 pairs, the last partial
    "mfma_multisort": LayerConfig("mfma_multisort", 214, T=1100, H=256, E=48, k=8, I=128,
                                  group=128, n_int2=8, group_int2=64),
}

_cache = {}


def _layer(cfg):
    key = (cfg.name, cfg.key)
    if key not in _cache:
        _cache[key] = make_layer(cfg)
    return _cache[key]


def _dev(cfg):
    from packed_bit_grouped_amd.layer import DeviceLayer
    print(f"[parity] {cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} I={cfg.I}",
          flush=True)
    return DeviceLayer.from_synth(_layer(cfg))


def _check_integer_stages(g, o, cfg):
    assert np.array_equal(g["ids"], o["ids"])
    assert np.allclose(g["w"], o["w"], rtol=2e-6, atol=1e-7)
    assert np.allclose(g["w"].sum(1), 1.0, atol=2e-6) or not cfg.renormalize
    for key in ("counts", "offsets", "sorted_pair", "pair_pos"):
        assert np.array_equal(g[key], o[key]), key
    assert np.array_equal(g["tiles"][:, :3], o["tiles"]), "tiles"
    assert g["err"] == 0


def _valid_h(h, cfg):
    """The written part of h: routed rows hold I values, shared rows I_shared."""
    P = cfg.T * cfg.k
    parts = [np.asarray(h[:P, :cfg.I], np.float64).ravel()]
    if cfg.n_shared:
        parts.append(np.asarray(h[P:, :cfg.I_shared], np.float64).ravel())
    return np.concatenate(parts)


def _check_layer(cfg, act=None, tile_m=16, flags=0):
    act = act or cfg.act
    dl = _dev(cfg)
    g, B = run_layer_gpu(dl, act, tile_m, flags)
    g32, _ = run_layer_gpu(dl, act, tile_m, flags, out_f32=True)
    o = oracle.oracle_layer(_layer(cfg), act=act, tile_m=tile_m)
    _check_integer_stages(g, o, cfg)
    gh, oh = (g["h"], o["h"]) if act == "a16" else (g["h32"], o["h32"])
    ok, rl2, worst = h_gate(_valid_h(gh, cfg), _valid_h(oh, cfg), act)
    assert ok, ("h", rl2, worst)
    check_out(g, g32, o["out"], f"{cfg.name} {act} flags={flags}")
    return g, o, dl, B


@pytest.mark.parametrize("name", list(MINIS) + list(MID))
def test_small_layers(name):
    cfg = MINIS.get(name) or MID[name]
    _check_layer(cfg, flags=1)


@pytest.mark.parametrize("name", ["c0", "mixed_shared", "mid_mixed"])
def test_small_layers_as_a8(name):
    cfg = MINIS.get(name) or MID[name]
    _check_layer(cfg, act="a8")


@pytest.mark.parametrize("tile_m", [1, 3, 16, 64])
def test_tile_sizes(tile_m):
    _check_layer(MID["mid_mixed"], tile_m=tile_m)


@pytest.mark.parametrize("name", list(MFMA))
def test_mfma_path_layers(name):
    _check_layer(MFMA[name], tile_m=128, flags=2)


@pytest.mark.parametrize("tile_m", [16, 64, 200])
def test_mfma_path_tile_sizes(tile_m):
    _check_layer(MFMA["mfma_mixed"], tile_m=tile_m, flags=2)


GATED = {
    "gated_mfma": LayerConfig("mfma_gated", 213, T=300, H=512, E=8, k=2, I=256, group=128,
                              n_int2=2, group_int2=64, n_shared=1, I_shared=384,
                              shared_gate=True),
    "gated_c1": LAYERS["decode_w4a16_t1"].replace(name="decode_w4a16_t1_gated",
                                                  shared_gate=True),
    "gated_t12": LAYERS["specdecode_w4a16_t12"].replace(name="specdecode_w4a16_t12_gated",
                                                        shared_gate=True),
}


@pytest.mark.parametrize("name,act,flags,tile_m", [
    ("gated_shared", "a16", 0, 16), ("gated_shared", "a16", 1, 16),
    ("gated_shared", "a16", 3, 16), ("gated_shared", "a8", 0, 16),
    ("gated_shared_a8", "a8", 3, 16), ("gated_shared_a8", "a8", 1, 16),
    ("gated_mfma", "a16", 2, 160), ("gated_mfma", "a16", 0, 16),
    ("gated_c1", "a16", 0, 16), ("gated_t12", "a16", 0, 16)])
def test_sigmoid_gated_shared_experts(name, act, flags, tile_m):
    """Shared experts gated per token by sigmoid(gate logit), on every
    combine: the decode kernel's fused combine, the combine kernel after the
    split-K, 16-row and matrix-core paths."""
    cfg = MINIS.get(name) or GATED[name]
    _check_layer(cfg, act=act, tile_m=tile_m, flags=flags)


@pytest.mark.parametrize("name", ["gated_c1", "gated_shared"])
def test_sigmoid_gate_one_launch_matches_two_calls(name):
    """The one-launch decode layer applies the same gate as the two calls,
    bit for bit."""
    from packed_bit_grouped_amd import _lib as L
    cfg = MINIS.get(name) or GATED[name]
    dl = _dev(cfg)
    assert L.moe_w4_layer_one_launch(0, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.n_shared,
                                     cfg.I_shared, 16, L.MOE_LAYER_ONE_LAUNCH) == 1
    g1, _ = run_layer_gpu(dl, "a16", 16, flags=L.MOE_LAYER_ONE_LAUNCH)
    g2, _ = run_layer_gpu(dl, "a16", 16)
    assert np.array_equal(g1["out"], g2["out"]) and g1["err"] == 0
    o = oracle.oracle_layer(_layer(cfg))
    ok, rl2, mabs, rms = float_gate(g1["out"], o["out"])
    assert rl2 <= 5e-3


def test_mfma_path_rejects_a8_and_odd_shapes():
    from packed_bit_grouped_amd import _lib as L
    dl = _dev(MID["mid_mixed"])       # I_shared = 192: not a multiple of 128
    B = dl.buffers("a16", 16)
    st = L.moe_w4_gateup_silu(0, dl.x, 100, 512, 256, 16, 4, dl.bank.w13, dl.bank.w13_sh, 1,
                              192, B.offsets, B.sorted_pair, B.tiles, B.n_tiles, 16, B.h,
                              B.ws, B.ws_bytes, 2, check=False)
    assert st == L.MOE_E_UNSUPPORTED


@pytest.mark.parametrize("lname", ["tiny_w4a16", "decode_w4a16_t1", "specdecode_w4a16_t12",
                                   "decode_w4a8_t64"])
def test_benchmark_layers_full(lname):
    _check_layer(LAYERS[lname])


# 16-row MFMA tiles (flags 3): every small layer (int4 and int2 experts,
# groups 32..256, shared experts, E = 1, k = E), both activation modes,
# ragged tile sizes, and the decode layers at full size.
@pytest.mark.parametrize("name", list(MINIS) + list(MID))
def test_m16_path_layers(name):
    cfg = MINIS.get(name) or MID[name]
    _check_layer(cfg, flags=3)


@pytest.mark.parametrize("name", ["c0", "mixed_shared", "mid_mixed", "mid_g256", "e288"])
def test_m16_path_as_a8(name):
    cfg = MINIS.get(name) or MID[name]
    _check_layer(cfg, act="a8", flags=3)


@pytest.mark.parametrize("tile_m", [1, 5, 16])
def test_m16_tile_sizes(tile_m):
    _check_layer(MID["mid_mixed"], tile_m=tile_m, flags=3)


@pytest.mark.parametrize("lname", ["decode_w4a16_t1", "specdecode_w4a16_t12", "decode_w4a8_t64"])
def test_m16_benchmark_layers(lname):
    _check_layer(LAYERS[lname], flags=3)


@pytest.mark.parametrize("name", ["c3", "mid_mixed_a8", "c0_a8", "mixed_shared_a8"])
def test_m16_a8_kernel_quantizer_matches_row_quantizer(name):
    """W4A8 gate/up on the 16-row tiles makes the int8 x rows inside the
    kernel; with MOE_QUANT_SEPARATE the row quantizer launch (bit-exact to
    the oracle, test_a8_quantizer_bit_exact) makes them instead.  Same codes
    and scales give the same MFMA inputs, so h and out agree bit for bit."""
    cfg = LAYERS["decode_w4a8_t64"] if name == "c3" else (MINIS.get(name) or MID[name])
    dl = _dev(cfg)
    g1, _ = run_layer_gpu(dl, "a8", 16, 3)
    g2, _ = run_layer_gpu(dl, "a8", 16, 3 | 4)
    assert np.array_equal(_valid_h(g1["h32"], cfg), _valid_h(g2["h32"], cfg))
    assert np.array_equal(g1["out"], g2["out"])
    assert g1["err"] == 0 and g2["err"] == 0


def test_route_ties_and_large_E():
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    rng = np.random.default_rng(1)
    for T, E, k in [(37, 288, 8), (5, 1024, 33), (9, 4, 4), (64, 64, 64), (3, 1, 1)]:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        lg[:, 1::7] = lg[:, 0:1]                 # many exact ties
        lg[0] = 0.5
        if E > 3:
            lg[1, 3] = -0.0
            lg[1, 2] = 0.0
        dl = torch.from_numpy(lg).cuda()
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        for renorm in (1, 0):
            L.moe_route_topk(dl, T, E, k, renorm, ids, w)
            torch.cuda.synchronize()
            oi, ow = oracle.route_topk(lg, k, renorm)
            assert np.array_equal(to_np(ids), oi), (T, E, k)
            assert np.allclose(to_np(w), ow, rtol=2e-6, atol=1e-7)


def test_permute_edge_cases():
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    rng = np.random.default_rng(2)
    cases = [(1, 8, 128, 16), (4096, 8, 256, 64), (333, 5, 17, 7), (50, 4, 512, 1),
             (2, 3, 3, 4096)]
    for T, k, E, tile_m in cases:
        ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
        _permute_check(torch, L, ids, E, tile_m)
    # duplicates within a token and a skewed distribution
    ids = rng.integers(0, 3, size=(200, 6)).astype(np.int32)
    _permute_check(torch, L, ids, 40, 5)


def _permute_check(torch, L, ids, E, tile_m):
    T, k = ids.shape
    P = T * k
    d = torch.from_numpy(ids).cuda()
    mt = L.moe_permute_max_tiles(T, k, E, tile_m)
    bufs = [torch.full((n,), -7, dtype=torch.int32, device="cuda")
            for n in (E, E + 1, P, P)]
    tiles = torch.full((max(mt, 1), 4), -7, dtype=torch.int32, device="cuda")
    nt = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.moe_permute(d, T, k, E, tile_m, *bufs, tiles, nt)
    torch.cuda.synchronize()
    o = oracle.permute(ids, E, tile_m)
    for key, b in zip(("counts", "offsets", "sorted_pair", "pair_pos"), bufs):
        assert np.array_equal(to_np(b), o[key]), (key, T, k, E, tile_m)
    n = int(nt.item())
    assert n == len(o["tiles"]) <= mt
    assert np.array_equal(to_np(tiles)[:n, :3], o["tiles"])


def test_fused_route_permute_matches_separate_calls():
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    rng = np.random.default_rng(5)
    for T, E, k, tile_m, renorm in [(1, 128, 8, 16, 1), (12, 128, 8, 16, 1),
                                    (64, 128, 8, 16, 1), (64, 512, 64, 3, 1),
                                    (7, 288, 8, 1, 0), (33, 8, 8, 4096, 1),
                                    # one-wave sort: up to 128 pairs, pairs in both
                                    # lane slots, ragged tiles, E up to 512
                                    (15, 64, 8, 5, 1), (9, 40, 14, 2, 0), (13, 512, 9, 7, 1),
                                    (11, 16, 11, 3, 1), (8, 128, 16, 1, 1), (3, 6, 5, 4096, 0)]:
        lg = rng.standard_normal((T, E)).astype(np.float32)
        lg[:, 3::5] = lg[:, 1:2]
        d = torch.from_numpy(lg).cuda()
        outs = []
        for fused in (True, False):
            P = T * k
            mt = L.moe_permute_max_tiles(T, k, E, tile_m)
            b = [torch.full((T, k), -7, dtype=torch.int32, device="cuda"),
                 torch.full((T, k), -7.0, dtype=torch.float32, device="cuda"),
                 torch.full((E,), -7, dtype=torch.int32, device="cuda"),
                 torch.full((E + 1,), -7, dtype=torch.int32, device="cuda"),
                 torch.full((P,), -7, dtype=torch.int32, device="cuda"),
                 torch.full((P,), -7, dtype=torch.int32, device="cuda"),
                 torch.full((mt, 4), -7, dtype=torch.int32, device="cuda"),
                 torch.zeros(1, dtype=torch.int32, device="cuda")]
            if fused:
                L.moe_route_permute(d, T, E, k, renorm, tile_m, *b)
            else:
                L.moe_route_topk(d, T, E, k, renorm, b[0], b[1])
                L.moe_permute(b[0], T, k, E, tile_m, *b[2:])
            torch.cuda.synchronize()
            n = int(b[7].item())
            outs.append([to_np(x) for x in b[:6]] + [to_np(b[6])[:n]])
        for a_, b_ in zip(*outs):
            assert np.array_equal(a_, b_), (T, E, k)
        oi, ow = oracle.route_topk(lg, k, renorm)
        assert np.array_equal(outs[0][0], oi)
        o = oracle.permute(oi, E, tile_m)
        assert np.array_equal(outs[0][6][:, :3], o["tiles"])


@pytest.mark.parametrize("name", ["c0", "c1", "e288", "k1", "mixed_shared", "norenorm",
                                  "kE", "e1"])
def test_fused_route_gateup_matches_separate_calls(name):
    """moe_w4_layer (one launch for bf16 decode batches) and
    moe_w4_route_gateup_silu + moe_w4_down_combine write the same routing
    tables, the same h and the same output, bit for bit, as the separate
    calls (moe_route_permute / moe_route_topk + moe_permute, gate/up, down)."""
    from packed_bit_grouped_amd import _lib as L
    cfg = {"c0": LAYERS["tiny_w4a16"], "c1": LAYERS["decode_w4a16_t1"], **MINIS}[name]
    dl = _dev(cfg)
    one = L.MOE_LAYER_ONE_LAUNCH
    expect_one = name not in ("e288",)
    assert L.moe_w4_layer_one_launch(0, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, cfg.n_shared,
                                     cfg.I_shared, 16, one) == int(expect_one)
    g0, B0 = run_layer_gpu(dl, "a16", 16, flags=one, fused=True, one_call=True)
    g3, _ = run_layer_gpu(dl, "a16", 16, fused=True, one_call=True)
    g1, _ = run_layer_gpu(dl, "a16", 16, fused=True, one_call=False)
    g2, _ = run_layer_gpu(dl, "a16", 16, fused=False)
    for g in (g0, g1, g3):
        for key in ("ids", "w", "counts", "offsets", "sorted_pair", "pair_pos", "tiles",
                    "n_tiles", "out"):
            assert np.array_equal(g[key], g2[key]), key
        assert np.array_equal(_valid_h(g["h"], cfg), _valid_h(g2["h"], cfg))
        assert g["err"] == 0
    # the error word is clear and the grid-wide barrier's flags are all equal
    hdr = to_np(B0.ws[:4352].view(torch_mod().int32))
    assert hdr[0] == 0 and len(set(hdr[64:].tolist())) == 1


def test_layer_one_launch_repeated_and_mixed_shapes():
    """Back-to-back one-launch layers on one workspace and stream (every
    launch leaves the barrier flags equal), interleaved with another shape
    of another grid size, each bit-identical to its two-call form."""
    torch = torch_mod()
    cfgs = [LAYERS["decode_w4a16_t1"], MINIS["mixed_shared"]]
    dls = [_dev(c) for c in cfgs]
    refs = [run_layer_gpu(d, "a16", 16, fused=False)[0] for d in dls]
    ws = None
    bufs = []
    for d, c in zip(dls, cfgs):
        B = d.buffers("a16", 16)
        if ws is None or B.ws_bytes > ws.numel():
            ws = torch.zeros(max(B.ws_bytes, ws.numel() if ws is not None else 0),
                             dtype=torch.uint8, device="cuda")
        bufs.append(B)
    for B in bufs:
        B.ws, B.ws_bytes = ws, ws.numel()
    from packed_bit_grouped_amd import _lib as L
    for d, c in zip(dls, cfgs):
        assert L.moe_w4_layer_one_launch(0, c.T, c.H, c.I, c.E, c.k, c.n_shared, c.I_shared,
                                         16, L.MOE_LAYER_ONE_LAUNCH) == 1
    for rep in range(6):
        i = rep % 2
        dls[i].run(bufs[i], L.MOE_LAYER_ONE_LAUNCH)
        if rep % 3 == 2:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    for d, B, ref in zip(dls, bufs, refs):
        got = collect(B)
        assert np.array_equal(got["out"], ref["out"])
    hdr = to_np(ws[:4352].view(torch.int32))
    assert hdr[0] == 0 and len(set(hdr[64:].tolist())) == 1


def test_permute_skips_out_of_range_ids():
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    ids = np.array([[0, 5], [7, 1], [-1, 2], [3, 8]], dtype=np.int32)   # E = 8
    T, k, E = 4, 2, 8
    d = torch.from_numpy(ids).cuda()
    c, off = (torch.zeros(E, dtype=torch.int32, device="cuda"),
              torch.zeros(E + 1, dtype=torch.int32, device="cuda"))
    sp, pp = (torch.zeros(8, dtype=torch.int32, device="cuda"),
              torch.zeros(8, dtype=torch.int32, device="cuda"))
    tiles = torch.zeros((L.moe_permute_max_tiles(T, k, E, 4), 4), dtype=torch.int32,
                        device="cuda")
    nt = torch.zeros(1, dtype=torch.int32, device="cuda")
    L.moe_permute(d, T, k, E, 4, c, off, sp, pp, tiles, nt)
    torch.cuda.synchronize()
    valid = ids.ravel()[(ids.ravel() >= 0) & (ids.ravel() < E)]
    assert int(to_np(off)[E]) == valid.size == 6
    assert to_np(pp)[4] == -1 and to_np(pp)[7] == -1
    assert list(to_np(sp)[6:]) == [-1, -1]
    assert np.array_equal(to_np(c), np.bincount(valid, minlength=E))


def test_a8_quantizer_bit_exact():
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    rng = np.random.default_rng(3)
    rows = (rng.standard_normal((50, 777)) * rng.uniform(1e-3, 300, (50, 1))).astype(np.float32)
    rows[4] = 0
    rows[5, :] = rows[5, 0]
    rows[6, ::3] = 127.0 * 0.5      # exact ties at amax = 127 * 0.5 * ...
    for src_is_f32 in (1, 0):
        if src_is_f32:
            src = torch.from_numpy(rows).cuda()
            ref_rows = rows
        else:
            from synth.gen import bf16_bits_from_f32
            bits = bf16_bits_from_f32(rows)
            src = torch.from_numpy(bits.view(np.int16)).cuda()
            ref_rows = bf16_bits_to_f64(bits).astype(np.float32)
        q = torch.empty((50, 777), dtype=torch.int8, device="cuda")
        s = torch.empty(50, dtype=torch.float32, device="cuda")
        L.moe_quant_a8_rows(src, src_is_f32, 50, 777, 777, q, s)
        torch.cuda.synchronize()
        oq, os_ = oracle.quant_rows_a8(ref_rows)
        assert np.array_equal(to_np(q), oq)
        assert np.array_equal(to_np(s), os_)


A8_PARTIAL_CASES = [(n, f, False) for n in ("c3", "mid_mixed_a8", "mid_g128_a8_shared",
                                             "mixed_shared_a8", "mid_g256", "e288")
                    for f in (0, 1)] + \
                   [("mixed_shared_a8", 0, True), ("mid_mixed_a8", 0, True),
                    ("mid_g128_a8_shared", 1, True), ("c3", 0, True)]


@pytest.mark.parametrize("name,flags,raw", A8_PARTIAL_CASES)
def test_a8_partials_bit_exact(name, flags, raw):
    """Stage 1: int32 per-group partials of int8 x against int codes equal
    the oracle's exactly.  Stage 2: the down call's int8 h codes equal the
    oracle quantizer applied to the GPU's fp32 h, and its int32 partials
    equal the oracle's partials computed from those codes.  flags 0 runs
    the kernels the product runs for the shape (the 16-row int8 matrix
    tiles, with the int8 x rows made in the gate/up kernel), flags 1 the
    split-K GEMV; raw: code bytes drawn uniformly (int4 -8, int2 -2)."""
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    from packed_bit_grouped_amd.layer import DeviceLayer
    from synth import with_random_codes
    cfg = LAYERS["decode_w4a8_t64"] if name == "c3" else (MINIS.get(name) or MID[name])
    layer = _layer(cfg)
    if raw:
        layer = with_random_codes(layer, seed=3)
    print(f"[parity] partials {cfg.name} flags={flags} raw={raw}", flush=True)
    dl = DeviceLayer.from_synth(layer)
    B = dl.buffers("a8", 16)
    c = cfg
    L.moe_route_topk(dl.logits, c.T, c.E, c.k, c.renormalize, B.ids, B.w)
    L.moe_permute(B.ids, c.T, c.k, c.E, B.tile_m, B.counts, B.offsets, B.sorted_pair,
                  B.pair_pos, B.tiles, B.n_tiles)
    ng1 = c.H // 32
    ng2 = B.ld_h // 32
    p1 = torch.full((B.R, 2 * B.ld_h, ng1), -(1 << 30), dtype=torch.int32, device="cuda")
    p2 = torch.full((B.R, c.H, ng2), -(1 << 30), dtype=torch.int32, device="cuda")
    L.moe_dbg_w4a8_gateup_partials(dl.x, c.T, c.H, c.I, c.E, c.k, dl.bank.w13,
                                   dl.bank.w13_sh, c.n_shared, c.I_shared, B.offsets,
                                   B.sorted_pair, B.tiles, B.n_tiles, B.tile_m, B.h,
                                   B.ws, B.ws_bytes, p1, ng1, flags=flags)
    L.moe_dbg_w4a8_down_partials(B.h, c.T, c.H, c.I, c.E, c.k, dl.bank.w2, dl.bank.w2_sh,
                                 c.n_shared, c.I_shared, B.w, B.offsets, B.sorted_pair,
                                 B.pair_pos, B.tiles, B.n_tiles, B.tile_m, B.out, B.ws,
                                 B.ws_bytes, p2, ng2, flags=flags)
    torch.cuda.synchronize()
    g = collect(B)
    ids, _ = oracle.route_topk(layer.logits, c.k, c.renormalize)
    perm = oracle.permute(ids, c.E, 16)
    o1 = oracle.gateup_a8(layer, perm, want_partials=True)
    P1 = to_np(p1)
    for (e, s), (rows, Pg) in o1["partials"].items():
        ex = layer.experts[e] if s is None else layer.shared[s]
        n2, ng = ex.w13.N, ex.w13.K // ex.w13.group
        assert np.array_equal(P1[rows, :n2, :ng], Pg), ("stage1", e, s)
    # stage 2 from the GPU's own fp32 h
    h32 = g["h32"]
    qh = np.zeros((B.R, B.ld_h), np.int8)
    sh = np.zeros(B.R, np.float32)
    for e_, rows, s, toks in oracle.expert_rows(perm, c.E, c.T, c.n_shared):
        I_e = (layer.experts[e_] if s is None else layer.shared[s]).w2.K
        q_, s_ = oracle.quant_rows_a8(h32[rows, :I_e])
        qh[rows, :I_e] = q_
        sh[rows] = s_
    qg = torch.empty((B.R, B.ld_h), dtype=torch.int8, device="cuda")
    sg = torch.empty(B.R, dtype=torch.float32, device="cuda")
    # the same rows quantized by the library's own quantizer
    qg.zero_()
    for e_, rows, s, toks in oracle.expert_rows(perm, c.E, c.T, c.n_shared):
        I_e = (layer.experts[e_] if s is None else layer.shared[s]).w2.K
        r0 = int(rows[0])
        qt = torch.empty((len(rows), I_e), dtype=torch.int8, device="cuda")
        L.moe_quant_a8_rows(B.h[r0:], 1, len(rows), I_e, B.ld_h, qt, sg[r0:])
        qg[r0:r0 + len(rows), :I_e] = qt
    torch.cuda.synchronize()
    assert np.array_equal(to_np(qg), qh)
    assert np.array_equal(to_np(sg), sh)
    _, parts2 = oracle.down_a8(layer, perm, qh, sh, want_partials=True)
    P2 = to_np(p2)
    for (e, s), (rows, Pg) in parts2.items():
        ex = layer.experts[e] if s is None else layer.shared[s]
        ng = ex.w2.K // ex.w2.group
        assert np.array_equal(P2[rows, :, :ng], Pg), ("stage2", e, s)
    assert g["err"] == 0
    # the hooks compute what the product calls compute
    g2, _ = run_layer_gpu(dl, "a8", 16, flags)
    assert np.array_equal(g2["h32"][:c.T * c.k], g["h32"][:c.T * c.k])
    assert np.array_equal(g2["out"], g["out"])
    g32, _ = run_layer_gpu(dl, "a8", 16, flags, out_f32=True)
    o = oracle.oracle_layer(layer, act="a8", tile_m=16)
    check_out(g2, g32, o["out"], f"partials {cfg.name}")


def test_prefill_layer_sampled_tokens():
    """The prefill layer at full size (4096 tokens, 256 experts, 192 int4 +
    64 int2): integer stages in full, outputs on a token sample."""
    cfg = LAYERS["prefill_mixed_t4096"]
    layer = _layer(cfg)
    dl = _dev(cfg)
    tile_m = 64
    g, B = run_layer_gpu(dl, "a16", tile_m)
    g32, _ = run_layer_gpu(dl, "a16", tile_m, out_f32=True)
    ids, w = oracle.route_topk(layer.logits, cfg.k)
    perm = oracle.permute(ids, cfg.E, tile_m)
    assert np.array_equal(g["ids"], ids)
    assert np.allclose(g["w"], w, rtol=2e-6, atol=1e-7)
    for key in ("counts", "offsets", "sorted_pair", "pair_pos"):
        assert np.array_equal(g[key], perm[key]), key
    assert np.array_equal(g["tiles"][:, :3], perm["tiles"])
    assert g["err"] == 0
    toks = list(np.random.default_rng(4).choice(cfg.T, 24, replace=False)) + [0, cfg.T - 1]
    s = oracle.oracle_token_outputs(layer, toks)
    sub = lambda d: {"out": d["out"][toks],
                     "out_bits": None if d["out_bits"] is None else d["out_bits"][toks]}
    check_out(sub(g), sub(g32), s["out"], "prefill sample")
    # h rows of the sampled tokens' pairs (bf16 on both sides)
    for n, t in enumerate(toks[:6]):
        for j in range(cfg.k):
            r = perm["pair_pos"][t * cfg.k + j]
            ok, rl2, worst = h_gate(g["h"][r, :cfg.I], s["h"][(t, j)], "a16")
            assert ok, ("h", t, j, rl2, worst)


_C4 = {}


def _c4_oracle():
    """The fp64 oracle of the whole prefill layer, once per test session
    (printed stage by stage: it runs for a minute or two)."""
    if not _C4:
        import time
        cfg = LAYERS["prefill_mixed_t4096"]
        layer = _layer(cfg)
        t0 = time.time()
        ids, w = oracle.route_topk(layer.logits, cfg.k)
        perm = oracle.permute(ids, cfg.E, 160)
        h, _ = oracle.gateup_a16(layer, perm)
        print(f"[parity] prefill oracle: gate/up done at {time.time() - t0:.0f} s", flush=True)
        y = oracle.down_a16(layer, perm, h)
        print(f"[parity] prefill oracle: down done at {time.time() - t0:.0f} s", flush=True)
        out = oracle.combine(layer, perm, w, y)
        del y
        _C4.update(ids=ids, w=w, h=h, out=out)
    return _C4


@pytest.mark.timeout(900)
@pytest.mark.parametrize("tile_m", [160, 64])
def test_prefill_layer_full(tile_m):
    """The prefill layer at full size (4096 tokens, 256 experts, 192 int4 +
    64 int2) against the oracle on every output: the routing tables bit for
    bit, all 32,768 x 1536 values of h and all 4096 x 4096 outputs, at the
    tile height the library prefers (160, the matrix-core chunk) and at 64."""
    cfg = LAYERS["prefill_mixed_t4096"]
    o = _c4_oracle()
    dl = _dev(cfg)
    g, B = run_layer_gpu(dl, "a16", tile_m)
    g32, _ = run_layer_gpu(dl, "a16", tile_m, out_f32=True)
    perm = oracle.permute(o["ids"], cfg.E, tile_m)
    assert np.array_equal(g["ids"], o["ids"])
    assert np.allclose(g["w"], o["w"], rtol=2e-6, atol=1e-7)
    for key in ("counts", "offsets", "sorted_pair", "pair_pos"):
        assert np.array_equal(g[key], perm[key]), key
    assert np.array_equal(g["tiles"][:, :3], perm["tiles"])
    assert g["err"] == 0
    P = cfg.T * cfg.k
    ok, rl2, worst = h_gate(g["h"][:P, :cfg.I], o["h"][:P, :cfg.I], "a16")
    print(f"[parity] prefill tile_m={tile_m}: h rel-L2 {rl2:.2e} worst/bound {worst:.2f}",
          flush=True)
    assert ok, ("h", rl2, worst)
    assert np.array_equal(g32["h"], g["h"])
    check_out(g, g32, o["out"], f"prefill tile_m={tile_m}")


def test_repeat_bitwise_identical():
    dl = _dev(LAYERS["specdecode_w4a16_t12"])
    g1, _ = run_layer_gpu(dl, "a16", 16)
    g2, _ = run_layer_gpu(dl, "a16", 16)
    assert np.array_equal(g1["out"], g2["out"])
    assert np.array_equal(g1["h"], g2["h"])
    g3, _ = run_layer_gpu(dl, "a8", 16)
    g4, _ = run_layer_gpu(dl, "a8", 16)
    assert np.array_equal(g3["out"], g4["out"])


@pytest.mark.parametrize("name,one", [("c1", False), ("c1", True), ("mixed_shared", False),
                                      ("mixed_shared", True), ("mfma_mixed", False)])
def test_graph_replay_matches_eager(name, one):
    """The whole step captured in a HIP graph (decode, one-launch layer,
    split-K GEMV and matrix-core forms): every replay, with eager work and
    synchronizations in between, reproduces the eager step bit for bit."""
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    fl = L.MOE_LAYER_ONE_LAUNCH if one else 0
    cfg = {"c1": LAYERS["decode_w4a16_t1"], **MINIS, **MFMA}[name]
    dl = _dev(cfg)
    B = dl.buffers()
    dl.run(B, fl)
    torch.cuda.synchronize()
    ref = collect(B)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dl.run(B, fl)
    for rep in range(3):
        B.out.zero_()
        B.h.zero_()
        B.sorted_pair.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = collect(B)
        for key in ("ids", "counts", "offsets", "sorted_pair", "pair_pos", "tiles", "out"):
            assert np.array_equal(got[key], ref[key]), (rep, key)
        assert np.array_equal(_valid_h(got["h"], cfg), _valid_h(ref["h"], cfg)), (rep, "h")
        dl.run(B, fl)
        torch.cuda.synchronize()


def test_side_stream_with_event_handoff():
    """Inputs written on one stream, the layer run on another after an
    event; the producer then overwrites its buffer only after the layer's
    event has completed (buffers stay alive and unmodified until the stream
    passes the call)."""
    torch = torch_mod()
    cfg = MINIS["mixed_shared"]
    dl = _dev(cfg)
    o = oracle.oracle_layer(_layer(cfg))
    prod, cons = torch.cuda.Stream(), torch.cuda.Stream()
    x_host = dl.x.clone()
    with torch.cuda.stream(prod):
        dl.x.zero_()
        dl.x.copy_(x_host)
        ev = torch.cuda.Event()
        ev.record(prod)
    B = dl.buffers()
    cons.wait_event(ev)
    dl.run(B, 0, cons)
    done = torch.cuda.Event()
    done.record(cons)
    prod.wait_event(done)
    with torch.cuda.stream(prod):
        dl.x.zero_()
    torch.cuda.synchronize()
    g = collect(B)
    ok, rl2, mabs, rms = float_gate(g["out"], o["out"])
    assert ok


def test_empty_batch_is_a_no_op():
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    from packed_bit_grouped_amd.layer import LayerBuffers
    cfg = MINIS["c0"]
    dl = _dev(cfg)
    B = LayerBuffers(0, cfg.H, cfg.I, cfg.E, cfg.k, device="cuda")
    B.out.fill_(123)
    L.moe_route_topk(dl.logits, 0, cfg.E, cfg.k, 1, B.ids, B.w)
    L.moe_w4_gateup_silu(0, dl.x, 0, cfg.H, cfg.I, cfg.E, cfg.k, dl.bank.w13, None, 0, 0,
                         B.offsets, B.sorted_pair, B.tiles, B.n_tiles, 16, B.h, B.ws,
                         B.ws_bytes)
    torch.cuda.synchronize()
    assert int(B.out[0, 0].item()) == 123


def test_unusable_descriptor_sets_error_word():
    """A descriptor with an unsupported bit width is skipped by the kernels
    (its rows are not computed) and reported in the workspace error word."""
    torch = torch_mod()
    import ctypes
    from packed_bit_grouped_amd import _lib as L
    cfg = MINIS["c0"]
    dl = _dev(cfg)
    raw = to_np(dl.bank.w13).copy()
    desc = L.QMatDesc.from_buffer(raw, 0)
    desc.bits = 3
    dl.bank.w13.copy_(torch.from_numpy(raw))
    g, B = run_layer_gpu(dl, "a16", 16)
    assert g["err"] & 1


@pytest.mark.parametrize("name,tile_m", [("mfma_mixed", 160), ("mfma_g32_int2", 128),
                                         ("mfma_g256", 64), ("gated_mfma", 160)])
def test_prepacked_bank_matches_canonical(name, tile_m):
    """moe_w4_prepack re-tiles every code matrix into the matrix-core
    layout; the layer run on the prepacked bank (MOE_W_PREPACKED) gives the
    same h and output bits as on the canonical bank, which meets the gate
    against the oracle."""
    cfg = MFMA.get(name) or GATED[name]
    dl = _dev(cfg)
    g0, _ = run_layer_gpu(dl, "a16", tile_m, flags=2)
    dl.bank = dl.bank.prepack()
    g1, _ = run_layer_gpu(dl, "a16", tile_m, flags=2)
    g32, _ = run_layer_gpu(dl, "a16", tile_m, flags=2, out_f32=True)
    assert g1["err"] == 0
    assert np.array_equal(g1["h"], g0["h"]) and np.array_equal(g1["out"], g0["out"])
    o = oracle.oracle_layer(_layer(cfg), tile_m=tile_m)
    check_out(g1, g32, o["out"], f"prepacked {cfg.name}")


@pytest.mark.parametrize("name,tile_m", [("mfma_mixed", 40), ("mfma_mixed", 80),
                                         ("mfma_mixed", 112), ("mfma_mixed", 144),
                                         ("mfma_g32_int2", 48)])
def test_mfma_half_row_blocks(name, tile_m):
    """Chunks of 32 m + 1 .. 32 m + 16 rows (m = 1 .. 4) run their last 16
    rows as a half block on the 16x16x32 matrix instruction: tiles of 40,
    48, 80, 112 and 144 rows (and the ragged last tile of each expert) put
    half blocks after one to four whole blocks in both projections, on the
    canonical and the prepacked bank; both meet the gate against the
    oracle and agree bit for bit."""
    cfg = MFMA[name]
    dl = _dev(cfg)
    g0, _ = run_layer_gpu(dl, "a16", tile_m, flags=2)
    g32, _ = run_layer_gpu(dl, "a16", tile_m, flags=2, out_f32=True)
    o = oracle.oracle_layer(_layer(cfg), tile_m=tile_m)
    _check_integer_stages(g0, o, cfg)
    ok, rl2, worst = h_gate(_valid_h(g0["h"], cfg), _valid_h(o["h"], cfg), "a16")
    assert ok, ("h", rl2, worst)
    check_out(g0, g32, o["out"], f"{cfg.name} tile_m={tile_m}")
    dl.bank = dl.bank.prepack()
    g1, _ = run_layer_gpu(dl, "a16", tile_m, flags=2)
    assert g1["err"] == 0
    assert np.array_equal(g1["h"], g0["h"]) and np.array_equal(g1["out"], g0["out"])


def test_prepacked_prefill_layer_matches_canonical():
    """The prefill layer (4096 tokens, 192 int4 + 64 int2 experts) on a
    prepacked bank: h and out identical to the canonical bank's, which is
    compared with the oracle in full by test_prefill_layer_full."""
    cfg = LAYERS["prefill_mixed_t4096"]
    dl = _dev(cfg)
    g0, _ = run_layer_gpu(dl, "a16", 160)
    dl.bank = dl.bank.prepack()
    g1, _ = run_layer_gpu(dl, "a16", 160)
    assert g1["err"] == 0
    assert np.array_equal(g1["h"], g0["h"]) and np.array_equal(g1["out"], g0["out"])


def _prepack_codes_ref(codes, bits, N, K, gate_up):
    """The documented moe_w4_prepack layout, written out from its definition:
    pieces of 64 lane slots, slot h*32 + c holding bytes [32 s + 16 h, +16)
    (int4) or [16 s + 8 h, +8) (int2, each 4-byte word's bytes reordered
    0, 2, 1, 3) of one row; down pieces (b, s) = rows 32b + c; gate/up pieces
    (b, s, p): p = 0 gate rows 32b + c, p = 1 up rows N/2 + 32b + c."""
    rb = K * bits // 8
    w = 16 if bits == 4 else 8
    rows = codes.reshape(N, rb)
    n_st = K // 64
    out = []
    nblk = (N // 2 if gate_up else N) // 32
    for blk in range(nblk):
        for st in range(n_st):
            for p in (range(2) if gate_up else range(1)):
                for h in range(2):
                    for c in range(32):
                        r = (N // 2 if (gate_up and p) else 0) + 32 * blk + c
                        piece = rows[r, st * 2 * w + h * w: st * 2 * w + h * w + w]
                        if bits == 2:
                            piece = piece.reshape(-1, 4)[:, [0, 2, 1, 3]].ravel()
                        out.append(piece)
    return np.concatenate(out)


def _prepack_scales_ref(scales, N, ng, gate_up):
    """The documented moe_w4_prepack_scales layout: word (b*ng + g)*32 + c =
    scale of group g of row r0 (low half) and row r1 (high half)."""
    s = scales.reshape(N, ng)
    out = np.zeros((N // 64, ng, 32, 2), np.uint16)
    for b in range(N // 64):
        for c in range(32):
            r0, r1 = (32 * b + c, N // 2 + 32 * b + c) if gate_up else (64 * b + c,
                                                                        64 * b + 32 + c)
            out[b, :, c, 0] = s[r0]
            out[b, :, c, 1] = s[r1]
    return out.ravel()


@pytest.mark.parametrize("bits,group,gate_up", [(4, 128, 1), (4, 32, 0), (2, 64, 1),
                                                (2, 256, 0)])
def test_prepack_layouts_match_their_definitions(bits, group, gate_up):
    """moe_w4_prepack and moe_w4_prepack_scales on random bytes against the
    layouts the header defines, re-tiled here on the host."""
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    rng = np.random.default_rng(bits * 1000 + group + gate_up)
    N, K = 192, 512
    ng = K // group
    codes = rng.integers(0, 256, size=N * K * bits // 8, dtype=np.uint8)
    scales = rng.integers(0, 1 << 16, size=N * ng, dtype=np.uint16)
    dc, ds = torch.from_numpy(codes).cuda(), torch.from_numpy(scales.view(np.int16)).cuda()
    oc, os_ = torch.zeros_like(dc), torch.zeros_like(ds)
    L.moe_w4_prepack(dc, bits, N, K, gate_up, oc)
    L.moe_w4_prepack_scales(ds, N, K, group, gate_up, os_)
    torch.cuda.synchronize()
    assert np.array_equal(oc.cpu().numpy(), _prepack_codes_ref(codes, bits, N, K, gate_up))
    assert np.array_equal(os_.cpu().numpy().view(np.uint16),
                          _prepack_scales_ref(scales, N, ng, gate_up))


def test_prepacked_bank_needs_the_matrix_core_path():
    from packed_bit_grouped_amd import _lib as L
    cfg = MINIS["mixed_shared"]
    dl = _dev(cfg)
    B = dl.buffers("a16", 16)
    st = L.moe_w4_gateup_silu(0, dl.x, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dl.bank.w13,
                              dl.bank.w13_sh, cfg.n_shared, cfg.I_shared, B.offsets,
                              B.sorted_pair, B.tiles, B.n_tiles, 16, B.h, B.ws, B.ws_bytes,
                              L.MOE_W_PREPACKED, check=False)
    assert st == L.MOE_E_UNSUPPORTED


BIG_SORT = LayerConfig("mfma_big_sort", 214, T=1100, H=256, E=40, k=8, I=128, group=64,
                       n_int2=7, group_int2=32)
# 33600 pairs: 17 chunks of 2048, the last one partial
SORT_TWO_LAUNCH = LayerConfig("mfma_sort_two_launch", 216, T=4200, H=256, E=40, k=8, I=128,
                              group=64, n_int2=7, group_int2=32)


@pytest.mark.parametrize("name", ["mfma_mixed", "gated_mfma", "big_sort", "sort_two_launch",
                                  "prefill"])
def test_layer_call_matches_separate_calls_on_matrix_cores(name):
    """moe_w4_layer on the matrix-core path (its routing launch makes the fp16
    copy of x, its gate/up epilogue writes the fp16 h rows the down
    projection reads; from 8192 pairs the sort runs over many workgroups
    with its counts in the workspace) gives the same routing tables, h and
    output bits as the separate calls (one-workgroup sort, fp16 x and h made
    by conversion passes)."""
    cfg = {"mfma_mixed": MFMA["mfma_mixed"], "gated_mfma": GATED["gated_mfma"],
           "big_sort": BIG_SORT, "sort_two_launch": SORT_TWO_LAUNCH,
           "prefill": LAYERS["prefill_mixed_t4096"]}[name]
    dl = _dev(cfg)
    g1, _ = run_layer_gpu(dl, "a16", 160)
    g2, _ = run_layer_gpu(dl, "a16", 160, fused=False)
    for key in ("ids", "w", "counts", "offsets", "sorted_pair", "pair_pos", "tiles",
                "n_tiles", "out", "h"):
        assert np.array_equal(g1[key], g2[key]), key
    assert g1["err"] == 0
    if name in ("big_sort", "sort_two_launch"):
        o = oracle.oracle_layer(_layer(cfg), tile_m=160)
        _check_integer_stages(g1, o, cfg)
        g32, _ = run_layer_gpu(dl, "a16", 160, out_f32=True)
        check_out(g1, g32, o["out"], name)


def test_gateup_reads_fp16_copy_left_by_the_layer_call():
    """MOE_X_PREPARED on the matrix-core path: the routing launch of the
    layer call leaves the fp16 copy of x in the workspace; a gate/up call
    that reads it (no conversion of its own) writes the layer's h bits."""
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    cfg = MFMA["mfma_mixed"]
    dl = _dev(cfg)
    g1, B = run_layer_gpu(dl, "a16", 160)
    B.h.zero_()
    L.moe_w4_gateup_silu(B.act, dl.x, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dl.bank.w13,
                         dl.bank.w13_sh, cfg.n_shared, cfg.I_shared, B.offsets,
                         B.sorted_pair, B.tiles, B.n_tiles, B.tile_m, B.h, B.ws, B.ws_bytes,
                         L.MOE_X_PREPARED)
    torch.cuda.synchronize()
    g2 = collect(B)
    assert np.array_equal(g1["h"], g2["h"])
    assert g2["err"] == 0


@pytest.mark.parametrize("name", ["c1", "c3", "mixed_shared"])
def test_cached_routing_tables_are_reused(name):
    """Routing cache: the routing tables a step computed (ids, gate weights,
    counts, offsets, sorted pairs, pair positions, tile list) are inputs of
    the projection calls, so later calls over the same tokens reuse them
    without routing again.  Routed once, then the logits are overwritten;
    gate/up + down on the cached tables reproduce the routed step bit for
    bit, twice, and a second bank run on the same tables matches its own
    routed run."""
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    cfg = {"c1": LAYERS["decode_w4a16_t1"], "c3": LAYERS["decode_w4a8_t64"]}.get(name) or MINIS[name]
    act = cfg.act
    dl = _dev(cfg)
    ref, B = run_layer_gpu(dl, act, 16)
    dl.logits.fill_(float("nan"))      # the cached tables must not need the logits again
    c = cfg
    for rep in range(2):
        B.h.zero_()
        B.out.zero_()
        L.moe_w4_gateup_silu(B.act, dl.x, c.T, c.H, c.I, c.E, c.k, dl.bank.w13, dl.bank.w13_sh,
                             c.n_shared, c.I_shared, B.offsets, B.sorted_pair, B.tiles,
                             B.n_tiles, B.tile_m, B.h, B.ws, B.ws_bytes)
        L.moe_w4_down_combine(B.act, B.h, c.T, c.H, c.I, c.E, c.k, dl.bank.w2, dl.bank.w2_sh,
                              c.n_shared, c.I_shared, B.w, B.offsets, B.sorted_pair, B.pair_pos,
                              B.tiles, B.n_tiles, B.tile_m, B.out, B.ws, B.ws_bytes)
        torch.cuda.synchronize()
        got = collect(B)
        assert np.array_equal(got["out"], ref["out"]), rep
        for key in ("ids", "sorted_pair", "pair_pos", "tiles"):
            assert np.array_equal(got[key], ref[key]), key
