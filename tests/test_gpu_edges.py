"""GPU parity on the method's edge cases, through the C ABI against the CPU
oracle.

* Raw code bytes: the quantizer never emits int4 -8 or int2 -2 (its codes
  stay within +-7 and +-1), but the packed format holds them and every
  unpack must decode them.  Layers whose code bytes are uniformly random
  run on every path (automatic choice, split-K GEMV, matrix-core prefill
  tiles, 16-row matrix tiles) in both activation modes.
* Activation rows at the edges: an all-zero token (its output is exactly
  zero on every path), a token whose largest |x| is ~2e-37 (the int8 row
  scale is then subnormal and has no finite reciprocal), a one-hot token
  and a token scaled by 50.
* Determinism: ten repeats of the speculative-decode layer (both modes)
  give identical bits.
"""
import numpy as np
import pytest

import oracle
from synth import LAYERS, LayerConfig, make_layer, with_random_codes, with_x_rows
from tests.gpu_util import check_out, h_gate, run_layer_gpu
from tests.minis import MINIS

pytestmark = pytest.mark.gpu

LAYERS_E = {
    "mixed_shared": MINIS["mixed_shared"],
    "mixed_shared_a8": MINIS["mixed_shared_a8"],
    "e288": MINIS["e288"],
    "mid_mixed_a8": LayerConfig("mid_mixed_a8", 201, T=70, H=512, E=12, k=3, I=320,
                                group=32, n_int2=4, group_int2=32, act="a8"),
    "mid_g256": LayerConfig("mid_g256", 203, T=9, H=768, E=10, k=2, I=512, group=256,
                            n_int2=2, group_int2=256),
    "mfma_mixed": LayerConfig("mfma_mixed", 210, T=600, H=512, E=16, k=4, I=256,
                              group=128, n_int2=4, group_int2=64, n_shared=1,
                              I_shared=384),
    "mfma_g32_int2": LayerConfig("mfma_g32_int2", 211, T=257, H=384, E=6, k=2, I=128,
                                 group=64, n_int2=3, group_int2=32),
    "c1": LAYERS["decode_w4a16_t1"],
    "c3_t16": LAYERS["decode_w4a8_t64"].replace(name="decode_w4a8_t16", T=16),
}

_cache = {}


def _base(name):
    if name not in _cache:
        _cache[name] = make_layer(LAYERS_E[name])
    return _cache[name]


def _run_and_check(layer, act, flags, tile_m=None):
    from packed_bit_grouped_amd.layer import DeviceLayer
    cfg = layer.cfg
    tile_m = tile_m or (128 if flags == 2 else 16)
    print(f"[edges] {cfg.name} act={act} flags={flags} tile_m={tile_m}", flush=True)
    dl = DeviceLayer.from_synth(layer)
    g, _ = run_layer_gpu(dl, act, tile_m, flags)
    g32, _ = run_layer_gpu(dl, act, tile_m, flags, out_f32=True)
    o = oracle.oracle_layer(layer, act=act, tile_m=tile_m)
    assert np.array_equal(g["ids"], o["ids"])
    for key in ("counts", "offsets", "sorted_pair", "pair_pos"):
        assert np.array_equal(g[key], o[key]), key
    assert g["err"] == 0
    P = cfg.T * cfg.k
    if act == "a16":
        gh = np.concatenate([g["h"][:P, :cfg.I].ravel(), g["h"][P:, :cfg.I_shared].ravel()])
        oh = np.concatenate([o["h"][:P, :cfg.I].ravel(), o["h"][P:, :cfg.I_shared].ravel()])
    else:
        gh = np.concatenate([g["h32"][:P, :cfg.I].ravel(), g["h32"][P:, :cfg.I_shared].ravel()])
        oh = np.concatenate([o["h32"][:P, :cfg.I].ravel(), o["h32"][P:, :cfg.I_shared].ravel()])
    ok, rl2, worst = h_gate(gh, oh, act)
    assert ok, ("h", rl2, worst)
    check_out(g, g32, o["out"], f"{cfg.name} {act} flags={flags}")
    return g, o


RAW = [("mixed_shared", "a16", f) for f in (0, 1, 3)] + \
      [("mixed_shared", "a8", f) for f in (0, 1, 3)] + \
      [("mixed_shared_a8", "a8", f) for f in (0, 1, 3)] + \
      [("e288", "a16", 0), ("e288", "a8", 3)] + \
      [("mid_mixed_a8", "a8", f) for f in (0, 1, 3)] + \
      [("mid_g256", act, f) for act in ("a16", "a8") for f in (0, 1, 3)] + \
      [("mfma_mixed", "a16", 2), ("mfma_g32_int2", "a16", 2), ("mfma_g32_int2", "a16", 0),
       ("c1", "a16", 0), ("c1", "a16", 3), ("c3_t16", "a8", 0)]


@pytest.mark.parametrize("name,act,flags", RAW)
def test_raw_code_bytes(name, act, flags):
    """Codes from random bytes (int4 -8 and int2 -2 included) on every path."""
    layer = with_random_codes(_base(name), seed=7)
    # every code value occurs in the bank
    for ex in layer.experts[:2] + layer.shared:
        for qm in (ex.w13, ex.w2):
            c = oracle.unpack_codes(qm.codes, qm.bits, qm.K)
            lo = -(1 << (qm.bits - 1))
            assert c.min() == lo and c.max() == -lo - 1
    _run_and_check(layer, act, flags)


def _edge_rows(layer):
    H = layer.cfg.H
    rng = np.random.default_rng(11)
    tiny = (rng.uniform(-1.0, 1.0, H) * 2e-37).astype(np.float32)
    tiny[::5] = 0.0
    tiny[3] = 2e-37                                 # amax 2e-37: scale 2e-37 / 127 < 2^-128
    one_hot = np.zeros(H, np.float32)
    one_hot[7] = 1.5
    big = (rng.standard_normal(H) * 50.0).astype(np.float32)
    rows = {0: np.zeros(H, np.float32), 1: tiny, 2: one_hot, 3: big}
    return with_x_rows(layer, {t: v for t, v in rows.items() if t < layer.cfg.T})


EDGE = [("mixed_shared", "a16", f) for f in (0, 1, 3)] + \
       [("mixed_shared", "a8", f) for f in (0, 1, 3)] + \
       [("mid_mixed_a8", "a8", f) for f in (0, 3)] + \
       [("mfma_g32_int2", "a16", 2), ("c1", "a16", 0), ("c3_t16", "a8", 0)]


@pytest.mark.parametrize("name,act,flags", EDGE)
def test_edge_activation_rows(name, act, flags):
    """Zero, tiny, one-hot and large tokens: the zero token's output is
    exactly zero, the rest pass the float gate."""
    layer = _edge_rows(_base(name))
    g, o = _run_and_check(layer, act, flags)
    assert np.all(g["out"][0] == 0.0) and np.all(o["out"][0] == 0.0)


@pytest.mark.parametrize("name", ["mixed_shared", "c3_t16"])
def test_int8_rows_of_every_maker_match_row_quantizer_on_edge_rows(name):
    """W4A8 x rows are made three ways: by the routing launch of the layer
    call (extra workgroups), by the 16-row gate/up kernel itself (separate
    calls), and by the row quantizer launch (MOE_QUANT_SEPARATE).  On the
    edge rows (zero row, subnormal row scale, zero elements) all three give
    the same codes and scales, so h and out agree bit for bit."""
    from packed_bit_grouped_amd.layer import DeviceLayer
    layer = _edge_rows(_base(name))
    dl = DeviceLayer.from_synth(layer)
    g1, _ = run_layer_gpu(dl, "a8", 16, 3)
    g2, _ = run_layer_gpu(dl, "a8", 16, 3 | 4)
    g3, _ = run_layer_gpu(dl, "a8", 16, 3, fused=False)
    for g in (g2, g3):
        assert np.array_equal(g1["h32"], g["h32"])
        assert np.array_equal(g1["out"], g["out"])
    assert g1["err"] == 0 and g2["err"] == 0 and g3["err"] == 0


@pytest.mark.parametrize("name", ["mixed_shared_a8", "c3_t16"])
def test_gateup_reads_int8_rows_left_by_the_layer_call(name):
    """MOE_X_PREPARED: after a W4A8 layer call the workspace holds x's int8
    rows; a gate/up call that reads them writes the same h as the layer."""
    from packed_bit_grouped_amd import _lib as L
    from packed_bit_grouped_amd.layer import DeviceLayer
    torch = pytest.importorskip("torch")
    layer = _base(name)
    cfg = layer.cfg
    dl = DeviceLayer.from_synth(layer)
    g1, B = run_layer_gpu(dl, "a8", 16, 0)
    B.h.zero_()
    L.moe_w4_gateup_silu(B.act, dl.x, cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dl.bank.w13,
                         dl.bank.w13_sh, cfg.n_shared, cfg.I_shared, B.offsets,
                         B.sorted_pair, B.tiles, B.n_tiles, B.tile_m, B.h, B.ws, B.ws_bytes,
                         L.MOE_X_PREPARED)
    torch.cuda.synchronize()
    h = B.h.cpu().numpy()[:B.R].astype(np.float32)
    assert np.array_equal(h, g1["h32"])


@pytest.mark.parametrize("act", ["a16", "a8"])
def test_ten_repeats_bitwise_identical(act):
    from packed_bit_grouped_amd.layer import DeviceLayer
    layer = make_layer(LAYERS["specdecode_w4a16_t12"])
    dl = DeviceLayer.from_synth(layer)
    ref, _ = run_layer_gpu(dl, act, 16)
    hk = "h" if act == "a16" else "h32"
    for rep in range(9):
        g, _ = run_layer_gpu(dl, act, 16)
        assert np.array_equal(g["out"], ref["out"]), rep
        assert np.array_equal(g[hk], ref[hk]), rep


@pytest.mark.parametrize("tile_m", [160, 64])
def test_prefill_ten_repeats_bitwise_identical(tile_m):
    """The prefill layer (matrix-core path, fixed-order combine) repeated
    ten times: h and out identical bit for bit (compared on the device).
    Tiles of 64 rows give chunks of one or two 32-row blocks, whose K steps
    are the shortest: the hand-counted waits for the activation loads of the
    first steps are exercised hardest there; the separate calls must give
    the same bits as the layer call."""
    import torch
    from packed_bit_grouped_amd.layer import DeviceLayer
    layer = make_layer(LAYERS["prefill_mixed_t4096"])
    dl = DeviceLayer.from_synth(layer)
    B = dl.buffers("a16", tile_m)
    dl.run(B)
    torch.cuda.synchronize()
    h0, out0 = B.h.clone(), B.out.clone()
    for rep in range(9):
        B.h.zero_()
        B.out.zero_()
        dl.run(B)
        torch.cuda.synchronize()
        assert torch.equal(B.h, h0) and torch.equal(B.out, out0), rep
    assert B.error_word() == 0
    B2 = dl.buffers("a16", tile_m)
    dl.run(B2, fused=False)
    torch.cuda.synchronize()
    assert torch.equal(B2.h, h0) and torch.equal(B2.out, out0)
