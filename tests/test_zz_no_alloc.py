"""moe_w4_layer_noalloc (the layer with the library's static device
scratch array as its workspace) against moe_w4_layer with a caller
workspace: identical routing tables, h and outputs, bit for bit, on two
calls in a row, the second with a smaller layer (the array keeps the first
call's contents), then the one-launch form (its barrier flags live in the
array too)."""
import numpy as np
import pytest

from synth import LAYERS, make_layer
from tests.gpu_util import collect

pytestmark = pytest.mark.gpu


def _noalloc(L, dl, B, flags, err):
    c = dl.cfg
    L.moe_w4_layer_noalloc(B.act, dl.logits, dl.x, c.T, c.H, c.I, c.E, c.k, c.renormalize,
                           dl.bank.w13, dl.bank.w2, dl.bank.w13_sh, dl.bank.w2_sh,
                           c.n_shared, c.I_shared, B.tile_m, B.ids, B.w, B.counts, B.offsets,
                           B.sorted_pair, B.pair_pos, B.tiles, B.n_tiles, B.h, B.out, err,
                           flags | B.out_flags)


def test_noalloc_matches_workspace_calls():
    import torch
    from packed_bit_grouped_amd import _lib as L
    from packed_bit_grouped_amd.layer import DeviceLayer
    cases = [("decode_w4a8_t64", "a8", 0), ("decode_w4a16_t1", "a16", 0),
             ("decode_w4a16_t1", "a16", L.MOE_LAYER_ONE_LAUNCH),
             ("specdecode_w4a16_t12", "a16", 0)]
    for name, act, flags in cases:
        cfg = LAYERS[name]
        print(f"[noalloc] {name} act={act} flags={flags}", flush=True)
        dl = DeviceLayer.from_synth(make_layer(cfg))
        ref_b = dl.buffers(act)
        assert ref_b.ws_bytes <= L.MOE_NOALLOC_SCRATCH_BYTES
        dl.run(ref_b, flags)
        torch.cuda.synchronize()
        ref = collect(ref_b)
        B = dl.buffers(act)
        B.out.fill_(0x7FFF)
        err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        _noalloc(L, dl, B, flags, err)
        torch.cuda.synchronize()
        got = collect(B)
        for key in ("ids", "w", "counts", "offsets", "sorted_pair", "pair_pos", "tiles",
                    "n_tiles", "out"):
            assert np.array_equal(got[key], ref[key]), (name, key)
        hk = "h" if act == "a16" else "h32"
        assert np.array_equal(got[hk], ref[hk]), (name, "h")
        assert int(err.item()) == 0 and ref["err"] == 0


def test_noalloc_rejects_shapes_beyond_the_scratch():
    from packed_bit_grouped_amd import _lib as L
    import torch
    t = torch.zeros(64, dtype=torch.int32, device="cuda")
    # the prefill chunk needs ~0.6 GB of workspace: rejected on the host
    st = L.moe_w4_layer_noalloc(0, t, t, 4096, 4096, 1536, 256, 8, 1, t, t, None, None, 0, 0,
                                160, t, t, t, t, t, t, t, t, t, t, None, 0, check=False)
    assert st == L.MOE_E_WORKSPACE
