"""The on-device router (moe_router_topk) against the fp64 oracle.

Logits are fp32 sums on the device, so they are compared within the
rounding bound of such a sum; the routing of the returned logits must be
exact (ids bit for bit, gate weights to fp32 rounding), and wherever the
exact logits leave margins wider than twice that bound around the chosen
experts the ids must equal those of the exact router."""
import numpy as np
import pytest

import oracle
from synth import LAYERS
from synth.gen import bf16_bits_from_f32
from tests.gpu_util import to_np, torch_mod

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _run(xb, W, prior, k, renorm=1):
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    T, H = xb.shape
    E = W.shape[1]
    dx = torch.from_numpy(xb.view(np.int16).copy()).cuda()
    dw = torch.from_numpy(np.ascontiguousarray(W, dtype=np.float32)).cuda()
    dp = None if prior is None else torch.from_numpy(prior.astype(np.float32)).cuda()
    lg = torch.full((max(T, 1), E), float("nan"), dtype=torch.float32, device="cuda")
    ids = torch.full((max(T, 1), k), -7, dtype=torch.int32, device="cuda")
    w = torch.full((max(T, 1), k), -7.0, dtype=torch.float32, device="cuda")
    nb = L.moe_router_workspace_bytes(T, H, E)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device="cuda")
    L.moe_router_topk(dx, T, H, dw, dp, E, k, renorm, lg, ids, w, ws, nb)
    torch.cuda.synchronize()
    return to_np(lg)[:T], to_np(ids)[:T], to_np(w)[:T]


def _chunks(T, H, E):
    """The library's split of H for a batch (its header: the chunking
    depends only on T, H and E): about 256 workgroups of 64 tokens x 64
    experts, chunks a multiple of 32 long."""
    groups = -(-T // 64) * -(-E // 64)
    n = min(max(-(-256 // groups), 1), -(-H // 32))
    hc = -(-(-(-H // n)) // 32) * 32
    return -(-H // hc), hc


def _check(xb, W, prior, k, renorm=1, min_safe=0.0):
    T, H = xb.shape
    E = W.shape[1]
    pr = None if prior is None else prior.astype(np.float32)
    lg, ids, w = _run(xb, W, pr, k, renorm)
    exact = oracle.router_logits(xb, W, pr)
    # rounding bound of the device's sums: a chain of at most hc fused
    # multiply-adds per chunk (each rounded once), n_chunks chunk sums, the
    # prior and the final rounding, with 1% slack for second-order terms
    n_chunks, hc = _chunks(T, H, E)
    mag = np.abs(oracle.x_float(xb)) @ np.abs(W.astype(np.float64))
    if pr is not None:
        mag = mag + np.abs(pr.astype(np.float64))[None, :]
    bound = 1.01 * (hc + n_chunks + 2) * U32 * mag + U32 * np.abs(exact) + 1e-30
    err = np.abs(lg.astype(np.float64) - exact)
    assert np.all(err <= bound), float((err / bound).max())
    assert np.linalg.norm(err) <= 1e-5 * np.linalg.norm(exact) + 1e-12
    # exact routing of the device's own logits
    oi, ow = oracle.route_topk(lg, k, renorm)
    assert np.array_equal(ids, oi)
    assert np.allclose(w, ow, rtol=2e-6, atol=1e-7)
    # margin-aware agreement with the exact router
    ei, _ = oracle.route_topk(exact.astype(np.float32), k, renorm)
    srt = -np.sort(-exact, axis=1)[:, :min(k + 1, E)]
    gaps = srt[:, :-1] - srt[:, 1:] if srt.shape[1] > 1 else np.full((T, 1), np.inf)
    tb = bound.max(axis=1)
    safe = np.all(gaps > 2 * tb[:, None], axis=1)
    assert np.array_equal(ids[safe], ei[safe])
    assert safe.mean() >= min_safe, safe.mean()
    return safe.mean()


@pytest.mark.parametrize("lname", ["tiny_w4a16", "decode_w4a16_t1", "specdecode_w4a16_t12",
                                   "decode_w4a8_t64"])
def test_router_on_benchmark_layer_inputs(lname):
    """The benchmark layers' own router inputs (the speculative-decode layer
    with its Zipf prior)."""
    from tests.test_gpu_parity import _layer
    layer = _layer(LAYERS[lname])
    cfg = layer.cfg
    print(f"[router] {lname}: T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k}", flush=True)
    frac = _check(layer.x_bf16, layer.router_w, layer.bias, cfg.k, cfg.renormalize,
                  min_safe=0.5 if cfg.T >= 12 else 0.0)
    print(f"[router] {lname}: {frac:.2f} of the tokens have margins over the bound",
          flush=True)


@pytest.mark.parametrize("T,H,E,k,renorm,seed,min_safe", [
    (4096, 4096, 256, 8, 1, 0, 0.1),   # prefill-sized batch: one 4096-long chunk (loose bound)
    (33, 96, 300, 5, 1, 1, 0.5),       # two expert groups, H not a multiple of 128
    (1, 64, 1, 1, 1, 2, 1.0),          # E = 1
    (7, 4000, 64, 64, 0, 3, 0.0),      # k = E, no renormalisation, ragged H chunks
    (17, 2048, 1024, 8, 1, 4, 0.3),    # E at its limit
])
def test_router_synthetic_shapes(T, H, E, k, renorm, seed, min_safe):
    """Seeded inputs with the benchmark's distributions (x ~ N(0, 1) as
    bf16, router weights ~ N(0, 0.02))."""
    rng = np.random.default_rng(1000 + seed)
    print(f"[router] T={T} H={H} E={E} k={k}", flush=True)
    xb = bf16_bits_from_f32(rng.standard_normal((T, H), dtype=np.float32))
    W = (rng.standard_normal((H, E), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    frac = _check(xb, W, None, k, renorm, min_safe)
    print(f"[router] {frac:.2f} of the tokens have margins over the bound", flush=True)


def test_router_zero_batch_and_ties():
    """T = 0 launches nothing; tokens whose logits tie exactly (duplicate
    router columns) route to the lower index, as the exact router does."""
    torch = torch_mod()
    from packed_bit_grouped_amd import _lib as L
    assert L.moe_router_topk(None, 0, 64, None, None, 8, 2, 1, None, None, None, None, 0) == 0
    rng = np.random.default_rng(7)
    H, E = 256, 16
    W = (rng.standard_normal((H, E), dtype=np.float32) * np.float32(0.02)).astype(np.float32)
    W[:, 9] = W[:, 2]          # experts 2 and 9 always tie
    W[:, 12] = W[:, 2] * 3.0   # and 12 dominates them
    xb = bf16_bits_from_f32(rng.standard_normal((5, H), dtype=np.float32))
    lg, ids, _ = _run(xb, W, None, 3)
    assert np.array_equal(lg[:, 2], lg[:, 9])
    oi, _ = oracle.route_topk(lg, 3, 1)
    assert np.array_equal(ids, oi)
    torch.cuda.synchronize()
