"""Seeded random shapes across the small domain, each checked against the oracle.

Every case draws N, d, V, K, tau, the dtype, the chunk size and the loss options
together, so ragged tails in every dimension meet each other: the cache build is
bit-exact against the oracle's top-K, then the loss (plain or with a mask and a
cross-entropy mix) on that cache is within the parity tolerances.
"""
import numpy as np
import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd
import oracle
from gpu_util import GRAD_TOL, LOSS_RTOL, LSE_RTOL, bf16_bits_of, device, rel_max_err, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _case(seed):
    g = np.random.default_rng(1000 + seed)
    n = int(g.integers(1, 700))
    d = 8 * int(g.integers(1, 66))
    k = int(g.integers(1, 120))
    v = int(g.integers(max(k, 2), 3000))
    tau = float(np.round(g.uniform(0.3, 3.0), 3))
    dtype = "bf16" if g.random() < 0.7 else "f32"
    chunk = int(g.choice([0, 256, 512]))
    opt = int(g.integers(0, 3))       # 0 plain, 1 mask only, 2 mask and mix
    return n, d, v, k, tau, dtype, chunk, opt


CASES = [_case(s) for s in range(24)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_random_shape(case):
    n, d, v, k, tau, dtype, chunk, opt = case
    print(f"[case] {case}", flush=True)
    vdt = "bf16" if dtype == "bf16" else "f32"
    p = kd_synth.small_problem(n, d, v, seed=n + d + v, dtype=dtype)
    H = kd_synth.to_float64(p["H"], dtype)
    W = kd_synth.to_float64(p["W"], dtype)
    WT = kd_synth.to_float64(p["WT"], dtype)
    idx, valb, _ = oracle.topk_cache(H, WT, k, vdt)
    val = kd_synth.to_float64(valb, vdt)
    h, w = to_dev(p["H"], dtype), to_dev(p["W"], dtype)
    gi, gv = kd.kd_topk_cache_build(h, to_dev(p["WT"], dtype), k, chunk_tokens=chunk)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gi.cpu().numpy(), idx)
    if vdt == "bf16":
        np.testing.assert_array_equal(bf16_bits_of(gv), valb)
    else:
        np.testing.assert_array_equal(gv.cpu().numpy().view(np.uint32), valb.view(np.uint32))

    labels, a = None, 0.0
    if opt:
        g = np.random.default_rng(n * 7 + k)
        labels = g.integers(0, v, size=n).astype(np.int32)
        labels[g.random(n) < 0.2] = -100
        a = 0.35 if opt == 2 else 0.0
        ref_loss, ref_lse, ref_rows = oracle.variant_forward(H, W, idx, val, tau, labels, -100, a)
        ref_dH, ref_dW = oracle.variant_backward(H, W, idx, val, tau, labels, -100, a, grad=0.6)
        kw = dict(labels=torch.from_numpy(labels).to(device()), ce_weight=a)
    else:
        ref_loss, ref_lse, ref_rows = oracle.kl_forward(H, W, idx, val, tau)
        ref_dH, ref_dW = oracle.kl_backward(H, W, idx, val, tau, grad=0.6)
        kw = {}
    gt = torch.tensor(0.6, dtype=torch.float32, device=device())
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, gi, gv, tau, with_rows=True, chunk_tokens=chunk, **kw)
    dh, dw = kd.kd_chunked_kl_bwd(h, w, gi, gv, tau, lse, gt, chunk_tokens=chunk, **kw)
    torch.cuda.synchronize()
    assert abs(loss.item() - ref_loss) <= LOSS_RTOL * max(abs(ref_loss), 1e-6)
    np.testing.assert_allclose(to_f64(lse), ref_lse, rtol=LSE_RTOL)
    np.testing.assert_allclose(to_f64(rows), ref_rows, rtol=5e-3, atol=5e-3)
    if np.abs(ref_dH).max() > 0:
        assert rel_max_err(to_f64(dh), ref_dH) <= GRAD_TOL
        assert rel_max_err(to_f64(dw), ref_dW) <= GRAD_TOL
    else:
        assert not dh.any() and not dw.any()
