"""Parity at the limits of the shape domain (include/kdkl.h).

* the largest K of the loss (65,535), also with a mixed-in label, whose entry
  index k = K = 65,535 is the last value of the bucket entry's 16-bit field;
* the largest vocabulary (2,097,088 = 2^21 - 64, 8,192 tiles, where one 256-row
  tile of dZ or W^T nears the 2^31-byte reach of the loads' offsets) at the
  smallest hidden size (d = 8), for the loss and the cache build;
* the largest K of the cache build (4,096), through both selection paths;
* a cache of more than 2^31 entries (N K), so every offset into idx and val
  must be 64-bit; checked on sampled rows and through the loss's definition as
  the mean of its rows.
"""
import numpy as np
import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd
import oracle
from gpu_util import (GRAD_TOL, LOSS_RTOL, LSE_RTOL, bf16_bits_of, device, rel_max_err, to_dev, to_f64)

pytestmark = pytest.mark.gpu

KMAX = 65535
VMAX = 2097088


def _loss_case(n, d, v, k, seed, tau=1.0, labels=None, a=0.0, chunk=0):
    p = kd_synth.small_problem(n, d, v, seed=seed)
    H = kd_synth.to_float64(p["H"], "bf16")
    W = kd_synth.to_float64(p["W"], "bf16")
    idx, valb = kd_synth.random_cache(n, v, k, seed=seed + 1)
    val = kd_synth.to_float64(valb, "bf16")
    if labels is None:
        ref_loss, ref_lse, ref_rows = oracle.kl_forward(H, W, idx, val, tau)
        ref_dH, ref_dW = oracle.kl_backward(H, W, idx, val, tau)
    else:
        ref_loss, ref_lse, ref_rows = oracle.variant_forward(H, W, idx, val, tau, labels, -100, a)
        ref_dH, ref_dW = oracle.variant_backward(H, W, idx, val, tau, labels, -100, a)
    h, w = to_dev(p["H"], "bf16"), to_dev(p["W"], "bf16")
    ti, tv = torch.from_numpy(idx).to(device()), to_dev(valb, "bf16")
    opt = {} if labels is None else dict(labels=torch.from_numpy(labels).to(device()), ce_weight=a)
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, ti, tv, tau, with_rows=True, chunk_tokens=chunk, **opt)
    dh, dw = kd.kd_chunked_kl_bwd(h, w, ti, tv, tau, lse, None, chunk_tokens=chunk, **opt)
    torch.cuda.synchronize()
    assert abs(loss.item() - ref_loss) <= LOSS_RTOL * abs(ref_loss)
    np.testing.assert_allclose(to_f64(lse), ref_lse, rtol=LSE_RTOL)
    np.testing.assert_allclose(to_f64(rows), ref_rows, rtol=5e-3, atol=5e-3)
    assert rel_max_err(to_f64(dh), ref_dH) <= GRAD_TOL
    assert rel_max_err(to_f64(dw), ref_dW) <= GRAD_TOL


def test_largest_k():
    print(f"[case] K={KMAX}", flush=True)
    _loss_case(40, 16, 70000, KMAX, seed=61)


def test_largest_k_with_mixed_label():
    """The label is gathered as entry k = K = 65,535."""
    print(f"[case] K={KMAX} with labels", flush=True)
    n, v = 40, 70000
    labels = np.random.default_rng(62).integers(0, v, size=n).astype(np.int32)
    labels[[3, 17]] = -100
    _loss_case(n, 16, v, KMAX, seed=63, labels=labels, a=0.4)


def test_largest_vocabulary_loss():
    print(f"[case] V={VMAX} d=8", flush=True)
    _loss_case(32, 8, VMAX, 8, seed=64, tau=2.0)


def test_largest_vocabulary_cache_build():
    print(f"[case] cache build V={VMAX} d=8", flush=True)
    n, d, v, k = 24, 8, VMAX, 8
    p = kd_synth.small_problem(n, d, v, seed=65)
    ref_idx, ref_val, _ = oracle.topk_cache(kd_synth.to_float64(p["H"], "bf16"),
                                            kd_synth.to_float64(p["WT"], "bf16"), k, "bf16")
    gi, gv = kd.kd_topk_cache_build(to_dev(p["H"], "bf16"), to_dev(p["WT"], "bf16"), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gi.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(bf16_bits_of(gv), ref_val)


@pytest.mark.parametrize("n,v", [(300, 20000), (16, 600000)], ids=["radix", "fast-bound"])
def test_largest_cache_build_k(n, v):
    """K = 4,096.  At V = 20,000 the tiles' top-2 pairs are fewer than K, so every
    row takes the radix selection; at V = 600,000 they are more, so the fast
    path's bound applies first (and hands over rows whose candidates overflow)."""
    k = 4096
    print(f"[case] cache build K={k} N={n} V={v}", flush=True)
    p = kd_synth.small_problem(n, 16, v, seed=66)
    ref_idx, ref_val, _ = oracle.topk_cache(kd_synth.to_float64(p["H"], "bf16"),
                                            kd_synth.to_float64(p["WT"], "bf16"), k, "bf16")
    gi, gv = kd.kd_topk_cache_build(to_dev(p["H"], "bf16"), to_dev(p["WT"], "bf16"), k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gi.cpu().numpy(), ref_idx)
    np.testing.assert_array_equal(bf16_bits_of(gv), ref_val)


def test_cache_larger_than_2_31_entries():
    """N K = 2,307,197,200 > 2^31 entries (9.2 GB of indices, 4.6 GB of values).
    The cache is built on the device from a closed form (distinct indices per row:
    7 is invertible mod 2,048) in row blocks; sampled rows go to the oracle."""
    n, d, v, k = (1 << 21) + 300, 8, 2048, 1100
    print(f"[case] N*K={n * k}", flush=True)
    p = kd_synth.small_problem(n, d, v, seed=67)
    h, w = to_dev(p["H"], "bf16"), to_dev(p["W"], "bf16")
    idx = torch.empty((n, k), dtype=torch.int32, device=device())
    val = torch.empty((n, k), dtype=torch.bfloat16, device=device())
    kk = torch.arange(k, device=device(), dtype=torch.int64)
    for r0 in range(0, n, 1 << 17):
        r1 = min(n, r0 + (1 << 17))
        rr = torch.arange(r0, r1, device=device(), dtype=torch.int64)[:, None]
        idx[r0:r1] = ((rr * 131 + kk[None, :] * 7) % v).to(torch.int32)
        val[r0:r1] = (torch.sin(rr.double() * 0.37 + kk[None, :].double() * 0.011) * 3.0).to(torch.bfloat16)
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, idx, val, 1.0, with_rows=True)
    dh, dw = kd.kd_chunked_kl_bwd(h, w, idx, val, 1.0, lse, None)
    torch.cuda.synchronize()
    g = np.random.default_rng(68)
    rs = np.unique(np.concatenate([[0, n - 1, (1 << 21) - 1, 1 << 21], g.choice(n, size=20, replace=False)]))
    rs_t = torch.from_numpy(rs).to(device())
    H64 = kd_synth.to_float64(p["H"][rs], "bf16")
    W64 = kd_synth.to_float64(p["W"], "bf16")
    i_s = idx[rs_t].cpu().numpy()
    v_s = val[rs_t].float().cpu().numpy().astype(np.float64)
    _, ref_lse, ref_rows = oracle.kl_forward(H64, W64, i_s, v_s, 1.0)
    np.testing.assert_allclose(to_f64(lse[rs_t]), ref_lse, rtol=LSE_RTOL)
    np.testing.assert_allclose(to_f64(rows[rs_t]), ref_rows, rtol=LOSS_RTOL, atol=LOSS_RTOL)
    ref_dH, _ = oracle.kl_backward(H64, W64, i_s, v_s, 1.0)
    assert rel_max_err(to_f64(dh[rs_t]), ref_dH * (len(rs) / n)) <= GRAD_TOL
    r_all = rows.double()
    assert torch.isfinite(r_all).all()
    assert abs(r_all.mean().item() - loss.item()) <= 1e-5 * abs(loss.item())
    assert torch.isfinite(dw).all()
