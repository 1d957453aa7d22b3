"""The student renormalised over the cached entries (kd_loss_opts.student =
KD_STUDENT_RENORM) against the float64 oracle (``oracle.renorm_forward`` /
``renorm_backward``): ragged shapes in bf16 and float32, two chunkings, with and
without a padding mask; repeated indices; the whole vocabulary cached (where it
equals the full-vocabulary loss); one cached entry (zero loss and gradient); W rows
outside every cache row get exactly zero gradient; autograd and the module; the
option errors; and 32,768 tokens at V = 128,256, d = 4,096 on sampled rows."""
import numpy as np
import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd
import oracle
from gpu_util import GRAD_TOL, LOSS_RTOL, LSE_RTOL, bf16_bits_of, device, rel_max_err, to_dev, to_f64

pytestmark = pytest.mark.gpu

IGN = -100
SHAPES = [
    (300, 136, 1000, 7, "bf16", 1.0),
    (520, 264, 1300, 33, "bf16", 2.0),
    (700, 128, 2600, 100, "f32", 1.5),
    (257, 512, 4099, 64, "bf16", 0.7),
    (1, 8, 50, 50, "bf16", 1.0),
]


def _setup(n, d, v, k, dtype, seed=0, distinct=True):
    p = kd_synth.small_problem(n, d, v, seed=seed, dtype=dtype)
    vdt = "bf16" if dtype == "bf16" else "f32"
    idx, valb = kd_synth.random_cache(n, v, k, seed=seed + 1, val_dtype=vdt, distinct=distinct)
    H = kd_synth.to_float64(p["H"], dtype)
    W = kd_synth.to_float64(p["W"], dtype)
    val = kd_synth.to_float64(valb, vdt)
    dev = (to_dev(p["H"], dtype), to_dev(p["W"], dtype), torch.from_numpy(idx).to(device()), to_dev(valb, vdt))
    return H, W, idx, val, dev


def _run(dev, tau, labels=None, chunk=0, g=None, dh_dtype=torch.float32):
    h, w, ti, tv = dev
    tl = None if labels is None else torch.from_numpy(labels).to(device())
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, ti, tv, tau, with_rows=True, chunk_tokens=chunk, labels=tl,
                                           student="renorm")
    gt = None if g is None else torch.tensor(g, dtype=torch.float32, device=device())
    dh, dw = kd.kd_chunked_kl_bwd(h, w, ti, tv, tau, lse, gt, dh_dtype=dh_dtype, chunk_tokens=chunk, labels=tl,
                                  student="renorm")
    torch.cuda.synchronize()
    return loss, lse, rows, dh, dw


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("chunk", [0, 256])
@pytest.mark.parametrize("masked", [False, True])
def test_renorm_matches_oracle(shape, chunk, masked):
    n, d, v, k, dtype, tau = shape
    H, W, idx, val, dev = _setup(n, d, v, k, dtype, seed=21)
    labels = None
    if masked:
        labels = np.zeros(n, dtype=np.int32)
        labels[np.random.default_rng(22).random(n) < 0.25] = IGN
        if n > 1:
            labels[0] = IGN
    g = 0.37
    ref_loss, ref_lse, ref_rows = oracle.renorm_forward(H, W, idx, val, tau, labels, IGN)
    ref_dH, ref_dW = oracle.renorm_backward(H, W, idx, val, tau, labels, IGN, grad=g)
    loss, lse, rows, dh, dw = _run(dev, tau, labels, chunk, g)
    assert abs(loss.item() - ref_loss) <= LOSS_RTOL * max(abs(ref_loss), 1e-6), (loss.item(), ref_loss)
    keep = np.isfinite(ref_lse)
    np.testing.assert_allclose(to_f64(lse)[keep], ref_lse[keep], rtol=LSE_RTOL)
    assert np.all(np.isnan(to_f64(lse)[~keep]))
    np.testing.assert_allclose(to_f64(rows), ref_rows, rtol=LOSS_RTOL, atol=LOSS_RTOL)
    assert rel_max_err(to_f64(dh), ref_dH) <= GRAD_TOL
    assert rel_max_err(to_f64(dw), ref_dW) <= GRAD_TOL
    if masked:
        assert not dh[torch.from_numpy(labels == IGN).to(device())].any()


def test_renorm_repeated_indices_bitwise_repeatable():
    n, d, v, k = 260, 64, 300, 40
    H, W, idx, val, dev = _setup(n, d, v, k, "bf16", seed=23, distinct=False)
    idx[:, 20:] = idx[:, :20]                      # every row repeats its first 20 indices
    dev = (dev[0], dev[1], torch.from_numpy(idx).to(device()), dev[3])
    ref_loss, _, _ = oracle.renorm_forward(H, W, idx, val, 1.0)
    ref_dH, ref_dW = oracle.renorm_backward(H, W, idx, val, 1.0)
    loss, lse, rows, dh, dw = _run(dev, 1.0)
    _, _, _, dh2, dw2 = _run(dev, 1.0)
    assert abs(loss.item() - ref_loss) <= LOSS_RTOL * abs(ref_loss)
    assert rel_max_err(to_f64(dh), ref_dH) <= GRAD_TOL and rel_max_err(to_f64(dw), ref_dW) <= GRAD_TOL
    assert torch.equal(dh, dh2) and torch.equal(dw, dw2)


def test_renorm_whole_vocabulary_equals_the_full_loss():
    """K = V: the cached set is the vocabulary, so the renormalised student is the
    full one; the two options agree (loss, lse, gradients) within the tolerances."""
    n, d, v = 200, 64, 500
    p = kd_synth.small_problem(n, d, v, seed=24, dtype="bf16")
    g = np.random.default_rng(25)
    idx = np.stack([g.permutation(v) for _ in range(n)]).astype(np.int32)
    valb = kd_synth.bf16_bits_from_f32(g.standard_normal((n, v)).astype(np.float32) * 2)
    h, w = to_dev(p["H"], "bf16"), to_dev(p["W"], "bf16")
    ti, tv = torch.from_numpy(idx).to(device()), to_dev(valb, "bf16")
    l_f, lse_f, _ = kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.2)
    dh_f, dw_f = kd.kd_chunked_kl_bwd(h, w, ti, tv, 1.2, lse_f)
    l_r, lse_r, _ = kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.2, student="renorm")
    dh_r, dw_r = kd.kd_chunked_kl_bwd(h, w, ti, tv, 1.2, lse_r, student="renorm")
    torch.cuda.synchronize()
    assert abs(l_f.item() - l_r.item()) <= LOSS_RTOL * abs(l_f.item())
    np.testing.assert_allclose(to_f64(lse_r), to_f64(lse_f), rtol=LSE_RTOL)
    assert rel_max_err(to_f64(dh_r), to_f64(dh_f)) <= GRAD_TOL
    assert rel_max_err(to_f64(dw_r), to_f64(dw_f)) <= GRAD_TOL


@pytest.mark.parametrize("case", ["one_long_row", "many_token_tiles"])
def test_renorm_dw_long_rows_and_many_token_tiles(case):
    """The dW kernel's limits: one vocabulary row holding thousands of a tile's entries
    (several LDS pieces, each overflowing a wave's row list, so the row's sum goes
    through partial sums in dW), and a chunk of more than 256 token tiles (the tiles'
    segment starts held in several groups)."""
    if case == "one_long_row":
        n, d, v, k, chunk = 1200, 64, 300, 8, 0
    else:
        n, d, v, k, chunk = 66000, 64, 700, 6, 131072
    H, W, idx, val, dev = _setup(n, d, v, k, "bf16", seed=28, distinct=False)
    if case == "one_long_row":
        idx[:, :4] = 5                              # row 5: 4,800 entries, every 4,096-entry piece
        dev = (dev[0], dev[1], torch.from_numpy(idx).to(device()), dev[3])
    ref_loss, _, _ = oracle.renorm_forward(H, W, idx, val, 1.0)
    ref_dH, ref_dW = oracle.renorm_backward(H, W, idx, val, 1.0)
    loss, lse, rows, dh, dw = _run(dev, 1.0, chunk=chunk)
    _, _, _, dh2, dw2 = _run(dev, 1.0, chunk=chunk)
    assert abs(loss.item() - ref_loss) <= LOSS_RTOL * abs(ref_loss)
    assert rel_max_err(to_f64(dh), ref_dH) <= GRAD_TOL and rel_max_err(to_f64(dw), ref_dW) <= GRAD_TOL
    assert torch.equal(dh, dh2) and torch.equal(dw, dw2)


def test_renorm_single_entry_and_off_set_rows():
    n, d, v = 300, 64, 2000
    H, W, idx, val, dev = _setup(n, d, v, 1, "bf16", seed=26)
    loss, lse, rows, dh, dw = _run(dev, 1.0)
    assert loss.item() == 0.0 and not rows.any() and not dh.any() and not dw.any()
    H, W, idx, val, dev = _setup(n, d, v, 8, "bf16", seed=27)
    _, _, _, _, dw = _run(dev, 1.0)
    off = np.setdiff1d(np.arange(v), idx.ravel())
    assert off.size > 0
    assert not dw[torch.from_numpy(off).to(device())].any()


def test_renorm_autograd_and_module():
    n, d, v, k = 96, 64, 700, 12
    H, W, idx, val, dev = _setup(n, d, v, k, "bf16", seed=28)
    h, w, ti, tv = dev
    hh = h.clone().requires_grad_(True)
    ww = w.clone().requires_grad_(True)
    crit = kd.ChunkedTopKKLLoss(tau=1.0, student="renorm")
    loss = crit(hh.view(2, 48, d), ww, ti.view(2, 48, k), tv.view(2, 48, k)) * 0.5
    loss.backward()
    ref_loss, _, _ = oracle.renorm_forward(H, W, idx, val, 1.0)
    ref_dH, ref_dW = oracle.renorm_backward(H, W, idx, val, 1.0, grad=0.5)
    assert abs(loss.item() - 0.5 * ref_loss) <= LOSS_RTOL * abs(0.5 * ref_loss)
    assert rel_max_err(to_f64(hh.grad), ref_dH) <= GRAD_TOL
    assert rel_max_err(to_f64(ww.grad), ref_dW) <= GRAD_TOL
    assert "student='renorm'" in repr(crit)


def test_renorm_option_errors():
    n, d, v, k = 64, 64, 300, 4
    _, _, _, _, (h, w, ti, tv) = _setup(n, d, v, k, "bf16", seed=29)
    lab = torch.zeros(n, dtype=torch.int32, device=device())
    with pytest.raises(kd.KDError) as e:
        kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.0, labels=lab, ce_weight=0.3, student="renorm")
    assert e.value.status == 14
    with pytest.raises(ValueError):
        kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.0, student="other")


def test_renorm_ctx32k_v128k_sampled_rows():
    """32,768 tokens at V = 128,256, d = 4,096 with the teacher cache built on the GPU:
    sampled rows' KL, normaliser and dH against the oracle; the loss is the mean of
    the rows; dW's columns sum to zero (each dZ row sums to zero) up to the bf16
    rounding of dZ."""
    w_ = kd_synth.WORKLOADS["ctx32k_v128k"]
    n, k = 32768, 100
    print(f"[renorm] {w_.name} N={n} K={k}", flush=True)
    Hb, Wb = kd_synth.hidden(w_, n), kd_synth.student_head(w_)
    h, w = to_dev(Hb, "bf16"), to_dev(Wb, "bf16")
    wt = to_dev(kd_synth.teacher_head(w_), "bf16")
    ti, tv = kd.kd_topk_cache_build(h, wt, k)
    del wt
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, ti, tv, w_.tau, with_rows=True, student="renorm")
    dh, dw = kd.kd_chunked_kl_bwd(h, w, ti, tv, w_.tau, lse, None, dh_dtype=torch.bfloat16, student="renorm")
    torch.cuda.synchronize()
    rs = np.unique(np.concatenate([[0, n - 1, 16383, 16384], np.random.default_rng(30).choice(n, 28, replace=False)]))
    rs_t = torch.from_numpy(rs).to(device())
    H64 = kd_synth.to_float64(Hb[rs], "bf16")
    W64 = kd_synth.to_float64(Wb, "bf16")
    ih = ti[rs_t].cpu().numpy()
    v64 = kd_synth.to_float64(bf16_bits_of(tv[rs_t]), "bf16")
    _, ref_lse, ref_rows = oracle.renorm_forward(H64, W64, ih, v64, w_.tau)
    np.testing.assert_allclose(to_f64(lse[rs_t]), ref_lse, rtol=LSE_RTOL)
    np.testing.assert_allclose(to_f64(rows[rs_t]), ref_rows, rtol=LOSS_RTOL, atol=LOSS_RTOL)
    ref_dH, _ = oracle.renorm_backward(H64, W64, ih, v64, w_.tau)
    ref_dH *= len(rs) / n
    assert rel_max_err(to_f64(dh[rs_t]), ref_dH) <= GRAD_TOL
    r_all = rows.double()
    assert torch.isfinite(r_all).all()
    assert abs(r_all.mean().item() - loss.item()) <= 1e-5 * abs(loss.item())
    dw64 = dw.double()
    colsum = dw64.sum(0).abs()
    bound = 2.0 ** -7 / n * h.double().abs().sum(0) * 1.01 + 2.0 ** -20 * dw64.abs().sum(0)
    assert bool((colsum <= bound).all()), float((colsum / bound).max())
