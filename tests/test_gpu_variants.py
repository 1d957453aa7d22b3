"""Parity of the loss variants (padding mask, hard-label cross-entropy mix; the
``kd_chunked_kl_fwd_ex`` / ``kd_chunked_kl_bwd_ex`` calls) with the float64
oracle (``oracle.variant_forward`` / ``variant_backward``).

Ignored rows carry garbage cache entries (out-of-range indices, NaN logits):
the kernels must not read them, so any read would show up as NaN.  Labels are
drawn over the vocabulary, and some repeat one of their row's cached indices,
so the label and a cached entry meet in the gradient scatter.
"""
import os

import numpy as np
import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd
import oracle
from gpu_util import GRAD_TOL, LOSS_RTOL, LSE_RTOL, device, rel_max_err, to_dev, to_f64

pytestmark = pytest.mark.gpu

IGN = -100

# (N, d, V, K, dtype, tau): ragged tails in every dimension, as in the plain parity tests
SHAPES = [
    (300, 136, 1000, 7, "bf16", 1.0),
    (520, 264, 1300, 33, "bf16", 2.0),
    (700, 128, 2600, 100, "f32", 1.5),
    (33, 8, 257, 5, "f32", 0.7),
]


def _inputs(n, d, v, k, dtype, seed, ignore_frac=0.15):
    p = kd_synth.small_problem(n, d, v, seed=seed, dtype=dtype)
    vdt = "bf16" if dtype == "bf16" else "f32"
    idx, valb = kd_synth.random_cache(n, v, k, seed=seed + 1, val_dtype=vdt)
    g = np.random.default_rng(seed + 2)
    labels = g.integers(0, v, size=n).astype(np.int32)
    hit = g.random(n) < 0.3
    labels[hit] = idx[hit, g.integers(0, k, size=int(hit.sum()))]      # label = a cached index
    ign = g.random(n) < ignore_frac
    if n > 2:
        ign[[0, n - 1]] = [True, False]
    labels[ign] = IGN
    idx[ign] = v + 7                                                     # garbage, never read
    valb = valb.copy()
    valb[ign] = 0x7FC0 if vdt == "bf16" else np.float32(np.nan)
    return p, vdt, idx, valb, labels


def _gpu(p, dtype, idx, valb, labels, vdt):
    h, w = to_dev(p["H"], dtype), to_dev(p["W"], dtype)
    return h, w, torch.from_numpy(idx).to(device()), to_dev(valb, vdt), torch.from_numpy(labels).to(device())


def _val64(valb, vdt):
    with np.errstate(invalid="ignore"):
        return kd_synth.to_float64(valb, vdt)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("a", [0.0, 0.3, 1.0])
@pytest.mark.parametrize("chunk", [0, 256])
def test_variants_match_oracle(shape, a, chunk):
    n, d, v, k, dtype, tau = shape
    print(f"[case] variants {shape} a={a} chunk={chunk}", flush=True)
    p, vdt, idx, valb, labels = _inputs(n, d, v, k, dtype, seed=n + k)
    H = kd_synth.to_float64(p["H"], dtype)
    W = kd_synth.to_float64(p["W"], dtype)
    val = _val64(valb, vdt)
    ref_loss, ref_lse, ref_rows = oracle.variant_forward(H, W, idx, val, tau, labels, IGN, a)
    g = 0.37
    ref_dH, ref_dW = oracle.variant_backward(H, W, idx, val, tau, labels, IGN, a, grad=g)

    h, w, ti, tv, tl = _gpu(p, dtype, idx, valb, labels, vdt)
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, ti, tv, tau, with_rows=True, chunk_tokens=chunk,
                                           labels=tl, ignore_index=IGN, ce_weight=a)
    gt = torch.tensor(g, dtype=torch.float32, device=device())
    dh, dw = kd.kd_chunked_kl_bwd(h, w, ti, tv, tau, lse, gt, chunk_tokens=chunk, labels=tl,
                                  ignore_index=IGN, ce_weight=a)
    torch.cuda.synchronize()

    assert abs(loss.item() - ref_loss) <= LOSS_RTOL * abs(ref_loss)
    np.testing.assert_allclose(to_f64(lse), ref_lse, rtol=LSE_RTOL)
    np.testing.assert_allclose(to_f64(rows), ref_rows, rtol=5e-3, atol=5e-3)
    ign = labels == IGN
    assert np.all(to_f64(rows)[ign] == 0.0)
    assert rel_max_err(to_f64(dh), ref_dH) <= GRAD_TOL
    assert rel_max_err(to_f64(dw), ref_dW) <= GRAD_TOL
    assert not to_f64(dh)[ign].any()


def test_no_ignored_rows_and_no_mix_is_bitwise_the_plain_loss():
    """Labels that leave no row out, with no mix, give the plain call's bits."""
    n, d, v, k = 600, 128, 1500, 16
    p = kd_synth.small_problem(n, d, v, seed=21)
    idx, valb = kd_synth.random_cache(n, v, k, seed=22)
    labels = np.random.default_rng(23).integers(0, v, size=n).astype(np.int32)
    h, w, ti, tv, tl = _gpu(p, "bf16", idx, valb, labels, "bf16")
    gt = torch.tensor(0.5, dtype=torch.float32, device=device())
    a = kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.3, with_rows=True, chunk_tokens=256)
    b = kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.3, with_rows=True, chunk_tokens=256, labels=tl, ignore_index=IGN)
    ga = kd.kd_chunked_kl_bwd(h, w, ti, tv, 1.3, a[1], gt, chunk_tokens=256)
    gb = kd.kd_chunked_kl_bwd(h, w, ti, tv, 1.3, b[1], gt, chunk_tokens=256, labels=tl, ignore_index=IGN)
    torch.cuda.synchronize()
    for x, y in zip(a + ga, b + gb):
        assert torch.equal(x, y)


def test_every_row_ignored():
    n, d, v, k = 300, 64, 700, 4
    p = kd_synth.small_problem(n, d, v, seed=24)
    idx = np.full((n, k), -1, np.int32)
    valb = np.full((n, k), 0x7FC0, np.uint16)
    labels = np.full(n, IGN, np.int32)
    h, w, ti, tv, tl = _gpu(p, "bf16", idx, valb, labels, "bf16")
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.0, with_rows=True, labels=tl, ce_weight=0.5)
    dh, dw = kd.kd_chunked_kl_bwd(h, w, ti, tv, 1.0, lse, None, labels=tl, ce_weight=0.5)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and not rows.any() and torch.isfinite(lse).all()
    assert not dh.any() and not dw.any()
    ref_lse = oracle.logsumexp_rows(kd_synth.to_float64(p["H"], "bf16") @ kd_synth.to_float64(p["W"], "bf16").T)
    np.testing.assert_allclose(to_f64(lse), ref_lse, rtol=LSE_RTOL)


def test_out_of_range_label_gives_nan_row_not_a_fault():
    n, d, v, k = 300, 64, 600, 5
    p = kd_synth.small_problem(n, d, v, seed=25)
    idx, valb = kd_synth.random_cache(n, v, k, seed=26)
    labels = np.random.default_rng(27).integers(0, v, size=n).astype(np.int32)
    labels[[17, 200]] = [v, -3]
    h, w, ti, tv, tl = _gpu(p, "bf16", idx, valb, labels, "bf16")
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.0, with_rows=True, labels=tl, ce_weight=0.5)
    dh, dw = kd.kd_chunked_kl_bwd(h, w, ti, tv, 1.0, lse, None, labels=tl, ce_weight=0.5)
    torch.cuda.synchronize()
    r = rows.cpu().numpy()
    assert np.isnan(r[17]) and np.isnan(r[200]) and np.isfinite(np.delete(r, [17, 200])).all()
    assert torch.isfinite(dh).all() and torch.isfinite(dw).all()
    # with no mix the labels only mask, and their values are not used
    loss0, _, rows0 = kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.0, with_rows=True, labels=tl, ce_weight=0.0)
    torch.cuda.synchronize()
    assert torch.isfinite(rows0).all()


def test_autograd_with_options():
    n, d, v, k = 400, 64, 900, 8
    p, vdt, idx, valb, labels = _inputs(n, d, v, k, "bf16", seed=28)
    h, w, ti, tv, tl = _gpu(p, "bf16", idx, valb, labels, vdt)
    hb, wb = h.clone().requires_grad_(), w.clone().requires_grad_()
    loss = kd.chunked_kl_loss(hb, wb, ti, tv, 1.5, labels=tl, ignore_index=IGN, ce_weight=0.25)
    (2.0 * loss).backward()
    H = kd_synth.to_float64(p["H"], "bf16")
    W = kd_synth.to_float64(p["W"], "bf16")
    val = _val64(valb, vdt)
    ref_loss, _, _ = oracle.variant_forward(H, W, idx, val, 1.5, labels, IGN, 0.25)
    ref_dH, ref_dW = oracle.variant_backward(H, W, idx, val, 1.5, labels, IGN, 0.25, grad=2.0)
    assert abs(loss.item() - ref_loss) <= LOSS_RTOL * abs(ref_loss)
    assert rel_max_err(to_f64(hb.grad), ref_dH) <= GRAD_TOL
    assert rel_max_err(to_f64(wb.grad), ref_dW) <= GRAD_TOL


def test_option_errors():
    p = kd_synth.small_problem(64, 64, 300, seed=29)
    h, w = to_dev(p["H"], "bf16"), to_dev(p["W"], "bf16")
    idx, valb = kd_synth.random_cache(64, 300, 4, seed=30)
    ti, tv = torch.from_numpy(idx).to(device()), to_dev(valb, "bf16")
    tl = torch.zeros(64, dtype=torch.int32, device=device())
    for kw in ({"ce_weight": 0.5}, {"labels": tl, "ce_weight": 1.5}, {"labels": tl, "ce_weight": float("nan")}):
        with pytest.raises(kd.KDError) as e:
            kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.0, **kw)
        assert e.value.status == 14
    with pytest.raises(ValueError):
        kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.0, labels=tl[:63].contiguous())
    for ii in (2**31, -2**31 - 1):
        with pytest.raises(ValueError, match="ignore_index"):
            kd.kd_chunked_kl_fwd(h, w, ti, tv, 1.0, labels=tl, ignore_index=ii)


def test_kd_check_reports_out_of_range_label():
    """KD_CHECK=1 (read once per process, hence a child process): with a mix, a
    label outside [0, V) that is not the ignore index returns
    KD_ERR_IDX_OUT_OF_RANGE; the same labels with no mix (mask only) pass."""
    import subprocess
    import sys
    script = r'''
import numpy as np, torch, sys
import kd_synth, lm_head_kl_amd as kd
p = kd_synth.small_problem(300, 64, 600, seed=6)
to = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to("cuda:0")
h, w = to(p["H"]), to(p["W"])
val = torch.zeros((300, 5), dtype=torch.bfloat16, device="cuda:0")
idx = torch.from_numpy(np.random.default_rng(1).integers(0, 600, size=(300, 5)).astype(np.int32)).to("cuda:0")
lab = np.random.default_rng(2).integers(0, 600, size=300).astype(np.int32)
lab[5] = -100
lab[9] = 600
tl = torch.from_numpy(lab).to("cuda:0")
loss, _, _ = kd.kd_chunked_kl_fwd(h, w, idx, val, 1.0, labels=tl, ce_weight=0.0)
assert np.isfinite(loss.item())
try:
    kd.kd_chunked_kl_fwd(h, w, idx, val, 1.0, labels=tl, ce_weight=0.5)
except kd.KDError as e:
    assert e.status == 10, e.status
    print("status", e.status)
    sys.exit(0)
sys.exit(3)
'''
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, KD_CHECK="1", PYTHONPATH=root + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-c", script], env=env, cwd=root, stdout=subprocess.PIPE,
                       stderr=subprocess.STDOUT, text=True, timeout=180)
    assert r.returncode == 0 and "status 10" in r.stdout, r.stdout[-2000:]


def test_loss_module_over_batch_and_sequence_axes():
    """ChunkedTopKKLLoss on [batch, seq, d] hidden states and [batch, seq, K]
    caches equals chunked_kl_loss on the flattened rows, loss and gradients."""
    b, t, d, v, k = 3, 170, 64, 900, 8
    p, vdt, idx, valb, labels = _inputs(b * t, d, v, k, "bf16", seed=31)
    h, w, ti, tv, tl = _gpu(p, "bf16", idx, valb, labels, vdt)
    mod = kd.ChunkedTopKKLLoss(tau=1.5, ce_weight=0.2)
    h3 = h.view(b, t, d).clone().requires_grad_()
    w1 = w.clone().requires_grad_()
    loss = mod(h3, w1, ti.view(b, t, k), tv.view(b, t, k), tl.view(b, t))
    loss.backward()
    h2, w2 = h.clone().requires_grad_(), w.clone().requires_grad_()
    ref = kd.chunked_kl_loss(h2, w2, ti, tv, 1.5, labels=tl, ce_weight=0.2)
    ref.backward()
    torch.cuda.synchronize()
    assert torch.equal(loss, ref)
    assert torch.equal(h3.grad.view(-1, d), h2.grad) and torch.equal(w1.grad, w2.grad)
    with pytest.raises(ValueError):
        mod(h3, w1, ti, tv)
    # int64 labels, as cross_entropy takes them, give the same loss bit for bit
    l64 = mod(h3.detach(), w, ti.view(b, t, k), tv.view(b, t, k), tl.view(b, t).to(torch.int64))
    torch.cuda.synchronize()
    assert torch.equal(l64, ref.detach())
    # an int64 label that int32 cannot hold is out of range (a NaN row), never wrapped
    # onto a valid class: 2^32 + 5 would truncate to 5
    wide = tl.view(b, t).to(torch.int64).clone()
    wide[1, 7] = 2**32 + 5
    lw = mod(h3.detach(), w, ti.view(b, t, k), tv.view(b, t, k), wide)
    five = tl.view(b, t).to(torch.int64).clone()
    five[1, 7] = 5
    l5 = mod(h3.detach(), w, ti.view(b, t, k), tv.view(b, t, k), five)
    torch.cuda.synchronize()
    assert torch.isnan(lw) and torch.isfinite(l5)
