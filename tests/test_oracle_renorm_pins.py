"""Pins of the oracle's renormalised-student loss (``oracle.renorm_forward`` /
``renorm_backward``: the student's softmax taken over the row's K cached entries
only).  Each check compares the oracle with something other than itself:

* K = V (every vocabulary entry cached, rows permuted): the cached set is the
  whole vocabulary, so the loss is scipy's full relative entropy, and the
  gradients equal the full-vocabulary oracle's;
* torch's log_softmax over the gathered logits and its kl_div (a library route);
* the closed form KL = 0 when the student restricted to the cached set equals the
  teacher, whatever mass the student puts elsewhere (where the full-vocabulary KL
  is -log of the student's cached mass instead);
* central finite differences of dH and dW, with repeated indices and a mask;
* the gradient vanishes off the cached set: W rows outside every cache row get no
  gradient and do not change dH;
* K = 1: the loss and gradients are exactly zero;
* a mask: ignored rows are neither read nor counted.
A plausible mistake (a full-vocabulary normaliser, a dropped p log p term, a sign
error, a transposed product) fails at least one of them.
"""
import math

import numpy as np
import scipy.special as sps
import torch

import oracle

IGN = -100


def _problem(n, d, v, k, seed, distinct=True):
    g = np.random.default_rng(seed)
    H = g.standard_normal((n, d))
    W = g.standard_normal((v, d)) / math.sqrt(d) * 2.0
    if distinct:
        idx = np.stack([g.choice(v, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    else:
        idx = g.integers(0, v, size=(n, k)).astype(np.int32)
    val = g.standard_normal((n, k)) * 2.0
    return H, W, idx, val


def test_full_cache_is_scipy_full_kl_and_the_full_vocabulary_gradients():
    n, d, v, tau = 7, 5, 12, 1.7
    g = np.random.default_rng(11)
    H = g.standard_normal((n, d))
    W = g.standard_normal((v, d))
    zt = g.standard_normal((n, v)) * 3
    perm = np.stack([g.permutation(v) for _ in range(n)]).astype(np.int32)
    val = np.take_along_axis(zt, perm, axis=1)
    loss, lse, rows = oracle.renorm_forward(H, W, perm, val, tau)
    kl = sps.rel_entr(sps.softmax(zt / tau, axis=1), sps.softmax(H @ W.T, axis=1)).sum(axis=1)
    np.testing.assert_allclose(rows, kl, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, sps.logsumexp(H @ W.T, axis=1), rtol=1e-13)
    assert abs(loss - kl.mean()) < 1e-12
    dH, dW = oracle.renorm_backward(H, W, perm, val, tau, grad=0.37)
    fH, fW = oracle.kl_backward(H, W, perm, val, tau, grad=0.37)
    np.testing.assert_allclose(dH, fH, rtol=1e-11, atol=1e-14)
    np.testing.assert_allclose(dW, fW, rtol=1e-11, atol=1e-14)


def test_torch_log_softmax_over_the_gathered_logits():
    n, d, v, k, tau = 9, 6, 30, 5, 0.8
    H, W, idx, val = _problem(n, d, v, k, seed=12, distinct=False)
    loss, lse, rows = oracle.renorm_forward(H, W, idx, val, tau)
    z = torch.tensor(H @ W.T)
    zk = torch.gather(z, 1, torch.tensor(idx).long())
    log_q = torch.log_softmax(zk, dim=1)
    log_p = torch.log_softmax(torch.tensor(val) / tau, dim=1)
    per = torch.nn.functional.kl_div(log_q, log_p, log_target=True, reduction="none").sum(dim=1).numpy()
    np.testing.assert_allclose(rows, per, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, torch.logsumexp(zk, dim=1).numpy(), rtol=1e-13)
    assert abs(loss - per.mean()) < 1e-12


def test_kl_is_zero_when_the_renormalised_student_is_the_teacher():
    # student logits at the cached entries equal the teacher's (val / tau) up to a
    # row constant; the student keeps a large mass outside the cached set
    n, d, v, k, tau = 5, 8, 40, 6, 1.3
    H, W, idx, _ = _problem(n, d, v, k, seed=13)
    z = H @ W.T
    zk = np.take_along_axis(z, idx.astype(np.int64), axis=1)
    c = np.arange(n)[:, None] * 0.7 - 1.0
    val = tau * (zk + c)
    _, _, rows = oracle.renorm_forward(H, W, idx, val, tau)
    assert np.all(np.abs(rows) < 1e-13), rows
    # the full-vocabulary KL of the same inputs is -log(student mass on the cached set) > 0
    _, lse, full = oracle.kl_forward(H, W, idx, val, tau)
    s = np.exp(zk - lse[:, None]).sum(axis=1)
    np.testing.assert_allclose(full, -np.log(s), rtol=1e-11)
    assert np.all(full > 0.01)
    dH, dW = oracle.renorm_backward(H, W, idx, val, tau)
    assert np.abs(dH).max() < 1e-14 and np.abs(dW).max() < 1e-14


def _fd(f, x, h=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        g[i] = (f(xp) - f(xm)) / (2 * h)
    return g


def test_finite_differences_with_repeated_indices_and_a_mask():
    n, d, v, k, tau = 6, 4, 9, 4, 0.9
    H, W, idx, val = _problem(n, d, v, k, seed=14, distinct=False)
    idx[2, 1] = idx[2, 3]                     # a repeated index
    labels = np.arange(n).astype(np.int32)
    labels[[1, 4]] = IGN
    g = 0.6

    def loss_h(x):
        return g * oracle.renorm_forward(x, W, idx, val, tau, labels, IGN)[0]

    def loss_w(x):
        return g * oracle.renorm_forward(H, x, idx, val, tau, labels, IGN)[0]

    dH, dW = oracle.renorm_backward(H, W, idx, val, tau, labels, IGN, grad=g)
    np.testing.assert_allclose(dH, _fd(loss_h, H), rtol=1e-6, atol=1e-9)
    np.testing.assert_allclose(dW, _fd(loss_w, W), rtol=1e-6, atol=1e-9)
    assert np.all(dH[[1, 4]] == 0.0)


def test_gradient_vanishes_off_the_cached_set():
    n, d, v, k, tau = 8, 5, 50, 4, 1.0
    H, W, idx, val = _problem(n, d, v, k, seed=15)
    dH, dW = oracle.renorm_backward(H, W, idx, val, tau)
    off = np.setdiff1d(np.arange(v), idx.ravel())
    assert off.size > 0 and np.all(dW[off] == 0.0)
    on = np.unique(idx.ravel())
    assert np.all(np.abs(dW[on]).sum(axis=1) > 0)
    W2 = W.copy()
    W2[off] = np.random.default_rng(16).standard_normal((off.size, d)) * 10
    dH2, _ = oracle.renorm_backward(H, W2, idx, val, tau)
    l1 = oracle.renorm_forward(H, W, idx, val, tau)[0]
    l2 = oracle.renorm_forward(H, W2, idx, val, tau)[0]
    np.testing.assert_allclose(dH2, dH, rtol=1e-12, atol=1e-15)
    assert abs(l1 - l2) < 1e-12


def test_single_entry_cache_gives_zero():
    H, W, idx, val = _problem(5, 4, 10, 1, seed=17)
    loss, lse, rows = oracle.renorm_forward(H, W, idx, val, 2.0)
    assert loss == 0.0 and np.all(rows == 0.0)
    np.testing.assert_allclose(lse, np.take_along_axis(H @ W.T, idx.astype(np.int64), axis=1)[:, 0], rtol=1e-14)
    dH, dW = oracle.renorm_backward(H, W, idx, val, 2.0)
    assert np.all(dH == 0.0) and np.all(dW == 0.0)


def test_mask_ignored_rows_are_not_read_nor_counted():
    n, d, v, k, tau = 10, 5, 20, 3, 1.1
    H, W, idx, val = _problem(n, d, v, k, seed=18)
    labels = np.zeros(n, dtype=np.int32)
    ign = [0, 3, 9]
    labels[ign] = IGN
    idx2, val2 = idx.copy(), val.copy()
    idx2[ign] = 10 ** 6                       # garbage an unread row may hold
    val2[ign] = np.nan
    loss, lse, rows = oracle.renorm_forward(H, W, idx2, val2, tau, labels, IGN)
    keep = labels != IGN
    sub, _, sub_rows = oracle.renorm_forward(H[keep], W, idx[keep], val[keep], tau)
    assert abs(loss - sub) < 1e-13
    np.testing.assert_allclose(rows[keep], sub_rows, rtol=1e-13)
    assert np.all(rows[~keep] == 0.0) and np.all(np.isnan(lse[~keep]))
    dH, dW = oracle.renorm_backward(H, W, idx2, val2, tau, labels, IGN)
    sH, sW = oracle.renorm_backward(H[keep], W, idx[keep], val[keep], tau)
    np.testing.assert_allclose(dH[keep], sH, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dW, sW, rtol=1e-12, atol=1e-15)
    assert np.all(dH[~keep] == 0.0)
    # every row ignored
    assert oracle.renorm_forward(H, W, idx2, val2, tau, np.full(n, IGN, np.int32), IGN)[0] == 0.0
