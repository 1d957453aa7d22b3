"""Pins of the loss-variant oracle (padding mask, hard-label cross-entropy mix).

Each check compares ``oracle.variant_forward`` / ``variant_backward`` with
something other than themselves: torch's cross-entropy with an ignore index,
scipy's relative entropy over the counted rows, their linear mix, central finite
differences, and the invariants a mask implies (ignored rows neither read nor
counted).  None needs a GPU.
"""
import math

import numpy as np
import pytest
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
    labels = g.integers(0, v, size=n).astype(np.int32)
    return H, W, idx, val, labels


def _full_cache(n, v, seed):
    """A cache that holds every vocabulary entry (K = V, rows permuted) with its
    teacher logits, and those logits as a dense matrix."""
    g = np.random.default_rng(seed)
    zt = g.standard_normal((n, v)) * 3
    perm = np.stack([g.permutation(v) for _ in range(n)]).astype(np.int32)
    return perm, np.take_along_axis(zt, perm, axis=1), zt


# ce_weight = 1: torch's mean cross-entropy, with its ignore index.
@pytest.mark.parametrize("ignore_index", [IGN, 3])
def test_pure_ce_is_torch_cross_entropy_with_ignore_index(ignore_index):
    H, W, idx, val, labels = _problem(23, 6, 17, 4, seed=1)
    labels[[0, 5, 6, 19]] = ignore_index
    loss, _, rows = oracle.variant_forward(H, W, idx, val, 1.3, labels, ignore_index, 1.0)
    ref = torch.nn.functional.cross_entropy(torch.tensor(H @ W.T), torch.tensor(labels).long(),
                                            ignore_index=ignore_index)
    assert abs(loss - ref.item()) < 1e-12
    per = torch.nn.functional.cross_entropy(torch.tensor(H @ W.T), torch.tensor(labels).long(),
                                            ignore_index=ignore_index, reduction="none").numpy()
    np.testing.assert_allclose(rows, per, rtol=1e-12, atol=1e-14)


# ce_weight = 0 with a mask and K = V: scipy's full KL, averaged over the counted rows.
@pytest.mark.parametrize("tau", [1.0, 2.0])
def test_masked_full_cache_is_full_kl_over_counted_rows(tau):
    n, d, v = 9, 5, 13
    g = np.random.default_rng(2)
    H = g.standard_normal((n, d))
    W = g.standard_normal((v, d))
    idx, val, zt = _full_cache(n, v, seed=3)
    labels = g.integers(0, v, size=n).astype(np.int32)
    labels[[1, 4]] = IGN
    keep = labels != IGN
    loss, _, rows = oracle.variant_forward(H, W, idx, val, tau, labels, IGN, 0.0)
    kl = sps.rel_entr(sps.softmax(zt / tau, axis=1), sps.softmax(H @ W.T, axis=1)).sum(axis=1)
    np.testing.assert_allclose(rows[keep], kl[keep], rtol=1e-12, atol=1e-13)
    assert np.all(rows[~keep] == 0.0)
    assert abs(loss - kl[keep].mean()) < 1e-12


# A mix: (1 - a) * scipy KL + a * torch CE, both over the counted rows.
def test_mix_is_linear_in_the_two_library_losses():
    n, d, v, a, tau = 11, 4, 9, 0.35, 0.7
    g = np.random.default_rng(4)
    H = g.standard_normal((n, d))
    W = g.standard_normal((v, d))
    idx, val, zt = _full_cache(n, v, seed=5)
    labels = g.integers(0, v, size=n).astype(np.int32)
    labels[[0, 10]] = IGN
    keep = labels != IGN
    loss, _, _ = oracle.variant_forward(H, W, idx, val, tau, labels, IGN, a)
    kl = sps.rel_entr(sps.softmax(zt / tau, axis=1), sps.softmax(H @ W.T, axis=1)).sum(axis=1)[keep].mean()
    ce = torch.nn.functional.cross_entropy(torch.tensor(H @ W.T), torch.tensor(labels).long(),
                                           ignore_index=IGN).item()
    assert abs(loss - ((1 - a) * kl + a * ce)) < 1e-12


# Gradients against central finite differences, with ignored rows, repeated
# cached indices and a label that is also one of its row's cached indices.
@pytest.mark.parametrize("a", [0.0, 0.4, 1.0])
def test_variant_gradients_match_finite_differences(a):
    n, d, v, k, tau, g_up = 7, 6, 20, 5, 1.5, 0.37
    H, W, idx, val, labels = _problem(n, d, v, k, seed=6, distinct=False)
    labels[2] = IGN
    labels[3] = idx[3, 1]
    dH, dW = oracle.variant_backward(H, W, idx, val, tau, labels, IGN, a, grad=g_up)
    h = 1e-6

    def f(Hx, Wx):
        return g_up * oracle.variant_forward(Hx, Wx, idx, val, tau, labels, IGN, a)[0]

    fdH = np.zeros_like(H)
    for i in range(n):
        for j in range(d):
            e = np.zeros_like(H)
            e[i, j] = h
            fdH[i, j] = (f(H + e, W) - f(H - e, W)) / (2 * h)
    assert np.abs(fdH - dH).max() <= 1e-7 * max(1.0, np.abs(dH).max())
    g = np.random.default_rng(7)
    for _ in range(40):
        r, c = int(g.integers(v)), int(g.integers(d))
        e = np.zeros_like(W)
        e[r, c] = h
        fd = (f(H, W + e) - f(H, W - e)) / (2 * h)
        assert abs(fd - dW[r, c]) <= 1e-7 * max(1.0, np.abs(dW).max())
    assert np.all(dH[2] == 0.0)


# An ignored row's cache entries, label and hidden state do not matter: garbage
# there (NaN logits, out-of-range indices) changes nothing, and its dH row is 0.
def test_ignored_rows_are_not_read():
    H, W, idx, val, labels = _problem(10, 5, 12, 3, seed=8)
    labels[[3, 7]] = IGN
    base = oracle.variant_forward(H, W, idx, val, 1.0, labels, IGN, 0.5)
    bH, bW = oracle.variant_backward(H, W, idx, val, 1.0, labels, IGN, 0.5)
    idx2, val2, H2 = idx.copy(), val.copy(), H.copy()
    idx2[[3, 7]] = 10 ** 6
    val2[[3, 7]] = np.nan
    H2[3] *= 5.0
    out = oracle.variant_forward(H2, W, idx2, val2, 1.0, labels, IGN, 0.5)
    oH, oW = oracle.variant_backward(H2, W, idx2, val2, 1.0, labels, IGN, 0.5)
    assert out[0] == base[0]
    np.testing.assert_array_equal(out[2], base[2])
    np.testing.assert_array_equal(oW, bW)
    np.testing.assert_array_equal(oH[[0, 1, 2, 4, 5, 6, 8, 9]], bH[[0, 1, 2, 4, 5, 6, 8, 9]])
    assert np.all(oH[[3, 7]] == 0.0)
    # the counted mean: appending ignored rows leaves loss and gradients unchanged
    Hp = np.vstack([H, np.ones((4, 5))])
    ip = np.vstack([idx, np.zeros((4, 3), np.int32)])
    vp = np.vstack([val, np.zeros((4, 3))])
    lp = np.concatenate([labels, np.full(4, IGN, np.int32)])
    assert abs(oracle.variant_forward(Hp, W, ip, vp, 1.0, lp, IGN, 0.5)[0] - base[0]) < 1e-15
    np.testing.assert_allclose(oracle.variant_backward(Hp, W, ip, vp, 1.0, lp, IGN, 0.5)[1], bW, atol=1e-16)


def test_every_row_ignored_and_empty():
    H, W, idx, val, labels = _problem(4, 3, 7, 2, seed=9)
    labels[:] = IGN
    loss, lse, rows = oracle.variant_forward(H, W, idx, val, 1.0, labels, IGN, 0.5)
    assert loss == 0.0 and np.all(rows == 0.0) and np.all(np.isfinite(lse))
    dH, dW = oracle.variant_backward(H, W, idx, val, 1.0, labels, IGN, 0.5)
    assert not dH.any() and not dW.any()
    e = np.zeros((0, 3))
    assert oracle.variant_forward(e, W, idx[:0], val[:0], 1.0, labels[:0], IGN, 0.5)[0] == 0.0


# Without labels (or with none ignored and no mix) the variant is the plain KL of
# oracle.kl, which has its own pins.
def test_no_option_is_the_plain_loss():
    H, W, idx, val, labels = _problem(12, 6, 15, 4, seed=10)
    plain = oracle.kl_forward(H, W, idx, val, 2.0)
    for lab in (None, labels):
        v = oracle.variant_forward(H, W, idx, val, 2.0, lab, IGN, 0.0)
        assert abs(v[0] - plain[0]) < 1e-14
        np.testing.assert_allclose(v[2], plain[2], rtol=1e-14, atol=1e-15)
        np.testing.assert_allclose(oracle.variant_backward(H, W, idx, val, 2.0, lab, IGN, 0.0)[1],
                                   oracle.kl_backward(H, W, idx, val, 2.0)[1], atol=1e-15)


def test_option_domain():
    H, W, idx, val, labels = _problem(3, 3, 5, 2, seed=11)
    with pytest.raises(ValueError):
        oracle.variant_forward(H, W, idx, val, 1.0, None, IGN, 0.5)
    with pytest.raises(ValueError):
        oracle.variant_forward(H, W, idx, val, 1.0, labels, IGN, 1.5)
