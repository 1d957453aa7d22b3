"""Pins of the float64 oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something other than itself: a
library routine (scipy / torch CPU), a closed form, brute force, finite
differences or an invariant.  None needs a GPU.
"""
import math

import numpy as np
import pytest
import scipy.special as sps
import torch

import oracle
from oracle import kl as okl
from oracle import topk as otk
from kd_synth import bf16_bits_from_f32, f32_from_bf16_bits, small_problem, to_float64


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_problem(n, d, v, k, seed, distinct=True):
    g = _rng(seed)
    H = g.standard_normal((n, d))
    W = g.standard_normal((v, d)) / math.sqrt(d)
    if distinct:
        idx = np.stack([g.choice(v, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    else:
        idx = g.integers(0, v, size=(n, k)).astype(np.int32)
    val = g.standard_normal((n, k)) * 2.0
    return H, W, idx, val


# ---------------------------------------------------------------------------
# P-1: K = |V| reduces to the full KL(P_T || P_S) of two softmax distributions.
@pytest.mark.parametrize("tau", [1.0, 2.0, 0.5])
def test_full_vocab_cache_is_full_kl(tau):
    n, d, v = 6, 5, 11
    g = _rng(1)
    H = g.standard_normal((n, d))
    W = g.standard_normal((v, d))
    zt = g.standard_normal((n, v)) * 3
    perm = np.stack([g.permutation(v) for _ in range(n)]).astype(np.int32)
    val = np.take_along_axis(zt, perm, axis=1)           # cache holds every entry, any order
    loss, _, kl_rows = oracle.kl_forward(H, W, perm, val, tau)
    z = H @ W.T
    pt = sps.softmax(zt / tau, axis=1)
    ps = sps.softmax(z, axis=1)
    ref_rows = sps.rel_entr(pt, ps).sum(axis=1)
    np.testing.assert_allclose(kl_rows, ref_rows, rtol=1e-12, atol=1e-13)
    # the torch form of the dense loss (student log-probs, teacher log-probs)
    ref_t = torch.nn.functional.kl_div(torch.log_softmax(torch.tensor(z), 1),
                                       torch.log_softmax(torch.tensor(zt / tau), 1),
                                       log_target=True, reduction="sum").item() / n
    assert abs(loss - ref_t) < 1e-12 * max(1.0, abs(ref_t))


# P-2: K = 1 reduces to the mean cross-entropy with the cached index as hard label.
def test_single_entry_cache_is_cross_entropy():
    H, W, idx, val = _rand_problem(9, 7, 13, 1, seed=2)
    loss, _, _ = oracle.kl_forward(H, W, idx, val, 1.0)
    ref = torch.nn.functional.cross_entropy(torch.tensor(H @ W.T), torch.tensor(idx[:, 0]).long()).item()
    assert abs(loss - ref) < 1e-12


# P-3: KL >= 0; KL = 0 iff the student restricted to the cached set equals the
# teacher and the student puts no mass off the set; otherwise KL = -log s.
def test_kl_nonnegative_random():
    for seed in range(5):
        H, W, idx, val = _rand_problem(16, 8, 40, 6, seed)
        _, _, kl_rows = oracle.kl_forward(H, W, idx, val, 1.3)
        assert (kl_rows >= -1e-12).all()


def _identity_head(z):
    """Inputs with d = V and W = I so that the logits equal ``z`` exactly."""
    return np.asarray(z, np.float64), np.eye(z.shape[1])


def test_kl_zero_when_student_matches_teacher_on_set():
    g = _rng(3)
    n, v, k, tau = 4, 20, 5, 1.7
    idx = np.stack([g.choice(v, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    val = g.standard_normal((n, k)) * 2
    z = np.full((n, v), -800.0)                               # no mass off the set (exp underflows)
    np.put_along_axis(z, idx, val / tau + 4.0, axis=1)      # student logits = teacher/tau + const on set
    H, W = _identity_head(z)
    _, _, kl_rows = oracle.kl_forward(H, W, idx, val, tau)
    assert np.abs(kl_rows).max() < 1e-12


def test_kl_is_minus_log_mass_when_only_off_set_mass_differs():
    g = _rng(4)
    n, v, k = 3, 30, 4
    idx = np.stack([g.choice(v, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    val = g.standard_normal((n, k))
    z = g.standard_normal((n, v))
    np.put_along_axis(z, idx, val + 1.5, axis=1)
    H, W = _identity_head(z)
    _, _, kl_rows = oracle.kl_forward(H, W, idx, val, 1.0)
    ps = sps.softmax(z, axis=1)
    s = np.take_along_axis(ps, idx, axis=1).sum(axis=1)
    np.testing.assert_allclose(kl_rows, -np.log(s), rtol=1e-12, atol=1e-13)


# P-4: adding a constant to a row of student logits (through the head) or of
# cached teacher logits changes nothing.
def test_shift_invariance():
    H, W, idx, val = _rand_problem(10, 6, 25, 4, seed=5)
    c = _rng(6).standard_normal(10) * 5
    Ha = np.concatenate([H, c[:, None]], axis=1)             # [H | c] . [W | 1]^T = z + c
    Wa = np.concatenate([W, np.ones((25, 1))], axis=1)
    l0, lse0, kl0 = oracle.kl_forward(H, W, idx, val, 1.0)
    l1, lse1, kl1 = oracle.kl_forward(Ha, Wa, idx, val, 1.0)
    np.testing.assert_allclose(kl1, kl0, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse1, lse0 + c, rtol=1e-12, atol=1e-12)
    dH0, dW0 = oracle.kl_backward(H, W, idx, val, 1.0)
    dH1, dW1 = oracle.kl_backward(Ha, Wa, idx, val, 1.0)
    np.testing.assert_allclose(dH1[:, :6], dH0, atol=1e-13)
    np.testing.assert_allclose(dW1[:, :6], dW0, atol=1e-13)
    l2, _, _ = oracle.kl_forward(H, W, idx, val + c[:, None], 1.0)
    assert abs(l2 - l0) < 1e-12


# P-5: equal cached values give a uniform teacher; closed form of the loss.
def test_equal_values_closed_form():
    H, W, idx, _ = _rand_problem(7, 5, 19, 6, seed=7)
    val = np.full((7, 6), 0.25)
    _, _, kl_rows = oracle.kl_forward(H, W, idx, val, 3.0)
    z = H @ W.T
    log_ps = z - sps.logsumexp(z, axis=1, keepdims=True)
    ref = -math.log(6) - np.take_along_axis(log_ps, idx, axis=1).mean(axis=1)
    np.testing.assert_allclose(kl_rows, ref, rtol=1e-12)


# P-6: the normalisers against the library routines.
def test_lse_and_teacher_softmax_match_scipy():
    g = _rng(8)
    z = g.standard_normal((5, 300)) * 20
    np.testing.assert_allclose(okl.logsumexp_rows(z), sps.logsumexp(z, axis=1), rtol=1e-14)
    val = g.standard_normal((5, 9)) * 4
    p, log_p = okl.teacher_probs(val, 0.7)
    np.testing.assert_allclose(p, sps.softmax(val / 0.7, axis=1), rtol=1e-13)
    np.testing.assert_allclose(log_p, sps.log_softmax(val / 0.7, axis=1), rtol=1e-13, atol=1e-14)


# Hand-derived worked example: z = (0, ln 2, ln 3) so p_S = (1/6, 2/6, 3/6);
# cache (idx 2 -> ln 3, idx 1 -> 0) so p_T = (3/4, 1/4) on entries (2, 1).
def test_worked_example_closed_form():
    z = np.array([[0.0, math.log(2.0), math.log(3.0)]])
    H, W = _identity_head(z)
    idx = np.array([[2, 1]], dtype=np.int32)
    val = np.array([[math.log(3.0), 0.0]])
    loss, lse, _ = oracle.kl_forward(H, W, idx, val, 1.0)
    assert abs(lse[0] - math.log(6.0)) < 1e-15
    ref = 0.75 * math.log(0.75 / 0.5) + 0.25 * math.log(0.25 / (2.0 / 6.0))
    assert abs(loss - ref) < 1e-15
    dH, dW = oracle.kl_backward(H, W, idx, val, 1.0, grad=1.0)
    # dZ = p_S - scatter(p_T) = (1/6, 1/3 - 1/4, 1/2 - 3/4); with W = I, dH = dZ
    np.testing.assert_allclose(dH[0], [1 / 6, 1 / 12, -1 / 4], atol=1e-15)
    # dW = dZ^T H = outer(dZ, z)
    np.testing.assert_allclose(dW, np.outer([1 / 6, 1 / 12, -1 / 4], z[0]), atol=1e-15)


# P-7: analytic gradients against central finite differences of the loss.
@pytest.mark.parametrize("distinct", [True, False])
def test_gradients_match_finite_differences(distinct):
    n, d, v, k, tau, g_up = 8, 16, 64, 4, 1.5, 0.37
    H, W, idx, val = _rand_problem(n, d, v, k, seed=9, distinct=distinct)
    dH, dW = oracle.kl_backward(H, W, idx, val, tau, grad=g_up)
    h = 1e-6

    def f(Hx, Wx):
        return g_up * oracle.kl_forward(Hx, Wx, idx, val, tau)[0]

    fdH = np.zeros_like(H)
    for i in range(n):
        for j in range(d):
            e = np.zeros_like(H)
            e[i, j] = h
            fdH[i, j] = (f(H + e, W) - f(H - e, W)) / (2 * h)
    g = _rng(10)
    fdW = {}
    for _ in range(60):
        a, b = int(g.integers(v)), int(g.integers(d))
        e = np.zeros_like(W)
        e[a, b] = h
        fdW[(a, b)] = (f(H, W + e) - f(H, W - e)) / (2 * h)
    assert np.abs(fdH - dH).max() <= 1e-7 * max(1.0, np.abs(dH).max()) + 1e-9
    for (a, b), val_fd in fdW.items():
        assert abs(val_fd - dW[a, b]) <= 1e-7 * max(1.0, np.abs(dW).max()) + 1e-9


# P-8: each dZ row sums to zero over the vocabulary, so dW's rows sum to zero.
def test_dw_rows_sum_to_zero():
    H, W, idx, val = _rand_problem(12, 9, 50, 7, seed=11)
    _, dW = oracle.kl_backward(H, W, idx, val, 1.0)
    assert np.abs(dW.sum(axis=0)).max() < 1e-15 * 50 * 12 + 1e-16
    assert np.abs(dW).max() > 1e-6


# The dense route of the pages (dense teacher matrix zero off the cache) gives
# the same loss as the per-entry form when the cached indices are distinct.
def test_dense_reconstruction_equals_sparse_form():
    H, W, idx, val = _rand_problem(11, 6, 37, 5, seed=12)
    for tau in (1.0, 2.0):
        assert abs(oracle.kl_forward(H, W, idx, val, tau)[0]
                   - oracle.kl_dense_reconstruction(H, W, idx, val, tau)) < 1e-12


# With repeated indices the two forms differ by a term that does not depend on
# the student, so both have the same gradient (scatter-add).
def test_repeated_indices_gradient_is_scatter_add():
    n, d, v, k = 5, 4, 6, 5
    H, W, idx, val = _rand_problem(n, d, v, k, seed=13, distinct=False)
    assert any(len(set(r)) < k for r in idx)
    dH, _ = oracle.kl_backward(H, W, idx, val, 1.0)
    h = 1e-6
    for i in range(n):
        for j in range(d):
            e = np.zeros_like(H)
            e[i, j] = h
            fd = (oracle.kl_dense_reconstruction(H + e, W, idx, val, 1.0)
                  - oracle.kl_dense_reconstruction(H - e, W, idx, val, 1.0)) / (2 * h)
            assert abs(fd - dH[i, j]) < 1e-7


# P-10: row-block size does not change the result; the mean loss and the
# gradients are additive over token chunks.
def test_block_invariance_and_chunk_additivity():
    H, W, idx, val = _rand_problem(40, 8, 30, 5, seed=14)
    l1, lse1, _ = oracle.kl_forward(H, W, idx, val, 1.0, block=7)
    l2, lse2, _ = oracle.kl_forward(H, W, idx, val, 1.0, block=256)
    assert abs(l1 - l2) < 1e-13
    np.testing.assert_allclose(lse1, lse2, rtol=1e-15)
    _, dW = oracle.kl_backward(H, W, idx, val, 1.0)
    parts = [(0, 13), (13, 31), (31, 40)]
    acc_l = 0.0
    acc_w = np.zeros_like(W)
    for a, b in parts:
        acc_l += (b - a) / 40 * oracle.kl_forward(H[a:b], W, idx[a:b], val[a:b], 1.0)[0]
        acc_w += (b - a) / 40 * oracle.kl_backward(H[a:b], W, idx[a:b], val[a:b], 1.0)[1]
    assert abs(acc_l - l2) < 1e-13
    np.testing.assert_allclose(acc_w, dW, atol=1e-15)


# ---------------------------------------------------------------------------
# Top-K cache.
def test_topk_matches_brute_force_sort():
    g = _rng(15)
    n, d, v, k = 6, 5, 40, 7
    HT = g.standard_normal((n, d))
    WT = g.standard_normal((v, d))
    WT[17] = WT[3]                       # an exact tie: index 3 must come first
    HT[0] = WT[3] * 10                   # make the tie land inside row 0's top-K
    idx, _, sc = oracle.topk_cache(HT, WT, k, "f32")
    s = HT @ WT.T
    for i in range(n):
        ref = sorted(range(v), key=lambda c: (-s[i, c], c))[:k]
        assert list(idx[i]) == ref
        assert set(idx[i]) == set(np.argpartition(-s[i], k - 1)[:k]) or len(set(s[i])) < v
    row0 = list(idx[0])
    assert 3 in row0 and 17 in row0 and row0.index(17) == row0.index(3) + 1
    np.testing.assert_array_equal(sc, np.take_along_axis(s, idx.astype(np.int64), axis=1))


def test_topk_full_vocab_is_permutation():
    g = _rng(16)
    HT = g.standard_normal((4, 3))
    WT = g.standard_normal((25, 3))
    idx, val, sc = oracle.topk_cache(HT, WT, 25, "f32")
    for r in idx:
        assert sorted(r) == list(range(25))
    assert (np.diff(sc, axis=1) <= 0).all()
    np.testing.assert_array_equal(val, sc.astype(np.float32))


def test_topk_prefix_property():
    g = _rng(17)
    HT = g.standard_normal((5, 8))
    WT = g.standard_normal((90, 8))
    i10, _, _ = oracle.topk_cache(HT, WT, 10)
    i4, _, _ = oracle.topk_cache(HT, WT, 4)
    np.testing.assert_array_equal(i10[:, :4], i4)


# Rounding of cached values: float64 -> bfloat16, nearest even, one rounding.
def test_round_to_bf16_matches_torch_on_float32_inputs():
    g = _rng(18)
    x32 = np.concatenate([g.standard_normal(20000).astype(np.float32) * 4,
                          np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130, 3e38],
                                   dtype=np.float32)])
    ref = torch.tensor(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = otk.bf16_bits(otk.round_to_bf16(x32.astype(np.float64)))
    np.testing.assert_array_equal(got, ref)


def test_round_to_bf16_single_rounding_from_float64():
    # Just above the midpoint between 1 and 1 + 2^-7; through float32 it would
    # land on the midpoint and tie down to 1.  A single rounding goes up.
    x = 1.0 + 2 ** -8 + 2 ** -30
    assert float(np.float32(x)) == 1.0 + 2 ** -8
    assert otk.round_to_bf16(np.array([x]))[0] == 1.0 + 2 ** -7
    assert otk.round_to_bf16(np.array([-x]))[0] == -(1.0 + 2 ** -7)
    # exact midpoints tie to even
    assert otk.round_to_bf16(np.array([1.0 + 2 ** -8]))[0] == 1.0
    assert otk.round_to_bf16(np.array([1.0 + 3 * 2 ** -8]))[0] == 1.0 + 2 ** -6
    # brute force against the two neighbouring bf16 values
    g = _rng(19)
    xs = g.standard_normal(3000) * 10.0 ** g.integers(-5, 5, 3000)
    r = otk.round_to_bf16(xs)
    for xv, rv in zip(xs, r):
        e = math.floor(math.log2(abs(xv)))
        q = 2.0 ** (e - 7)
        lo = math.floor(abs(xv) / q) * q
        hi = lo + q
        best = lo if (abs(xv) - lo) < (hi - abs(xv)) else hi
        if (abs(xv) - lo) == (hi - abs(xv)):
            best = lo if (lo / q) % 2 == 0 else hi
        assert abs(rv) == best and math.copysign(1, rv) == math.copysign(1, xv)


# ---------------------------------------------------------------------------
# Generators: prefix property and storage rounding.
def test_generator_prefix_and_rounding():
    import kd_synth
    w = kd_synth.WORKLOADS["seq4k_v32k"]
    a = kd_synth.hidden(w, 8192 + 3)
    b = kd_synth.hidden(w, 100)
    np.testing.assert_array_equal(a[:100], b)
    rows = np.array([5, 4097, 8194, 0])
    np.testing.assert_array_equal(kd_synth.hidden_rows(w, rows), a[rows])
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    ref = torch.tensor(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_bits_from_f32(x), ref)
    np.testing.assert_array_equal(f32_from_bf16_bits(ref), torch.tensor(x).to(torch.bfloat16).float().numpy())
    p = small_problem(10, 16, 40, seed=1)
    assert to_float64(p["H"], "bf16").dtype == np.float64
