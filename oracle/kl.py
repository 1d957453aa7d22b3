"""Float64 definition of the top-K KL loss and its gradients (test infrastructure).

Definition (readings of the pages, see the package docstring for sources):

    z[i, v]   = sum_j H[i, j] * W[v, j]                       student logits, all V
    lse[i]    = log sum_v exp(z[i, v])                        student normaliser, all V
    p[i, k]   = exp(val[i,k]/tau) / sum_k' exp(val[i,k']/tau) teacher, renormalised over its K cached entries
    KL[i]     = sum_k p[i,k] * (log p[i,k] - (z[i, idx[i,k]] - lse[i]))
    loss      = (1/N) * sum_i KL[i]
    dZ[i, v]  = (g/N) * (exp(z[i,v] - lse[i]) - sum_{k: idx[i,k] = v} p[i,k])
    dH        = dZ @ W,   dW = dZ^T @ H

Readings taken where the pages are silent or ambiguous:

* The student's log-probabilities are normalised over the whole vocabulary
  (the dense variant compares the rebuilt teacher with the student's *dense*
  log-probability matrix).
* The temperature applies to the cached teacher logits only; the student is
  not tempered and there is no tau^2 factor.
* The reduction is the mean over the N token rows (every row counts; no
  padding mask).
* Teacher mass outside the cached K entries is dropped (the teacher is
  renormalised over the K entries).
* ``p * log p`` is taken as 0 where ``p`` underflows to 0.
* Repeated indices within a row: every cached entry is its own teacher atom
  (the loss sums per entry, the gradient scatter-adds).  With distinct indices
  this is exactly the dense reconstruction (:func:`kl_dense_reconstruction`).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

_BLOCK = 256


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def logsumexp_rows(Z) -> np.ndarray:
    """``log sum_v exp(Z[i, v])`` per row, shifted by the row max for range."""
    Z = _f64(Z)
    m = Z.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(Z - m).sum(axis=1, keepdims=True)))[:, 0]


def teacher_probs(val, tau: float) -> Tuple[np.ndarray, np.ndarray]:
    """Teacher distribution over the K cached entries: ``softmax(val / tau)``.

    Returns ``(p, log_p)``; both float64 ``[N, K]``.
    """
    a = _f64(val) / float(tau)
    a = a - a.max(axis=1, keepdims=True)
    log_p = a - np.log(np.exp(a).sum(axis=1, keepdims=True))
    return np.exp(log_p), log_p


def _xlogy_self(p: np.ndarray, log_p: np.ndarray) -> np.ndarray:
    return np.where(p > 0.0, p * log_p, 0.0)


def kl_forward(H, W, idx, val, tau: float, block: int = _BLOCK
               ) -> Tuple[float, np.ndarray, np.ndarray]:
    """Loss, per-row log-sum-exp and per-row KL.

    Returns ``(loss, lse[N], kl_rows[N])`` in float64.  Rows are processed in
    blocks of ``block`` rows; each block materialises its full logit rows.
    """
    H = _f64(H)
    W = _f64(W)
    idx = np.asarray(idx, dtype=np.int64)
    n = H.shape[0]
    p, log_p = teacher_probs(val, tau)
    lse = np.empty(n)
    kl = np.empty(n)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        z = H[r0:r1] @ W.T
        l = logsumexp_rows(z)
        z_cached = np.take_along_axis(z, idx[r0:r1], axis=1)
        log_q = z_cached - l[:, None]                     # student log-prob at cached entries
        kl[r0:r1] = (_xlogy_self(p[r0:r1], log_p[r0:r1]) - p[r0:r1] * log_q).sum(axis=1)
        lse[r0:r1] = l
    loss = float(kl.sum() / n) if n else 0.0
    return loss, lse, kl


def kl_backward(H, W, idx, val, tau: float, grad: float = 1.0, block: int = _BLOCK
                ) -> Tuple[np.ndarray, np.ndarray]:
    """``(dH, dW)`` for upstream gradient ``grad`` of the mean loss."""
    H = _f64(H)
    W = _f64(W)
    idx = np.asarray(idx, dtype=np.int64)
    n = H.shape[0]
    p, _ = teacher_probs(val, tau)
    dH = np.zeros_like(H)
    dW = np.zeros_like(W)
    if n == 0:
        return dH, dW
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        z = H[r0:r1] @ W.T
        l = logsumexp_rows(z)
        dz = np.exp(z - l[:, None])
        rows = np.repeat(np.arange(r1 - r0), idx.shape[1])
        np.add.at(dz, (rows, idx[r0:r1].ravel()), -p[r0:r1].ravel())   # scatter-add of the teacher
        dz *= float(grad) / n
        dH[r0:r1] = dz @ W
        dW += dz.T @ H[r0:r1]
    return dH, dW


def kl_dense_reconstruction(H, W, idx, val, tau: float) -> float:
    """Loss by the dense route: rebuild a dense ``[N, V]`` teacher matrix that is
    zero outside the cached entries, then ``sum P_T * log(P_T / P_S)`` over the
    whole vocabulary, divided by N.  Only for small shapes; used as a second,
    independent route to the same value."""
    H = _f64(H)
    W = _f64(W)
    idx = np.asarray(idx, dtype=np.int64)
    n = H.shape[0]
    z = H @ W.T
    log_ps = z - logsumexp_rows(z)[:, None]
    p, _ = teacher_probs(val, tau)
    PT = np.zeros_like(z)
    np.add.at(PT, (np.repeat(np.arange(n), idx.shape[1]), idx.ravel()), p.ravel())
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(PT > 0.0, PT * (np.log(np.where(PT > 0, PT, 1.0)) - log_ps), 0.0)
    return float(terms.sum() / n)
