"""Float64 definition of the loss variants: a padding mask, a hard-label
cross-entropy mix, and a student renormalised over the cached entries (test
infrastructure, like the rest of this package).

The pages report ablations of the loss design and of sequence packing (the
paper's abstract) without defining either.  What is computed here is the plain
reading of those two ideas in next-token training, on top of the KL of
:mod:`oracle.kl`:

    C         = { i : labels[i] != ignore_index }      counted rows (all rows without labels)
    CE[i]     = lse[i] - z[i, labels[i]]               cross-entropy with the hard label
    l[i]      = (1 - a) * KL[i] + a * CE[i]  for i in C, 0 otherwise     (a = ce_weight in [0, 1])
    loss      = (1 / |C|) * sum_i l[i]                 (0 when C is empty)
    dZ[i, v]  = (g / |C|) * (exp(z[i,v] - lse[i]) - (1 - a) * sum_{k: idx[i,k] = v} p[i,k]
                              - a * [v == labels[i]])   for i in C; 0 otherwise
    dH        = dZ @ W,   dW = dZ^T @ H

Readings:

* The mean runs over the counted rows only (a padded position neither adds to
  the loss nor dilutes it), as in a cross-entropy with an ignore index.
* The cache rows (idx, val) of an ignored row are never read: padding may hold
  anything there.  Its lse is still defined (it depends on H and W only).
* With ``a = 0`` the labels serve only as the mask; their values are not read
  otherwise.
* The cross-entropy uses the same untempered student log-probabilities as the
  KL (full-vocabulary normaliser).
"""
from __future__ import annotations

from typing import Optional, Tuple

import numpy as np

from .kl import _f64, _xlogy_self, logsumexp_rows, teacher_probs

_BLOCK = 256


def counted_rows(labels: Optional[np.ndarray], n: int, ignore_index: int) -> np.ndarray:
    """Boolean mask of the rows that count: every row without labels, else the
    rows whose label differs from ``ignore_index``."""
    if labels is None:
        return np.ones(n, dtype=bool)
    return np.asarray(labels, dtype=np.int64) != int(ignore_index)


def _check(labels, ce_weight):
    a = float(ce_weight)
    if not (0.0 <= a <= 1.0):
        raise ValueError("ce_weight must lie in [0, 1]")
    if labels is None and a != 0.0:
        raise ValueError("a cross-entropy mix needs labels")
    return a


def variant_forward(H, W, idx, val, tau: float, labels=None, ignore_index: int = -100,
                    ce_weight: float = 0.0, block: int = _BLOCK
                    ) -> Tuple[float, np.ndarray, np.ndarray]:
    """Loss, per-row log-sum-exp and per-row loss term ``l[i]``.

    Returns ``(loss, lse[N], l[N])`` in float64.
    """
    a = _check(labels, ce_weight)
    H = _f64(H)
    W = _f64(W)
    n = H.shape[0]
    keep = counted_rows(labels, n, ignore_index)
    lab = None if labels is None else np.asarray(labels, dtype=np.int64)
    lse = np.empty(n)
    rows = np.zeros(n)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        z = H[r0:r1] @ W.T
        l = logsumexp_rows(z)
        lse[r0:r1] = l
        sel = np.nonzero(keep[r0:r1])[0]              # counted rows of the block
        if sel.size == 0:
            continue
        p, log_p = teacher_probs(np.asarray(val)[r0 + sel], tau)
        zc = np.take_along_axis(z[sel], np.asarray(idx, dtype=np.int64)[r0 + sel], axis=1)
        kl = (_xlogy_self(p, log_p) - p * (zc - l[sel, None])).sum(axis=1)
        ce = l[sel] - z[sel, lab[r0 + sel]] if a > 0.0 else np.zeros(sel.size)
        rows[r0 + sel] = (1.0 - a) * kl + a * ce
    count = int(keep.sum())
    loss = float(rows.sum() / count) if count else 0.0
    return loss, lse, rows


def variant_backward(H, W, idx, val, tau: float, labels=None, ignore_index: int = -100,
                     ce_weight: float = 0.0, grad: float = 1.0, block: int = _BLOCK
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """``(dH, dW)`` for upstream gradient ``grad`` of the loss above."""
    a = _check(labels, ce_weight)
    H = _f64(H)
    W = _f64(W)
    n = H.shape[0]
    keep = counted_rows(labels, n, ignore_index)
    lab = None if labels is None else np.asarray(labels, dtype=np.int64)
    count = int(keep.sum())
    dH = np.zeros_like(H)
    dW = np.zeros_like(W)
    if count == 0:
        return dH, dW
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        sel = np.nonzero(keep[r0:r1])[0]
        if sel.size == 0:
            continue
        z = H[r0 + sel] @ W.T
        dz = np.exp(z - logsumexp_rows(z)[:, None])
        p, _ = teacher_probs(np.asarray(val)[r0 + sel], tau)
        ii = np.asarray(idx, dtype=np.int64)[r0 + sel]
        np.add.at(dz, (np.repeat(np.arange(sel.size), ii.shape[1]), ii.ravel()), -(1.0 - a) * p.ravel())
        if a > 0.0:
            np.add.at(dz, (np.arange(sel.size), lab[r0 + sel]), -a)
        dz *= float(grad) / count
        dH[r0 + sel] = dz @ W
        dW += dz.T @ H[r0 + sel]
    return dH, dW


def renorm_forward(H, W, idx, val, tau: float, labels=None, ignore_index: int = -100, block: int = _BLOCK
                   ) -> Tuple[float, np.ndarray, np.ndarray]:
    """The KL against a student renormalised over the row's K cached entries.

    The paper's abstract reports ablations of the loss design without defining
    them; the plainest alternative to a student normalised over the whole
    vocabulary is one restricted to the same K entries as the teacher:

        z[i, k]  = H[i] . W[idx[i, k]]                 student logits at the cached entries
        lseK[i]  = log sum_k exp(z[i, k])              normaliser over those K entries
        q[i, k]  = exp(z[i, k] - lseK[i])
        KL[i]    = sum_k p[i, k] (log p[i, k] - log q[i, k])    (p log p = 0 at p = 0)
        loss     = mean of KL over the counted rows (every row without labels)

    Every cached entry is its own atom of both distributions (a repeated index
    counts once per entry).  Returns ``(loss, lseK[N], KL[N])``; ignored rows have
    ``lseK = nan`` (their cache rows are not read) and ``KL = 0``.
    """
    H = _f64(H)
    W = _f64(W)
    n = H.shape[0]
    keep = counted_rows(labels, n, ignore_index)
    lse = np.full(n, np.nan)
    rows = np.zeros(n)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        sel = np.nonzero(keep[r0:r1])[0]
        if sel.size == 0:
            continue
        z = H[r0 + sel] @ W.T
        zk = np.take_along_axis(z, np.asarray(idx, dtype=np.int64)[r0 + sel], axis=1)
        lk = logsumexp_rows(zk)
        p, log_p = teacher_probs(np.asarray(val)[r0 + sel], tau)
        rows[r0 + sel] = (_xlogy_self(p, log_p) - p * (zk - lk[:, None])).sum(axis=1)
        lse[r0 + sel] = lk
    count = int(keep.sum())
    loss = float(rows.sum() / count) if count else 0.0
    return loss, lse, rows


def renorm_backward(H, W, idx, val, tau: float, labels=None, ignore_index: int = -100, grad: float = 1.0,
                    block: int = _BLOCK) -> Tuple[np.ndarray, np.ndarray]:
    """``(dH, dW)`` of :func:`renorm_forward`'s loss for upstream gradient ``grad``:

        dZ[i, v] = (g / |C|) sum_{k: idx[i, k] = v} (q[i, k] - p[i, k])    for counted rows i
        dH = dZ @ W,   dW = dZ^T @ H

    (the p-weighted sum of the normaliser's gradient is q because sum_k p = 1).
    dZ is zero outside each row's cached entries.
    """
    H = _f64(H)
    W = _f64(W)
    n = H.shape[0]
    keep = counted_rows(labels, n, ignore_index)
    count = int(keep.sum())
    dH = np.zeros_like(H)
    dW = np.zeros_like(W)
    if count == 0:
        return dH, dW
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        sel = np.nonzero(keep[r0:r1])[0]
        if sel.size == 0:
            continue
        ii = np.asarray(idx, dtype=np.int64)[r0 + sel]
        zk = np.take_along_axis(H[r0 + sel] @ W.T, ii, axis=1)
        q = np.exp(zk - logsumexp_rows(zk)[:, None])
        p, _ = teacher_probs(np.asarray(val)[r0 + sel], tau)
        dz = np.zeros((sel.size, W.shape[0]))
        np.add.at(dz, (np.repeat(np.arange(sel.size), ii.shape[1]), ii.ravel()), (q - p).ravel())
        dz *= float(grad) / count
        dH[r0 + sel] = dz @ W
        dW += dz.T @ H[r0 + sel]
    return dH, dW
