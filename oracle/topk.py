"""Float64 definition of the offline teacher cache (test infrastructure).

Source: the paper's abstract (offline KD caches the teacher's top-K logits
once) and the llm-wiki study note, section "핵심 아이디어 1: Offline Top-K
Logits" / "사전 계산(Pre-computation) 파이프라인": the teacher is run once over
the data and, at every token position, the K highest logits are stored as
(vocab index, logit value) pairs.

Readings where the pages are silent:

* The teacher logits are ``S = H_T @ W_T^T`` evaluated exactly in float64 on
  the stored input values.
* Order within a row: descending logit; equal logits are ordered by the
  smaller vocabulary index first.  So the top-K' for K' < K is a prefix.
* Indices are int32 (the pages' int16 only covers vocabularies below 65,536;
  the vocabularies here reach 201,088).
* Stored values: the float64 logit rounded once, to nearest with ties to even,
  directly to bfloat16 (or to float32 for float32 caches); never through an
  intermediate float32 rounding.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_to_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even).

    bfloat16 keeps 8 significant bits and float32's exponent range; below
    2^-126 the spacing is the subnormal quantum 2^-133.  Returns float64
    values that are exactly representable in bfloat16.
    """
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, e = np.frexp(ax)                      # ax = m * 2^e with m in [0.5, 1)
    ex = np.maximum(e.astype(np.int64) - 1, -126)
    q = np.ldexp(1.0, (ex - 7).astype(np.int32))
    with np.errstate(over="ignore", invalid="ignore"):
        r = np.rint(ax / q) * q              # np.rint rounds halves to even
    r = np.where(np.isfinite(ax), r, ax)
    r = np.where(r > _BF16_MAX, np.inf, r)
    r = np.where(ax == 0.0, 0.0, r)
    out = np.copysign(r, x)
    return np.where(np.isnan(x), np.nan, out)


def bf16_bits(values_exact) -> np.ndarray:
    """Bit patterns of float64 values that are already exact bfloat16 values."""
    f = np.asarray(values_exact, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def topk_cache(H_T, W_T, k: int, val_dtype: str = "bf16", block: int = 256
               ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Exact per-row top-K of the teacher logits.

    Returns ``(idx int32 [N,K], val [N,K], scores float64 [N,K])``; ``val`` is
    bf16 bit patterns (``uint16``) or ``float32`` values per ``val_dtype``.
    """
    H_T = np.asarray(H_T, np.float64)
    W_T = np.asarray(W_T, np.float64)
    n = H_T.shape[0]
    v = W_T.shape[0]
    if not 1 <= k <= v:
        raise ValueError("need 1 <= k <= V")
    idx = np.empty((n, k), dtype=np.int32)
    sc = np.empty((n, k), dtype=np.float64)
    for r0 in range(0, n, block):
        r1 = min(n, r0 + block)
        s = H_T[r0:r1] @ W_T.T
        order = np.argsort(-s, axis=1, kind="stable")[:, :k]     # ties keep ascending index
        idx[r0:r1] = order
        sc[r0:r1] = np.take_along_axis(s, order, axis=1)
    if val_dtype == "bf16":
        val = bf16_bits(round_to_bf16(sc))
    elif val_dtype == "f32":
        val = sc.astype(np.float32)           # float64 -> float32 cast rounds to nearest even
    else:
        raise ValueError(val_dtype)
    return idx, val, sc
