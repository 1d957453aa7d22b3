"""Seeded synthetic inputs for the top-K KL distillation loss over an LM head.

This module only draws numbers and stores them in the dtypes the loss consumes.
It holds none of the loss's arithmetic; the float64 checker and the GPU library
both receive exactly the arrays made here, and neither is imported here.

What is drawn (all float32 normals, then rounded once to the storage dtype):

* student head ``W[V, d] ~ N(0, 1/d)``;
* teacher head ``W_T = W + N(0, 0.5^2/d)`` (a perturbed copy), or for the
  "independent teacher" workload ``W_T ~ N(0, 1/d)`` drawn separately;
* hidden states ``H[N, d] ~ N(0, 1)`` and teacher hidden states ``H_T = H``
  (the synthetic teacher shares the student's final hidden states; only the
  heads differ).

Every matrix is generated in blocks of ``BLOCK_ROWS`` rows.  Each block has its
own PCG64 stream keyed by ``(2026, workload id, point, tensor tag, block)``, so
the result does not depend on how many threads generate it, and a smaller token
count is always a row prefix of a larger one (nested checks across a sweep).

Storage: bfloat16 tensors are returned as ``uint16`` bit patterns (round to
nearest even from float32); float32 tensors as ``float32``.

The sizes follow the web pages' workloads: vocabularies of 32,000, 128,256 and
201,088 entries, top-100 caches (50-500 range), and 4K-256K token batches.
The model hidden sizes are not given on the pages and are fixed per workload.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import Dict, Optional, Tuple

import numpy as np

BLOCK_ROWS = 4096

# Tags for the per-tensor streams.
_TAG_W = 1
_TAG_E = 2       # teacher perturbation noise
_TAG_WT = 3      # independent teacher head
_TAG_H = 4


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload.  ``tokens`` may list several N for a sweep."""
    name: str
    wid: int                    # numeric id used in the seeds
    tokens: Tuple[int, ...]
    d: int
    vocab: int
    ks: Tuple[int, ...]         # cache sizes K exercised on this workload
    tau: float
    dtype: str                  # "bf16" or "f32" for H, W, H_T, W_T
    teacher: str                # "perturbed" or "independent"

    @property
    def val_dtype(self) -> str:
        return "f32" if self.dtype == "f32" else "bf16"


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        # Tiny fp32 case the float64 checker finishes in well under a second;
        # K=16 plus a K=|V| full-distribution variant.
        Workload("tiny_fp32", 0, (256,), 256, 4096, (16, 4096), 1.0, "f32", "perturbed"),
        # One 4096-token sequence, 32,000-entry vocabulary.
        Workload("seq4k_v32k", 1, (4096,), 2048, 32000, (100,), 1.0, "bf16", "perturbed"),
        # One 32,768-token sequence over a 201,088-entry vocabulary.
        Workload("long32k_v201k", 2, (32768,), 2880, 201088, (100,), 1.0, "bf16", "perturbed"),
        # Four packed 32,768-token sequences, 128,256 vocabulary, tau=2,
        # teacher head drawn independently of the student's (high-KL regime).
        Workload("packed131k_v128k", 3, (131072,), 4096, 128256, (100,), 2.0, "bf16", "independent"),
        # Token sweep at the 128,256 vocabulary.
        Workload("sweep_v128k", 4, (4096, 16384, 65536, 262144), 4096, 128256, (50, 100, 500), 1.0,
                 "bf16", "perturbed"),
        # One 32,768-token sequence at the 128,256 vocabulary (the long-context
        # point at which the fused loss is asked to reach half of MFMA peak).
        Workload("ctx32k_v128k", 5, (32768,), 4096, 128256, (100,), 1.0, "bf16", "perturbed"),
    )
}


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(wid: int, point: int, tag: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, wid, point, tag, block])))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _blocked(rows: int, cols: int, fill, out: np.ndarray) -> np.ndarray:
    """Fill ``out`` block by block with ``fill(block_index, r0, r1) -> array``."""
    nblk = (rows + BLOCK_ROWS - 1) // BLOCK_ROWS

    def job(b: int) -> None:
        r0 = b * BLOCK_ROWS
        r1 = min(rows, r0 + BLOCK_ROWS)
        out[r0:r1] = fill(b, r0, r1)

    if nblk == 1:
        job(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(job, range(nblk)))
    return out


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_from_f32(x32) if dtype == "bf16" else x32.astype(np.float32, copy=False)


def _empty(rows: int, cols: int, dtype: str) -> np.ndarray:
    return np.empty((rows, cols), dtype=np.uint16 if dtype == "bf16" else np.float32)


def student_head(w: Workload, point: int = 0) -> np.ndarray:
    """``W[V, d]`` in storage dtype."""
    sc = np.float32(1.0 / np.sqrt(w.d))

    def fill(b, r0, r1):
        return _store(_rng(w.wid, point, _TAG_W, b).standard_normal((r1 - r0, w.d), dtype=np.float32) * sc,
                      w.dtype)

    return _blocked(w.vocab, w.d, fill, _empty(w.vocab, w.d, w.dtype))


def teacher_head(w: Workload, point: int = 0) -> np.ndarray:
    """``W_T[V, d]`` in storage dtype (see module docstring)."""
    sc = np.float32(1.0 / np.sqrt(w.d))
    if w.teacher == "independent":
        def fill(b, r0, r1):
            return _store(_rng(w.wid, point, _TAG_WT, b).standard_normal((r1 - r0, w.d), dtype=np.float32) * sc,
                          w.dtype)
    else:
        noise = np.float32(0.5 / np.sqrt(w.d))

        def fill(b, r0, r1):
            base = _rng(w.wid, point, _TAG_W, b).standard_normal((r1 - r0, w.d), dtype=np.float32) * sc
            if w.dtype == "bf16":
                base = f32_from_bf16_bits(bf16_bits_from_f32(base))
            e = _rng(w.wid, point, _TAG_E, b).standard_normal((r1 - r0, w.d), dtype=np.float32) * noise
            return _store(base + e, w.dtype)

    return _blocked(w.vocab, w.d, fill, _empty(w.vocab, w.d, w.dtype))


def hidden(w: Workload, n_tokens: int, point: int = 0, row0: int = 0) -> np.ndarray:
    """Rows ``[row0, row0 + n_tokens)`` of ``H`` in storage dtype.

    ``row0`` must be a multiple of ``BLOCK_ROWS``; any prefix of a longer draw
    is identical to a shorter draw.
    """
    if row0 % BLOCK_ROWS:
        raise ValueError("row0 must be a multiple of BLOCK_ROWS")
    b0 = row0 // BLOCK_ROWS

    def fill(b, r0, r1):
        g = _rng(w.wid, point, _TAG_H, b0 + b)
        return _store(g.standard_normal((r1 - r0, w.d), dtype=np.float32), w.dtype)

    return _blocked(n_tokens, w.d, fill, _empty(n_tokens, w.d, w.dtype))


def hidden_rows(w: Workload, rows: np.ndarray, point: int = 0) -> np.ndarray:
    """Selected rows of ``H`` (any order) without drawing the whole matrix."""
    rows = np.asarray(rows, dtype=np.int64)
    out = _empty(len(rows), w.d, w.dtype)
    for b in np.unique(rows // BLOCK_ROWS):
        g = _rng(w.wid, point, _TAG_H, int(b))
        last = int(rows[rows // BLOCK_ROWS == b].max() % BLOCK_ROWS)
        blk = _store(g.standard_normal((last + 1, w.d), dtype=np.float32), w.dtype)
        sel = np.nonzero(rows // BLOCK_ROWS == b)[0]
        out[sel] = blk[rows[sel] % BLOCK_ROWS]
    return out


def to_float64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of stored inputs (bf16 bits or float32)."""
    return (f32_from_bf16_bits(x) if dtype == "bf16" else np.asarray(x, np.float32)).astype(np.float64)


def random_cache(n_tokens: int, vocab: int, k: int, seed: int = 0, scale: float = 3.0,
                 val_dtype: str = "bf16", distinct: bool = True) -> Tuple[np.ndarray, np.ndarray]:
    """A cache of the right shape not tied to any head: ``k`` distinct indices per
    row (or with repeats when ``distinct`` is False) and normal values, sorted
    descending.  Used where a cache's provenance does not matter."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, 99, seed])))
    if distinct:
        idx = np.empty((n_tokens, k), dtype=np.int32)
        for i in range(n_tokens):
            idx[i] = g.choice(vocab, size=k, replace=False)
    else:
        idx = g.integers(0, vocab, size=(n_tokens, k), dtype=np.int32)
    val = -np.sort(-g.standard_normal((n_tokens, k), dtype=np.float32) * np.float32(scale), axis=1)
    return idx, _store(val, val_dtype)


def small_problem(n: int, d: int, v: int, seed: int, dtype: str = "bf16",
                  teacher_noise: float = 0.5, logit_scale: float = 1.0) -> Dict[str, np.ndarray]:
    """Arbitrary small shapes (ragged tails etc.) with the workload recipe:
    ``H ~ N(0,1)``, ``W ~ N(0,1/d)``, ``W_T = W + N(0, noise^2/d)``.  ``logit_scale``
    multiplies H before rounding (logits ~ N(0, scale^2): the stress variant for the
    online max / rescaling)."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([2026, 7, seed, n, d, v])))
    sc = np.float32(1.0 / np.sqrt(d))
    w32 = g.standard_normal((v, d), dtype=np.float32) * sc
    w = _store(w32, dtype)
    base = f32_from_bf16_bits(w) if dtype == "bf16" else w32
    wt = _store(base + g.standard_normal((v, d), dtype=np.float32) * np.float32(teacher_noise) * sc, dtype)
    h = _store(g.standard_normal((n, d), dtype=np.float32) * np.float32(logit_scale), dtype)
    return {"H": h, "W": w, "WT": wt, "dtype": dtype}
