"""The stored full-size oracle results (``tests/golden/fullsize/``) against the
oracle and input generator as they stand, on a few rows of every workload: each
sampled row's teacher cache is rebuilt with ``oracle.topk_cache`` and its
log-sum-exp and KL with ``oracle.kl_forward``, which must equal the stored float32
values up to the float32 rounding of a float64 that a different BLAS blocking can
move in its last bits.  A stored file that no longer matches what the committed
oracle and generator produce fails here, on the CPU, before any GPU run compares
with it.  (Every row's cache is pinned by the GPU tests through block digests.)"""
import gc
import json
import os

import numpy as np
import pytest

import kd_synth
import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fullsize")

# (file, number of rows stored, K of the stored KL rows)
POINTS = [
    ("seq4k_v32k", 4096, 100),
    ("long32k_v201k", 32768, 100),
    ("ctx32k_v128k", 32768, 100),
    ("packed131k_v128k", 131072, 100),
    ("sweep_v128k", 262144, 100),
]


@pytest.mark.parametrize("name,n,k", POINTS, ids=[p[0] for p in POINTS])
def test_stored_rows_match_the_oracle(name, n, k):
    with open(os.path.join(GOLDEN, f"{name}.json")) as f:
        meta = json.load(f)
    arrays = dict(np.load(os.path.join(GOLDEN, f"{name}.npz")))
    w = kd_synth.WORKLOADS[meta["workload"]]
    assert meta["n"] == n and (meta["d"], meta["vocab"], meta["tau"]) == (w.d, w.vocab, w.tau)
    rows = np.array([0, 1, n // 2 + 3, n - 1], dtype=np.int64)
    H = kd_synth.to_float64(kd_synth.hidden_rows(w, rows), w.dtype)
    WT = kd_synth.to_float64(kd_synth.teacher_head(w), w.dtype)
    idx, val, _ = oracle.topk_cache(H, WT, meta["k_built"], w.val_dtype)
    del WT
    gc.collect()
    val64 = kd_synth.to_float64(val, w.val_dtype)
    W = kd_synth.to_float64(kd_synth.student_head(w), w.dtype)
    _, lse, kl = oracle.kl_forward(H, W, idx[:, :k], val64[:, :k], w.tau)
    del W
    gc.collect()
    np.testing.assert_allclose(lse.astype(np.float32), arrays["lse"][rows], rtol=2e-7, atol=0)
    np.testing.assert_allclose(kl.astype(np.float32), arrays[f"kl_k{k}_n{n}"][rows], rtol=2e-6, atol=1e-7)
