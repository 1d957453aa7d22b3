"""Writes tests/golden/fullsize/: the float64 oracle's results on every row of the
full-size workloads, for the GPU parity tests to compare against.

For each workload of ``kd_synth.WORKLOADS`` except the tiny float32 one
(4,096 tokens at V = 32,000; 32,768 at V = 201,088; 32,768 and 131,072 at
V = 128,256; the 262,144-token sweep draw at V = 128,256, whose shorter token
counts are its row prefixes):

* the teacher cache that ``oracle.topk_cache`` builds for every row, stored as
  SHA-256 digests of each 4,096-row block: the int32 indices (little-endian,
  row-major ``[rows, K]``) and the stored value bits (bf16 as uint16, float32 as
  uint32).  For the sweep the cache is built once at K = 500; by the oracle's
  ordering (descending logit, ties to the smaller index) the K = 50 and K = 100
  caches are its column prefixes, and their digests are taken from those
  prefixes;
* ``oracle.kl_forward`` on that cache: every row's log-sum-exp and KL (stored as
  float32 in ``<point>.npz``) and the loss (float64, in the JSON).  For the
  sweep, K = 100 over all 262,144 rows, and K = 50 and K = 500 over the first
  16,384 rows.

Calls only ``oracle`` and the input generator ``kd_synth``.  Rows are split into
slices that worker threads hand to the oracle's functions unchanged (each oracle
call sees a contiguous slice of rows; its results do not depend on the slicing,
which the oracle's block-invariance pin covers).  The run takes one to two hours
on eight cores; finished points are kept and skipped when the script is rerun.

    python tests/golden/make_fullsize_golden.py [--threads 8] [--only NAME ...]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import kd_synth  # noqa: E402
import oracle  # noqa: E402

OUT_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "fullsize")
DIGEST_ROWS = 4096
SLICE = 1024          # rows per oracle call in a worker

# (point name, workload, N, K of the cache built, [(K, rows) of the forward])
POINTS = [
    ("seq4k_v32k", "seq4k_v32k", 4096, 100, [(100, 4096)]),
    ("long32k_v201k", "long32k_v201k", 32768, 100, [(100, 32768)]),
    ("ctx32k_v128k", "ctx32k_v128k", 32768, 100, [(100, 32768)]),
    ("packed131k_v128k", "packed131k_v128k", 131072, 100, [(100, 131072)]),
    ("sweep_v128k", "sweep_v128k", 262144, 500, [(100, 262144), (50, 16384), (500, 16384)]),
]
SWEEP_PREFIX_KS = (50, 100, 500)


def log(msg: str) -> None:
    print(f"[golden {time.strftime('%H:%M:%S')}] {msg}", flush=True)


def block_digests(a: np.ndarray) -> list:
    """SHA-256 of each DIGEST_ROWS-row block of a C-contiguous little-endian array."""
    out = []
    for r0 in range(0, a.shape[0], DIGEST_ROWS):
        blk = np.ascontiguousarray(a[r0:r0 + DIGEST_ROWS], dtype=a.dtype.newbyteorder("<"))
        out.append(hashlib.sha256(blk.tobytes()).hexdigest())
    return out


def val_bits(val: np.ndarray, val_dtype: str) -> np.ndarray:
    return val.view(np.uint16) if val_dtype == "bf16" else np.ascontiguousarray(val, np.float32).view(np.uint32)


def run_slices(n: int, job, threads: int, what: str) -> None:
    t0 = time.time()
    done = 0
    with cf.ThreadPoolExecutor(threads) as ex:
        futs = [ex.submit(job, r0, min(n, r0 + SLICE)) for r0 in range(0, n, SLICE)]
        for f in cf.as_completed(futs):
            f.result()
            done += 1
            if done % 16 == 0 or done == len(futs):
                log(f"  {what}: {done}/{len(futs)} slices, {time.time() - t0:.0f} s")


def make_point(name: str, wname: str, n: int, kc: int, fwd: list, threads: int) -> None:
    w = kd_synth.WORKLOADS[wname]
    jpath = os.path.join(OUT_DIR, f"{name}.json")
    if os.path.exists(jpath):
        log(f"{name}: present, skipped")
        return
    log(f"{name}: N={n} d={w.d} V={w.vocab} K={kc} tau={w.tau} {w.dtype}")
    H = kd_synth.hidden(w, n)
    W64 = kd_synth.to_float64(kd_synth.student_head(w), w.dtype)
    WT64 = kd_synth.to_float64(kd_synth.teacher_head(w), w.dtype)

    idx = np.empty((n, kc), dtype=np.int32)
    val = np.empty((n, kc), dtype=np.uint16 if w.val_dtype == "bf16" else np.float32)

    def teacher(r0, r1):
        hs = kd_synth.to_float64(H[r0:r1], w.dtype)
        i, v, _ = oracle.topk_cache(hs, WT64, kc, w.val_dtype)
        idx[r0:r1] = i
        val[r0:r1] = v

    run_slices(n, teacher, threads, "teacher top-K")
    del WT64

    ks = SWEEP_PREFIX_KS if name == "sweep_v128k" else (kc,)
    digests = {}
    for k in ks:
        ik = np.ascontiguousarray(idx[:, :k])
        vk = np.ascontiguousarray(val[:, :k])
        digests[str(k)] = {"idx": block_digests(ik), "val": block_digests(val_bits(vk, w.val_dtype))}

    arrays = {}
    losses = {}
    lse_all = None
    for k, rows in fwd:
        lse = np.empty(rows)
        kl = np.empty(rows)
        ik = np.ascontiguousarray(idx[:rows, :k])
        v64 = kd_synth.to_float64(np.ascontiguousarray(val[:rows, :k]), w.val_dtype)

        def forward(r0, r1):
            hs = kd_synth.to_float64(H[r0:r1], w.dtype)
            _, l, r = oracle.kl_forward(hs, W64, ik[r0:r1], v64[r0:r1], w.tau)
            lse[r0:r1] = l
            kl[r0:r1] = r

        run_slices(rows, forward, threads, f"forward K={k} on {rows} rows")
        losses[f"{k}_{rows}"] = {"k": k, "rows": rows, "loss": float(kl.sum() / rows)}
        arrays[f"kl_k{k}_n{rows}"] = kl.astype(np.float32)
        if lse_all is None or rows > lse_all.shape[0]:
            lse_all = lse
    arrays["lse"] = lse_all.astype(np.float32)
    np.savez_compressed(os.path.join(OUT_DIR, f"{name}.npz"), **arrays)
    meta = {
        "workload": wname, "n": n, "d": w.d, "vocab": w.vocab, "tau": w.tau, "dtype": w.dtype,
        "val_dtype": w.val_dtype, "teacher": w.teacher, "k_built": kc, "digest_rows": DIGEST_ROWS,
        "digest": "sha256 of each block: idx int32 little-endian [rows, K]; val bits (bf16 uint16 / f32 uint32)",
        "cache": digests, "forward": losses,
        "arrays": {k: list(v.shape) for k, v in arrays.items()},
        "writer": "tests/golden/make_fullsize_golden.py (oracle.topk_cache, oracle.kl_forward)",
    }
    with open(jpath + ".tmp", "w") as f:
        json.dump(meta, f, indent=1)
        f.write("\n")
    os.replace(jpath + ".tmp", jpath)
    summary = ", ".join("K=%d loss=%.6f" % (v["k"], v["loss"]) for v in losses.values())
    log(f"{name}: written ({summary})")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--threads", type=int, default=len(os.sched_getaffinity(0)))
    ap.add_argument("--only", nargs="*", default=None)
    args = ap.parse_args()
    os.makedirs(OUT_DIR, exist_ok=True)
    from threadpoolctl import threadpool_limits
    with threadpool_limits(1):      # one BLAS thread per worker; the workers run in parallel
        for name, wname, n, kc, fwd in POINTS:
            if args.only and name not in args.only:
                continue
            make_point(name, wname, n, kc, fwd, args.threads)
    return 0


if __name__ == "__main__":
    sys.exit(main())
