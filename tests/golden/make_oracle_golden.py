"""Writes tests/golden/oracle_tiny_fp32.json: the float64 oracle's results on the
tiny float32 workload (256 tokens, d = 256, V = 4,096, tau = 1; teacher caches of
K = 16 and K = V built by the oracle).  Calls only ``oracle`` and the input
generator ``kd_synth``; rerun it (python tests/golden/make_oracle_golden.py) only
for a change to the oracle's arithmetic that a passage of the pages justifies."""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import kd_synth  # noqa: E402
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny_fp32.json")


def compute():
    w = kd_synth.WORKLOADS["tiny_fp32"]
    H = kd_synth.to_float64(kd_synth.hidden(w, w.tokens[0]), w.dtype)
    W = kd_synth.to_float64(kd_synth.student_head(w), w.dtype)
    WT = kd_synth.to_float64(kd_synth.teacher_head(w), w.dtype)
    out = {"workload": w.name, "n": int(H.shape[0]), "d": int(H.shape[1]), "v": int(W.shape[0]), "tau": w.tau,
           "cases": {}}
    for k in w.ks:
        idx, val, _ = oracle.topk_cache(H, WT, k, "f32")
        v64 = kd_synth.to_float64(val, "f32")
        loss, lse, rows = oracle.kl_forward(H, W, idx, v64, w.tau)
        dH, dW = oracle.kl_backward(H, W, idx, v64, w.tau)
        out["cases"][str(k)] = {
            "idx_first_row": idx[0, :8].tolist(),
            "val_bits_first_row": val[0, :8].view(np.uint32).tolist(),
            "loss": float(loss),
            "lse_first": lse[:8].tolist(),
            "kl_rows_first": rows[:8].tolist(),
            "kl_rows_sum": float(rows.sum()),
            "dH_fro": float(np.linalg.norm(dH)),
            "dW_fro": float(np.linalg.norm(dW)),
            "dW_first": dW[0, :8].tolist(),
        }
    return out


if __name__ == "__main__":
    data = compute()
    with open(OUT, "w") as f:
        json.dump(data, f, indent=1)
        f.write("\n")
    print(f"wrote {OUT}")
