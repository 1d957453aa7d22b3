"""The C ABI from plain C: tests/c_abi/kd_client (built by the package's build step
with gcc against libkdkl.so and the HIP runtime's C API, no torch) builds the
teacher cache, runs the forward and the backward; its outputs must match the
float64 oracle on the same inputs.  It also writes the cache to shard files and
streams them back with the loader (include/kdcache.h): the loss from that copy must
be the same float.  Last it runs the _ex calls with a padding mask and a hard-label
mix (kd_loss_opts), checked against ``oracle.variant_forward`` / ``variant_backward``,
and streams the device cache to shards with the streaming writer."""
import os
import subprocess

import numpy as np
import pytest

import kd_synth
import oracle
from gpu_util import GRAD_TOL, LOSS_RTOL, LSE_RTOL, rel_max_err

pytestmark = pytest.mark.gpu

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "kd_client")


def test_c_client_matches_oracle(tmp_path):
    assert os.path.exists(CLIENT), f"{CLIENT} is not built (python -m lm_head_kl_amd.build)"
    n, d, v, k, tau = 300, 64, 1000, 8, 1.5
    p = kd_synth.small_problem(n, d, v, seed=12, dtype="bf16")
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([n, d, v], dtype=np.int64).tobytes())
        f.write(np.array([k], dtype=np.int32).tobytes())
        f.write(np.array([tau], dtype=np.float32).tobytes())
        for a in (p["H"], p["W"], p["WT"]):
            f.write(np.ascontiguousarray(a).view(np.uint16).tobytes())
    print(f"[c-client] N={n} d={d} V={v} K={k}", flush=True)
    r = subprocess.run([CLIENT, str(inp), str(out), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    buf = open(out, "rb").read()
    off = 0

    def take(dtype, count):
        nonlocal off
        a = np.frombuffer(buf, dtype=dtype, count=count, offset=off)
        off += a.nbytes
        return a

    assert take(np.int32, 1)[0] == 0
    g_idx = take(np.int32, n * k).reshape(n, k)
    g_val = take(np.uint16, n * k).reshape(n, k)
    g_loss = float(take(np.float32, 1)[0])
    g_lse = take(np.float32, n)
    g_dh = take(np.float32, n * d).reshape(n, d)
    g_dw = take(np.float32, v * d).reshape(v, d)
    g_loss2 = take(np.float32, 1)[0]
    g_loss3 = float(take(np.float32, 1)[0])
    g_dh3 = take(np.float32, n * d).reshape(n, d)
    g_dw3 = take(np.float32, v * d).reshape(v, d)
    writer_ok = take(np.int32, 1)[0]
    assert off == len(buf)
    assert writer_ok == 1                                 # the streaming writer's shards hold the cache
    assert np.float32(g_loss) == g_loss2                 # same cache bytes, same loss
    assert (tmp_path / "c0.kdc").exists() and (tmp_path / "c1.kdc").exists()

    H = kd_synth.to_float64(p["H"], "bf16")
    W = kd_synth.to_float64(p["W"], "bf16")
    WT = kd_synth.to_float64(p["WT"], "bf16")
    idx, val, _ = oracle.topk_cache(H, WT, k, "bf16")
    np.testing.assert_array_equal(g_idx, idx)
    np.testing.assert_array_equal(g_val, val)
    v64 = kd_synth.to_float64(val, "bf16")
    ref_loss, ref_lse, _ = oracle.kl_forward(H, W, idx, v64, tau)
    ref_dH, ref_dW = oracle.kl_backward(H, W, idx, v64, tau)
    assert abs(g_loss - ref_loss) <= LOSS_RTOL * abs(ref_loss)
    np.testing.assert_allclose(g_lse.astype(np.float64), ref_lse, rtol=LSE_RTOL)
    assert rel_max_err(g_dh.astype(np.float64), ref_dH) <= GRAD_TOL
    assert rel_max_err(g_dw.astype(np.float64), ref_dW) <= GRAD_TOL

    i = np.arange(n)
    labels = np.where(i % 7 == 3, -100, (131 * i) % v).astype(np.int32)
    ref_loss3, _, _ = oracle.variant_forward(H, W, idx, v64, tau, labels, -100, 0.25)
    ref_dH3, ref_dW3 = oracle.variant_backward(H, W, idx, v64, tau, labels, -100, 0.25)
    assert abs(g_loss3 - ref_loss3) <= LOSS_RTOL * abs(ref_loss3)
    assert rel_max_err(g_dh3.astype(np.float64), ref_dH3) <= GRAD_TOL
    assert rel_max_err(g_dw3.astype(np.float64), ref_dW3) <= GRAD_TOL
    assert not g_dh3[i % 7 == 3].any()
