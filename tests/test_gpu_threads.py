"""Calls from several host threads at once.

The compute calls keep no shared mutable state (each call brings its own workspace;
the only cache, the per-device architecture check, is atomic), so threads may call
them concurrently, each on its own stream.  ctypes releases the interpreter lock
during a foreign call, so the library's host code really runs concurrently here.
Every thread's results must equal, bit for bit, those of the same calls made one
after another (the library's results are bitwise reproducible).
"""
import threading

import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd
from gpu_util import device, to_dev

pytestmark = pytest.mark.gpu


def _inputs(i):
    n, d, v, k = 700 + 37 * i, 128, 2000 + 100 * i, 12
    p = kd_synth.small_problem(n, d, v, seed=90 + i)
    return to_dev(p["H"], "bf16"), to_dev(p["W"], "bf16"), to_dev(p["WT"], "bf16"), k


def _run(h, w, wt, k):
    idx, val = kd.kd_topk_cache_build(h, wt, k, chunk_tokens=256)
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, idx, val, 1.3, with_rows=True, chunk_tokens=256)
    dh, dw = kd.kd_chunked_kl_bwd(h, w, idx, val, 1.3, lse, None, chunk_tokens=256)
    return idx, val, loss, lse, rows, dh, dw


def test_concurrent_calls_from_threads():
    print("[case] 4 threads, 4 streams", flush=True)
    inputs = [_inputs(i) for i in range(4)]
    ref = [_run(*x) for x in inputs]
    torch.cuda.synchronize()
    out = [None] * 4
    errors = []
    streams = [torch.cuda.Stream(device=device()) for _ in range(4)]
    start = threading.Barrier(4)

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                start.wait()
                got = []
                for _ in range(3):       # repeated, so the calls of the threads interleave
                    got.append(_run(*inputs[i]))
                streams[i].synchronize()
                out[i] = got
        except Exception as e:           # reported below, in the main thread
            errors.append((i, repr(e)))

    threads = [threading.Thread(target=work, args=(i,)) for i in range(4)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(4):
        for rep in out[i]:
            for a, b in zip(rep, ref[i]):
                assert torch.equal(a, b), f"thread {i}"
