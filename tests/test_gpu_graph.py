"""The library under HIP graph capture.

Every call enqueues kernels only on the caller's stream (no host synchronisation,
no memset nodes, no allocation inside the library), so a training loop can capture
the cache build, the forward and the backward once and replay them.  The captured
graph is replayed several times, with eager work and synchronisations of the
program between the replays, and every replay must equal the eager results bit
for bit (the library's results are bitwise reproducible).  New inputs are then fed
through the captured buffers and the replay must follow them.
"""
import numpy as np
import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd
from gpu_util import device, to_dev

pytestmark = pytest.mark.gpu


def _static_inputs(n, d, v, seed):
    p = kd_synth.small_problem(n, d, v, seed=seed)
    g = np.random.default_rng(seed + 1)
    labels = g.integers(0, v, size=n).astype(np.int32)
    labels[g.random(n) < 0.1] = -100
    return (to_dev(p["H"], "bf16"), to_dev(p["W"], "bf16"), to_dev(p["WT"], "bf16"),
            torch.from_numpy(labels).to(device()))


# (N, d, V, K, chunk): two chunks with ragged tails; and a vocabulary of 274 tiles at
# d = 64, whose dW runs 256 tiles in one launch and the other 18 as split-K partials
# with their sum (first chunk; the short last chunk is not split)
GRAPH_SHAPES = [(1000, 256, 3000, 16, 512), (3000, 64, 70000, 16, 2048)]


@pytest.mark.parametrize("shape", GRAPH_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("with_options", [False, True])
def test_graph_replays_equal_eager(with_options, shape):
    n, d, v, k, chunk = shape
    tau = 1.5
    print(f"[case] graph options={with_options} shape={shape}", flush=True)
    h, w, wt, lab = _static_inputs(n, d, v, seed=51)
    gsc = torch.tensor(0.7, dtype=torch.float32, device=device())
    opt = dict(labels=lab, ignore_index=-100, ce_weight=0.3) if with_options else {}

    def step():
        idx, val = kd.kd_topk_cache_build(h, wt, k, chunk_tokens=chunk)
        loss, lse, rows = kd.kd_chunked_kl_fwd(h, w, idx, val, tau, with_rows=True, chunk_tokens=chunk, **opt)
        dh, dw = kd.kd_chunked_kl_bwd(h, w, idx, val, tau, lse, gsc, chunk_tokens=chunk, **opt)
        return idx, val, loss, lse, rows, dh, dw

    ref = step()
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = step()
    torch.cuda.synchronize()

    x = torch.randn(512, 512, device=device())
    for r in range(3):
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(out, ref):
            assert torch.equal(a, b), f"replay {r}"
        # the program's own eager work between replays: another library call and
        # an unrelated product
        e = step()
        y = x @ x
        torch.cuda.synchronize()
        assert torch.equal(e[2], ref[2]) and torch.isfinite(y).all()
        del e, y

    # new inputs through the captured buffers
    h2, _, _, lab2 = _static_inputs(n, d, v, seed=52)
    h.copy_(h2)
    lab.copy_(lab2)
    ref2 = step()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    for a, b in zip(out, ref2):
        assert torch.equal(a, b)
    assert not torch.equal(ref2[2], ref[2])


@pytest.mark.parametrize("student", ["full", "renorm"])
def test_graph_noalloc_forward(student):
    """The allocation-free forward under capture (the case it exists for: nothing to
    allocate while capturing), with the padding mask and both student normalisers:
    every replay equals the forward with a caller's workspace, bit for bit."""
    n, d, v, k, tau = 3000, 128, 5000, 16, 1.3
    print(f"[case] graph noalloc student={student}", flush=True)
    h, w, wt, lab = _static_inputs(n, d, v, seed=53)
    idx, val = kd.kd_topk_cache_build(h, wt, k)
    ref_loss, ref_lse, ref_rows = kd.kd_chunked_kl_fwd(h, w, idx, val, tau, with_rows=True, labels=lab,
                                                       student=student)
    loss = torch.empty((), dtype=torch.float32, device=device())
    lse = torch.empty((n,), dtype=torch.float32, device=device())
    rows = torch.empty((n,), dtype=torch.float32, device=device())
    kd.kd_chunked_kl_fwd_noalloc(h, w, idx, val, tau, loss, lse, rows, labels=lab, student=student)   # eager
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        kd.kd_chunked_kl_fwd_noalloc(h, w, idx, val, tau, loss, lse, rows, labels=lab, student=student)
    torch.cuda.synchronize()
    for r in range(3):
        loss.zero_()
        lse.zero_()
        rows.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss.view(torch.int32), ref_loss.view(torch.int32)), f"replay {r}"
        assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
        assert torch.equal(rows.view(torch.int32), ref_rows.view(torch.int32))
        e, _, _ = kd.kd_chunked_kl_fwd(h, w, idx, val, tau, labels=lab, student=student)   # eager work between
        torch.cuda.synchronize()
        assert torch.equal(e, ref_loss)
