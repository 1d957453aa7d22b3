"""The allocation-free forward (kd_chunked_kl_fwd_noalloc, through the C ABI) against
the forward with a caller's workspace (kd_chunked_kl_fwd / _ex): two calls in a row on
the library's one scratch array, the second on a smaller problem, with and without the
loss options.  The forward's results do not depend on the chunk, so the two entry
points agree bit for bit."""
import ctypes

import numpy as np
import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd
from gpu_util import device, to_dev


def _problem(n, d, v, k, seed, dtype="bf16"):
    p = kd_synth.small_problem(n, d, v, seed=seed, dtype=dtype)
    h, w = to_dev(p["H"], dtype), to_dev(p["W"], dtype)
    idx, val = kd_synth.random_cache(n, v, k, seed=seed, val_dtype="bf16" if dtype == "bf16" else "f32")
    return h, w, torch.from_numpy(idx).to(device()), to_dev(val, "bf16" if dtype == "bf16" else "f32")


def _bits(t):
    return t.view(torch.int32)


@pytest.mark.gpu
@pytest.mark.parametrize("with_labels", [False, True])
def test_noalloc_matches_the_workspace_forward_twice(with_labels):
    # first call: 3,000 tokens over three 1,024-token chunks; second: a smaller problem
    cases = [(3000, 256, 5000, 16, 1.0, 1024, 31), (700, 128, 3001, 8, 2.0, 0, 32)]
    for n, d, v, k, tau, chunk, seed in cases:
        print(f"[noalloc] N={n} d={d} V={v} K={k} chunk={chunk} labels={with_labels}", flush=True)
        h, w, idx, val = _problem(n, d, v, k, seed)
        labels, a = None, 0.0
        if with_labels:
            g = np.random.default_rng(seed)
            lab = g.integers(0, v, size=n).astype(np.int32)
            lab[g.random(n) < 0.2] = -100
            labels, a = torch.from_numpy(lab).to(device()), 0.3
        ref_loss, ref_lse, ref_rows = kd.kd_chunked_kl_fwd(h, w, idx, val, tau, with_rows=True, chunk_tokens=chunk,
                                                           labels=labels, ce_weight=a)
        loss = torch.full((), float("nan"), dtype=torch.float32, device=device())
        lse = torch.full((n,), float("nan"), dtype=torch.float32, device=device())
        rows = torch.full((n,), float("nan"), dtype=torch.float32, device=device())
        kd.kd_chunked_kl_fwd_noalloc(h, w, idx, val, tau, loss, lse, rows, chunk_tokens=chunk, labels=labels,
                                     ce_weight=a)
        torch.cuda.synchronize()
        assert torch.isfinite(ref_loss)
        assert torch.equal(_bits(loss), _bits(ref_loss)), (loss.item(), ref_loss.item())
        assert torch.equal(_bits(lse), _bits(ref_lse))
        assert torch.equal(_bits(rows), _bits(ref_rows))


@pytest.mark.gpu
def test_noalloc_float32_and_default_chunk_at_a_large_vocabulary():
    # V = 128,256 with K = 100: the default 16K chunk needs more than the scratch
    # holds, so the call takes the largest chunk that fits (13,824 tokens here)
    n, d, v, k = 20000, 64, 128256, 100
    print(f"[noalloc] N={n} d={d} V={v} K={k} default chunk", flush=True)
    h, w, idx, val = _problem(n, d, v, k, 33)
    ref_loss, ref_lse, _ = kd.kd_chunked_kl_fwd(h, w, idx, val, 1.0)
    loss = torch.empty((), dtype=torch.float32, device=device())
    lse = torch.empty((n,), dtype=torch.float32, device=device())
    kd.kd_chunked_kl_fwd_noalloc(h, w, idx, val, 1.0, loss, lse)
    torch.cuda.synchronize()
    assert torch.equal(_bits(loss), _bits(ref_loss)) and torch.equal(_bits(lse), _bits(ref_lse))
    # float32 inputs, then back to bf16 on a smaller problem
    for dtype, (n2, d2, v2, k2) in (("f32", (513, 64, 2000, 4)), ("bf16", (300, 64, 1000, 3))):
        h, w, idx, val = _problem(n2, d2, v2, k2, 34, dtype=dtype)
        ref_loss, ref_lse, _ = kd.kd_chunked_kl_fwd(h, w, idx, val, 0.5)
        loss = torch.empty((), dtype=torch.float32, device=device())
        lse = torch.empty((n2,), dtype=torch.float32, device=device())
        kd.kd_chunked_kl_fwd_noalloc(h, w, idx, val, 0.5, loss, lse)
        torch.cuda.synchronize()
        assert torch.equal(_bits(loss), _bits(ref_loss)) and torch.equal(_bits(lse), _bits(ref_lse)), dtype


def test_noalloc_rejects_problems_beyond_the_scratch():
    # no device work: the refusal comes before any HIP call
    lib = kd.load_library()
    # an explicit chunk whose workspace exceeds the 64 MiB scratch, and a problem for
    # which even a 256-token chunk does not fit; both refused before any launch
    for prob in (kd.make_problem(65536, 64, 128256, 100, 1.0, kd.KD_BF16, kd.KD_BF16, kd.KD_F32, 16384),
                 kd.make_problem(1024, 64, 2097088, 65535, 1.0, kd.KD_BF16, kd.KD_BF16, kd.KD_F32, 0)):
        st = lib.kd_chunked_kl_fwd_noalloc(ctypes.byref(prob), None, None, None, None, None, None, None, None, None)
        assert st == 15, st   # KD_ERR_SCRATCH_TOO_SMALL
