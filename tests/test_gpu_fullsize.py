"""Parity at the workloads' full sizes, in the launch configuration the benchmark
uses (library-default chunking).

The float64 oracle cannot evaluate every row at these sizes, so each workload is
checked on a seeded sample of rows (always including the first and last row and
rows on both sides of a chunk boundary) that the oracle computes one by one:
top-K indices and values bit-exact, per-row log-sum-exp and KL, and dH rows.  dW
needs every row; it is checked element-wise at the 4K-token workload and through
properties that hold at any size elsewhere (every row of dZ sums to zero, so the
columns of dW sum to zero; the loss is the mean of the per-row KL).
"""
import numpy as np
import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd
import oracle
from gpu_util import GRAD_TOL, LOSS_RTOL, LSE_RTOL, bf16_bits_of, device, rel_max_err, to_dev, to_f64

pytestmark = pytest.mark.gpu

CHUNK = 16384   # the library's default tokens per chunk


def sample_rows(n, count, seed):
    g = np.random.default_rng(seed)
    fixed = [0, n - 1] + [c + o for c in range(CHUNK, n, CHUNK) for o in (-1, 0)][:6]
    rest = g.choice(n, size=max(0, count - len(fixed)), replace=False)
    return np.unique(np.array(fixed + list(rest), dtype=np.int64))


def run_workload(name, n, k, rows_count=24, full_dw=False):
    w = kd_synth.WORKLOADS[name]
    print(f"[fullsize] {name} N={n} K={k}", flush=True)
    H = kd_synth.hidden(w, n)
    W = kd_synth.student_head(w)
    WT = kd_synth.teacher_head(w)
    h, wd, wt = to_dev(H, w.dtype), to_dev(W, w.dtype), to_dev(WT, w.dtype)
    idx, val = kd.kd_topk_cache_build(h, wt, k)
    del wt
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, wd, idx, val, w.tau, with_rows=True)
    dh, dw = kd.kd_chunked_kl_bwd(h, wd, idx, val, w.tau, lse, None,
                                  dh_dtype=torch.float32)
    torch.cuda.synchronize()

    rs = sample_rows(n, rows_count, seed=n + k)
    rs_t = torch.from_numpy(rs).to(device())
    H64 = kd_synth.to_float64(H[rs], w.dtype)
    W64 = kd_synth.to_float64(W, w.dtype)
    WT64 = kd_synth.to_float64(WT, w.dtype)
    ref_idx, ref_val, _ = oracle.topk_cache(H64, WT64, k, w.val_dtype)
    g_idx = idx[rs_t].cpu().numpy()
    np.testing.assert_array_equal(g_idx, ref_idx)
    g_val = val[rs_t]
    if w.val_dtype == "bf16":
        np.testing.assert_array_equal(bf16_bits_of(g_val), ref_val)
    else:
        np.testing.assert_array_equal(g_val.cpu().numpy().view(np.uint32), ref_val.view(np.uint32))

    vref = kd_synth.to_float64(ref_val, w.val_dtype)
    _, ref_lse, ref_rows = oracle.kl_forward(H64, W64, ref_idx, vref, w.tau)
    np.testing.assert_allclose(to_f64(lse[rs_t]), ref_lse, rtol=LSE_RTOL)
    np.testing.assert_allclose(to_f64(rows[rs_t]), ref_rows, rtol=LOSS_RTOL, atol=LOSS_RTOL)
    # dH rows: the oracle normalises by its own row count; rescale to 1/N
    ref_dH, _ = oracle.kl_backward(H64, W64, ref_idx, vref, w.tau)
    ref_dH *= len(rs) / n
    assert rel_max_err(to_f64(dh[rs_t]), ref_dH) <= GRAD_TOL

    # properties at any size
    r_all = rows.double()
    assert torch.isfinite(r_all).all() and (r_all >= -1e-4).all()
    assert abs(r_all.mean().item() - loss.item()) <= 1e-5 * abs(loss.item())
    # Columns of dW sum to zero up to the bf16 rounding of dZ: each dZ row sums to
    # zero exactly, rounding moves each element by at most 2^-8 of its size, and
    # sum_v |dZ[t, v]| <= 2 / N, so |sum_v dW[v, j]| <= 2^-7 / N * sum_t |H[t, j]|.
    dw64 = dw.double()
    colsum = dw64.sum(0).abs()
    bound = 2.0 ** -7 / n * h.double().abs().sum(0) * 1.01 + 2.0 ** -20 * dw64.abs().sum(0)
    assert bool((colsum <= bound).all()), float((colsum / bound).max())
    del dw64
    if n > CHUNK:
        # chunk additivity: dW over all N tokens equals the token-weighted sum of
        # dW over each chunk alone (checks the cross-chunk accumulation)
        acc = torch.zeros_like(dw, dtype=torch.float64)
        for c0 in range(0, n, CHUNK):
            c1 = min(n, c0 + CHUNK)
            hc, ic, vc = h[c0:c1].contiguous(), idx[c0:c1].contiguous(), val[c0:c1].contiguous()
            _, lc, _ = kd.kd_chunked_kl_fwd(hc, wd, ic, vc, w.tau)
            _, dwc = kd.kd_chunked_kl_bwd(hc, wd, ic, vc, w.tau, lc, None, dh_dtype=torch.float32)
            acc += dwc.double() * ((c1 - c0) / n)
            del dwc
        torch.cuda.synchronize()
        assert (acc - dw.double()).abs().max().item() <= 1e-4 * dw.abs().max().item()
        del acc

    if full_dw:
        # Every element: the oracle builds its own cache for all rows; the GPU
        # cache must equal it, and the GPU loss and gradients are recomputed on
        # the oracle's cache bytes.
        Hall = kd_synth.to_float64(H, w.dtype)
        oi, ov, _ = oracle.topk_cache(Hall, WT64, k, w.val_dtype)
        np.testing.assert_array_equal(idx.cpu().numpy(), oi)
        ref_loss, ref_lse_all, _ = oracle.kl_forward(Hall, W64, oi, kd_synth.to_float64(ov, w.val_dtype), w.tau)
        ref_dH_all, ref_dW = oracle.kl_backward(Hall, W64, oi, kd_synth.to_float64(ov, w.val_dtype), w.tau)
        ti, tv = torch.from_numpy(oi).to(device()), to_dev(ov, w.val_dtype)
        loss2, lse2, _ = kd.kd_chunked_kl_fwd(h, wd, ti, tv, w.tau)
        dh2, dw2 = kd.kd_chunked_kl_bwd(h, wd, ti, tv, w.tau, lse2, None, dh_dtype=torch.float32)
        torch.cuda.synchronize()
        assert abs(loss2.item() - ref_loss) <= LOSS_RTOL * abs(ref_loss)
        np.testing.assert_allclose(to_f64(lse2), ref_lse_all, rtol=LSE_RTOL)
        assert rel_max_err(to_f64(dh2), ref_dH_all) <= GRAD_TOL
        assert rel_max_err(to_f64(dw2), ref_dW) <= GRAD_TOL
    return loss.item()


def test_seq4k_v32k_full():
    """4,096 tokens, d=2048, V=32,000, K=100: every output element checked,
    including the whole teacher cache and dW."""
    run_workload("seq4k_v32k", 4096, 100, rows_count=32, full_dw=True)


def test_long32k_v201k():
    run_workload("long32k_v201k", 32768, 100)


def test_ctx32k_v128k():
    run_workload("ctx32k_v128k", 32768, 100)


def test_packed131k_v128k():
    run_workload("packed131k_v128k", 131072, 100, rows_count=16)


@pytest.mark.parametrize("n,k", [(4096, 50), (4096, 500), (262144, 100)])
def test_sweep_points(n, k):
    run_workload("sweep_v128k", n, k, rows_count=12)


def test_peak_memory_linear_in_tokens():
    """Peak device memory of forward + backward grows linearly with N, with a
    slope of a few KB per token (inputs, cache and gradients), far below the
    2 x V bytes per token an N x V bf16 logit tensor would add.  The HIP runtime's
    used-memory count (hipMemGetInfo) moves with torch's reserved memory: no device
    memory is allocated outside the caller's allocator."""
    w = kd_synth.WORKLOADS["sweep_v128k"]
    torch.cuda.synchronize()
    free0, total0 = torch.cuda.mem_get_info()
    runtime_base = (total0 - free0) - torch.cuda.memory_reserved()   # context and other non-torch use
    W = to_dev(kd_synth.student_head(w), "bf16")
    Hfull = kd_synth.hidden(w, 131072)
    peaks = {}
    for n in (16384, 32768, 65536, 131072):     # at or above one chunk: the workspace is fixed
        h = to_dev(Hfull[:n], "bf16")
        idx, val = kd_synth.random_cache(n, w.vocab, 100, seed=n)
        ti, tv = torch.from_numpy(idx).to(device()), to_dev(val, "bf16")
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        loss, lse, _ = kd.kd_chunked_kl_fwd(h, W, ti, tv, 1.0)
        dh, dw = kd.kd_chunked_kl_bwd(h, W, ti, tv, 1.0, lse, None, dh_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        peaks[n] = torch.cuda.max_memory_allocated() - base + (h.numel() * 2 + idx.size * 6)
        del loss, lse, dh, dw, h, ti, tv
    # the runtime's view agrees with torch's: the library allocates no device memory
    # of its own (everything, workspace included, comes through the caching allocator)
    free, total = torch.cuda.mem_get_info()
    assert (total - free) - torch.cuda.memory_reserved() - runtime_base < 256 << 20
    ns = np.array(sorted(peaks), dtype=np.float64)
    ps = np.array([peaks[int(x)] for x in ns])
    b, a = np.polyfit(ns, ps, 1)
    resid = np.abs(ps - (a + b * ns)).max() / ps.max()
    print(f"[fullsize] peak bytes {dict(zip(ns.astype(int).tolist(), ps.tolist()))}, slope {b:.0f} B/token")
    assert resid < 0.02
    assert b < 0.1 * 2 * w.vocab      # no N x V term
    assert b > 2 * w.d                 # at least H itself


def test_loss_options_ctx32k_v128k():
    """The loss options at full size, in the benchmark's launch configuration:
    32,768 tokens, V = 128,256, d = 4,096, a synthetic cache of K = 100, labels
    over the vocabulary with the last 1/16 of each 8,192 tokens ignored (padding)
    and a cross-entropy weight of 0.5.  Sampled rows against the oracle (row
    terms, lse, dH rows); the loss is the mean of the row terms over the counted
    rows; dW's columns sum to zero (each counted dZ row still sums to zero)."""
    w = kd_synth.WORKLOADS["ctx32k_v128k"]
    n, k, a, ign = 32768, 100, 0.5, -100
    print(f"[fullsize] loss options {w.name} N={n} K={k} a={a}", flush=True)
    H = kd_synth.hidden(w, n)
    W = kd_synth.student_head(w)
    idx, valb = kd_synth.random_cache(n, w.vocab, k, seed=41)
    g = np.random.default_rng(42)
    labels = g.integers(0, w.vocab, size=n).astype(np.int32)
    labels[np.arange(n) % 8192 >= 8192 - 512] = ign
    h, wd = to_dev(H, w.dtype), to_dev(W, w.dtype)
    ti, tv, tl = torch.from_numpy(idx).to(device()), to_dev(valb, "bf16"), torch.from_numpy(labels).to(device())
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, wd, ti, tv, w.tau, with_rows=True, labels=tl, ce_weight=a)
    dh, dw = kd.kd_chunked_kl_bwd(h, wd, ti, tv, w.tau, lse, None, dh_dtype=torch.float32, labels=tl, ce_weight=a)
    torch.cuda.synchronize()

    count = int((labels != ign).sum())
    rs = np.unique(np.concatenate([sample_rows(n, 20, seed=43), [8192 - 1, 8192 - 512, 8192 - 513]]))
    rs_t = torch.from_numpy(rs).to(device())
    H64 = kd_synth.to_float64(H[rs], w.dtype)
    W64 = kd_synth.to_float64(W, w.dtype)
    v64 = kd_synth.to_float64(valb[rs], "bf16")
    _, ref_lse, ref_rows = oracle.variant_forward(H64, W64, idx[rs], v64, w.tau, labels[rs], ign, a)
    np.testing.assert_allclose(to_f64(lse[rs_t]), ref_lse, rtol=LSE_RTOL)
    np.testing.assert_allclose(to_f64(rows[rs_t]), ref_rows, rtol=LOSS_RTOL, atol=LOSS_RTOL)
    # dH rows: the oracle divides by the sample's counted rows; rescale to the batch's
    c_s = int((labels[rs] != ign).sum())
    ref_dH, _ = oracle.variant_backward(H64, W64, idx[rs], v64, w.tau, labels[rs], ign, a)
    ref_dH *= c_s / count
    assert rel_max_err(to_f64(dh[rs_t]), ref_dH) <= GRAD_TOL
    assert not dh[torch.from_numpy(labels == ign).to(device())].any()

    r_all = rows.double()
    assert torch.isfinite(r_all).all()
    assert abs(r_all.sum().item() / count - loss.item()) <= 1e-5 * abs(loss.item())
    dw64 = dw.double()
    colsum = dw64.sum(0).abs()
    bound = 2.0 ** -7 / count * h.double().abs().sum(0) * 1.01 + 2.0 ** -20 * dw64.abs().sum(0)
    assert bool((colsum <= bound).all()), float((colsum / bound).max())
