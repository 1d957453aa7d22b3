"""Parity at the workloads' full sizes, with the step run exactly as the benchmark
runs it: ``kd_chunked_kl_fwd`` with the library's default chunk and no per-row
output, then ``kd_chunked_kl_bwd`` with bf16 dH (the bf16-store epilogue of the dH
product, unsplit at 16K-token chunks) and the default chunk.

What is compared, per workload:

* the teacher cache of every row, bit for bit: SHA-256 digests of each 4,096-row
  block of the GPU's idx and val against those of the oracle's cache, stored in
  ``tests/golden/fullsize/`` by ``tests/golden/make_fullsize_golden.py`` (oracle and
  input generator only);
* every row's lse and KL and the loss against the oracle's, stored by the same
  script (KL rows from a second forward call with the per-row output, whose loss
  must equal the benchmark call's bit for bit);
* dH and dW: at 4,096 and 32,768 tokens (both 32K workloads) and at 16,384 tokens
  of the sweep, every element against the oracle's backward, run here on the GPU
  host (one to two minutes each).  At 65,536 and more tokens the oracle's
  backward over every row would take several minutes, so dH is compared on seeded
  sample rows, and dW through properties that hold at any size: each dZ row sums
  to zero, so dW's columns do; dW over all tokens equals the token-weighted sum of
  dW over each chunk alone.
"""
import hashlib
import json
import os

import numpy as np
import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd
import oracle
from gpu_util import GRAD_TOL, LOSS_RTOL, LSE_RTOL, bf16_bits_of, device, rel_max_err, to_dev, to_f64

pytestmark = pytest.mark.gpu

CHUNK = 16384   # the library's default tokens per chunk
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fullsize")


def golden(name):
    with open(os.path.join(GOLDEN, f"{name}.json")) as f:
        meta = json.load(f)
    arrays = dict(np.load(os.path.join(GOLDEN, f"{name}.npz")))
    return meta, arrays


def sample_rows(n, count, seed):
    g = np.random.default_rng(seed)
    fixed = [0, n - 1] + [c + o for c in range(CHUNK, n, CHUNK) for o in (-1, 0)][:6]
    rest = g.choice(n, size=max(0, count - len(fixed)), replace=False)
    return np.unique(np.array(fixed + list(rest), dtype=np.int64))


def check_cache(idx, val, meta, k, n):
    """Every row of the GPU cache against the oracle's block digests."""
    rows = meta["digest_rows"]
    assert n % rows == 0
    want = meta["cache"][str(k)]
    ih = idx.cpu().numpy()
    vh = bf16_bits_of(val) if meta["val_dtype"] == "bf16" else val.cpu().numpy().view(np.uint32)
    bad = []
    for b in range(n // rows):
        r0, r1 = b * rows, (b + 1) * rows
        di = hashlib.sha256(np.ascontiguousarray(ih[r0:r1], dtype="<i4").tobytes()).hexdigest()
        dv = hashlib.sha256(np.ascontiguousarray(vh[r0:r1], dtype=vh.dtype.newbyteorder("<")).tobytes()).hexdigest()
        if di != want["idx"][b] or dv != want["val"][b]:
            bad.append((b, di != want["idx"][b], dv != want["val"][b]))
    assert not bad, f"cache blocks (block, idx differs, val differs) of {rows} rows: {bad[:10]}"


def chunked_rel_err(got: torch.Tensor, ref: np.ndarray, rows: int = 8192) -> float:
    """max |got - ref| / max |ref| without a second full-size float64 copy on the host."""
    scale = float(np.abs(ref).max())
    err = 0.0
    for r0 in range(0, ref.shape[0], rows):
        g = got[r0:r0 + rows].double().cpu().numpy()
        err = max(err, float(np.abs(g - ref[r0:r0 + rows]).max()))
    return err / (scale if scale > 0 else 1.0)


def bench_step(h, wd, idx, val, tau, dh_dtype):
    """The benchmark's step (bench.py: measure.step)."""
    loss, lse, rows = kd.kd_chunked_kl_fwd(h, wd, idx, val, tau, chunk_tokens=0)
    assert rows is None
    dh, dw = kd.kd_chunked_kl_bwd(h, wd, idx, val, tau, lse, None, dh_dtype=dh_dtype, chunk_tokens=0)
    return loss, lse, dh, dw


def run_workload(name, n, k, full_oracle, sample=64, golden_name=None):
    w = kd_synth.WORKLOADS[name]
    meta, arrays = golden(golden_name or name)
    assert (meta["workload"], meta["d"], meta["vocab"], meta["tau"]) == (w.name, w.d, w.vocab, w.tau)
    print(f"[fullsize] {name} N={n} K={k}", flush=True)
    H = kd_synth.hidden(w, n)
    W = kd_synth.student_head(w)
    h, wd, wt = to_dev(H, w.dtype), to_dev(W, w.dtype), to_dev(kd_synth.teacher_head(w), w.dtype)
    idx, val = kd.kd_topk_cache_build(h, wt, k)
    del wt
    dh_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    loss, lse, dh, dw = bench_step(h, wd, idx, val, w.tau, dh_dtype)
    loss2, lse2, rows = kd.kd_chunked_kl_fwd(h, wd, idx, val, w.tau, with_rows=True)
    torch.cuda.synchronize()

    # the cache, every row
    check_cache(idx, val, meta, k, n)
    print(f"[fullsize]   cache: {n // meta['digest_rows']} blocks equal the oracle's", flush=True)
    # loss, lse and KL, every row
    fw = meta["forward"].get(f"{k}_{n}")
    kl_key = next((key for key in arrays if key.startswith(f"kl_k{k}_n") and int(key.split("_n")[1]) >= n), None)
    assert kl_key is not None, f"no stored KL rows for K={k} covering {n} rows"
    ref_kl = arrays[kl_key][:n].astype(np.float64)
    ref_loss = fw["loss"] if fw is not None else float(ref_kl.sum() / n)
    assert torch.equal(loss.view(torch.int32), loss2.view(torch.int32))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    assert abs(loss.item() - ref_loss) <= LOSS_RTOL * abs(ref_loss), (loss.item(), ref_loss)
    np.testing.assert_allclose(to_f64(lse), arrays["lse"][:n].astype(np.float64), rtol=LSE_RTOL)
    np.testing.assert_allclose(to_f64(rows), ref_kl, rtol=LOSS_RTOL, atol=LOSS_RTOL)
    print(f"[fullsize]   loss {loss.item():.6f} (oracle {ref_loss:.6f}); lse and KL of every row", flush=True)

    W64 = kd_synth.to_float64(W, w.dtype)
    if full_oracle:
        H64 = kd_synth.to_float64(H, w.dtype)
        v64 = kd_synth.to_float64(bf16_bits_of(val) if w.val_dtype == "bf16" else val.cpu().numpy(), w.val_dtype)
        ref_dH, ref_dW = oracle.kl_backward(H64, W64, idx.cpu().numpy(), v64, w.tau, block=512)
        e_dh, e_dw = chunked_rel_err(dh, ref_dH), chunked_rel_err(dw, ref_dW)
        print(f"[fullsize]   every element: dH err {e_dh:.2e}, dW err {e_dw:.2e}", flush=True)
        assert e_dh <= GRAD_TOL and e_dw <= GRAD_TOL
        return
    # dH on sampled rows (the oracle normalises by its own row count; rescale to 1/N)
    rs = sample_rows(n, sample, seed=n + k)
    rs_t = torch.from_numpy(rs).to(device())
    H64 = kd_synth.to_float64(H[rs], w.dtype)
    ih = idx[rs_t].cpu().numpy()
    vv = val[rs_t]
    v64 = kd_synth.to_float64(bf16_bits_of(vv) if w.val_dtype == "bf16" else vv.cpu().numpy(), w.val_dtype)
    ref_dH, _ = oracle.kl_backward(H64, W64, ih, v64, w.tau)
    ref_dH *= len(rs) / n
    assert rel_max_err(to_f64(dh[rs_t]), ref_dH) <= GRAD_TOL
    # Columns of dW sum to zero up to the bf16 rounding of dZ: each dZ row sums to
    # zero exactly, rounding moves each element by at most 2^-8 of its size, and
    # sum_v |dZ[t, v]| <= 2 / N, so |sum_v dW[v, j]| <= 2^-7 / N * sum_t |H[t, j]|.
    dw64 = dw.double()
    colsum = dw64.sum(0).abs()
    bound = 2.0 ** -7 / n * h.double().abs().sum(0) * 1.01 + 2.0 ** -20 * dw64.abs().sum(0)
    assert bool((colsum <= bound).all()), float((colsum / bound).max())
    del dw64
    print(f"[fullsize]   dH on {len(rs)} sampled rows; dW column sums", flush=True)
    return h, wd, idx, val, dw


def test_seq4k_v32k():
    """4,096 tokens, d=2048, V=32,000, K=100 (split-K dH)."""
    run_workload("seq4k_v32k", 4096, 100, full_oracle=True)


@pytest.mark.timeout(900)
def test_long32k_v201k():
    """32,768 tokens, d=2880, V=201,088: every element of dH and dW."""
    run_workload("long32k_v201k", 32768, 100, full_oracle=True)


@pytest.mark.timeout(900)
def test_ctx32k_v128k():
    """32,768 tokens at V=128,256, d=4,096: the point where half of MFMA peak is
    asked for; every element of dH and dW."""
    run_workload("ctx32k_v128k", 32768, 100, full_oracle=True)


@pytest.mark.timeout(600)
def test_packed131k_v128k():
    """131,072 tokens, tau = 2, independent teacher: the benchmark's default
    workload.  Also chunk additivity of dW over the eight 16K-token chunks."""
    h, wd, idx, val, dw = run_workload("packed131k_v128k", 131072, 100, full_oracle=False)
    w = kd_synth.WORKLOADS["packed131k_v128k"]
    n = h.shape[0]
    acc = torch.zeros_like(dw, dtype=torch.float64)
    for c0 in range(0, n, CHUNK):
        c1 = min(n, c0 + CHUNK)
        hc, ic, vc = h[c0:c1].contiguous(), idx[c0:c1].contiguous(), val[c0:c1].contiguous()
        _, lc, _ = kd.kd_chunked_kl_fwd(hc, wd, ic, vc, w.tau)
        _, dwc = kd.kd_chunked_kl_bwd(hc, wd, ic, vc, w.tau, lc, None, dh_dtype=torch.bfloat16)
        acc += dwc.double() * ((c1 - c0) / n)
        del dwc
    torch.cuda.synchronize()
    assert (acc - dw.double()).abs().max().item() <= 1e-4 * dw.abs().max().item()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("n,k", [(4096, 50), (4096, 500), (16384, 50), (16384, 500), (65536, 100),
                                 (262144, 100)])
def test_sweep_points(n, k):
    run_workload("sweep_v128k", n, k, full_oracle=False, sample=32)


@pytest.mark.timeout(900)
def test_sweep_16k_full():
    """16,384 tokens of the sweep at K = 100: every element of dH and dW."""
    run_workload("sweep_v128k", 16384, 100, full_oracle=True)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("k", [50, 500])
def test_sweep_262k_cache(k):
    """The teacher cache of all 262,144 sweep tokens at K = 50 and K = 500, every row."""
    w = kd_synth.WORKLOADS["sweep_v128k"]
    meta, _ = golden("sweep_v128k")
    n = 262144
    print(f"[fullsize] sweep_v128k cache N={n} K={k}", flush=True)
    h = to_dev(kd_synth.hidden(w, n), w.dtype)
    wt = to_dev(kd_synth.teacher_head(w), w.dtype)
    idx, val = kd.kd_topk_cache_build(h, wt, k)
    torch.cuda.synchronize()
    check_cache(idx, val, meta, k, n)


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
    dh, dw = kd.kd_chunked_kl_bwd(h, wd, ti, tv, w.tau, lse, None, dh_dtype=torch.bfloat16, labels=tl, ce_weight=a)
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
