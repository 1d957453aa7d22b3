#!/usr/bin/env python
"""Throughput of the fused, chunked top-K KL loss (forward + backward) on one MI355X.

A step is one forward (``kd_chunked_kl_fwd``) and one backward
(``kd_chunked_kl_bwd``) pass over one batch of synthetic tokens: logits
recomputed tile by tile in both passes, online log-sum-exp, cached-entry
gather, dZ, dH and dW.  The teacher cache is built once beforehand with
``kd_topk_cache_build`` (the offline pass) and timed separately.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused LM-head+top-K KL fwd+bwd tokens/s (V=128256,d=4096); MFMA util; peak GB"
BF16_DENSE_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
FP32_DENSE_PEAK_TFLOPS = 157.3
HBM_PEAK_GBS = 8000.0
# the GEMM kernels and the host code that sets their launch shapes: the committed
# traffic table is used only while these are unchanged
KERNEL_SOURCES = ("lm_head_kl_amd/csrc/kd_gemm.hpp", "lm_head_kl_amd/csrc/kd_common.hpp",
                  "lm_head_kl_amd/csrc/kdkl.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_for(kind: str):
    """HBM bytes per launch of `kind` from the committed counter summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash():
        return None
    k = t.get("kernels", {}).get(kind)
    return None if k is None else k.get("bytes_per_launch")


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


class ClockSampler:
    """Samples the GPU's metrics table (amdsmi, every 25 ms) in a background thread
    between start() and stop(): the graphics clock, the socket power and the
    firmware's count of time spent at the package power limit (PPT).  stop() returns
    {"mhz", "snapshots", "power_w", "ppt_frac"}, or None when the clock cannot be read
    (no amdsmi, or not exactly one GPU visible to it) or fewer than two fresh readings
    came in; power_w and ppt_frac are None when the table lacks them.  The firmware
    refreshes the table about once a second, so readings are kept once per table
    snapshot (its system clock counter), and the snapshot current at start() is left
    out: it predates the measured work.  ppt_frac is the growth of the PPT residency
    counter over that of the table's accumulation counter between the first and the
    last fresh snapshot.  A timed region under two seconds therefore reports nothing."""

    MIN_SNAPSHOTS = 2

    def __init__(self):
        self.samples = []
        self.handle = None
        self.power_cap_w = None
        self._stop = None
        self._thread = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            if len(hs) == 1:
                self.handle = hs[0]
                self._amdsmi = amdsmi
                self._read()
                try:   # reported in microwatts
                    cap = amdsmi.amdsmi_get_power_cap_info(self.handle).get("power_cap")
                    self.power_cap_w = round(cap / 1e6, 1) if isinstance(cap, (int, float)) and cap > 0 else None
                except Exception:
                    self.power_cap_w = None
        except Exception:
            self.handle = None

    @staticmethod
    def _num(x):
        return x if isinstance(x, (int, float)) and not isinstance(x, bool) else None

    def _read(self):
        # (snapshot id, MHz, W, PPT residency, accumulation counter): the per-XCD
        # graphics clocks of the GPU metrics table, averaged; else the clock query's
        # single value (no snapshot id, no power)
        try:
            m = self._amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
            xs = [float(x) for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and 0 < x < 5000]
            ts = m.get("system_clock_counter")
            if xs:
                return ((ts if isinstance(ts, int) else None), sum(xs) / len(xs), self._num(m.get("current_socket_power")),
                        self._num(m.get("ppt_residency_acc")), self._num(m.get("accumulation_counter")))
        except Exception:
            pass
        c = self._amdsmi.amdsmi_get_clock_info(self.handle, self._amdsmi.AmdSmiClkType.GFX)
        return None, float(c["clk"]), None, None, None

    def _run(self):
        import time as _t
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except Exception:
                pass
            _t.sleep(0.025)

    def start(self):
        if self.handle is None:
            return
        import threading
        try:
            self._stale = self._read()[0]
        except Exception:
            self._stale = None
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        if self.handle is None or self._thread is None:
            return None
        self._stop.set()
        self._thread.join()
        self._thread = None
        seen, kept = set(), []
        for smp in self.samples:
            ts, mhz = smp[0], smp[1]
            if mhz <= 0:
                continue
            if ts is not None:
                if ts == self._stale or ts in seen:
                    continue
                seen.add(ts)
            kept.append(smp)
        if len(kept) < self.MIN_SNAPSHOTS:
            return None
        watts = [k[2] for k in kept if k[2] is not None and k[2] > 0]
        ppt = None
        first, last = kept[0], kept[-1]
        if None not in (first[3], first[4], last[3], last[4]) and last[4] > first[4]:
            ppt = max(0.0, min(1.0, (last[3] - first[3]) / (last[4] - first[4])))
        return {"mhz": sum(k[1] for k in kept) / len(kept), "snapshots": len(kept),
                "power_w": (sum(watts) / len(watts)) if watts else None, "ppt_frac": ppt}


def cpu_baseline(workload, n_rows: int, k: int):
    """The float64 oracle, as it stands, on the first ``n_rows`` tokens of the same
    workload (full vocabulary and hidden size) with a synthetic cache of the same
    shape; returns tokens/s of its forward + backward."""
    import numpy as np
    import kd_synth
    import oracle
    blas = None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in libs] or [1])
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')} ({libs[0].get('threading_layer')})"
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    H = kd_synth.to_float64(kd_synth.hidden(workload, n_rows), workload.dtype)
    W = kd_synth.to_float64(kd_synth.student_head(workload), workload.dtype)
    idx, valb = kd_synth.random_cache(n_rows, workload.vocab, k, seed=5, val_dtype=workload.val_dtype)
    val = kd_synth.to_float64(valb, workload.val_dtype)
    t0 = time.perf_counter()
    oracle.kl_forward(H, W, idx, val, workload.tau)
    oracle.kl_backward(H, W, idx, val, workload.tau)
    dt = time.perf_counter() - t0
    return {"value": n_rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": host_cpu_model(), "blas": blas, "numpy": np.__version__,
            "sample": f"first {n_rows} tokens of the workload (full V={workload.vocab}, d={workload.d}, K={k}), "
                      f"float64 forward+backward, synthetic cache of the same shape; {dt:.1f} s"}


def run_point(kd, torch, w, h, wd, wt, n, k, steps, warmup, chunk=0):
    """Cache build (timed once) and `steps` timed fwd+bwd steps on the first n rows of h."""
    hn = h[:n]
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    idx, val = kd.kd_topk_cache_build(hn, wt, k)
    e1.record()
    torch.cuda.synchronize()
    cache_ms = e0.elapsed_time(e1)
    dh_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    torch.cuda.empty_cache()
    # peak of this point alone: the step's own inputs (H rows, W, cache) plus everything
    # the step allocates (outputs, workspace); other resident tensors are excluded
    own = hn.numel() * hn.element_size() + wd.numel() * wd.element_size() + \
        idx.numel() * idx.element_size() + val.numel() * val.element_size()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()

    def step():
        loss, lse, _ = kd.kd_chunked_kl_fwd(hn, wd, idx, val, w.tau, chunk_tokens=chunk)
        dh, dw = kd.kd_chunked_kl_bwd(hn, wd, idx, val, w.tau, lse, None, dh_dtype=dh_dtype, chunk_tokens=chunk)
        return loss

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        loss = step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    peak_gb = (torch.cuda.max_memory_allocated() - base + own) / 1e9
    flops = 8.0 * n * w.vocab * w.d
    peak_tf = BF16_DENSE_PEAK_TFLOPS if w.dtype == "bf16" else FP32_DENSE_PEAK_TFLOPS
    out = {"workload": w.name, "n_tokens": n, "d": w.d, "vocab": w.vocab, "k": k, "tau": w.tau,
           "tokens_per_s": round(n / (ms / 1e3), 1), "ms_per_step": round(ms, 3),
           "mfma_util": round(flops / (ms / 1e3) / (peak_tf * 1e12), 4), "peak_gb": round(peak_gb, 3),
           "cache_build_ms": round(cache_ms, 2), "loss": round(loss.item(), 5)}
    del idx, val
    return out


def sweep(kd, torch, np, kd_synth, steps, warmup):
    points = [("seq4k_v32k", None), ("long32k_v201k", None), ("ctx32k_v128k", None), ("packed131k_v128k", None),
              ("sweep_v128k", None)]
    rows = []
    for name, _ in points:
        w = kd_synth.WORKLOADS[name]
        dev = torch.device("cuda:0")

        def to_dev(x):
            if w.dtype == "bf16":
                return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(x).to(dev)

        nmax = max(w.tokens)
        t0 = time.perf_counter()
        h = to_dev(kd_synth.hidden(w, nmax))      # shorter token counts are row prefixes
        wd = to_dev(kd_synth.student_head(w))
        wt = to_dev(kd_synth.teacher_head(w))
        log(f"{name}: inputs for N<={nmax} in {time.perf_counter() - t0:.1f}s")
        for n in w.tokens:
            for k in w.ks:
                r = run_point(kd, torch, w, h, wd, wt, n, k, steps, warmup)
                rows.append(r)
                print(json.dumps(r), flush=True)
                log(f"  N={n:7d} K={k:3d}: {r['tokens_per_s']:10.0f} tokens/s  {r['ms_per_step']:9.2f} ms  "
                    f"MFMA {100 * r['mfma_util']:.1f}%  peak {r['peak_gb']:.2f} GB  cache {r['cache_build_ms']:.1f} ms")
        del h, wd, wt
        torch.cuda.empty_cache()
    log("| workload | N | d | V | K | tokens/s | ms/step | MFMA util (8NVd, 2.5 PF) | peak GB | cache build ms |")
    log("|---|---|---|---|---|---|---|---|---|---|")
    for r in rows:
        log(f"| {r['workload']} | {r['n_tokens']:,} | {r['d']:,} | {r['vocab']:,} | {r['k']} | {r['tokens_per_s']:,.0f} | "
            f"{r['ms_per_step']:.2f} | {100 * r['mfma_util']:.1f} % | {r['peak_gb']:.2f} | {r['cache_build_ms']:.1f} |")
    for fit in peak_memory_fits(np, rows):
        print(json.dumps(fit), flush=True)
        log(f"peak memory, {fit['workload']} K={fit['k']}: {fit['intercept_gb']:.3f} GB + {fit['slope_bytes_per_token']:,.0f} "
            f"B/token (expected {fit['expected_bytes_per_token']:,} = H, bf16 dH, cache, lse), largest residual "
            f"{100 * fit['max_rel_residual']:.2f} %, over N = {fit['n_tokens']}; an N x V bf16 tensor would add "
            f"{2 * fit['vocab']:,} B/token")
    return 0


def peak_memory_fits(np, rows, chunk=16384):
    """Least-squares line peak(N) = a + b N per (workload, K) over the sweep points at
    or above one token chunk (below it the backward's workspace is smaller).  Linear
    memory means b is the per-token inputs and outputs only: H and dH (2d bytes each in
    bf16), the cache (4 + 2 bytes per entry) and lse (4 bytes), with no term in V."""
    out = []
    groups = {}
    for r in rows:
        if r["n_tokens"] >= chunk:
            groups.setdefault((r["workload"], r["k"]), []).append(r)
    for (name, k), rs in groups.items():
        if len(rs) < 3:
            continue
        ns = np.array([r["n_tokens"] for r in rs], dtype=np.float64)
        ps = np.array([r["peak_gb"] * 1e9 for r in rs])
        b, a = np.polyfit(ns, ps, 1)
        d = rs[0]["d"]
        out.append({"peak_memory_fit": True, "workload": name, "k": k, "vocab": rs[0]["vocab"],
                    "n_tokens": [int(x) for x in ns], "intercept_gb": round(float(a) / 1e9, 4),
                    "slope_bytes_per_token": round(float(b), 1), "expected_bytes_per_token": 2 * d + 2 * d + 6 * k + 4,
                    "max_rel_residual": round(float(np.abs(ps - (a + b * ns)).max() / ps.max()), 5)})
    return out


def cache_io(kd, torch, idx, val, vocab, shards=4, batch=16384, prefetch=3, with_paths=None):
    """Write the built cache to shards in a temporary directory and stream it back
    to the device with the loader (the files were just written, so this measures the
    page cache and the upload path, not a disk).  Checks the streamed cache is the
    original, bit for bit."""
    import shutil
    import tempfile
    ih, vh = idx.cpu(), val.cpu()
    n = ih.shape[0]
    d = tempfile.mkdtemp(prefix="kdcache_")
    try:
        paths = [os.path.join(d, f"part{i:03d}.kdc") for i in range(shards)]
        cuts = [n * i // shards for i in range(shards + 1)]
        t0 = time.perf_counter()
        for i, p in enumerate(paths):
            kd.kd_cache_write(p, ih[cuts[i]:cuts[i + 1]].contiguous(), vh[cuts[i]:cuts[i + 1]].contiguous(), vocab)
        t_write = time.perf_counter() - t0
        nbytes = sum(os.path.getsize(p) for p in paths)
        bits = kd.kd_cache_info_read(paths[0])["idx_bits"]
        li, lv = torch.empty_like(idx), torch.empty_like(val)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h = kd.kd_cache_loader_open(paths, batch, prefetch)
        try:
            row = 0
            while True:
                r = kd.kd_cache_loader_next(h, li[row:row + batch], lv[row:row + batch])
                if r == 0:
                    break
                row += r
        finally:
            kd.kd_cache_loader_close(h)
        torch.cuda.synchronize()
        t_load = time.perf_counter() - t0
        exact = bool(torch.equal(li, idx)) and bool(torch.equal(lv.view(torch.int16 if lv.dtype == torch.bfloat16
                                                                         else torch.int32),
                                                                val.view(torch.int16 if val.dtype == torch.bfloat16
                                                                         else torch.int32)))
        if not exact or row != n:
            raise RuntimeError("cache streamed back through the loader differs from the cache written")
        out = {"bytes": nbytes, "shards": shards, "idx_bits": bits, "batch_tokens": batch,
               "write_gbs": nbytes / t_write / 1e9, "load_gbs": nbytes / t_load / 1e9,
               "load_tokens_per_s": n / t_load, "exact": exact,
               "note": "files in the page cache; host->device through pinned buffers"}
        if with_paths is not None:
            out["loss_fed_by_loader"] = with_paths(paths)
        return out
    finally:
        shutil.rmtree(d, ignore_errors=True)


def loader_fed_steps(kd, torch, h, wd, idx, val, w, dh_dtype, paths, batch=16384):
    """Training fed from the cache files: the loader streams the shards in batches of
    `batch` tokens while each batch's forward and backward run on the GPU.  The same
    per-batch loop with the cache already in device memory is timed beside it, so
    the difference is what reading the cache costs the loss."""
    def step(i, v, r0, rows):
        hb = h[r0:r0 + rows]
        loss, lse, _ = kd.kd_chunked_kl_fwd(hb, wd, i, v, w.tau)
        kd.kd_chunked_kl_bwd(hb, wd, i, v, w.tau, lse, None, dh_dtype=dh_dtype)

    n = h.shape[0]
    step(idx[:batch], val[:batch], 0, min(batch, n))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for r0 in range(0, n, batch):
        rows = min(batch, n - r0)
        step(idx[r0:r0 + rows], val[r0:r0 + rows], r0, rows)
    torch.cuda.synchronize()
    t_mem = time.perf_counter() - t0
    t0 = time.perf_counter()
    r0 = 0
    with kd.CacheLoader(paths, batch, 3, str(h.device)) as ld:
        for i, v in ld:
            step(i, v, r0, i.shape[0])
            r0 += i.shape[0]
    torch.cuda.synchronize()
    t_ld = time.perf_counter() - t0
    if r0 != n:
        raise RuntimeError("the loader handed out a different number of rows than the cache holds")
    return {"tokens_per_s": n / t_ld, "from_memory_tokens_per_s": n / t_mem, "batch_tokens": batch,
            "ratio": round(t_mem / t_ld, 4)}


def cache_pipeline(kd, torch, h, wt, k, vocab, ref_idx, ref_val, batch=32768, shard=32768):
    """The offline pass end to end: the teacher cache built batch by batch on the
    GPU and handed to the streaming writer as it is produced, until every shard is
    on disk (page cache).  Checks the shards against the cache built in one call.
    Reports the writer's fixed costs (opening: pinned buffers; closing: the last
    shard's write after the GPU is done) beside the whole."""
    import shutil
    import tempfile
    n = h.shape[0]
    d = tempfile.mkdtemp(prefix="kdpipe_")
    try:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        wr = kd.CacheWriter(os.path.join(d, "cache"), shard, vocab, k, ref_val.dtype, batch)
        t1 = time.perf_counter()
        for r0 in range(0, n, batch):
            i, v = kd.kd_topk_cache_build(h[r0:r0 + batch], wt, k)
            wr.put(i, v)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        wr.close()
        t3 = time.perf_counter()
        got_i = torch.cat([kd.kd_cache_read(p)[0] for p in wr.paths])
        got_v = torch.cat([kd.kd_cache_read(p)[1] for p in wr.paths])
        bits = torch.int16 if got_v.dtype == torch.bfloat16 else torch.int32
        if not (torch.equal(got_i, ref_idx.cpu()) and torch.equal(got_v.view(bits), ref_val.cpu().view(bits))):
            raise RuntimeError("shards written by the pipeline differ from the cache built in one call")
        t = t3 - t0
        return {"tokens_per_s": n / t, "ms": round(t * 1e3, 1), "batch_tokens": batch, "shard_tokens": shard,
                "shards": len(wr.paths), "bytes": sum(os.path.getsize(p) for p in wr.paths), "exact": True,
                "open_ms": round((t1 - t0) * 1e3, 1), "gpu_ms": round((t2 - t1) * 1e3, 1),
                "close_ms": round((t3 - t2) * 1e3, 1)}
    finally:
        shutil.rmtree(d, ignore_errors=True)


def variants(kd, torch, h, wd, idx, val, w, dh_dtype, steps, chunk, ce_weight=0.5, seq=32768, pad_frac=1 / 16):
    """The same step with the loss options on: labels drawn over the vocabulary,
    the last ``pad_frac`` of every ``seq``-token sequence marked as padding
    (ignore index -100), and a cross-entropy mix of weight ``ce_weight``.  Tokens/s
    counts every token of the batch, padded or not."""
    n = h.shape[0]
    g = torch.Generator().manual_seed(7)
    lab = torch.randint(0, w.vocab, (n,), generator=g, dtype=torch.int32)
    pos = torch.arange(n) % seq
    lab[pos >= seq - int(seq * pad_frac)] = -100
    ignored = float((lab == -100).float().mean())
    lab = lab.to(h.device)

    def vstep():
        loss, lse, _ = kd.kd_chunked_kl_fwd(h, wd, idx, val, w.tau, chunk_tokens=chunk, labels=lab,
                                            ce_weight=ce_weight)
        dh, dw = kd.kd_chunked_kl_bwd(h, wd, idx, val, w.tau, lse, None, dh_dtype=dh_dtype, chunk_tokens=chunk,
                                      labels=lab, ce_weight=ce_weight)
        return loss, dh, dw

    vstep()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    out = None
    for _ in range(steps):
        out = None
        out = vstep()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    loss = out[0].item()
    del out
    out = {"tokens_per_s": n / (ms / 1e3), "ms_per_step": round(ms, 3), "ce_weight": ce_weight,
           "ignored_frac": round(ignored, 4), "loss": round(loss, 5),
           "options": f"labels over V, last 1/{round(1 / pad_frac)} of every {seq}-token sequence ignored"}

    # the student renormalised over the cached entries (no mix), same mask
    def rstep():
        loss, lse, _ = kd.kd_chunked_kl_fwd(h, wd, idx, val, w.tau, chunk_tokens=chunk, labels=lab,
                                            student="renorm")
        dh, dw = kd.kd_chunked_kl_bwd(h, wd, idx, val, w.tau, lse, None, dh_dtype=dh_dtype, chunk_tokens=chunk,
                                      labels=lab, student="renorm")
        return loss, dh, dw

    rstep()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r = None
        r = rstep()
    torch.cuda.synchronize()
    rms = (time.perf_counter() - t0) * 1e3 / steps
    out["student_renorm"] = {"tokens_per_s": n / (rms / 1e3), "ms_per_step": round(rms, 3),
                             "loss": round(r[0].item(), 5)}
    del r
    # its dominant kernel against HBM bandwidth: the gathered rows (K W rows per token
    # for the logits and for dH, K H rows per token for dW) are its algorithmic bytes
    kd.profile_begin()
    r = rstep()
    torch.cuda.synchronize()
    stats = kd.profile_end()
    del r
    dom_kind, dom = max(stats.items(), key=lambda kv: kv[1]["total_ms"])
    avg_s = dom["total_ms"] / dom["launches"] / 1e3
    achieved = dom["bytes"] / dom["launches"] / avg_s / 1e9
    out["student_renorm"]["roofline"] = {
        "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4), "kernel": dom_kind, "avg_launch_ms": round(avg_s * 1e3, 4),
        "bytes_per_launch": dom["bytes"] / dom["launches"]}
    out["student_renorm"]["kernels_ms_per_step"] = {k2: round(v["total_ms"], 4) for k2, v in stats.items()}
    return out


def inputs_and_cache(kd, torch, np, kd_synth, w, n, k, dev, timed=True):
    """Device inputs of workload ``w`` (first n tokens) and its teacher cache, built
    with kd_topk_cache_build (H_T = H: the synthetic teacher shares the hidden
    states); the second build is timed."""
    def to_dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    t0 = time.perf_counter()
    h = to_dev(kd_synth.hidden(w, n))
    wd = to_dev(kd_synth.student_head(w))
    wt = to_dev(kd_synth.teacher_head(w))
    torch.cuda.synchronize()
    log(f"{w.name}: N={n} d={w.d} V={w.vocab} K={k} tau={w.tau} {w.dtype}; inputs in "
        f"{time.perf_counter() - t0:.1f}s")
    idx, val = kd.kd_topk_cache_build(h, wt, k)
    torch.cuda.synchronize()
    cache = None
    if timed:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        idx, val = kd.kd_topk_cache_build(h, wt, k)
        e1.record()
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1)
        cache = {"ms": round(cms, 3), "tokens_per_s": n / (cms / 1e3),
                 "mfma_frac": 2.0 * n * w.vocab * w.d / (cms / 1e3) / (BF16_DENSE_PEAK_TFLOPS * 1e12)}
        log(f"cache build {cms:.1f} ms ({cache['tokens_per_s']:.0f} tokens/s)")
    del wt
    return h, wd, idx, val, cache


def measure(kd, torch, w, h, wd, idx, val, n, k, steps, warmup, chunk, clock, min_seconds=0.0):
    """`warmup` untimed and `steps` timed fwd+bwd steps.  Whole-run wall time gives
    tokens/s; HIP events on the launch stream give each step's time (median, min)
    and, through the library's profiling hooks, each kernel's average launch time
    (the roofline of the dominant kernel).  The graphics clock is sampled meanwhile.
    With `min_seconds`, more steps are timed if `steps` would take less than that
    (estimated from the last warmup step), so the clock sampler sees enough of the
    GPU's metrics snapshots (about one a second)."""
    dev = h.device
    dh_dtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def step():
        loss, lse, _ = kd.kd_chunked_kl_fwd(h, wd, idx, val, w.tau, chunk_tokens=chunk)
        dh, dw = kd.kd_chunked_kl_bwd(h, wd, idx, val, w.tau, lse, None, dh_dtype=dh_dtype, chunk_tokens=chunk)
        return loss, dh, dw

    est = None
    nwarm = max(warmup, 1 if min_seconds > 0 else 0)
    for i in range(nwarm):
        t0 = time.perf_counter()
        wl = step()[0].item()
        torch.cuda.synchronize()
        est = time.perf_counter() - t0
        log(f"warmup {i + 1}/{nwarm} loss={wl:.5f}")
    if min_seconds > 0 and est and steps * est < min_seconds:
        steps = int(min_seconds / est) + 1
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    kd.profile_begin()
    clock.start()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    out = None
    ev[0].record()
    for i in range(steps):
        out = None          # a training loop has consumed the previous step's gradients
        out = step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    clk = clock.stop()
    stats = kd.profile_end()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    # peak of the step: what it allocates (outputs, workspace) on top of the resident
    # inputs (H, W, cache), counted in full
    own = sum(t.numel() * t.element_size() for t in (h, wd, idx, val))
    peak_gb = (torch.cuda.max_memory_allocated(dev) - base + own) / 1e9
    loss_val = out[0].item()
    del out
    ms = t_total * 1e3 / steps
    flops_step = 8.0 * n * w.vocab * w.d
    peak_tf = BF16_DENSE_PEAK_TFLOPS if w.dtype == "bf16" else FP32_DENSE_PEAK_TFLOPS
    mfma_util = flops_step / (ms / 1e3) / (peak_tf * 1e12)
    mid = per_step[len(per_step) // 2] if steps % 2 else 0.5 * (per_step[steps // 2 - 1] + per_step[steps // 2])
    # utilisation against the peak at the clock measured meanwhile (the peak scales with
    # it); a reading that would put the MFMA pipes above their peak is not a clock the
    # kernels ran at (e.g. under a profiler), and is dropped
    if clk is not None and mfma_util * 2400.0 / clk["mhz"] > 1.0:
        log(f"clock samples ({clk['mhz']:.0f} MHz) inconsistent with the measured throughput; not reported")
        clk = None
    clock_mhz = None if clk is None else round(clk["mhz"], 1)
    util_clk = None if clk is None else round(mfma_util * 2400.0 / clk["mhz"], 4)
    power_w = None if clk is None or clk["power_w"] is None else round(clk["power_w"], 1)
    ppt = None if clk is None or clk["ppt_frac"] is None else round(clk["ppt_frac"], 4)
    log(f"{steps} steps: {ms:.2f} ms/step (median {mid:.2f}, min {per_step[0]:.2f}), {n / (ms / 1e3):.0f} tokens/s, "
        f"MFMA {100 * mfma_util:.1f}% of dense peak at 2.4 GHz"
        + (f", {100 * util_clk:.1f}% at the measured {clock_mhz:.0f} MHz ({clk['snapshots']} metrics snapshots)"
           if clk else "")
        + (f", {power_w:.0f} W" + (f" of the {clock.power_cap_w:.0f} W cap" if clock.power_cap_w else "")
           if power_w is not None else "")
        + (f", at the power limit {100 * ppt:.0f}% of the time" if ppt is not None else "")
        + f", peak {peak_gb:.2f} GB, loss={loss_val:.5f}")
    tot = sum(v["total_ms"] for v in stats.values())
    for kind, st in sorted(stats.items(), key=lambda kv: -kv[1]["total_ms"]):
        avg = st["total_ms"] / max(1, st["launches"])
        tf = st["flops"] / (st["total_ms"] / 1e3) / 1e12 if st["flops"] and st["total_ms"] else 0.0
        gbs = st["bytes"] / (st["total_ms"] / 1e3) / 1e9 if st["total_ms"] else 0.0
        log(f"  {kind:14s} {st['launches']:5d} launches  {st['total_ms'] / steps:9.3f} ms/step "
            f"({100 * st['total_ms'] / tot:5.1f}%)  avg {avg:8.3f} ms  {tf:7.1f} TFLOP/s  {gbs:7.1f} GB/s")
    dom_kind, dom = max(stats.items(), key=lambda kv: kv[1]["total_ms"])
    avg_s = dom["total_ms"] / dom["launches"] / 1e3
    per_launch_flops = dom["flops"] / dom["launches"]
    if per_launch_flops > 0:
        achieved = per_launch_flops / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(achieved / peak_tf, 4), "traffic": traffic_for(dom_kind), "kernel": dom_kind,
                "avg_launch_ms": round(avg_s * 1e3, 4), "flops_per_launch": per_launch_flops}
    else:
        achieved = dom["bytes"] / dom["launches"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_for(dom_kind), "kernel": dom_kind,
                "avg_launch_ms": round(avg_s * 1e3, 4)}
    return {"workload": w.name, "n_tokens": n, "d": w.d, "vocab": w.vocab, "k": k, "tau": w.tau, "steps": steps,
            "tokens_per_s": round(n / (ms / 1e3), 1), "ms_per_step": round(ms, 3), "ms_median": round(mid, 3),
            "ms_min": round(per_step[0], 3), "mfma_util": round(mfma_util, 4),
            "mfma_util_measured_clock": util_clk, "clock_mhz": clock_mhz, "power_w": power_w,
            "power_limit_residency": ppt, "peak_gb": round(peak_gb, 3),
            "loss": round(loss_val, 5), "roofline": roof,
            "kernels_ms_per_step": {k2: round(v["total_ms"] / steps, 4) for k2, v in stats.items()},
            "_stats": stats}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="packed131k_v128k")
    ap.add_argument("--tokens", type=int, default=0, help="override N (e.g. a sweep point)")
    ap.add_argument("--k", type=int, default=0, help="override K")
    ap.add_argument("--chunk", type=int, default=0, help="tokens per chunk (0 = library default)")
    ap.add_argument("--cpu-rows", type=int, default=4096)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-cache-build-timing", action="store_true")
    ap.add_argument("--no-cache-io", action="store_true",
                    help="skip writing the cache to shards and streaming it back with the loader")
    ap.add_argument("--no-target-point", action="store_true",
                    help="skip timing the 32,768-token point (V=128,256, d=4,096, K=100) after the main workload")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip timing the step with the loss options (padding mask, cross-entropy mix)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (HBM counter calibration) and exit")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the single line: one JSON line per workload point (4K-256K tokens, "
                         "every K) and a markdown table on stderr")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path (the loss "
              "would shard over tokens, each GPU holding W, with one all-reduce of dW).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import kd_synth
    import lm_head_kl_amd as kd

    if args.calibrate_copy_mib:
        nbytes = args.calibrate_copy_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copied {args.calibrate_copy_mib} MiB twice (read {nbytes} B, write {nbytes} B per copy)")
        return 0

    kd.load_library()
    if args.sweep:
        return sweep(kd, torch, np, kd_synth, max(1, args.steps), args.warmup)
    dev = torch.device("cuda:0")
    clock = ClockSampler()
    w = kd_synth.WORKLOADS[args.workload]
    n = args.tokens or w.tokens[0]
    k = args.k or (100 if 100 in w.ks else w.ks[0])
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to_dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    h, wd, idx, val, cache = inputs_and_cache(kd, torch, np, kd_synth, w, n, k, dev,
                                              timed=not args.no_cache_build_timing)
    dh_dtype = tdt
    main_pt = measure(kd, torch, w, h, wd, idx, val, n, k, args.steps, args.warmup, args.chunk, clock)
    ms, value, mfma_util, peak_gb = (main_pt["ms_per_step"], main_pt["tokens_per_s"], main_pt["mfma_util"],
                                     main_pt["peak_gb"])
    roof = main_pt["roofline"]
    stats = main_pt["_stats"]

    var = None
    if not args.no_variants:
        var = variants(kd, torch, h, wd, idx, val, w, dh_dtype, max(1, min(args.steps, 3)), args.chunk)
        rr = var["student_renorm"]["roofline"]
        log(f"loss options (mask {100 * var['ignored_frac']:.2f} % of tokens, CE weight {var['ce_weight']}): "
            f"{var['ms_per_step']:.2f} ms/step, {var['tokens_per_s']:.0f} tokens/s; renormalised student: "
            f"{var['student_renorm']['ms_per_step']:.2f} ms/step, {var['student_renorm']['tokens_per_s']:.0f} tokens/s, "
            f"dominant kernel {rr['kernel']} {rr['achieved']:.0f} GB/s of gathered rows ({100 * rr['frac']:.1f} % of HBM)")

    cio = None
    if not args.no_cache_io:
        cio = cache_io(kd, torch, idx, val, w.vocab,
                       with_paths=lambda paths: loader_fed_steps(kd, torch, h, wd, idx, val, w, dh_dtype, paths))
        log(f"cache io: {cio['bytes'] / 1e6:.1f} MB in {cio['shards']} shards; write {cio['write_gbs']:.2f} GB/s, "
            f"loader to device {cio['load_gbs']:.2f} GB/s = {cio['load_tokens_per_s']:.0f} tokens/s")
        lf = cio["loss_fed_by_loader"]
        log(f"loss fed by the loader ({lf['batch_tokens']}-token batches): {lf['tokens_per_s']:.0f} tokens/s, "
            f"from device memory {lf['from_memory_tokens_per_s']:.0f} tokens/s (ratio {lf['ratio']:.3f})")
        wt = to_dev(kd_synth.teacher_head(w))
        cio["pipeline"] = cache_pipeline(kd, torch, h, wt, k, w.vocab, idx, val)
        del wt
        torch.cuda.empty_cache()
        cp = cio["pipeline"]
        log(f"cache build + streaming writer: {cp['ms']:.1f} ms = {cp['tokens_per_s']:.0f} tokens/s "
            f"(open {cp['open_ms']:.1f} ms, build and copies {cp['gpu_ms']:.1f} ms, last shard {cp['close_ms']:.1f} ms), "
            f"{cp['shards']} shards, {cp['bytes'] / 1e6:.1f} MB")

    target = None
    if not args.no_target_point and (args.workload, n, k) != ("ctx32k_v128k", 32768, 100):
        # the point at which the fused loss is asked to reach half of the MFMA peak:
        # one 32,768-token sequence at V = 128,256, d = 4,096, K = 100
        del h, wd, idx, val
        torch.cuda.empty_cache()
        wt_ = kd_synth.WORKLOADS["ctx32k_v128k"]
        h, wd, idx, val, tcache = inputs_and_cache(kd, torch, np, kd_synth, wt_, 32768, 100, dev, timed=True)
        target = measure(kd, torch, wt_, h, wd, idx, val, 32768, 100, args.steps, args.warmup, args.chunk, clock,
                         min_seconds=3.0)
        target.pop("_stats")
        target["cache_build"] = tcache
        uc = target["mfma_util_measured_clock"]
        log(f"target point ctx32k_v128k ({target['steps']} steps): {target['tokens_per_s']:.0f} tokens/s, "
            f"median {target['ms_median']:.2f} ms, MFMA {100 * target['mfma_util']:.1f}%"
            + (f" ({100 * uc:.1f}% at the measured {target['clock_mhz']:.0f} MHz)" if uc is not None else "")
            + f", peak {target['peak_gb']:.2f} GB")

    cpu = None
    if not args.no_cpu_baseline:
        del h, wd, idx, val
        torch.cuda.empty_cache()
        log(f"cpu baseline: float64 oracle on {args.cpu_rows} tokens ...")
        cpu = cpu_baseline(w, args.cpu_rows, k)
        log(f"cpu baseline {cpu['value']:.1f} tokens/s on {cpu['cores']} threads")

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": args.workload, "n_tokens": n, "d": w.d, "vocab": w.vocab, "k": k, "tau": w.tau,
                   "chunk_tokens": args.chunk or "default", "teacher": w.teacher},
        "mfma_util": round(mfma_util, 4), "peak_gb": round(peak_gb, 3),
        "ms_median": main_pt["ms_median"], "ms_min": main_pt["ms_min"],
        "clock_mhz": main_pt["clock_mhz"], "mfma_util_measured_clock": main_pt["mfma_util_measured_clock"],
        "power_w": main_pt["power_w"], "power_cap_w": clock.power_cap_w,
        "power_limit_residency": main_pt["power_limit_residency"],
        "roofline": roof, "cpu_baseline": cpu, "target_point": target, "cache_build": cache, "cache_io": cio,
        "loss_options": var,
        "kernels_ms_per_step": {k2: round(s["total_ms"] / args.steps, 4) for k2, s in stats.items()},
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
