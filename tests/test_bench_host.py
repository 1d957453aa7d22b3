"""Host logic of bench.py that runs without a GPU: the refusal of more than one
GPU, the least-squares fit of peak memory against N, the clock sampler's
handling of the GPU metrics table (one reading per snapshot, the snapshot
current at the start left out, mean power and the share of time at the power
limit), and the traffic table's source-hash guard."""
import os
import subprocess
import sys
import threading

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""


def _rows(slope, intercept, ns, k, noise=0.0, seed=0):
    g = np.random.default_rng(seed)
    return [{"workload": "w", "n_tokens": n, "k": k, "d": 4096, "vocab": 128256,
             "peak_gb": (intercept + slope * n) * (1 + noise * g.standard_normal()) / 1e9} for n in ns]


def test_peak_memory_fit_recovers_a_line_and_skips_points_below_one_chunk():
    rows = _rows(16988.0, 8.56e9, [16384, 65536, 262144], 100) + _rows(16688.0, 8.55e9, [16384, 65536, 262144], 50)
    # a point below one chunk (smaller workspace) must not enter the fit
    rows.append({"workload": "w", "n_tokens": 4096, "k": 100, "d": 4096, "vocab": 128256, "peak_gb": 4.31})
    fits = {f["k"]: f for f in bench.peak_memory_fits(np, rows)}
    assert set(fits) == {50, 100}
    assert fits[100]["n_tokens"] == [16384, 65536, 262144]
    assert abs(fits[100]["slope_bytes_per_token"] - 16988.0) < 1.0
    assert abs(fits[100]["intercept_gb"] - 8.56) < 1e-3
    assert fits[100]["expected_bytes_per_token"] == 2 * 4096 + 2 * 4096 + 6 * 100 + 4
    assert fits[50]["expected_bytes_per_token"] == 16688
    assert fits[100]["max_rel_residual"] < 1e-6


def test_peak_memory_fit_reports_the_residual_and_needs_three_points():
    rows = _rows(17000.0, 8.5e9, [16384, 32768, 65536, 131072], 100, noise=0.01, seed=3)
    (fit,) = bench.peak_memory_fits(np, rows)
    assert 0.0 < fit["max_rel_residual"] < 0.05
    assert bench.peak_memory_fits(np, _rows(17000.0, 8.5e9, [16384, 65536], 100)) == []


class _Done:
    def join(self):
        pass


def _sampler(samples, stale):
    c = object.__new__(bench.ClockSampler)
    c.handle = object()
    c._stop = threading.Event()
    c._thread = _Done()
    c._stale = stale
    c.samples = samples
    return c


def test_clock_sampler_keeps_one_reading_per_snapshot_and_drops_the_stale_one():
    # snapshot 7 was current when the timed region began; 8 and 9 are fresh, each
    # read several times between refreshes: (snapshot, MHz, W, PPT residency, accumulation)
    c = _sampler([(7, 2400.0, 250, 100, 1000), (7, 2400.0, 250, 100, 1000), (8, 1800.0, 1350, 130, 1040),
                  (8, 1800.0, 1350, 130, 1040), (9, 1900.0, 1370, 166, 1080), (9, 1900.0, 1370, 166, 1080),
                  (9, 1900.0, 1370, 166, 1080)], 7)
    r = c.stop()
    assert r["snapshots"] == 2 and abs(r["mhz"] - 1850.0) < 1e-9
    assert abs(r["power_w"] - 1360.0) < 1e-9
    # PPT residency grew by 36 of the accumulation counter's 40 between the fresh snapshots
    assert abs(r["ppt_frac"] - 0.9) < 1e-12


def test_clock_sampler_reports_nothing_from_fewer_than_two_snapshots():
    assert _sampler([(7, 2400.0, 250, 1, 1), (8, 1800.0, 1300, 2, 2), (8, 1800.0, 1300, 2, 2)], 7).stop() is None
    assert _sampler([], 7).stop() is None
    # readings without a snapshot id (the clock query) each count; non-positive ones
    # never; without power fields the power and residency are None
    r = _sampler([(None, 1700.0, None, None, None), (None, 0.0, None, None, None),
                  (None, 1900.0, None, None, None)], None).stop()
    assert r["snapshots"] == 2 and abs(r["mhz"] - 1800.0) < 1e-9
    assert r["power_w"] is None and r["ppt_frac"] is None


def test_traffic_table_is_ignored_once_the_kernel_sources_change(monkeypatch):
    if bench.traffic_for("gemm_dw") is None:
        return      # no table for these sources
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.traffic_for("gemm_dw") is None
