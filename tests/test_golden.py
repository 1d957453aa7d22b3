"""Stored fixtures under tests/golden/.

* ``cache_size_wiki.json``: the cache-size estimate the pages print (tokens x K x
  (2 + 2) bytes; one billion tokens at K = 100 is 400 GB).  The shard format with
  16-bit indices and bf16 values stores exactly that many bytes per token after
  its fixed 64-byte header.
* ``oracle_tiny_fp32.json``: the oracle's results on the tiny float32 workload,
  written by ``tests/golden/make_oracle_golden.py`` (oracle and input generator
  only).  Recomputing them catches any change to the oracle's arithmetic.
"""
import importlib.util
import json
import os

import numpy as np
import torch

import lm_head_kl_amd as kd

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_shard_bytes_match_the_pages_cache_size(tmp_path):
    g = json.load(open(os.path.join(GOLDEN, "cache_size_wiki.json")))
    n, k = 1000, g["k"]
    idx = torch.randint(0, 32000, (n, k), dtype=torch.int32)
    val = torch.randn(n, k).to(torch.bfloat16)
    p = str(tmp_path / "s.kdc")
    kd.kd_cache_write(p, idx, val, 32000)          # V <= 65,536: 16-bit indices
    info = kd.kd_cache_info_read(p)
    assert info["idx_bits"] == 16
    per_token = (os.path.getsize(p) - 64) / n      # 64-byte header, then idx and val
    assert per_token == k * (g["index_bytes"] + g["value_bytes"])
    assert per_token * g["tokens"] == g["total_bytes"]


def test_oracle_reproduces_stored_tiny_fp32_values():
    spec = importlib.util.spec_from_file_location("make_oracle_golden",
                                                  os.path.join(GOLDEN, "make_oracle_golden.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    stored = json.load(open(os.path.join(GOLDEN, "oracle_tiny_fp32.json")))
    now = mod.compute()
    assert {k: stored[k] for k in ("n", "d", "v", "tau")} == {k: now[k] for k in ("n", "d", "v", "tau")}
    assert stored["cases"].keys() == now["cases"].keys()
    for k, s in stored["cases"].items():
        c = now["cases"][k]
        assert s["idx_first_row"] == c["idx_first_row"] and s["val_bits_first_row"] == c["val_bits_first_row"]
        for key in ("loss", "kl_rows_sum", "dH_fro", "dW_fro"):
            assert abs(s[key] - c[key]) <= 1e-12 * max(1.0, abs(s[key])), (k, key)
        for key in ("lse_first", "kl_rows_first", "dW_first"):
            np.testing.assert_allclose(c[key], s[key], rtol=1e-12, atol=1e-15)
