"""Streaming cache loader on the GPU (include/kdcache.h): batches that cross shard
boundaries arrive bit-exact, prefetch slots are reused only after their copies, and
the loss computed from a cache that went through the files equals the loss from the
cache as built (same bytes in, same result out)."""

import pytest
import torch

import kd_synth
import lm_head_kl_amd as kd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _cache(n, k, vocab, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    idx = torch.randint(0, vocab, (n, k), dtype=torch.int32, generator=g)
    val = torch.randn((n, k), generator=g).to(dtype)
    return idx, val


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("batch,prefetch", [(700, 3), (1, 2), (64, 2), (5000, 4)])
def test_loader_streams_shards_in_order(tmp_path, batch, prefetch):
    print(f"[case] loader batch={batch} prefetch={prefetch}", flush=True)
    vocab, k = 32000, 16
    parts = [_cache(n, k, vocab, torch.bfloat16, seed) for seed, n in enumerate((1000, 0, 2500, 37))]
    paths = []
    for i, (idx, val) in enumerate(parts):
        p = str(tmp_path / f"s{i}.kdc")
        kd.kd_cache_write(p, idx, val, vocab, idx_bits=16 if i % 2 == 0 else 32)   # mixed index widths
        paths.append(p)
    want_i = torch.cat([p[0] for p in parts])
    want_v = torch.cat([p[1] for p in parts])
    got_i, got_v = [], []
    with kd.CacheLoader(paths, batch, prefetch, DEV) as ld:
        assert ld.info["n_tokens"] == want_i.shape[0] and ld.info["k"] == k
        # no host synchronisation between batches: slots are refilled while earlier
        # copies may still be in flight, which the loader must wait for
        for bi, (i_dev, v_dev) in enumerate(ld):
            got_i.append(i_dev)
            got_v.append(v_dev)
    torch.cuda.synchronize()
    got_i = torch.cat(got_i).cpu()
    got_v = torch.cat(got_v).cpu()
    assert torch.equal(got_i, want_i)
    assert torch.equal(_bits(got_v), _bits(want_v))
    n = want_i.shape[0]
    assert bi + 1 == -(-n // batch)


def test_loader_end_and_raw_calls(tmp_path):
    idx, val = _cache(10, 4, 100, torch.float32, 3)
    p = str(tmp_path / "a.kdc")
    kd.kd_cache_write(p, idx, val, 100)
    h = kd.kd_cache_loader_open([p], 4, 2)
    try:
        i_dev = torch.empty((4, 4), dtype=torch.int32, device=DEV)
        v_dev = torch.empty((4, 4), dtype=torch.float32, device=DEV)
        rows = [kd.kd_cache_loader_next(h, i_dev, v_dev) for _ in range(5)]
        assert rows == [4, 4, 2, 0, 0]
        torch.cuda.synchronize()
        assert torch.equal(i_dev[:2].cpu(), idx[8:10]) and torch.equal(v_dev[:2].cpu(), val[8:10])
    finally:
        kd.kd_cache_loader_close(h)


def test_loss_from_loaded_cache_is_identical(tmp_path):
    """Teacher cache built on the GPU, written to two shards, streamed back through the
    loader: the forward loss and lse are bitwise those of the cache as built."""
    print("[case] cache build -> shards -> loader -> loss", flush=True)
    w = kd_synth.WORKLOADS["seq4k_v32k"]
    n = 2048
    to_dev = lambda x: torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(DEV)
    h = to_dev(kd_synth.hidden(w, n))
    wd = to_dev(kd_synth.student_head(w))
    wt = to_dev(kd_synth.teacher_head(w))
    idx, val = kd.kd_topk_cache_build(h, wt, w.ks[0])
    ih, vh = idx.cpu(), val.cpu()
    paths = [str(tmp_path / "c0.kdc"), str(tmp_path / "c1.kdc")]
    kd.kd_cache_write(paths[0], ih[:1234].contiguous(), vh[:1234].contiguous(), w.vocab)
    kd.kd_cache_write(paths[1], ih[1234:].contiguous(), vh[1234:].contiguous(), w.vocab)
    with kd.CacheLoader(paths, n, 2, DEV) as ld:
        li, lv = next(ld)
    assert li.shape == idx.shape
    loss_a, lse_a, _ = kd.kd_chunked_kl_fwd(h, wd, idx, val, 1.0)
    loss_b, lse_b, _ = kd.kd_chunked_kl_fwd(h, wd, li.contiguous(), lv.contiguous(), 1.0)
    torch.cuda.synchronize()
    assert torch.equal(li, idx) and torch.equal(_bits(lv), _bits(val))
    assert torch.equal(loss_a, loss_b) and torch.equal(lse_a, lse_b)
