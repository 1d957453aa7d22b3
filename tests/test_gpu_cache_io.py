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


def test_raw_calls_check_tensors_against_the_handle(tmp_path):
    """The raw next/put calls take caller tensors: a batch of another K or value
    dtype, or too few rows for a loader batch, is refused before any copy is
    enqueued, and the handle keeps working."""
    idx, val = _cache(10, 4, 100, torch.float32, 5)
    p = str(tmp_path / "a.kdc")
    kd.kd_cache_write(p, idx, val, 100)
    h = kd.kd_cache_loader_open([p], 4, 2)
    try:
        bad = [((4, 5), torch.float32), ((4, 4), torch.bfloat16), ((3, 4), torch.float32)]
        for shape, vdt in bad:
            with pytest.raises(ValueError, match="kd_cache_loader_next"):
                kd.kd_cache_loader_next(h, torch.empty(shape, dtype=torch.int32, device=DEV),
                                        torch.empty(shape, dtype=vdt, device=DEV))
        i_dev = torch.empty((6, 4), dtype=torch.int32, device=DEV)   # more rows than a batch is fine
        v_dev = torch.empty((6, 4), dtype=torch.float32, device=DEV)
        assert kd.kd_cache_loader_next(h, i_dev, v_dev) == 4
        torch.cuda.synchronize()
        assert torch.equal(i_dev[:4].cpu(), idx[:4])
    finally:
        kd.kd_cache_loader_close(h)
    with pytest.raises(ValueError, match="not an open handle"):
        kd.kd_cache_loader_next(h, i_dev, v_dev)

    # slices of one buffer, as a caller filling a whole cache does: the last batch
    # gets a shorter slice and the end call an empty one
    li = torch.empty((10, 4), dtype=torch.int32, device=DEV)
    lv = torch.empty((10, 4), dtype=torch.float32, device=DEV)
    h = kd.kd_cache_loader_open([p], 4, 2)
    try:
        row, got = 0, []
        while True:
            r = kd.kd_cache_loader_next(h, li[row:row + 4], lv[row:row + 4])
            got.append(r)
            if r == 0:
                break
            row += r
    finally:
        kd.kd_cache_loader_close(h)
    torch.cuda.synchronize()
    assert got == [4, 4, 2, 0] and torch.equal(li.cpu(), idx) and torch.equal(lv.cpu(), val)

    with kd.CacheWriter(str(tmp_path / "w"), 8, 100, 4, torch.float32, 6) as wr:
        for shape, vdt in [((2, 5), torch.float32), ((2, 4), torch.bfloat16)]:
            with pytest.raises(ValueError, match="kd_cache_writer_put"):
                wr.put(torch.zeros(shape, dtype=torch.int32, device=DEV), torch.zeros(shape, dtype=vdt, device=DEV))
        wr.put(idx[:6].to(DEV), val[:6].to(DEV))
    assert len(wr.paths) == 1
    got_i, got_v = kd.kd_cache_read(wr.paths[0])
    assert torch.equal(got_i, idx[:6]) and torch.equal(got_v, val[:6])


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


def test_writer_pipeline_build_then_store(tmp_path):
    """The offline pass at small scale: the teacher cache is built on the GPU batch
    by batch, each batch handed to the streaming writer without a host sync, and
    the shards (1,500 rows each; the last one shorter) read back bit-exactly,
    through kd_cache_read and through the loader."""
    print("[case] writer pipeline", flush=True)
    n, d, v, k, batch, shard = 5000, 64, 3000, 24, 700, 1500
    p = kd_synth.small_problem(n, d, v, seed=51)
    to_dev = lambda x: torch.from_numpy(x.view("int16")).view(torch.bfloat16).to(DEV)
    h, wt = to_dev(p["H"]), to_dev(p["WT"])
    prefix = str(tmp_path / "cache")
    built_i, built_v = [], []
    with kd.CacheWriter(prefix, shard, v, k, torch.bfloat16, batch) as wr:
        for r0 in range(0, n, batch):
            i, val = kd.kd_topk_cache_build(h[r0:r0 + batch].contiguous(), wt, k)
            wr.put(i, val)
            built_i.append(i)
            built_v.append(val)
    assert wr.paths == [f"{prefix}_{j:05d}.kdc" for j in range(4)]
    sizes = [kd.kd_cache_info_read(path)["n_tokens"] for path in wr.paths]
    assert sizes == [1500, 1500, 1500, 500]
    assert all(kd.kd_cache_info_read(path)["idx_bits"] == 16 for path in wr.paths)
    want_i = torch.cat(built_i).cpu()
    want_v = torch.cat(built_v).cpu()
    got = [kd.kd_cache_read(path) for path in wr.paths]
    assert torch.equal(torch.cat([g[0] for g in got]), want_i)
    assert torch.equal(_bits(torch.cat([g[1] for g in got])), _bits(want_v))
    with kd.CacheLoader(wr.paths, 1024, 2, DEV) as ld:
        li = torch.cat([b[0] for b in ld]).cpu()
    assert torch.equal(li, want_i)


def test_writer_f32_and_index_errors(tmp_path):
    """float32 values with 32-bit indices round-trip; an out-of-range index fails
    its shard, and the error comes back from the next put and from close."""
    idx, val = _cache(300, 8, 100000, torch.float32, 7)
    prefix = str(tmp_path / "f")
    with kd.CacheWriter(prefix, 128, 100000, 8, torch.float32, 100, depth=2) as wr:
        for r0 in range(0, 300, 100):
            wr.put(idx[r0:r0 + 100].to(DEV), val[r0:r0 + 100].to(DEV))
    got = [kd.kd_cache_read(path) for path in wr.paths]
    assert [kd.kd_cache_info_read(path)["idx_bits"] for path in wr.paths] == [32, 32, 32]
    assert torch.equal(torch.cat([g[0] for g in got]), idx)
    assert torch.equal(_bits(torch.cat([g[1] for g in got])), _bits(val))

    # the bad index is in row 25, i.e. in the third shard of 10 rows
    bad = idx.clone()
    bad[25, 3] = 100000
    bdir = tmp_path / "bad"
    bdir.mkdir()
    wr2 = kd.CacheWriter(str(bdir / "b"), 10, 100000, 8, torch.float32, 100, depth=2)
    wr2.put(bad[:100].to(DEV), val[:100].to(DEV))
    # with two buffers the third put waits for the first batch's shards, whose
    # write has failed by then
    with pytest.raises(kd.KDError) as e:
        for _ in range(2):
            wr2.put(idx[100:200].to(DEV), val[100:200].to(DEV))
    assert e.value.status == 10
    with pytest.raises(kd.KDError) as e:
        wr2.close()
    assert e.value.status == 10
    # nothing is written after the failed shard: the two before it, complete
    assert wr2.paths == [str(bdir / "b_00000.kdc"), str(bdir / "b_00001.kdc")]
    assert sorted(p.name for p in bdir.iterdir()) == ["b_00000.kdc", "b_00001.kdc"]
    got = [kd.kd_cache_read(path) for path in wr2.paths]
    assert torch.equal(torch.cat([g[0] for g in got]), idx[:20])
