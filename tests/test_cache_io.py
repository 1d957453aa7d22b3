"""On-disk teacher cache shards (include/kdcache.h), host side: no GPU needed.

The byte layout is pinned by an independent reader written here from the layout
table in include/kdcache.h (struct + numpy), not by the library's own reader; the
file size is pinned by the cache-size estimate of the pages (llm-wiki note,
"운영 적용 가이드" / "캐시 크기 추정": tokens x K x (index bytes + value bytes), with
16-bit indices and bf16 values suggested in "사전 계산(Pre-computation) 파이프라인").
"""
import ctypes
import os
import struct

import numpy as np
import pytest
import torch

import lm_head_kl_amd as kd

KD_ERR_NULL_POINTER, KD_ERR_BAD_SHAPE, KD_ERR_BAD_DTYPE, KD_ERR_NO_DEVICE = 1, 2, 3, 7
KD_ERR_IDX_OUT_OF_RANGE, KD_ERR_IO, KD_ERR_BAD_FORMAT = 10, 12, 13


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kd.LIB_PATH):
        from lm_head_kl_amd import build
        build.build()
    return kd.load_library()


def _cache(n, k, vocab, dtype, seed=0):
    g = torch.Generator().manual_seed(seed)
    idx = torch.randint(0, vocab, (n, k), dtype=torch.int32, generator=g)
    val = torch.randn((n, k), generator=g).to(dtype)
    return idx, val


def parse_shard(path):
    """Independent reader of the documented layout."""
    raw = open(path, "rb").read()
    magic, version, hdr, n, vocab, k, bits, vdt, reserved, ioff, voff = struct.unpack_from("<8sIIQQIIIIQQ", raw, 0)
    assert (magic, version, hdr, reserved) == (b"KDCACHE1", 1, 64, 0)
    ib = {16: np.dtype("<u2"), 32: np.dtype("<i4")}[bits]
    vb = {0: np.dtype("<f4"), 1: np.dtype("<u2")}[vdt]
    assert ioff == 64 and voff == -(-(64 + n * k * ib.itemsize) // 64) * 64
    assert len(raw) == voff + n * k * vb.itemsize
    idx = np.frombuffer(raw, ib, n * k, ioff).astype(np.int32).reshape(n, k)
    val = np.frombuffer(raw, vb, n * k, voff).reshape(n, k)
    return dict(n=n, vocab=vocab, k=k, bits=bits, vdt=vdt), idx, val


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("n,k,vocab,dtype,bits,want_bits", [
    (300, 16, 32000, torch.bfloat16, 0, 16),     # config-1 vocabulary: 16-bit indices chosen
    (257, 100, 128256, torch.bfloat16, 0, 32),   # above 65,536 entries: int32
    (64, 8, 4096, torch.float32, 32, 32),        # fp32 values, forced int32
    (50, 3, 65536, torch.bfloat16, 16, 16),      # largest vocabulary that fits 16 bits
])
def test_round_trip_and_layout(lib, tmp_path, n, k, vocab, dtype, bits, want_bits):
    idx, val = _cache(n, k, vocab, dtype)
    if vocab == 65536:
        idx[0, 0] = 65535
    p = str(tmp_path / "s.kdc")
    kd.kd_cache_write(p, idx, val, vocab, idx_bits=bits)
    info = kd.kd_cache_info_read(p)
    assert info == {"n_tokens": n, "vocab": vocab, "k": k, "idx_bits": want_bits, "val_dtype": kd._dt(dtype)}
    hdr, pidx, pval = parse_shard(p)
    assert hdr["bits"] == want_bits and hdr["vocab"] == vocab
    assert np.array_equal(pidx, idx.numpy())
    assert np.array_equal(pval.view(np.int16 if dtype == torch.bfloat16 else np.int32), _bits(val).numpy())
    i2, v2 = kd.kd_cache_read(p)
    assert torch.equal(i2, idx) and torch.equal(_bits(v2), _bits(val))
    assert not [f for f in os.listdir(tmp_path) if ".tmp." in f]     # written under a temporary name


def test_size_matches_the_pages_estimate(tmp_path):
    """16-bit indices + bf16 values: exactly N*K*(2+2) bytes after the 64-byte header
    (N*K*2 a multiple of 64, so there is no padding)."""
    n, k = 512, 100
    idx, val = _cache(n, k, 32000, torch.bfloat16)
    p = str(tmp_path / "s.kdc")
    kd.kd_cache_write(p, idx, val, 32000)
    assert os.path.getsize(p) - 64 == n * k * (2 + 2)


def test_partial_reads(lib, tmp_path):
    idx, val = _cache(1000, 7, 50000, torch.bfloat16)
    p = str(tmp_path / "s.kdc")
    kd.kd_cache_write(p, idx, val, 50000)
    for r0, rows in ((0, 1), (999, 1), (123, 456), (1000, 0), (0, 1000)):
        i2, v2 = kd.kd_cache_read(p, r0, rows)
        assert torch.equal(i2, idx[r0:r0 + rows]) and torch.equal(_bits(v2), _bits(val[r0:r0 + rows]))
    buf_i = torch.empty((2, 7), dtype=torch.int32)
    buf_v = torch.empty((2, 7), dtype=torch.bfloat16)
    for r0, rows in ((999, 2), (-1, 1), (0, -1), (1001, 0)):
        st = lib.kd_cache_read(p.encode(), r0, rows, buf_i.data_ptr(), buf_v.data_ptr())
        assert st == KD_ERR_BAD_SHAPE, (r0, rows)


def test_empty_shard(tmp_path):
    idx, val = _cache(0, 5, 1000, torch.float32)
    p = str(tmp_path / "e.kdc")
    kd.kd_cache_write(p, idx, val, 1000)
    assert kd.kd_cache_info_read(p)["n_tokens"] == 0
    assert os.path.getsize(p) == 64
    i2, v2 = kd.kd_cache_read(p)
    assert i2.shape == (0, 5) and v2.shape == (0, 5)


def _raw_write(lib, path, n, k, vocab, bits, vdt, idx, val):
    info = kd.KDCacheInfo(n, vocab, k, bits, vdt)
    return lib.kd_cache_write(path.encode(), ctypes.byref(info), idx, val)


def test_write_rejects_bad_input(lib, tmp_path):
    p = str(tmp_path / "x.kdc")
    idx, val = _cache(4, 3, 100, torch.float32)
    ip, vp = idx.data_ptr(), val.data_ptr()
    bad = idx.clone()
    bad[2, 1] = 100
    assert _raw_write(lib, p, 4, 3, 100, 0, 0, bad.data_ptr(), vp) == KD_ERR_IDX_OUT_OF_RANGE
    bad[2, 1] = -1
    assert _raw_write(lib, p, 4, 3, 100, 0, 0, bad.data_ptr(), vp) == KD_ERR_IDX_OUT_OF_RANGE
    assert _raw_write(lib, p, 4, 3, 70000, 16, 0, ip, vp) == KD_ERR_BAD_SHAPE     # 16 bits cannot hold V
    assert _raw_write(lib, p, 4, 3, 100, 8, 0, ip, vp) == KD_ERR_BAD_SHAPE        # idx_bits 8
    assert _raw_write(lib, p, 4, 101, 100, 0, 0, ip, vp) == KD_ERR_BAD_SHAPE      # k > V
    assert _raw_write(lib, p, -1, 3, 100, 0, 0, ip, vp) == KD_ERR_BAD_SHAPE
    assert _raw_write(lib, p, 4, 3, 100, 0, 7, ip, vp) == KD_ERR_BAD_DTYPE
    assert _raw_write(lib, p, 4, 3, 100, 0, 0, None, vp) == KD_ERR_NULL_POINTER
    assert lib.kd_cache_write(None, None, ip, vp) == KD_ERR_NULL_POINTER
    assert _raw_write(lib, str(tmp_path / "no" / "dir.kdc"), 4, 3, 100, 0, 0, ip, vp) == KD_ERR_IO
    assert not os.path.exists(p)


def _good(tmp_path, name="g.kdc"):
    idx, val = _cache(40, 4, 1000, torch.bfloat16)
    p = str(tmp_path / name)
    kd.kd_cache_write(p, idx, val, 1000)
    return p


def _info_status(lib, p):
    info = kd.KDCacheInfo()
    return lib.kd_cache_info_read(p.encode(), ctypes.byref(info))


def _patched(tmp_path, src, offset, data, name):
    raw = bytearray(open(src, "rb").read())
    raw[offset:offset + len(data)] = data
    q = str(tmp_path / name)
    open(q, "wb").write(bytes(raw))
    return q


def test_reader_rejects_damaged_shards(lib, tmp_path):
    p = _good(tmp_path)
    assert _info_status(lib, p) == 0
    assert _info_status(lib, str(tmp_path / "missing.kdc")) == KD_ERR_IO
    cases = {
        "magic": (0, b"KDCACHE2"),
        "version": (8, struct.pack("<I", 2)),
        "header": (12, struct.pack("<I", 128)),
        "rows": (16, struct.pack("<Q", 41)),            # file too short for the stated rows
        "bits": (36, struct.pack("<I", 8)),
        "dtype": (40, struct.pack("<I", 5)),
        "reserved": (44, struct.pack("<I", 1)),
        "valoff": (56, struct.pack("<Q", 64 + 40 * 4 * 2 + 64)),
    }
    for name, (off, data) in cases.items():
        assert _info_status(lib, _patched(tmp_path, p, off, data, name + ".kdc")) == KD_ERR_BAD_FORMAT, name
    raw = open(p, "rb").read()
    for name, body in (("short", raw[:-1]), ("long", raw + b"\0"), ("stub", raw[:40])):
        q = str(tmp_path / (name + ".kdc"))
        open(q, "wb").write(body)
        assert _info_status(lib, q) == KD_ERR_BAD_FORMAT, name
    with pytest.raises(kd.KDError):
        kd.kd_cache_read(str(tmp_path / "short.kdc"))


def test_loader_argument_checks(lib, tmp_path):
    """Everything the loader checks before it allocates pinned host memory."""
    a = _good(tmp_path, "a.kdc")
    idx, val = _cache(10, 5, 1000, torch.bfloat16)     # k differs from a.kdc
    b = str(tmp_path / "b.kdc")
    kd.kd_cache_write(b, idx, val, 1000)

    def open_status(paths, batch=16, prefetch=2):
        arr = (ctypes.c_char_p * max(1, len(paths)))(*[x.encode() for x in paths])
        h = ctypes.c_void_p()
        return lib.kd_cache_loader_open(arr, len(paths), batch, prefetch, ctypes.byref(h)), h

    assert open_status([a], batch=0)[0] == KD_ERR_BAD_SHAPE
    assert open_status([a], prefetch=1)[0] == KD_ERR_BAD_SHAPE
    assert open_status([])[0] == KD_ERR_BAD_SHAPE
    assert open_status([a, b])[0] == KD_ERR_BAD_FORMAT
    assert open_status([a, str(tmp_path / "none.kdc")])[0] == KD_ERR_IO
    assert lib.kd_cache_loader_close(None) == 0
    if not torch.cuda.is_available():
        st, h = open_status([a])
        assert st == KD_ERR_NO_DEVICE and not h.value


def test_writer_argument_errors_before_any_device_call():
    """The streaming writer validates its arguments before touching the HIP runtime
    (these run on a host without a GPU)."""
    import ctypes
    lib = kd.load_library()
    out = ctypes.c_void_p()
    info = kd.KDCacheInfo(1000, 32000, 16, 0, kd.KD_BF16)
    assert lib.kd_cache_writer_open(None, ctypes.byref(info), 100, 2, ctypes.byref(out)) == 1
    assert lib.kd_cache_writer_open(b"/tmp/x", None, 100, 2, ctypes.byref(out)) == 1
    for bad, st in ((kd.KDCacheInfo(0, 32000, 16, 0, kd.KD_BF16), 2),        # no rows per shard
                    (kd.KDCacheInfo(1000, 100000, 16, 16, kd.KD_BF16), 2),   # 16-bit indices, V > 65536
                    (kd.KDCacheInfo(1000, 32000, 0, 0, kd.KD_BF16), 2),      # K = 0
                    (kd.KDCacheInfo(1000, 32000, 16, 0, 7), 3)):             # unknown value dtype
        assert lib.kd_cache_writer_open(b"/tmp/x", ctypes.byref(bad), 100, 2, ctypes.byref(out)) == st
    assert lib.kd_cache_writer_open(b"/tmp/x", ctypes.byref(info), 0, 2, ctypes.byref(out)) == 2
    assert lib.kd_cache_writer_open(b"/tmp/x", ctypes.byref(info), 100, 1, ctypes.byref(out)) == 2
    assert lib.kd_cache_writer_put(None, None, None, 1, None) == 1
    assert lib.kd_cache_writer_close(None, None) == 0
