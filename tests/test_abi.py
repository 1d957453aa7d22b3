"""C-ABI contract tests that need no GPU: the library loads, exports every symbol
the header declares, and every argument error is reported before any device
work (so these run on a host without a GPU)."""
import ctypes
import glob
import math
import os
import re
import subprocess

import pytest

import lm_head_kl_amd as kd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kd.LIB_PATH):
        from lm_head_kl_amd import build
        build.build()
    return kd.load_library()


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kd_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(kd.EXPORTED), names


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", kd.LIB_PATH], stdout=subprocess.PIPE, text=True).stdout
    exported = set(re.findall(r"\sT\s+(\w+)$", out, flags=re.M))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    assert lib.kd_version() == 102


def test_status_strings(lib):
    for code, name in kd.STATUS_NAMES.items():
        s = lib.kd_status_string(code).decode()
        assert s and s != "unknown status", name
    assert lib.kd_status_string(999).decode() == "unknown status"


def _P(**kw):
    base = dict(n=64, d=128, v=1000, k=8, tau=1.0, x_dtype=kd.KD_BF16, val_dtype=None, dh_dtype=kd.KD_F32,
                chunk_tokens=0)
    base.update(kw)
    return kd.make_problem(base["n"], base["d"], base["v"], base["k"], base["tau"], base["x_dtype"],
                           base["val_dtype"], base["dh_dtype"], base["chunk_tokens"])


def _ws(lib, op, prob):
    out = ctypes.c_size_t(0)
    st = lib.kd_workspace_size(op, ctypes.byref(prob), ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("kw,status", [
    (dict(d=0), 2), (dict(d=12), 2), (dict(v=0), 2), (dict(k=0), 2), (dict(k=1001), 2), (dict(n=-1), 2),
    (dict(v=2097089, k=1), 2), (dict(k=70000, v=100000), 2), (dict(chunk_tokens=-5), 2),
    (dict(tau=0.0), 4), (dict(tau=-1.0), 4), (dict(tau=float("nan")), 4), (dict(tau=float("inf")), 4),
    (dict(x_dtype=7), 3), (dict(val_dtype=kd.KD_F32), 3), (dict(x_dtype=kd.KD_F32, val_dtype=kd.KD_BF16), 3),
])
def test_workspace_size_rejects_bad_problems(lib, kw, status):
    for op in (kd.KD_OP_KL_FWD, kd.KD_OP_KL_BWD):
        st, _ = _ws(lib, op, _P(**kw))
        assert st == status, (kw, op, st)


@pytest.mark.parametrize("x_dtype", [kd.KD_BF16, kd.KD_F32])
def test_domain_limits_are_exact(lib, x_dtype):
    """The header's largest V (2,097,088), K (65,535; 4,096 for the cache build),
    d, N and chunk are accepted by every call and one more is refused."""
    for op in (kd.KD_OP_TOPK_BUILD, kd.KD_OP_KL_FWD, kd.KD_OP_KL_BWD):
        assert _ws(lib, op, _P(v=2097088, x_dtype=x_dtype))[0] == 0, op
        assert _ws(lib, op, _P(v=2097089, x_dtype=x_dtype))[0] == 2, op
        kmax = 4096 if op == kd.KD_OP_TOPK_BUILD else 65535
        assert _ws(lib, op, _P(v=70000, k=kmax, x_dtype=x_dtype))[0] == 0, op
        assert _ws(lib, op, _P(v=70000, k=kmax + 1, x_dtype=x_dtype))[0] == 2, op
        # d <= 2^20, N <= 2^31 - 256, and the chunk as used <= 2,096,896 tokens
        assert _ws(lib, op, _P(d=1 << 20, x_dtype=x_dtype))[0] == 0, op
        assert _ws(lib, op, _P(d=(1 << 20) + 8, x_dtype=x_dtype))[0] == 2, op
        assert _ws(lib, op, _P(n=(1 << 31) - 256, x_dtype=x_dtype))[0] == 0, op
        assert _ws(lib, op, _P(n=(1 << 31) - 255, x_dtype=x_dtype))[0] == 2, op
        assert _ws(lib, op, _P(n=1 << 22, chunk_tokens=2096896, x_dtype=x_dtype))[0] == 0, op
        assert _ws(lib, op, _P(n=1 << 22, chunk_tokens=2096897, x_dtype=x_dtype))[0] == 2, op
        assert _ws(lib, op, _P(n=2096896, chunk_tokens=(1 << 31) - 1, x_dtype=x_dtype))[0] == 0, op
        assert _ws(lib, op, _P(n=2096897, chunk_tokens=(1 << 31) - 1, x_dtype=x_dtype))[0] == 2, op


def test_workspace_size_null_and_bad_op(lib):
    prob = _P()
    assert lib.kd_workspace_size(kd.KD_OP_KL_FWD, ctypes.byref(prob), None) == 1
    assert lib.kd_workspace_size(kd.KD_OP_KL_FWD, None, ctypes.byref(ctypes.c_size_t())) == 1
    assert lib.kd_workspace_size(9, ctypes.byref(prob), ctypes.byref(ctypes.c_size_t())) == 2
    st, _ = _ws(lib, kd.KD_OP_KL_BWD, _P(dh_dtype=5))
    assert st == 3
    st, _ = _ws(lib, kd.KD_OP_TOPK_BUILD, _P(k=5000, v=10000))
    assert st == 2           # the cache build holds at most 4096 entries per row
    st, _ = _ws(lib, kd.KD_OP_TOPK_BUILD, _P(tau=0.0))
    assert st == 0           # tau is not used by the cache build


def test_workspace_is_chunk_sized_not_token_sized(lib):
    """Peak-memory linearity: the big workspace terms depend on the chunk, not N."""
    sizes = {}
    for n in (16384, 65536, 262144):    # at or above one chunk (below 4K tokens the backward skips W^T)
        for op in (kd.KD_OP_KL_FWD, kd.KD_OP_KL_BWD):
            st, b = _ws(lib, op, _P(n=n, d=4096, v=128256, k=100, chunk_tokens=16384))
            assert st == 0
            sizes[(op, n)] = b
    # backward: independent of N once N >= chunk
    assert sizes[(kd.KD_OP_KL_BWD, 16384)] == sizes[(kd.KD_OP_KL_BWD, 262144)]
    # forward: only an O(N) term grows, the float64 KL sum of each block of 16 rows
    # (0.5 byte per token, against 8 KB per token of H itself)
    grow = sizes[(kd.KD_OP_KL_FWD, 262144)] - sizes[(kd.KD_OP_KL_FWD, 16384)]
    assert 0 <= grow <= (262144 - 16384) // 16 * 8 + 512
    # and nothing of size N x V: 262144 x 128256 x 2 bytes would be 67 GB
    assert max(sizes.values()) < 16e9


def _null_calls(lib, prob, ws_bytes):
    """Each entry point with NULL data pointers but a valid problem."""
    vp = ctypes.c_void_p
    fake = vp(4096)   # aligned, never dereferenced: validation fails first
    return {
        "topk_null_h": lib.kd_topk_cache_build(ctypes.byref(prob), None, fake, fake, fake, fake, ws_bytes, None),
        "fwd_null_loss": lib.kd_chunked_kl_fwd(ctypes.byref(prob), fake, fake, fake, fake, None, fake, None, fake,
                                               ws_bytes, None),
        "bwd_null_dw": lib.kd_chunked_kl_bwd(ctypes.byref(prob), fake, fake, fake, fake, fake, None, fake, None,
                                             fake, ws_bytes, None),
    }


def test_null_pointers_rejected_before_device_work(lib):
    prob = _P()
    res = _null_calls(lib, prob, 1 << 40)
    assert all(v == 1 for v in res.values()), res


def test_misaligned_and_small_workspace(lib):
    prob = _P()
    _, need = _ws(lib, kd.KD_OP_KL_FWD, prob)
    a, m = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 4)
    st = lib.kd_chunked_kl_fwd(ctypes.byref(prob), m, a, a, a, a, a, None, a, need, None)
    assert st == 5
    st = lib.kd_chunked_kl_fwd(ctypes.byref(prob), a, a, a, a, a, a, None, a, need - 1, None)
    assert st == 6
    _, need_b = _ws(lib, kd.KD_OP_KL_BWD, prob)
    st = lib.kd_chunked_kl_bwd(ctypes.byref(prob), a, a, a, a, a, None, a, a, a, need_b - 1, None)
    assert st == 6
    _, need_t = _ws(lib, kd.KD_OP_TOPK_BUILD, prob)
    st = lib.kd_topk_cache_build(ctypes.byref(prob), a, a, a, a, a, need_t - 1, None)
    assert st == 6


def test_valid_call_without_gpu_reports_no_device(lib):
    """With valid arguments the next step is the device check; on a host with no
    GPU it must fail cleanly (and enqueue nothing)."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    prob = _P()
    _, need = _ws(lib, kd.KD_OP_KL_FWD, prob)
    a = ctypes.c_void_p(4096)
    st = lib.kd_chunked_kl_fwd(ctypes.byref(prob), a, a, a, a, a, a, None, a, need, None)
    assert st == 7


def test_python_binding_refuses_cpu_tensors():
    import torch
    h = torch.zeros(4, 8, dtype=torch.bfloat16)
    w = torch.zeros(10, 8, dtype=torch.bfloat16)
    idx = torch.zeros(4, 2, dtype=torch.int32)
    val = torch.zeros(4, 2, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        kd.kd_chunked_kl_fwd(h, w, idx, val, 1.0)


def test_python_binding_checks_shapes_before_pointers():
    """The library sees pointers and sizes only, so the binding refuses inputs
    whose shapes or dtypes disagree before it takes a pointer (here on CPU tensors,
    so the shape error comes before the no-CPU-fallback one)."""
    import torch
    bf = torch.bfloat16
    h = torch.zeros(4, 8, dtype=bf)
    idx = torch.zeros(4, 2, dtype=torch.int32)
    val = torch.zeros(4, 2, dtype=bf)
    lse = torch.zeros(4, dtype=torch.float32)
    bad = [
        (dict(w=torch.zeros(10, 16, dtype=bf)), "w \\[V, d\\]"),        # W of another hidden size
        (dict(w=torch.zeros(10, 8, dtype=torch.float32)), "one dtype"),  # W of another dtype
        (dict(w=torch.zeros(80, dtype=bf)), "w \\[V, d\\]"),            # W not 2-D
        (dict(idx=torch.zeros(3, 2, dtype=torch.int32), val=torch.zeros(3, 2, dtype=bf)), "idx must be"),
        (dict(idx=torch.zeros(4, 2, dtype=torch.int64)), "idx must be"),
        (dict(val=torch.zeros(4, 3, dtype=bf)), "idx must be"),
    ]
    for kw, msg in bad:
        a = dict(h=h, w=torch.zeros(10, 8, dtype=bf), idx=idx, val=val)
        a.update(kw)
        with pytest.raises(ValueError, match=msg):
            kd.kd_chunked_kl_fwd(a["h"], a["w"], a["idx"], a["val"], 1.0)
        with pytest.raises(ValueError, match=msg):
            kd.kd_chunked_kl_bwd(a["h"], a["w"], a["idx"], a["val"], 1.0, lse)
    w = torch.zeros(10, 8, dtype=bf)
    for bad_lse in (torch.zeros(3, dtype=torch.float32), torch.zeros(4, dtype=bf), torch.zeros(4, 1)):
        with pytest.raises(ValueError, match="lse must be"):
            kd.kd_chunked_kl_bwd(h, w, idx, val, 1.0, bad_lse)
    with pytest.raises(ValueError, match="h_t must be"):
        kd.kd_topk_cache_build(h, torch.zeros(10, 16, dtype=bf), 2)
    with pytest.raises(ValueError, match="h_t must be"):
        kd.kd_topk_cache_build(h, torch.zeros(10, 8, dtype=torch.float32), 2)
    # a well-formed call on CPU tensors still stops at the device check
    with pytest.raises(ValueError, match="GPU tensors only"):
        kd.kd_chunked_kl_fwd(h, w, idx, val, 1.0)


def test_empty_problem_workspace(lib):
    st, b = _ws(lib, kd.KD_OP_KL_FWD, _P(n=0))
    assert st == 0 and b > 0
    st, b = _ws(lib, kd.KD_OP_KL_BWD, _P(n=0))
    assert st == 0
