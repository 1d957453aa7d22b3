"""Python binding of the kdkl HIP library (fused, chunked top-K KL distillation loss).

Argument marshalling only: every step of the loss runs in the library's HIP
kernels (``lm_head_kl_amd/csrc``, C ABI in ``include/kdkl.h``).  PyTorch provides
device memory (through its caching allocator, so peak-memory statistics include
the workspace) and the current HIP stream.  There is no CPU fallback: if the
library is missing or a tensor is not on a GPU, the call raises.

Entry points (same names as the C ABI):

* :func:`kd_topk_cache_build` -- offline teacher cache: exact top-K (index,
  logit) pairs of ``H_T @ W_T^T`` per token.
* :func:`kd_chunked_kl_fwd` -- loss, per-row log-sum-exp (and per-row KL).
* :func:`kd_chunked_kl_bwd` -- ``dH`` and ``dW``.
  Both take optional ``labels`` / ``ignore_index`` / ``ce_weight`` (a padding
  mask and a hard-label cross-entropy mix), which select the C calls
  ``kd_chunked_kl_fwd_ex`` / ``kd_chunked_kl_bwd_ex``.
* :class:`KDChunkedKL` / :func:`chunked_kl_loss` -- autograd wrapper (forward
  saves ``lse``; backward calls :func:`kd_chunked_kl_bwd`);
  :class:`ChunkedTopKKLLoss` -- the same as a ``torch.nn.Module`` over
  ``[..., d]`` hidden states and ``[..., K]`` caches.
* :func:`kd_cache_write`, :func:`kd_cache_info_read`, :func:`kd_cache_read` --
  on-disk cache shards (C ABI in ``include/kdcache.h``);
  :func:`kd_cache_loader_open` / :func:`kd_cache_loader_next` /
  :func:`kd_cache_loader_close` and the iterator :class:`CacheLoader` -- streaming
  of shards to the device with prefetch; :func:`kd_cache_writer_open` /
  :func:`kd_cache_writer_put` / :func:`kd_cache_writer_close` and
  :class:`CacheWriter` -- device batches written to shards in the background.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkdkl.so")

KD_F32, KD_BF16 = 0, 1
KD_OP_TOPK_BUILD, KD_OP_KL_FWD, KD_OP_KL_BWD = 0, 1, 2

STATUS_NAMES = {
    0: "KD_OK", 1: "KD_ERR_NULL_POINTER", 2: "KD_ERR_BAD_SHAPE", 3: "KD_ERR_BAD_DTYPE", 4: "KD_ERR_BAD_TAU",
    5: "KD_ERR_MISALIGNED", 6: "KD_ERR_WORKSPACE_TOO_SMALL", 7: "KD_ERR_NO_DEVICE", 8: "KD_ERR_UNSUPPORTED_ARCH",
    9: "KD_ERR_LAUNCH", 10: "KD_ERR_IDX_OUT_OF_RANGE", 11: "KD_ERR_TOPK_OVERFLOW", 12: "KD_ERR_IO",
    13: "KD_ERR_BAD_FORMAT", 14: "KD_ERR_BAD_OPTION", 15: "KD_ERR_SCRATCH_TOO_SMALL",
}

# Every symbol the header declares (checked by the CPU test suite).
EXPORTED = ("kd_workspace_size", "kd_topk_cache_build", "kd_chunked_kl_fwd", "kd_chunked_kl_bwd",
            "kd_chunked_kl_fwd_ex", "kd_chunked_kl_bwd_ex", "kd_chunked_kl_fwd_noalloc", "kd_status_string", "kd_version", "kd_profile_begin", "kd_profile_end",
            "kd_cache_write", "kd_cache_info_read", "kd_cache_read", "kd_cache_loader_open",
            "kd_cache_loader_info", "kd_cache_loader_next", "kd_cache_loader_close",
            "kd_cache_writer_open", "kd_cache_writer_put", "kd_cache_writer_close")


class KDProblem(ctypes.Structure):
    """Mirror of ``kd_problem`` in include/kdkl.h."""
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("d_model", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("k", ctypes.c_int32),
        ("tau", ctypes.c_float),
        ("x_dtype", ctypes.c_int32),
        ("val_dtype", ctypes.c_int32),
        ("dh_dtype", ctypes.c_int32),
        ("chunk_tokens", ctypes.c_int32),
    ]


KD_STUDENT_FULL, KD_STUDENT_RENORM = 0, 1
_STUDENT = {"full": KD_STUDENT_FULL, "renorm": KD_STUDENT_RENORM}


class KDLossOpts(ctypes.Structure):
    """Mirror of ``kd_loss_opts``."""
    _fields_ = [
        ("labels", ctypes.c_void_p),
        ("ignore_index", ctypes.c_int32),
        ("ce_weight", ctypes.c_float),
        ("student", ctypes.c_int32),
    ]


class KDKernelStat(ctypes.Structure):
    """Mirror of ``kd_kernel_stat``."""
    _fields_ = [
        ("name", ctypes.c_char * 32),
        ("launches", ctypes.c_int64),
        ("total_ms", ctypes.c_double),
        ("flops", ctypes.c_double),
        ("bytes", ctypes.c_double),
    ]


class KDCacheInfo(ctypes.Structure):
    """Mirror of ``kd_cache_info`` in include/kdcache.h."""
    _fields_ = [
        ("n_tokens", ctypes.c_int64),
        ("vocab", ctypes.c_int64),
        ("k", ctypes.c_int32),
        ("idx_bits", ctypes.c_int32),
        ("val_dtype", ctypes.c_int32),
    ]


class KDError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({status_string(status)})")


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) the built shared library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"kdkl HIP library not built: {path} is missing "
                           f"(run `python -m lm_head_kl_amd.build`)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(KDProblem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.kd_workspace_size.argtypes = [ctypes.c_int, P, ctypes.POINTER(sz)]
    lib.kd_topk_cache_build.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_chunked_kl_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_chunked_kl_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    O = ctypes.POINTER(KDLossOpts)
    lib.kd_chunked_kl_fwd_ex.argtypes = [P, O, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_chunked_kl_bwd_ex.argtypes = [P, O, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kd_chunked_kl_fwd_noalloc.argtypes = [P, O, vp, vp, vp, vp, vp, vp, vp, vp]
    for f in ("kd_workspace_size", "kd_topk_cache_build", "kd_chunked_kl_fwd", "kd_chunked_kl_bwd",
              "kd_chunked_kl_fwd_ex", "kd_chunked_kl_bwd_ex", "kd_chunked_kl_fwd_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    lib.kd_status_string.argtypes = [ctypes.c_int]
    lib.kd_status_string.restype = ctypes.c_char_p
    lib.kd_version.argtypes = []
    lib.kd_version.restype = ctypes.c_int
    lib.kd_profile_begin.argtypes = []
    lib.kd_profile_begin.restype = ctypes.c_int
    lib.kd_profile_end.argtypes = [ctypes.POINTER(KDKernelStat), ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.kd_profile_end.restype = ctypes.c_int
    CI = ctypes.POINTER(KDCacheInfo)
    cp, i64, i32 = ctypes.c_char_p, ctypes.c_int64, ctypes.c_int32
    lib.kd_cache_write.argtypes = [cp, CI, vp, vp]
    lib.kd_cache_info_read.argtypes = [cp, CI]
    lib.kd_cache_read.argtypes = [cp, i64, i64, vp, vp]
    lib.kd_cache_loader_open.argtypes = [ctypes.POINTER(cp), i32, i64, i32, ctypes.POINTER(vp)]
    lib.kd_cache_loader_info.argtypes = [vp, CI]
    lib.kd_cache_loader_next.argtypes = [vp, vp, vp, ctypes.POINTER(i64), vp]
    lib.kd_cache_loader_close.argtypes = [vp]
    lib.kd_cache_writer_open.argtypes = [cp, CI, i64, i32, ctypes.POINTER(vp)]
    lib.kd_cache_writer_put.argtypes = [vp, vp, vp, i64, vp]
    lib.kd_cache_writer_close.argtypes = [vp, ctypes.POINTER(i64)]
    for f in ("kd_cache_write", "kd_cache_info_read", "kd_cache_read", "kd_cache_loader_open",
              "kd_cache_loader_info", "kd_cache_loader_next", "kd_cache_loader_close",
              "kd_cache_writer_open", "kd_cache_writer_put", "kd_cache_writer_close"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load_library().kd_status_string(int(status)).decode()
    except RuntimeError:
        return STATUS_NAMES.get(status, "unknown")


def _check(status: int, where: str) -> None:
    if status != 0:
        raise KDError(status, where)


def _dt(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return KD_BF16
    if t == torch.float32:
        return KD_F32
    raise TypeError(f"unsupported dtype {t}")


def make_problem(n: int, d: int, v: int, k: int, tau: float = 1.0, x_dtype: int = KD_BF16,
                 val_dtype: Optional[int] = None, dh_dtype: int = KD_F32, chunk_tokens: int = 0) -> KDProblem:
    return KDProblem(int(n), int(d), int(v), int(k), float(tau), int(x_dtype),
                     int(x_dtype if val_dtype is None else val_dtype), int(dh_dtype), int(chunk_tokens))


def workspace_size(op: int, prob: KDProblem) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().kd_workspace_size(int(op), ctypes.byref(prob), ctypes.byref(out)), "kd_workspace_size")
    return int(out.value)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need_gpu(*ts: torch.Tensor) -> torch.device:
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("kdkl works on GPU tensors only (no CPU fallback)")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous row-major")
        dev = t.device if dev is None else dev
        if t.device != dev:
            raise ValueError("all tensors must be on one device")
    return dev


def _loss_inputs(h: torch.Tensor, w: torch.Tensor, idx: torch.Tensor, val: torch.Tensor,
                 lse: Optional[torch.Tensor] = None) -> Tuple[int, int, int, int]:
    """Shapes and dtypes of the loss's inputs, checked before any pointer is taken:
    the library sees only pointers and the sizes passed here.  Returns (N, d, V, K)."""
    if h.dim() != 2 or w.dim() != 2 or w.shape[1] != h.shape[1]:
        raise ValueError(f"h must be [N, d] and w [V, d]; got {tuple(h.shape)} and {tuple(w.shape)}")
    if h.dtype != w.dtype or h.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"h and w must share one dtype, bfloat16 or float32; got {h.dtype} and {w.dtype}")
    if idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[0] != h.shape[0] or val.shape != idx.shape:
        raise ValueError("idx must be int32 [N, K] and val [N, K]")
    if lse is not None and (lse.dtype != torch.float32 or lse.shape != (h.shape[0],)):
        raise ValueError("lse must be float32 [N]")
    return h.shape[0], h.shape[1], w.shape[0], idx.shape[1]


def _workspace(op: int, prob: KDProblem, device: torch.device) -> torch.Tensor:
    return torch.empty(max(256, workspace_size(op, prob)), dtype=torch.uint8, device=device)


def kd_topk_cache_build(h_t: torch.Tensor, w_t: torch.Tensor, k: int, chunk_tokens: int = 0
                        ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact top-K teacher cache.  Returns ``(idx int32 [N,K], val [N,K])``; ``val``
    has the inputs' dtype (bf16 for bf16 heads, float32 for float32 heads)."""
    if h_t.dim() != 2 or w_t.dim() != 2 or w_t.shape[1] != h_t.shape[1] or w_t.dtype != h_t.dtype:
        raise ValueError("h_t must be [N, d] and w_t [V, d], of one dtype")
    dev = _need_gpu(h_t, w_t)
    n, d = h_t.shape
    v = w_t.shape[0]
    xdt = _dt(h_t.dtype)
    prob = make_problem(n, d, v, k, 1.0, xdt, xdt, KD_F32, chunk_tokens)
    idx = torch.empty((n, k), dtype=torch.int32, device=dev)
    val = torch.empty((n, k), dtype=h_t.dtype, device=dev)
    ws = _workspace(KD_OP_TOPK_BUILD, prob, dev)
    with torch.cuda.device(dev):
        st = _stream(dev)
        _check(load_library().kd_topk_cache_build(ctypes.byref(prob), _ptr(h_t), _ptr(w_t), _ptr(idx), _ptr(val),
                                                  _ptr(ws), ws.numel(), st), "kd_topk_cache_build")
    return idx, val


def _opts(labels: Optional[torch.Tensor], ignore_index: int, ce_weight: float, n: int, student: str = "full"
          ) -> Optional[KDLossOpts]:
    """The loss options, or None for the plain loss (no labels, no mix, the
    full-vocabulary student)."""
    if not -2**31 <= int(ignore_index) < 2**31:
        raise ValueError("ignore_index must fit in int32")
    if student not in _STUDENT:
        raise ValueError("student must be 'full' or 'renorm'")
    if labels is None and ce_weight == 0.0 and student == "full":
        return None
    if labels is not None and (labels.dtype != torch.int32 or labels.shape != (n,)):
        raise ValueError("labels must be int32 [N]")
    return KDLossOpts(_ptr(labels), int(ignore_index), float(ce_weight), _STUDENT[student])


def kd_chunked_kl_fwd(h: torch.Tensor, w: torch.Tensor, idx: torch.Tensor, val: torch.Tensor, tau: float,
                      with_rows: bool = False, chunk_tokens: int = 0, labels: Optional[torch.Tensor] = None,
                      ignore_index: int = -100, ce_weight: float = 0.0, student: str = "full"
                      ) -> Tuple[torch.Tensor, torch.Tensor, Optional[torch.Tensor]]:
    """Returns ``(loss [] float32, lse [N] float32, rows [N] float32 or None)``.

    With ``labels`` (int32 [N]), rows labelled ``ignore_index`` are left out and
    the mean runs over the others; ``ce_weight`` a mixes in the cross-entropy
    with the labels: row term ``(1 - a) KL + a CE`` (``rows`` holds those terms).
    ``student="renorm"`` takes the student's softmax over the row's K cached
    entries only (``lse`` then holds that normaliser)."""
    n, d, v, k = _loss_inputs(h, w, idx, val)
    dev = _need_gpu(h, w, idx, val, labels)
    prob = make_problem(n, d, v, k, tau, _dt(h.dtype), _dt(val.dtype), KD_F32, chunk_tokens)
    loss = torch.empty((), dtype=torch.float32, device=dev)
    lse = torch.empty((n,), dtype=torch.float32, device=dev)
    rows = torch.empty((n,), dtype=torch.float32, device=dev) if with_rows else None
    ws = _workspace(KD_OP_KL_FWD, prob, dev)
    opts = _opts(labels, ignore_index, ce_weight, n, student)
    lib = load_library()
    with torch.cuda.device(dev):
        if opts is None:
            _check(lib.kd_chunked_kl_fwd(ctypes.byref(prob), _ptr(h), _ptr(w), _ptr(idx), _ptr(val), _ptr(loss),
                                         _ptr(lse), _ptr(rows), _ptr(ws), ws.numel(), _stream(dev)),
                   "kd_chunked_kl_fwd")
        else:
            _check(lib.kd_chunked_kl_fwd_ex(ctypes.byref(prob), ctypes.byref(opts), _ptr(h), _ptr(w), _ptr(idx),
                                            _ptr(val), _ptr(loss), _ptr(lse), _ptr(rows), _ptr(ws), ws.numel(),
                                            _stream(dev)), "kd_chunked_kl_fwd_ex")
    return loss, lse, rows


def kd_chunked_kl_fwd_noalloc(h: torch.Tensor, w: torch.Tensor, idx: torch.Tensor, val: torch.Tensor, tau: float,
                              loss: torch.Tensor, lse: torch.Tensor, rows: Optional[torch.Tensor] = None,
                              chunk_tokens: int = 0, labels: Optional[torch.Tensor] = None,
                              ignore_index: int = -100, ce_weight: float = 0.0, student: str = "full") -> None:
    """The forward into caller-provided outputs (``loss`` float32 scalar, ``lse``
    float32 [N], ``rows`` float32 [N] or None), with the library's fixed scratch
    array as workspace: nothing is allocated, by the library or here."""
    n, d, v, k = _loss_inputs(h, w, idx, val, lse)
    dev = _need_gpu(h, w, idx, val, loss, lse, rows, labels)
    if loss.dtype != torch.float32 or loss.numel() != 1 or (rows is not None and (rows.dtype != torch.float32
                                                                                   or rows.shape != (n,))):
        raise ValueError("loss must be a float32 scalar and rows float32 [N]")
    prob = make_problem(n, d, v, k, tau, _dt(h.dtype), _dt(val.dtype), KD_F32, chunk_tokens)
    opts = _opts(labels, ignore_index, ce_weight, n, student)
    with torch.cuda.device(dev):
        _check(load_library().kd_chunked_kl_fwd_noalloc(ctypes.byref(prob), None if opts is None else ctypes.byref(opts),
                                                         _ptr(h), _ptr(w), _ptr(idx), _ptr(val), _ptr(loss), _ptr(lse),
                                                         _ptr(rows), _stream(dev)), "kd_chunked_kl_fwd_noalloc")


def kd_chunked_kl_bwd(h: torch.Tensor, w: torch.Tensor, idx: torch.Tensor, val: torch.Tensor, tau: float,
                      lse: torch.Tensor, grad: Optional[torch.Tensor] = None, dh_dtype: torch.dtype = torch.float32,
                      chunk_tokens: int = 0, labels: Optional[torch.Tensor] = None, ignore_index: int = -100,
                      ce_weight: float = 0.0, student: str = "full") -> Tuple[torch.Tensor, torch.Tensor]:
    """Returns ``(dH [N,d] dh_dtype, dW [V,d] float32)`` for upstream gradient
    ``grad`` (a device scalar; None means 1).  ``labels`` / ``ignore_index`` /
    ``ce_weight`` / ``student`` must be those of the forward call."""
    n, d, v, k = _loss_inputs(h, w, idx, val, lse)
    dev = _need_gpu(h, w, idx, val, lse, grad, labels)
    if grad is not None and (grad.dtype != torch.float32 or grad.numel() != 1):
        raise ValueError("grad must be a float32 scalar tensor")
    prob = make_problem(n, d, v, k, tau, _dt(h.dtype), _dt(val.dtype), _dt(dh_dtype), chunk_tokens)
    dh = torch.empty((n, d), dtype=dh_dtype, device=dev)
    dw = torch.empty((v, d), dtype=torch.float32, device=dev)
    ws = _workspace(KD_OP_KL_BWD, prob, dev)
    opts = _opts(labels, ignore_index, ce_weight, n, student)
    lib = load_library()
    with torch.cuda.device(dev):
        if opts is None:
            _check(lib.kd_chunked_kl_bwd(ctypes.byref(prob), _ptr(h), _ptr(w), _ptr(idx), _ptr(val), _ptr(lse),
                                         _ptr(grad), _ptr(dh), _ptr(dw), _ptr(ws), ws.numel(), _stream(dev)),
                   "kd_chunked_kl_bwd")
        else:
            _check(lib.kd_chunked_kl_bwd_ex(ctypes.byref(prob), ctypes.byref(opts), _ptr(h), _ptr(w), _ptr(idx),
                                            _ptr(val), _ptr(lse), _ptr(grad), _ptr(dh), _ptr(dw), _ptr(ws),
                                            ws.numel(), _stream(dev)), "kd_chunked_kl_bwd_ex")
    return dh, dw


def profile_begin() -> None:
    """Start bracketing every kernel launch of the library with HIP events."""
    _check(load_library().kd_profile_begin(), "kd_profile_begin")


def profile_end() -> dict:
    """Stop the session; returns ``{kind: {launches, total_ms, flops, bytes}}``."""
    buf = (KDKernelStat * 64)()
    n = ctypes.c_int(0)
    _check(load_library().kd_profile_end(buf, 64, ctypes.byref(n)), "kd_profile_end")
    return {buf[i].name.decode(): {"launches": int(buf[i].launches), "total_ms": float(buf[i].total_ms),
                                   "flops": float(buf[i].flops), "bytes": float(buf[i].bytes)}
            for i in range(min(n.value, 64))}


class KDChunkedKL(torch.autograd.Function):
    """``loss = KDChunkedKL.apply(H, W, idx, val, tau[, chunk_tokens, labels,
    ignore_index, ce_weight])``; gradients flow to H and W."""

    @staticmethod
    def forward(ctx, h, w, idx, val, tau, chunk_tokens=0, labels=None, ignore_index=-100, ce_weight=0.0,
                student="full"):
        loss, lse, _ = kd_chunked_kl_fwd(h, w, idx, val, tau, chunk_tokens=chunk_tokens, labels=labels,
                                         ignore_index=ignore_index, ce_weight=ce_weight, student=student)
        ctx.save_for_backward(h, w, idx, val, lse, labels)
        ctx.tau = tau
        ctx.chunk_tokens = chunk_tokens
        ctx.ignore_index = ignore_index
        ctx.ce_weight = ce_weight
        ctx.student = student
        return loss

    @staticmethod
    def backward(ctx, g):
        h, w, idx, val, lse, labels = ctx.saved_tensors
        g = g.detach().to(torch.float32).reshape(()).contiguous()
        dh, dw = kd_chunked_kl_bwd(h, w, idx, val, ctx.tau, lse, g,
                                   dh_dtype=torch.float32 if h.dtype == torch.float32 else torch.bfloat16,
                                   chunk_tokens=ctx.chunk_tokens, labels=labels, ignore_index=ctx.ignore_index,
                                   ce_weight=ctx.ce_weight, student=ctx.student)
        return dh.to(h.dtype), dw.to(w.dtype), None, None, None, None, None, None, None, None


def chunked_kl_loss(h, w, idx, val, tau: float = 1.0, chunk_tokens: int = 0, labels=None,
                    ignore_index: int = -100, ce_weight: float = 0.0, student: str = "full") -> torch.Tensor:
    """Mean top-K KL over the tokens (autograd).  ``labels`` (int32 [N]) leave out
    the rows labelled ``ignore_index``; ``ce_weight`` mixes in the cross-entropy
    with the labels; ``student="renorm"`` normalises the student over the cached
    entries only."""
    return KDChunkedKL.apply(h, w, idx, val, float(tau), int(chunk_tokens), labels, int(ignore_index),
                             float(ce_weight), student)


class ChunkedTopKKLLoss(torch.nn.Module):
    """Drop-in loss module: ``loss = ChunkedTopKKLLoss(tau)(hidden, head_weight,
    idx, val[, labels])``.

    ``hidden`` is ``[..., d]`` (for example ``[batch, seq, d]``), ``idx`` / ``val``
    are ``[..., K]`` and ``labels`` ``[...]`` over the same leading axes; they are
    flattened to rows as views (no copy, so they must be contiguous).  ``labels``
    may be int32 or int64 (as for ``cross_entropy``); int64 labels are converted on
    the device, and a value int32 cannot hold counts as out of range.  The head
    weight is ``[V, d]`` as in ``nn.Linear(d, V, bias=False).weight``.  Returns the
    mean top-K KL over the tokens (over the counted tokens with labels), mixed with
    the labels' cross-entropy when ``ce_weight`` > 0."""

    def __init__(self, tau: float = 1.0, ignore_index: int = -100, ce_weight: float = 0.0,
                 chunk_tokens: int = 0, student: str = "full"):
        super().__init__()
        self.tau = float(tau)
        self.ignore_index = int(ignore_index)
        self.ce_weight = float(ce_weight)
        self.chunk_tokens = int(chunk_tokens)
        if student not in _STUDENT:
            raise ValueError("student must be 'full' or 'renorm'")
        self.student = student

    def forward(self, hidden, weight, idx, val, labels=None):
        d = hidden.shape[-1]
        k = idx.shape[-1]
        if idx.shape[:-1] != hidden.shape[:-1] or val.shape != idx.shape:
            raise ValueError("idx / val must be [..., K] over the hidden states' leading axes")
        if labels is not None and labels.shape != hidden.shape[:-1]:
            raise ValueError("labels must have the hidden states' leading axes")
        h = hidden.view(-1, d)
        lab = None if labels is None else labels.view(-1)
        if lab is not None and lab.dtype == torch.int64:
            v = weight.shape[0]
            bad = v + 1 if v == self.ignore_index else v      # out of [0, V) and not the ignore index
            wide = (lab < -2**31) | (lab >= 2**31)
            lab = torch.where(wide, torch.full_like(lab, bad), lab).to(torch.int32)
        return chunked_kl_loss(h, weight, idx.view(-1, k), val.view(-1, k), self.tau, self.chunk_tokens, lab,
                               self.ignore_index, self.ce_weight, self.student)

    def extra_repr(self) -> str:
        return (f"tau={self.tau}, ignore_index={self.ignore_index}, ce_weight={self.ce_weight}, "
                f"chunk_tokens={self.chunk_tokens}, student={self.student!r}")


# ---- on-disk cache shards and the streaming loader (include/kdcache.h)

_VAL_TORCH = {KD_F32: torch.float32, KD_BF16: torch.bfloat16}

# open loader and writer handles -> [rows one call moves at most, K, value dtype,
# rows a loader has still to hand out (None for a writer)], so that the device
# tensors of next/put are checked against them before a copy is enqueued (the
# library sees only pointers)
_HANDLES = {}


def _batch_tensors(handle: ctypes.c_void_p, idx: torch.Tensor, val: torch.Tensor, where: str) -> list:
    spec = _HANDLES.get(handle.value if handle is not None else None)
    if spec is None:
        raise ValueError(f"{where}: not an open handle")
    k, vdt = spec[1], spec[2]
    if idx.dtype != torch.int32 or idx.dim() != 2 or idx.shape[1] != k or val.shape != idx.shape or val.dtype != vdt:
        raise ValueError(f"{where}: idx must be int32 [rows, {k}] and val {vdt} [rows, {k}]")
    return spec


def _host(t: torch.Tensor, dtype: torch.dtype, name: str) -> torch.Tensor:
    if t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous CPU tensor of dtype {dtype}")
    return t


def kd_cache_write(path: str, idx: torch.Tensor, val: torch.Tensor, vocab: int, idx_bits: int = 0) -> None:
    """Write one shard from host tensors ``idx`` int32 [N,K] and ``val`` bf16/float32
    [N,K].  ``idx_bits`` 0 picks 16 when ``vocab <= 65536``, else 32."""
    if idx.dim() != 2 or val.shape != idx.shape:
        raise ValueError("idx and val must both be [N, K]")
    _host(idx, torch.int32, "idx")
    vdt = _dt(val.dtype)
    _host(val, val.dtype, "val")
    info = KDCacheInfo(int(idx.shape[0]), int(vocab), int(idx.shape[1]), int(idx_bits), vdt)
    _check(load_library().kd_cache_write(os.fsencode(path), ctypes.byref(info), _ptr(idx), _ptr(val)),
           "kd_cache_write")


def kd_cache_info_read(path: str) -> dict:
    info = KDCacheInfo()
    _check(load_library().kd_cache_info_read(os.fsencode(path), ctypes.byref(info)), "kd_cache_info_read")
    return {"n_tokens": int(info.n_tokens), "vocab": int(info.vocab), "k": int(info.k),
            "idx_bits": int(info.idx_bits), "val_dtype": int(info.val_dtype)}


def kd_cache_read(path: str, row0: int = 0, rows: Optional[int] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Rows ``[row0, row0 + rows)`` of a shard as host tensors (idx int32, val)."""
    info = kd_cache_info_read(path)
    if rows is None:
        rows = info["n_tokens"] - row0
    idx = torch.empty((rows, info["k"]), dtype=torch.int32)
    val = torch.empty((rows, info["k"]), dtype=_VAL_TORCH[info["val_dtype"]])
    _check(load_library().kd_cache_read(os.fsencode(path), int(row0), int(rows), _ptr(idx), _ptr(val)),
           "kd_cache_read")
    return idx, val


def kd_cache_loader_open(paths, batch_tokens: int, prefetch: int = 2) -> ctypes.c_void_p:
    """Open a streaming loader over the shards ``paths`` (read in order)."""
    enc = [os.fsencode(p) for p in paths]
    arr = (ctypes.c_char_p * max(1, len(enc)))(*enc)
    h = ctypes.c_void_p()
    _check(load_library().kd_cache_loader_open(arr, len(enc), int(batch_tokens), int(prefetch), ctypes.byref(h)),
           "kd_cache_loader_open")
    info = kd_cache_loader_info(h)
    _HANDLES[h.value] = [int(batch_tokens), info["k"], _VAL_TORCH[info["val_dtype"]], info["n_tokens"]]
    return h


def kd_cache_loader_info(handle: ctypes.c_void_p) -> dict:
    info = KDCacheInfo()
    _check(load_library().kd_cache_loader_info(handle, ctypes.byref(info)), "kd_cache_loader_info")
    return {"n_tokens": int(info.n_tokens), "vocab": int(info.vocab), "k": int(info.k),
            "idx_bits": int(info.idx_bits), "val_dtype": int(info.val_dtype)}


def kd_cache_loader_next(handle: ctypes.c_void_p, idx_dev: torch.Tensor, val_dev: torch.Tensor) -> int:
    """Enqueue the next batch's copies into the device tensors (on the current
    stream of their device); returns its row count, 0 at the end.  The tensors
    hold at least that batch: idx int32 [>= rows, K], val [same] (rows =
    batch_tokens, fewer for the last batch, 0 at the end)."""
    spec = _batch_tensors(handle, idx_dev, val_dev, "kd_cache_loader_next")
    need = min(spec[0], spec[3])
    if idx_dev.shape[0] < need:
        raise ValueError(f"kd_cache_loader_next: the tensors hold {idx_dev.shape[0]} rows, the next batch {need}")
    rows = ctypes.c_int64(0)
    if need > 0:
        dev = _need_gpu(idx_dev, val_dev)
        with torch.cuda.device(dev):
            _check(load_library().kd_cache_loader_next(handle, _ptr(idx_dev), _ptr(val_dev), ctypes.byref(rows),
                                                       _stream(dev)), "kd_cache_loader_next")
    else:
        # every row handed out: the library returns 0 rows and touches no buffer
        _check(load_library().kd_cache_loader_next(handle, None, None, ctypes.byref(rows), None),
               "kd_cache_loader_next")
    spec[3] -= int(rows.value)
    return int(rows.value)


def kd_cache_loader_close(handle: ctypes.c_void_p) -> None:
    _HANDLES.pop(handle.value if handle is not None else None, None)
    _check(load_library().kd_cache_loader_close(handle), "kd_cache_loader_close")


class CacheLoader:
    """Iterates ``(idx, val)`` device tensors of ``batch_tokens`` rows (the last
    batch may be shorter) over cache shards, prefetching in a background thread.
    Each batch has its own device tensors, so a batch stays valid while the next
    one streams in."""

    def __init__(self, paths, batch_tokens: int, prefetch: int = 2, device: str = "cuda"):
        self.device = torch.device(device)
        self.handle = kd_cache_loader_open(paths, batch_tokens, prefetch)
        self.info = kd_cache_loader_info(self.handle)
        self.batch = int(batch_tokens)

    def __iter__(self):
        return self

    def __next__(self) -> Tuple[torch.Tensor, torch.Tensor]:
        if self.handle is None:
            raise StopIteration
        k = self.info["k"]
        idx = torch.empty((self.batch, k), dtype=torch.int32, device=self.device)
        val = torch.empty((self.batch, k), dtype=_VAL_TORCH[self.info["val_dtype"]], device=self.device)
        rows = kd_cache_loader_next(self.handle, idx, val)
        if rows == 0:
            self.close()
            raise StopIteration
        return idx[:rows], val[:rows]

    def close(self) -> None:
        if self.handle is not None:
            kd_cache_loader_close(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def kd_cache_writer_open(prefix: str, shard_tokens: int, vocab: int, k: int, val_dtype: torch.dtype,
                         max_batch_tokens: int, depth: int = 3, idx_bits: int = 0) -> ctypes.c_void_p:
    """Open a streaming writer of shards ``<prefix>_00000.kdc`` ... of
    ``shard_tokens`` rows each."""
    info = KDCacheInfo(int(shard_tokens), int(vocab), int(k), int(idx_bits), _dt(val_dtype))
    h = ctypes.c_void_p()
    _check(load_library().kd_cache_writer_open(os.fsencode(prefix), ctypes.byref(info), int(max_batch_tokens),
                                               int(depth), ctypes.byref(h)), "kd_cache_writer_open")
    _HANDLES[h.value] = [int(max_batch_tokens), int(k), val_dtype, None]
    return h


def kd_cache_writer_put(handle: ctypes.c_void_p, idx_dev: torch.Tensor, val_dev: torch.Tensor) -> None:
    """Hand over device rows ``idx_dev`` int32 [rows, K] and ``val_dev`` [rows, K];
    the copies run on the current stream of their device.  The tensors must stay
    unchanged until those copies have run (the next put or close waits for them
    only as far as buffer space requires)."""
    _batch_tensors(handle, idx_dev, val_dev, "kd_cache_writer_put")
    dev = _need_gpu(idx_dev, val_dev)
    with torch.cuda.device(dev):
        _check(load_library().kd_cache_writer_put(handle, _ptr(idx_dev), _ptr(val_dev), int(idx_dev.shape[0]),
                                                  _stream(dev)), "kd_cache_writer_put")


def kd_cache_writer_close(handle: ctypes.c_void_p) -> int:
    """Write the last shard and free the writer; returns the number of shards."""
    _HANDLES.pop(handle.value if handle is not None else None, None)
    n = ctypes.c_int64(0)
    _check(load_library().kd_cache_writer_close(handle, ctypes.byref(n)), "kd_cache_writer_close")
    return int(n.value)


class CacheWriter:
    """``with CacheWriter(prefix, shard_tokens, vocab, k, torch.bfloat16, max_batch) as w:
    w.put(idx, val)`` for each device batch; ``w.paths`` lists the shards written."""

    def __init__(self, prefix: str, shard_tokens: int, vocab: int, k: int, val_dtype: torch.dtype,
                 max_batch_tokens: int, depth: int = 3, idx_bits: int = 0):
        self.prefix = prefix
        self.handle = kd_cache_writer_open(prefix, shard_tokens, vocab, k, val_dtype, max_batch_tokens, depth,
                                           idx_bits)
        self.paths = []

    def put(self, idx_dev: torch.Tensor, val_dev: torch.Tensor) -> None:
        kd_cache_writer_put(self.handle, idx_dev, val_dev)

    def close(self) -> list:
        """Write the last shard and free the writer.  ``paths`` is set before an
        error is raised: the shards written before it are complete and in order."""
        if self.handle is not None:
            h, self.handle = self.handle, None
            _HANDLES.pop(h.value, None)
            n = ctypes.c_int64(0)
            st = load_library().kd_cache_writer_close(h, ctypes.byref(n))
            self.paths = [f"{self.prefix}_{i:05d}.kdc" for i in range(n.value)]
            _check(st, "kd_cache_writer_close")
        return self.paths

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
