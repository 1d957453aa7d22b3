/*
 * kdkl.h - C ABI of the fused, chunked top-K KL distillation loss over an LM head,
 * for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages about arXiv 2608.03796, "Efficient Knowledge Distillation for
 * LLMs: Offline Top-K Logits and a Fused Chunked KL Loss"):
 *   [abs]  the paper's abstract (chatpaper.ai page / Hugging Face papers mirror):
 *          offline KD caches the teacher's top-K logits once; the fused chunked KL
 *          loss never materialises the full vocabulary-sized logit tensor, so peak
 *          memory grows linearly with sequence length.
 *   [mv]   mind-verse.de, "Optimierung der Wissensdestillation ...", section
 *          "2. Ein zusammengeführter, chunked KL-Verlust", bullet "Fused chunked KL":
 *          the output projection is folded into the loss, one chunk at a time is
 *          projected, folded into the running loss and discarded; the backward pass
 *          recomputes each chunk, so the projection runs twice.
 *   [wiki] llm-wiki study note "LLM 지식 증류 효율화 ...", sections "표준 KD의 손실 함수"
 *          (KL(P_T || P_S) over the vocabulary), "핵심 아이디어 1: Offline Top-K Logits"
 *          (K (vocab index, logit) pairs per position), "기존 라이브러리 통합" (the
 *          teacher precompute and the fused loss are independent, drop-in pieces).
 *
 * Notation: N tokens, d hidden size, V vocabulary, K cached entries per token.
 *   H [N, d]   student final hidden states            (row-major)
 *   W [V, d]   student LM head, out x in (no bias)     (row-major)
 *   H_T, W_T   teacher hidden states / teacher head    (same layouts)
 *   idx [N, K] int32 cached vocabulary indices        (row-major)
 *   val [N, K] cached teacher logits                   (row-major)
 *
 * What is computed by the plain calls (all rows count; mean over N; a padding
 * mask and a hard-label mix are the _ex calls below):
 *   z[i,v]  = H[i,:] . W[v,:]                 student logits (never stored)
 *   lse[i]  = log sum_v exp(z[i,v])           over the whole vocabulary
 *   p[i,k]  = softmax_k(val[i,k] / tau)       teacher renormalised over its K entries
 *   KL[i]   = sum_k p[i,k] (log p[i,k] - z[i,idx[i,k]] + lse[i])   (p log p = 0 at p = 0)
 *   loss    = (1/N) sum_i KL[i]
 *   dZ[i,v] = (g/N) (exp(z[i,v] - lse[i]) - sum_{k: idx[i,k]=v} p[i,k])
 *   dH = dZ W,  dW = dZ^T H
 * tau applies to the teacher only (no tau^2 factor). Repeated indices in a row are
 * separate entries (the gradient scatter-adds them).
 *
 * Conventions for every call:
 *   - All data pointers are DEVICE pointers into contiguous row-major buffers,
 *     16-byte aligned. The caller owns every buffer; the library allocates no
 *     device memory and keeps no state besides a per-device architecture check
 *     and, for kd_chunked_kl_fwd_noalloc, a fixed scratch array per device and
 *     its address.
 *   - Scratch memory is the caller's workspace `ws` of at least
 *     kd_workspace_size() bytes (16-byte aligned); its contents on entry do not
 *     matter and are clobbered (kd_chunked_kl_fwd_noalloc uses the library's
 *     scratch array instead).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and
 *     the call returns without waiting. Two calls that share a workspace must be
 *     ordered on one stream.
 *   - Threads: the compute calls and kd_workspace_size may be made from several
 *     host threads at once (each call with its own workspace); the profiling hooks
 *     below are the exception.
 *   - Outputs are overwritten, never accumulated into.
 *   - Errors: every argument error returns a non-zero kd_status BEFORE anything is
 *     enqueued or any HIP call is made; KD_ERR_NO_DEVICE / KD_ERR_UNSUPPORTED_ARCH
 *     come from the device check that follows validation; KD_ERR_LAUNCH reports a
 *     failed kernel launch. Asynchronous device faults surface at the caller's next
 *     synchronisation. The library never aborts, prints or throws.
 *   - Shape domain: N >= 0, d >= 8 with d % 8 == 0, 1 <= V <= 2097088 (2^21 - 64),
 *     1 <= K <= min(V, 65535) (the cache build: K <= 4096), tau finite and > 0.
 *     Also N <= 2^31 - 256, d <= 2^20, chunk_tokens >= 0, and the chunk as used
 *     (chunk_tokens or the default, rounded up to 256, and at most N rounded up to
 *     256) at most 2096896 tokens: 256 rows of every operand, the chunk-strided
 *     transposed ones included, then stay within 2^31 bytes.
 *   - Cached indices must lie in [0, V). An out-of-range index is skipped by the
 *     kernels (no out-of-bounds access); it makes that row's KL NaN, and when the
 *     environment variable KD_CHECK=1 is set the forward call synchronises the
 *     stream and returns KD_ERR_IDX_OUT_OF_RANGE.
 *   - Results are bitwise reproducible for a given shape, chunk size and device:
 *     there are no floating-point atomics, every reduction has a fixed order, and
 *     repeated indices in a row are applied in k order.
 */
#ifndef KDKL_H
#define KDKL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KD_F32 = 0, KD_BF16 = 1 } kd_dtype;

typedef enum {
  KD_OK = 0,
  KD_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
  KD_ERR_BAD_SHAPE = 2,          /* a size is outside the domain above, or overflows */
  KD_ERR_BAD_DTYPE = 3,          /* unknown dtype, or an unsupported combination */
  KD_ERR_BAD_TAU = 4,            /* tau not finite or <= 0 */
  KD_ERR_MISALIGNED = 5,         /* a pointer is not 16-byte aligned */
  KD_ERR_WORKSPACE_TOO_SMALL = 6,/* ws_bytes < kd_workspace_size() */
  KD_ERR_NO_DEVICE = 7,          /* no HIP device is current */
  KD_ERR_UNSUPPORTED_ARCH = 8,   /* the current device is not gfx950 */
  KD_ERR_LAUNCH = 9,             /* a kernel launch failed */
  KD_ERR_IDX_OUT_OF_RANGE = 10,  /* only with KD_CHECK=1: a cached index (or mixed-in label) is outside [0, V) */
  KD_ERR_TOPK_OVERFLOW = 11,     /* only with KD_CHECK=1: too many near-ties at the K-th value */
  KD_ERR_IO = 12,                /* kdcache.h: a file could not be opened, read or written */
  KD_ERR_BAD_FORMAT = 13,        /* kdcache.h: a shard header or file size does not match the format */
  KD_ERR_BAD_OPTION = 14,        /* a kd_loss_opts field is outside its domain */
  KD_ERR_SCRATCH_TOO_SMALL = 15  /* kd_chunked_kl_fwd_noalloc: the problem needs more than the 64 MiB scratch */
} kd_status;

typedef enum { KD_OP_TOPK_BUILD = 0, KD_OP_KL_FWD = 1, KD_OP_KL_BWD = 2 } kd_op;

/* Problem description shared by all calls. */
typedef struct {
  int64_t n_tokens;     /* N */
  int64_t d_model;      /* d */
  int64_t vocab;        /* V */
  int32_t k;            /* K */
  float tau;            /* teacher temperature (KL calls; ignored by the cache build) */
  int32_t x_dtype;      /* kd_dtype of H, W, H_T, W_T: KD_BF16, or KD_F32 */
  int32_t val_dtype;    /* kd_dtype of val: KD_BF16 (with bf16 x) or KD_F32 (with f32 x) */
  int32_t dh_dtype;     /* kd_dtype of dH: KD_F32 or KD_BF16 (dW is always float32) */
  int32_t chunk_tokens; /* tokens per chunk; 0 = library default. Rounded up to 256. */
} kd_problem;

/* Workspace bytes that `op` needs for problem `p` (independent of the data).
 * The workspace grows with the chunk size, not with N, except for O(N) terms
 * of a few bytes per token. Returns KD_OK and writes *bytes, or an argument error. */
kd_status kd_workspace_size(kd_op op, const kd_problem* p, size_t* bytes);

/* Offline teacher cache ([abs]; [wiki] "핵심 아이디어 1", "사전 계산 파이프라인"):
 * S = H_T W_T^T evaluated tile by tile with bf16 (or f32) MFMA and float32
 * accumulation (kept in the workspace rounded to bf16, beside each row's two
 * largest float32 logits per 256-column tile), then a per-row top-K. Every logit
 * within a rigorous float32 error bound of the K-th value (widened by the bf16
 * rounding of the kept logits) is re-scored in float64: the products of bf16 (or f32) inputs are exact in float64
 * and are summed in a fixed order, each addition rounded to float64. Rows are
 * ranked by that float64 score, descending, equal scores putting the smaller index
 * first. So the chosen set and order are those of the exact logits wherever the
 * exact logits of two candidates differ by more than the float64 summation error
 * (at most about d 2^-53 sum_j |h_j w_j|); closer than that, the float64 scores
 * decide (and may tie).
 *   h_t   [N, d] x_dtype          w_t [V, d] x_dtype
 *   idx_out [N, K] int32          val_out [N, K] val_dtype: the float64 score rounded
 *                                 once (nearest, ties to even) to bf16 / f32.
 * A row with more than 6,144 logits within the error bound of its K-th value (a
 * massive near-tie, e.g. thousands of identical teacher rows at the top) exceeds
 * the candidate buffer: its idx are written as -1 and its val as NaN, and with
 * KD_CHECK=1 the call synchronises and returns KD_ERR_TOPK_OVERFLOW.
 * tau and dh_dtype are ignored. */
kd_status kd_topk_cache_build(const kd_problem* p, const void* h_t, const void* w_t,
                              int32_t* idx_out, void* val_out,
                              void* ws, size_t ws_bytes, void* stream);

/* Forward of the fused chunked KL ([mv] "Fused chunked KL"; [wiki] "표준 KD의 손실 함수").
 * Student logits are computed tile by tile (tokens x vocabulary) with MFMA; each
 * tile is folded into a per-row online log-sum-exp and the cached entries are
 * gathered from it; nothing of size N x V is stored.
 *   h [N, d], w [V, d] x_dtype;  idx [N, K] int32;  val [N, K] val_dtype
 *   loss_out   device float scalar: the mean KL over the N rows (0 when N = 0)
 *   lse_out    [N] float: per-row log-sum-exp (the input of the backward call)
 *   kl_rows_out[N] float per-row KL, or NULL. */
kd_status kd_chunked_kl_fwd(const kd_problem* p, const void* h, const void* w,
                            const int32_t* idx, const void* val,
                            float* loss_out, float* lse_out, float* kl_rows_out,
                            void* ws, size_t ws_bytes, void* stream);

/* Backward of the fused chunked KL ([mv] "Fused chunked KL": the backward pass
 * recomputes every chunk's logits). For each token chunk: recompute the logit
 * tiles, form dZ in bf16 (f32 for f32 inputs) in a chunk-sized buffer, then
 * dH = dZ W and dW += dZ^T H with MFMA; dW is accumulated in float32 in tiles
 * that each workgroup owns (no atomics).
 *   lse        [N] float from kd_chunked_kl_fwd on the same inputs
 *   grad_loss  device float scalar g (d loss_total / d loss), or NULL for g = 1
 *   dh_out     [N, d] dh_dtype (overwritten)
 *   dw_out     [V, d] float32  (overwritten; zero when N = 0) */
kd_status kd_chunked_kl_bwd(const kd_problem* p, const void* h, const void* w,
                            const int32_t* idx, const void* val,
                            const float* lse, const float* grad_loss,
                            void* dh_out, float* dw_out,
                            void* ws, size_t ws_bytes, void* stream);

/* ---- Loss variants: a padding mask and a hard-label cross-entropy mix.
 * The paper's abstract ([abs]) reports ablations of the loss design and of
 * sequence packing without defining them. These calls give the plain reading of
 * both in next-token training, on top of the KL above (a = ce_weight, y = labels):
 *   C       = { i : y[i] != ignore_index }   rows that count (every row when labels is NULL)
 *   CE[i]   = lse[i] - z[i, y[i]]            cross-entropy with the hard label
 *   l[i]    = (1 - a) KL[i] + a CE[i] for i in C, 0 for the other rows
 *   loss    = (1/|C|) sum_i l[i]             (0 when no row counts)
 *   dZ[i,v] = (g/|C|) (exp(z[i,v] - lse[i]) - (1 - a) sum_{k: idx[i,k]=v} p[i,k] - a [v = y[i]])
 *             for i in C; dZ[i,:] = 0 for the other rows
 * An ignored row's cache entries (idx, val) are not read, so padding may hold
 * anything there; its lse is still computed. With a = 0 the labels only mask.
 * With a > 0, a label outside [0, V) other than ignore_index makes its row's
 * term NaN (KD_CHECK=1: KD_ERR_IDX_OUT_OF_RANGE), like a cached index.
 *
 * student = KD_STUDENT_RENORM is the other loss-design reading: the student's
 * softmax over the row's K cached entries only, like the teacher's (a = 0 only):
 *   lseK[i] = log sum_k exp(z[i, idx[i,k]])          (every cached entry its own atom)
 *   KL[i]   = sum_k p[i,k] (log p[i,k] - z[i, idx[i,k]] + lseK[i]),  loss = mean over C
 *   dZ[i,v] = (g/|C|) sum_{k: idx[i,k]=v} (exp(z[i, idx[i,k]] - lseK[i]) - p[i,k])  for i in C
 * dZ is zero off the cached entries, so the logits are formed at the cached entries
 * only (no vocabulary-wide product in the forward; dH gathers W rows).  lse_out
 * receives lseK (NaN on ignored rows), and the backward takes it as `lse`.
 * KD_ERR_BAD_OPTION: student outside kd_student, or KD_STUDENT_RENORM with a > 0. */
typedef enum { KD_STUDENT_FULL = 0, KD_STUDENT_RENORM = 1 } kd_student;

typedef struct {
  const int32_t* labels;  /* [N] int32 DEVICE array (4-byte aligned), or NULL */
  int32_t ignore_index;   /* label value of a row left out (e.g. -100 for padding) */
  float ce_weight;        /* a in [0, 1]; > 0 needs labels */
  int32_t student;        /* kd_student: KD_STUDENT_FULL (0, the loss above) or KD_STUDENT_RENORM */
} kd_loss_opts;

/* kd_chunked_kl_fwd with loss options (NULL = kd_chunked_kl_fwd). rows_out [N]
 * (or NULL) receives l[i]; loss_out the mean over the counted rows.
 * KD_ERR_BAD_OPTION: ce_weight not finite or outside [0, 1], or > 0 without labels.
 * Workspace: kd_workspace_size(KD_OP_KL_FWD, ...), the same as the plain call. */
kd_status kd_chunked_kl_fwd_ex(const kd_problem* p, const kd_loss_opts* opts, const void* h, const void* w,
                               const int32_t* idx, const void* val,
                               float* loss_out, float* lse_out, float* rows_out,
                               void* ws, size_t ws_bytes, void* stream);

/* kd_chunked_kl_bwd with loss options (NULL = kd_chunked_kl_bwd); `opts` must
 * match the forward call that produced `lse`. dH rows of ignored tokens are 0.
 * Workspace: kd_workspace_size(KD_OP_KL_BWD, ...), the same as the plain call. */
kd_status kd_chunked_kl_bwd_ex(const kd_problem* p, const kd_loss_opts* opts, const void* h, const void* w,
                               const int32_t* idx, const void* val,
                               const float* lse, const float* grad_loss,
                               void* dh_out, float* dw_out,
                               void* ws, size_t ws_bytes, void* stream);

/* ---- Allocation-free forward, for callers that cannot allocate memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * kd_chunked_kl_fwd_ex (opts may be NULL for the plain loss) whose workspace is a
 * fixed 64 MiB scratch array inside the library (a device global, one per device,
 * held from module load until the process ends) instead of a caller's buffer.  It
 * calls no allocator.  Results are bitwise those of kd_chunked_kl_fwd_ex: the
 * forward's results do not depend on the chunk.
 *   - Chunk: p->chunk_tokens if > 0, else the largest multiple of 256 tokens up to
 *     the library default whose workspace fits 64 MiB.  The workspace is
 *     kd_workspace_size(KD_OP_KL_FWD, ...) at that chunk: about 4.9 KB per chunk
 *     token at V = 128,256, K = 100 (a 13,824-token chunk), plus 0.5 byte per token
 *     of N.  KD_ERR_SCRATCH_TOO_SMALL when the given chunk, or every chunk down to
 *     256 tokens, needs more than 64 MiB (large V, large K or very large N).
 *   - Every call on one device uses that device's single scratch array, and a call
 *     leaves its contents behind.  Calls that overlap in time on one device (on
 *     different streams or from different host threads without ordering) race on
 *     it: order them on one stream, or synchronise between them.
 *   - The first call on a device looks up that device's scratch address (with the
 *     device current); later calls reuse it.  Other errors as kd_chunked_kl_fwd_ex. */
kd_status kd_chunked_kl_fwd_noalloc(const kd_problem* p, const kd_loss_opts* opts, const void* h, const void* w,
                                    const int32_t* idx, const void* val,
                                    float* loss_out, float* lse_out, float* rows_out, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* kd_status_string(kd_status s);

/* ---- Measurement hooks (not part of the loss; for benchmarks and profiling).
 * Between kd_profile_begin() and kd_profile_end(), every kernel launch made by the
 * calls above is bracketed by a pair of HIP events recorded on the call's stream.
 * kd_profile_end() waits for those events, aggregates them per kernel kind and
 * disables the hooks. Not thread-safe: one profiling session per process. */
typedef struct {
  char name[32];          /* kernel kind, e.g. "gemm_kl_fwd", "gemm_dz", "bucket" */
  int64_t launches;       /* launches in the session */
  double total_ms;        /* sum of event-measured durations */
  double flops;           /* algorithmic FLOPs of all launches (GEMMs: 2*rows*cols*K; else 0) */
  double bytes;           /* algorithmic HBM bytes of all launches (operands once, outputs once) */
} kd_kernel_stat;

/* Starts a session (discarding any previous one). */
kd_status kd_profile_begin(void);

/* Ends the session; writes up to `max` entries to `out` and the number of kernel
 * kinds seen to *n. Returns KD_ERR_LAUNCH if an event could not be created, recorded
 * or read (the launches it would have timed are left out of the entries). */
kd_status kd_profile_end(kd_kernel_stat* out, int max, int* n);

/* Library ABI version (major * 100 + minor): 102 adds kd_loss_opts.student. */
int kd_version(void);

#ifdef __cplusplus
}
#endif
#endif /* KDKL_H */
