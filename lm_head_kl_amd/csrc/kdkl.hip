// Host side of the kdkl C ABI: argument validation, workspace planning and the
// launch sequences of the teacher-cache build and the chunked KL forward/backward.
// The declarations and the contract of every entry point are in include/kdkl.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <atomic>
#include <mutex>
#include <numeric>
#include <cstring>
#include <string>
#include <type_traits>
#include <vector>
#include <algorithm>

#include "kdkl.h"
#include "kd_aux.hpp"
#include "kd_gemm.hpp"

using namespace kd;

namespace {

// 2^21 - 64: the 256-row tiles of the operands with V-element rows (dZ, W^T; 4-byte
// elements in the float32 path, padded by pad_ld) then span less than 2^31 bytes, so
// the loads' out-of-range offset 0x80000000 stays past every tile's descriptor (the
// 32-bit offset check in validate() below).  8,192 vocabulary tiles.
constexpr int64_t kMaxVocab = 2097088;
constexpr int kMaxK = 65535;             // k fits the 16-bit field of a bucket entry
constexpr int kMaxKTopk = 4096;          // selection candidates are held in LDS
constexpr int64_t kDefaultChunkKL = 16384;
constexpr int64_t kDefaultChunkTopk = 8192;
constexpr int kGroup = 4;   // X tiles walked per Y tile (measured best for all four GEMM shapes)
constexpr int kMinTiles = 256;   // workgroups that fill MI355X's compute units (one 256 x 256 tile each)
constexpr int kMaxSplits = 16;
// Up to this many tokens the backward reads W K-major in the dH product instead of
// making W^T.  Both costs scale with V d: measured at V=128,256, d=4,096 the copy
// takes 0.83 ms and the transposing read adds ~0.09 ms per 1,024 tokens to dH, so
// the copy only pays from ~9K tokens (4K tokens: step 14.97 -> 14.28 ms; 16K: 53.7
// -> 56.1 ms, hence the bound).
constexpr int64_t kWkmMaxTokens = 4096;

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
// Leading dimension of an internal buffer: a multiple of 64 elements whose byte
// stride is not a multiple of 4 KiB (power-of-two strides put all rows of a tile
// on the same L2 channels; measured 25% slower on the dW GEMM).
inline int64_t pad_ld(int64_t n, int64_t esz) {
  int64_t l = round_up(n, 64);
  if ((l * esz) % 4096 == 0) l += 64;
  return l;
}

struct Plan {
  int64_t N, d, V;
  int K;
  float tau;
  kd_dtype xdt, vdt, dhdt;
  int64_t esz;      // bytes per H/W element
  int64_t Nc;       // tokens per chunk (multiple of 256)
  int64_t V_pad;    // vocabulary rounded up to 64 (K-extent of dH)
  int64_t ld_v;     // leading dimension of dZ, W^T and the teacher logits (>= V_pad)
  int64_t ld_t;     // leading dimension of dZ^T and H^T (>= Nc)
  int n_ty;         // 256-wide vocabulary tiles
};

// Workspace regions, each 256-byte aligned, in bytes from the workspace start.
struct Layout {
  size_t entries, offsets, zg, partials, block_sums, flags;       // forward
  size_t wt, ht, dz, dzt, dhp, lse_eff, pw, ew;                   // backward
  size_t count;                                                   // counted rows (+ gradient scale)
  size_t s, bmax, wmax, overflow, tops, todo;                     // cache build
  size_t total;
};

bool mul_ok(int64_t a, int64_t b, int64_t lim = INT64_MAX / 4) { return a == 0 || b <= lim / a; }

// The int a C caller stored in an enum argument, read without loading it as the
// enum type (whose C++ value range may not hold it).
template <typename E> int enum_bits(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

kd_status validate(kd_op op, const kd_problem* p, Plan* pl) {
  if (!p) return KD_ERR_NULL_POINTER;
  if (p->x_dtype != KD_F32 && p->x_dtype != KD_BF16) return KD_ERR_BAD_DTYPE;
  if (p->val_dtype != KD_F32 && p->val_dtype != KD_BF16) return KD_ERR_BAD_DTYPE;
  if (p->x_dtype == KD_BF16 && p->val_dtype != KD_BF16) return KD_ERR_BAD_DTYPE;
  if (p->x_dtype == KD_F32 && p->val_dtype != KD_F32) return KD_ERR_BAD_DTYPE;
  if (op == KD_OP_KL_BWD && p->dh_dtype != KD_F32 && p->dh_dtype != KD_BF16) return KD_ERR_BAD_DTYPE;
  if (p->n_tokens < 0 || p->d_model < 8 || (p->d_model % 8) != 0) return KD_ERR_BAD_SHAPE;
  if (p->vocab < 1 || p->vocab > kMaxVocab) return KD_ERR_BAD_SHAPE;
  if (p->k < 1 || p->k > kMaxK || p->k > p->vocab) return KD_ERR_BAD_SHAPE;
  if (op == KD_OP_TOPK_BUILD && p->k > kMaxKTopk) return KD_ERR_BAD_SHAPE;
  if (p->chunk_tokens < 0) return KD_ERR_BAD_SHAPE;
  if (p->d_model > (1 << 20) || p->n_tokens > (int64_t(1) << 31) - 256) return KD_ERR_BAD_SHAPE;
  if (!mul_ok(p->n_tokens, p->k) || !mul_ok(p->n_tokens, p->d_model) || !mul_ok(p->vocab, p->d_model))
    return KD_ERR_BAD_SHAPE;
  if (op != KD_OP_TOPK_BUILD && !(std::isfinite(p->tau) && p->tau > 0.f)) return KD_ERR_BAD_TAU;
  pl->N = p->n_tokens;
  pl->d = p->d_model;
  pl->V = p->vocab;
  pl->K = p->k;
  pl->tau = p->tau;
  pl->xdt = (kd_dtype)p->x_dtype;
  pl->vdt = (kd_dtype)p->val_dtype;
  pl->dhdt = (kd_dtype)p->dh_dtype;
  pl->esz = p->x_dtype == KD_BF16 ? 2 : 4;
  const int64_t def = op == KD_OP_TOPK_BUILD ? kDefaultChunkTopk : kDefaultChunkKL;
  int64_t c = p->chunk_tokens > 0 ? p->chunk_tokens : def;
  c = round_up(c, BX);
  c = std::min<int64_t>(c, round_up(std::max<int64_t>(pl->N, 1), BX));
  pl->Nc = c;
  pl->V_pad = round_up(pl->V, 64);
  pl->ld_v = pad_ld(pl->V_pad, op == KD_OP_TOPK_BUILD ? 2 : pl->esz);
  pl->ld_t = pad_ld(pl->Nc, pl->esz);
  pl->n_ty = (int)cdiv(pl->V, BY);
  // 32-bit byte offsets inside one 256-row tile of every GEMM operand
  if (!mul_ok(BX * 4, std::max<int64_t>(std::max<int64_t>(pl->ld_v, pl->ld_t), pl->d), INT32_MAX))
    return KD_ERR_BAD_SHAPE;
  return KD_OK;
}

// Split-K factor of the dH product for a chunk of nr tokens: when its output tiles
// cannot fill the device's compute units, each tile's V range is cut into parts
// (at least 8 K stages each) summed afterwards in a fixed order.
int dh_splits(const Plan& pl, int64_t nr) {
  const int64_t tiles = cdiv(nr, BX) * cdiv(pl.d, BY);
  if (nr <= 0 || tiles >= kMinTiles) return 1;
  const int64_t stages = cdiv(pl.V_pad, MainCfg::KB / pl.esz);
  int64_t s = std::min<int64_t>(kMaxSplits, kMinTiles / tiles);
  s = std::min<int64_t>(s, std::max<int64_t>(1, stages / 8));
  return (int)std::max<int64_t>(1, s);
}

// dW's output tiles in whole rounds of kMinTiles workgroups, and the rest.  When the
// tiles past the last whole round would leave most compute units idle for a final
// round (V = 128,256, d = 4,096: 8,016 tiles, 31 rounds and 80 tiles), those tiles are
// computed as S split-K partials (at least 8 K stages each) summed afterwards in a
// fixed order, so the final round takes about 1/S of a tile's time.  Returns S (1: one
// plain launch) and the X tiles (vocabulary tiles) of the whole rounds.
int dw_splits(const Plan& pl, int64_t nr64, int64_t* tx_main) {
  const int64_t n_tx = cdiv(pl.V, BX), n_ty = cdiv(pl.d, BY);
  const int64_t unit = kMinTiles / std::gcd<int64_t>(kMinTiles, n_ty);   // X tiles per whole rounds
  const int64_t txm = n_tx / unit * unit;
  const int64_t rem = (n_tx - txm) * n_ty;
  *tx_main = txm;
  if (txm == 0 || rem == 0) return 1;
  const int64_t stages = cdiv(nr64, MainCfg::KB / pl.esz);
  int64_t s = std::min<int64_t>(kMaxSplits, kMinTiles / rem);
  s = std::min<int64_t>(s, stages / 8);
  return (int)std::max<int64_t>(1, s);
}

size_t layout(kd_op op, const Plan& pl, Layout* L) {
  size_t cur = 0;
  auto take = [&](size_t bytes) {
    const size_t at = cur;
    cur = (size_t)round_up((int64_t)(cur + bytes), 256);
    return at;
  };
  std::memset(L, 0, sizeof(*L));
  const int64_t n_tx = pl.Nc / BX;
  if (op == KD_OP_KL_FWD) {
    // one more entry per row for a label (cross-entropy mix)
    L->entries = take(sizeof(uint32_t) * pl.Nc * (pl.K + 1));
    L->offsets = take(sizeof(int) * n_tx * (pl.n_ty + 1));
    L->zg = take(sizeof(float) * pl.Nc * (pl.K + 1));
    L->partials = take(sizeof(float2) * pl.n_ty * pl.Nc);
    L->block_sums = take(sizeof(double) * (size_t)std::max<int64_t>(1, cdiv(pl.N, RB_ROWS)));
    L->flags = take(sizeof(int) * 4);
    L->count = take(16);
  } else if (op == KD_OP_KL_BWD) {
    if (!(pl.xdt == KD_BF16 && pl.N <= kWkmMaxTokens)) L->wt = take((size_t)(pl.esz * pl.d * pl.ld_v));
    L->ht = take((size_t)(pl.esz * pl.d * pl.ld_t));
    L->dz = take((size_t)(pl.esz * pl.Nc * pl.ld_v));
    // bf16 reads dZ K-major in the dW product; float32 (no transposing LDS read)
    // keeps a transposed copy
    if (pl.xdt == KD_F32) L->dzt = take((size_t)(pl.esz * pl.V_pad * pl.ld_t));
    // split-K partials of dH and of dW's last tiles (one region: each product's partials
    // are summed before the next product starts), for the full chunks and the last one
    const int64_t last = pl.N % pl.Nc;
    const int64_t full = pl.N >= pl.Nc ? pl.Nc : 0;
    int64_t part = 0;
    for (int64_t nr : {full, last}) {
      if (nr <= 0) continue;
      if (dh_splits(pl, nr) > 1) part = std::max<int64_t>(part, dh_splits(pl, nr) * nr * pl.d);
      int64_t txm = 0;
      const int sw = dw_splits(pl, round_up(nr, 64), &txm);
      if (sw > 1) part = std::max<int64_t>(part, sw * (pl.V - txm * BX) * pl.d);
    }
    if (part) L->dhp = take((size_t)(4 * part));
    L->lse_eff = take(sizeof(float) * (size_t)pl.Nc);
    L->count = take(16);
    // the chunk's cached entries (and labels) bucketed per tile, with their weights
    L->entries = take(sizeof(uint32_t) * pl.Nc * (pl.K + 1));
    L->offsets = take(sizeof(int) * n_tx * (pl.n_ty + 1));
    L->pw = take(sizeof(float) * pl.Nc * (pl.K + 1));
    L->ew = take(sizeof(float) * pl.Nc * (pl.K + 1));
    L->flags = take(sizeof(int) * 4);
  } else {
    L->s = take(sizeof(bf16_t) * (size_t)(pl.Nc * pl.ld_v));
    L->bmax = take(sizeof(double) * 1024);
    L->wmax = take(sizeof(double));
    L->overflow = take(sizeof(int) * 4);
    L->tops = take(sizeof(float) * 2 * (size_t)(pl.n_ty * pl.Nc));
    L->todo = take(sizeof(int) * (size_t)pl.Nc);
  }
  L->total = cur;
  return cur;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }

// Per-device answer cached for later calls.  Calls may come from several threads at
// once: the caches are atomics (every thread that fills one stores the same value).
kd_status check_device() {
  static std::atomic<int> state[256];   // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KD_ERR_NO_DEVICE;
  const int known = dev < 256 ? state[dev].load(std::memory_order_relaxed) : 0;
  if (known) return known == 1 ? KD_OK : KD_ERR_UNSUPPORTED_ARCH;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return KD_ERR_NO_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 256) state[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? KD_OK : KD_ERR_UNSUPPORTED_ARCH;
}

bool debug_checks() {
  static std::atomic<int> v{-1};
  int c = v.load(std::memory_order_relaxed);
  if (c < 0) {
    const char* e = std::getenv("KD_CHECK");
    c = (e && e[0] == '1') ? 1 : 0;
    v.store(c, std::memory_order_relaxed);
  }
  return c == 1;
}

inline kd_status launched() { return hipGetLastError() == hipSuccess ? KD_OK : KD_ERR_LAUNCH; }

// ---- measurement hooks (kd_profile_begin / kd_profile_end)
struct ProfRec {
  int kind;
  hipEvent_t a, b;
  double flops, bytes;
};
struct Prof {
  bool on = false;
  bool failed = false;   // an event could not be created or recorded in this session
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  std::vector<std::string> kinds;
};
Prof& prof() {
  static Prof p;
  return p;
}
hipEvent_t prof_event() {
  Prof& p = prof();
  if (!p.pool.empty()) {
    hipEvent_t e = p.pool.back();
    p.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
int prof_kind(const char* name) {
  Prof& p = prof();
  for (size_t i = 0; i < p.kinds.size(); ++i)
    if (p.kinds[i] == name) return (int)i;
  p.kinds.emplace_back(name);
  return (int)p.kinds.size() - 1;
}

// Launch `f` (which enqueues one kernel on `st`); bracket it with events when profiling.
template <typename F>
kd_status launch(const char* kind, double flops, double bytes, hipStream_t st, F&& f) {
  Prof& p = prof();
  hipEvent_t a = nullptr, b = nullptr;
  bool timed = false;
  if (p.on) {
    a = prof_event();
    b = prof_event();
    timed = a && b && hipEventRecord(a, st) == hipSuccess;
  }
  f();
  const kd_status s = launched();
  if (p.on) {
    timed = timed && hipEventRecord(b, st) == hipSuccess;
    if (timed) {
      p.recs.push_back(ProfRec{prof_kind(kind), a, b, flops, bytes});
    } else {
      // the launch stays untimed; its events go back to the pool and the session reports the failure
      p.failed = true;
      if (a) p.pool.push_back(a);
      if (b) p.pool.push_back(b);
    }
  }
  return s;
}

#define KD_TRY(x)                 \
  do {                            \
    const kd_status _s = (x);     \
    if (_s != KD_OK) return _s;   \
  } while (0)

GemmArgs gemm_args(const void* X, int64_t ldx, int nx, const void* Y, int64_t ldy, int ny, int k) {
  GemmArgs g;
  std::memset(&g, 0, sizeof(g));
  g.X = X;
  g.ldx = ldx;
  g.nx = nx;
  g.Y = Y;
  g.ldy = ldy;
  g.ny = ny;
  g.k = k;
  g.n_tx = (int)cdiv(nx, BX);
  g.n_ty = (int)cdiv(ny, BY);
  g.group = kGroup;
  g.splits = 1;
  return g;
}

template <typename T, int EPI, int XKM = 0, int YKM = 0>
kd_status run_gemm(const char* kind, const GemmArgs& g, int64_t out_bytes, hipStream_t st) {
  if (g.nx <= 0 || g.ny <= 0) return KD_OK;
  const unsigned blocks = (unsigned)(g.n_tx * g.n_ty * g.splits);
  const double flops = 2.0 * g.nx * (double)g.ny * g.k;
  const double bytes = (double)sizeof(T) * ((double)g.nx + g.ny) * g.k + (double)out_bytes;
  return launch(kind, flops, bytes, st, [&] {
    hipLaunchKernelGGL((gemm_kernel<MainCfg, T, EPI, XKM, YKM>), dim3(blocks), dim3(MainCfg::NTHREADS), 0, st, g);
  });
}

kd_status zero_words(void* p, int64_t n_words, hipStream_t st) {
  const unsigned blocks = (unsigned)std::min<int64_t>(1024, std::max<int64_t>(1, cdiv(n_words, 256)));
  return launch("fill", 0.0, 4.0 * n_words, st, [&] {
    hipLaunchKernelGGL(fill_f32_kernel, dim3(blocks), dim3(256), 0, st, (float*)p, n_words, 0.0f);
  });
}

// Loss variants (kd_loss_opts): labels (NULL = every row counts, no mix), the
// label that marks an ignored row, and the cross-entropy weight.
struct Opts {
  const int32_t* labels = nullptr;
  int ignore = 0;
  float alpha = 0.f;
  bool renorm = false;   // student softmax over the row's K cached entries only
};

// Counted rows (double) and, with `scale`, g / count (float) into ws + L.count.
kd_status count_rows(const Plan& pl, const Layout& L, const Opts& o, const float* grad, bool scale, char* ws,
                     hipStream_t st) {
  double* cnt = (double*)(ws + L.count);
  float* gs = scale ? (float*)(ws + L.count + 8) : nullptr;
  return launch("count", 0.0, 4.0 * pl.N, st, [&] {
    hipLaunchKernelGGL(count_rows_kernel, dim3(1), dim3(1024), 0, st, o.labels, pl.N, o.ignore, grad, cnt, gs);
  });
}

// Bucketed cache entries of one chunk (bucket_kernel): one block per 256-token tile,
// as many waves (up to 16) as leave the per-wave tables of all waves in 64 KB of LDS
// with the kernel's 1 KB of labels and 256 bytes of scan scratch: counters, and with
// `ordered` (the backward's weighted entries, whose order inside each bucket is
// fixed) 64-bit lane masks; fewer waves mean more rows per wave.  A vocabulary too
// large for the mask table at one wave orders its buckets with ballots instead.
kd_status run_bucket(const Plan& pl, const int32_t* idx_c, const int32_t* lab_c, const Opts& o, int add_label, int nr,
                     int kz, bool ordered, const float* pw, uint32_t* entries, float* ew, int* offsets, int* flags,
                     hipStream_t st) {
  const int64_t budget = 16384 - 64 - 1 - BX;   // ints (64 of scan scratch, 1 of mask alignment)
  int mode = ordered ? 1 : 0;
  if (mode == 1 && 3 * (int64_t)pl.n_ty > budget) mode = 2;
  const int tables = mode == 1 ? 3 : 1;
  int nw = 16;
  while (nw > 1 && (int64_t)tables * nw * pl.n_ty > budget) nw >>= 1;
  const size_t lds = sizeof(int) * ((size_t)tables * nw * pl.n_ty + 64 + 1);
  const int n_tx = (int)cdiv(nr, BX);
  return launch(ordered ? "bucket_ordered" : "bucket", 0.0, 12.0 * nr * kz, st, [&] {
    hipLaunchKernelGGL(bucket_kernel, dim3(n_tx), dim3(64 * nw), lds, st, idx_c, lab_c, o.ignore, add_label, nr,
                       pl.K, kz, (int)pl.V, pl.n_ty, mode, pw, entries, ew, offsets, flags);
  });
}

// Forward with the student renormalised over the cached entries: the logits at the
// cached entries (gather_dot), then per row the normaliser over them, the teacher
// softmax and the KL; the loss as in the full forward.
template <typename T>
kd_status fwd_renorm_impl(const Plan& pl, const Layout& L, const void* h, const void* w, const int32_t* idx,
                          const void* val, float* loss, float* lse, float* kl_rows, char* ws, hipStream_t st,
                          const Opts& o) {
  float* zg = (float*)(ws + L.zg);
  double* bsums = (double*)(ws + L.block_sums);
  int* flags = (int*)(ws + L.flags);
  const bool check = debug_checks();
  if (check) KD_TRY(zero_words(flags, 4, st));
  const float inv_tau = 1.0f / pl.tau;
  const int64_t es = (int64_t)sizeof(T);
  if (o.labels) KD_TRY(count_rows(pl, L, o, nullptr, false, ws, st));
  for (int64_t r0 = 0; r0 < pl.N; r0 += pl.Nc) {
    const int nr = (int)std::min<int64_t>(pl.Nc, pl.N - r0);
    const int32_t* idx_c = idx + r0 * pl.K;
    const int32_t* lab_c = o.labels ? o.labels + r0 : nullptr;
    KD_TRY(launch("gather_dot", 2.0 * nr * pl.K * (double)pl.d, (double)nr * pl.K * (es * pl.d + 8.0), st, [&] {
      hipLaunchKernelGGL(gather_dot_kernel<T>, dim3(nr), dim3(256), 0, st, (const T*)h + r0 * pl.d, (const T*)w,
                         idx_c, nr, pl.K, (int)pl.d, (int)pl.V, lab_c, o.ignore, zg, flags);
    }));
    const int nb = (int)cdiv(nr, RB_ROWS);
    KD_TRY(launch("renorm_merge", 0.0, (double)nr * pl.K * (4.0 + (pl.vdt == KD_BF16 ? 2 : 4)), st, [&] {
      if (pl.vdt == KD_BF16)
        hipLaunchKernelGGL(renorm_merge_kernel<bf16_t>, dim3(nb), dim3(256), 0, st, zg,
                           (const bf16_t*)val + r0 * pl.K, nr, pl.K, inv_tau, lab_c, o.ignore, lse + r0,
                           kl_rows ? kl_rows + r0 : nullptr, bsums + r0 / RB_ROWS);
      else
        hipLaunchKernelGGL(renorm_merge_kernel<float>, dim3(nb), dim3(256), 0, st, zg, (const float*)val + r0 * pl.K,
                           nr, pl.K, inv_tau, lab_c, o.ignore, lse + r0, kl_rows ? kl_rows + r0 : nullptr,
                           bsums + r0 / RB_ROWS);
    }));
  }
  const int nb_all = (int)cdiv(pl.N, RB_ROWS);
  KD_TRY(launch("loss", 0.0, 8.0 * nb_all, st, [&] {
    hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(256), 0, st, bsums, nb_all, pl.N > 0 ? 1.0 / (double)pl.N : 0.0,
                       o.labels ? (const double*)(ws + L.count) : nullptr, loss);
  }));
  if (check) {
    int bad = 0;
    if (hipMemcpyAsync(&bad, flags, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return KD_ERR_LAUNCH;
    if (hipStreamSynchronize(st) != hipSuccess) return KD_ERR_LAUNCH;
    if (bad) return KD_ERR_IDX_OUT_OF_RANGE;
  }
  return KD_OK;
}

template <typename T>
kd_status fwd_impl(const Plan& pl, const Layout& L, const void* h, const void* w, const int32_t* idx,
                   const void* val, float* loss, float* lse, float* kl_rows, char* ws, hipStream_t st,
                   const Opts& o) {
  if (o.renorm) return fwd_renorm_impl<T>(pl, L, h, w, idx, val, loss, lse, kl_rows, ws, st, o);
  uint32_t* entries = (uint32_t*)(ws + L.entries);
  int* offsets = (int*)(ws + L.offsets);
  float* zg = (float*)(ws + L.zg);
  float2* partials = (float2*)(ws + L.partials);
  double* bsums = (double*)(ws + L.block_sums);
  int* flags = (int*)(ws + L.flags);
  const bool check = debug_checks();
  if (check) KD_TRY(zero_words(flags, 4, st));
  const float inv_tau = 1.0f / pl.tau;
  const int vsz = pl.vdt == KD_BF16 ? 2 : 4;
  const int add_label = o.alpha > 0.f ? 1 : 0;
  const int kz = pl.K + add_label;   // gathered logits per row: the K entries, then the label's
  if (o.labels) KD_TRY(count_rows(pl, L, o, nullptr, false, ws, st));
  for (int64_t r0 = 0; r0 < pl.N; r0 += pl.Nc) {
    const int nr = (int)std::min<int64_t>(pl.Nc, pl.N - r0);
    const int32_t* idx_c = idx + r0 * pl.K;
    const int32_t* lab_c = o.labels ? o.labels + r0 : nullptr;
    KD_TRY(run_bucket(pl, idx_c, lab_c, o, add_label, nr, kz, false, nullptr, entries, nullptr, offsets, flags, st));
    GemmArgs g = gemm_args((const T*)h + r0 * pl.d, pl.d, nr, w, pl.d, (int)pl.V, (int)pl.d);
    g.entries = entries;
    g.offsets = offsets;
    g.kc = kz;
    g.zg = zg;
    g.partials = partials;
    g.ld_part = pl.Nc;
    KD_TRY((run_gemm<T, EPI_KL_FWD>("gemm_kl_fwd", g, (int64_t)8 * nr * pl.n_ty, st)));
    const int nb = (int)cdiv(nr, RB_ROWS);
    const double mbytes = (double)nr * (8.0 * pl.n_ty + pl.K * (8.0 + vsz) + 8.0);
    KD_TRY(launch("merge", 0.0, mbytes, st, [&] {
      if (pl.vdt == KD_BF16)
        hipLaunchKernelGGL(merge_kernel<bf16_t>, dim3(nb), dim3(256), 0, st, partials, (int64_t)pl.Nc, pl.n_ty,
                           idx_c, (const bf16_t*)val + r0 * pl.K, zg, nr, pl.K, kz, (int)pl.V, inv_tau, lab_c,
                           o.ignore, o.alpha, lse + r0, kl_rows ? kl_rows + r0 : nullptr, bsums + r0 / RB_ROWS);
      else
        hipLaunchKernelGGL(merge_kernel<float>, dim3(nb), dim3(256), 0, st, partials, (int64_t)pl.Nc, pl.n_ty,
                           idx_c, (const float*)val + r0 * pl.K, zg, nr, pl.K, kz, (int)pl.V, inv_tau, lab_c,
                           o.ignore, o.alpha, lse + r0, kl_rows ? kl_rows + r0 : nullptr, bsums + r0 / RB_ROWS);
    }));
  }
  const int nb_all = (int)cdiv(pl.N, RB_ROWS);
  KD_TRY(launch("loss", 0.0, 8.0 * nb_all, st, [&] {
    hipLaunchKernelGGL(loss_kernel, dim3(1), dim3(256), 0, st, bsums, nb_all, pl.N > 0 ? 1.0 / (double)pl.N : 0.0,
                       o.labels ? (const double*)(ws + L.count) : nullptr, loss);
  }));
  if (check) {
    int bad = 0;
    if (hipMemcpyAsync(&bad, flags, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return KD_ERR_LAUNCH;
    if (hipStreamSynchronize(st) != hipSuccess) return KD_ERR_LAUNCH;
    if (bad) return KD_ERR_IDX_OUT_OF_RANGE;
  }
  return KD_OK;
}

template <typename T, int EPI>
kd_status run_dh(const GemmArgs& g, bool w_kmajor, int64_t out_bytes, hipStream_t st) {
  if constexpr (std::is_same<T, bf16_t>::value) {
    if (w_kmajor) return run_gemm<T, EPI, 0, 1>("gemm_dh", g, out_bytes, st);
  }
  return run_gemm<T, EPI>("gemm_dh", g, out_bytes, st);
}

// Backward with the student renormalised over the cached entries.  dZ is zero off
// each row's cached entries: per chunk the logits at the entries again (gather_dot),
// their gradient c = (g/N)(q - p), dH by a gather of W rows weighted by c, and dW by
// each vocabulary row's sum of c H[t] over its entries, in a fixed order.
template <typename T>
kd_status bwd_renorm_impl(const Plan& pl, const Layout& L, const void* h, const void* w, const int32_t* idx,
                          const void* val, const float* lse, const float* grad, void* dh, float* dw, char* ws,
                          hipStream_t st, const Opts& o) {
  float* zg = (float*)(ws + L.ew);
  float* cf = (float*)(ws + L.pw);
  uint32_t* entries = (uint32_t*)(ws + L.entries);
  int* offsets = (int*)(ws + L.offsets);
  int* flags = (int*)(ws + L.flags);
  float inv_n = 1.0f / (float)pl.N;
  const float inv_tau = 1.0f / pl.tau;
  const int64_t es = (int64_t)sizeof(T);
  if (o.labels) {
    KD_TRY(count_rows(pl, L, o, grad, true, ws, st));
    grad = (const float*)(ws + L.count + 8);
    inv_n = 1.0f;
  }
  for (int64_t r0 = 0; r0 < pl.N; r0 += pl.Nc) {
    const int nr = (int)std::min<int64_t>(pl.Nc, pl.N - r0);
    const T* hc = (const T*)h + r0 * pl.d;
    const int32_t* idx_c = idx + r0 * pl.K;
    const int32_t* lab_c = o.labels ? o.labels + r0 : nullptr;
    const int nb = (int)cdiv(nr, RB_ROWS);
    KD_TRY(launch("gather_dot", 2.0 * nr * pl.K * (double)pl.d, (double)nr * pl.K * (es * pl.d + 8.0), st, [&] {
      hipLaunchKernelGGL(gather_dot_kernel<T>, dim3(nr), dim3(256), 0, st, hc, (const T*)w, idx_c, nr, pl.K,
                         (int)pl.d, (int)pl.V, lab_c, o.ignore, zg, (int*)nullptr);
    }));
    KD_TRY(launch("renorm_coef", 0.0, (double)nr * pl.K * (8.0 + (pl.vdt == KD_BF16 ? 2 : 4)), st, [&] {
      if (pl.vdt == KD_BF16)
        hipLaunchKernelGGL(renorm_coef_kernel<bf16_t>, dim3(nb), dim3(256), 0, st, zg, (const bf16_t*)val + r0 * pl.K,
                           lse + r0, nr, pl.K, inv_tau, grad, inv_n, lab_c, o.ignore, cf);
      else
        hipLaunchKernelGGL(renorm_coef_kernel<float>, dim3(nb), dim3(256), 0, st, zg, (const float*)val + r0 * pl.K,
                           lse + r0, nr, pl.K, inv_tau, grad, inv_n, lab_c, o.ignore, cf);
    }));
    KD_TRY(launch("renorm_dh", 2.0 * nr * pl.K * (double)pl.d, (double)nr * pl.K * es * pl.d, st, [&] {
      if (pl.dhdt == KD_F32)
        hipLaunchKernelGGL((renorm_dh_kernel<T, float>), dim3(nr), dim3(256), 0, st, (const T*)w, idx_c, cf, nr,
                           pl.K, (int)pl.d, (int)pl.V, lab_c, o.ignore, (float*)dh + r0 * pl.d);
      else
        hipLaunchKernelGGL((renorm_dh_kernel<T, bf16_t>), dim3(nr), dim3(256), 0, st, (const T*)w, idx_c, cf, nr,
                           pl.K, (int)pl.d, (int)pl.V, lab_c, o.ignore, (bf16_t*)dh + r0 * pl.d);
    }));
    // dW: the entries with their gradients, bucketed per tile in a fixed order (the
    // gathered logits are no longer needed, so their buffer takes the weights), then
    // each vocabulary row's sum over its entries
    KD_TRY(run_bucket(pl, idx_c, lab_c, o, 0, nr, pl.K, true, cf, entries, zg, offsets, flags, st));
    KD_TRY(launch("renorm_dw", 2.0 * nr * pl.K * (double)pl.d, (double)nr * pl.K * es * pl.d + 4.0 * pl.V * pl.d, st,
                  [&] {
      hipLaunchKernelGGL(renorm_dw_kernel<T>, dim3((unsigned)pl.n_ty), dim3(RDW_WAVES * 64), 0, st, entries, zg, offsets,
                         (int)cdiv(nr, BX), pl.n_ty, pl.K, hc, (int)pl.d, (int)pl.V, r0 > 0 ? 1 : 0, dw);
    }));
  }
  return KD_OK;
}

template <typename T>
kd_status bwd_impl(const Plan& pl, const Layout& L, const void* h, const void* w, const int32_t* idx,
                   const void* val, const float* lse, const float* grad, void* dh, float* dw, char* ws,
                   hipStream_t st, const Opts& o) {
  if (pl.N == 0) return zero_words(dw, pl.V * pl.d, st);
  if (o.renorm) return bwd_renorm_impl<T>(pl, L, h, w, idx, val, lse, grad, dh, dw, ws, st, o);
  // W^T and H^T are cheap copies (W once, H per chunk).  dZ^T would cost a second
  // N x V write per chunk: bf16 reads dZ K-major in the dW product instead
  // (transposing LDS reads); float32 writes dZ^T from the dZ epilogue.
  constexpr bool kKm = std::is_same<T, bf16_t>::value;
  T* wt = (T*)(ws + L.wt);
  T* ht = (T*)(ws + L.ht);
  T* dz = (T*)(ws + L.dz);
  T* dzt = kKm ? nullptr : (T*)(ws + L.dzt);
  float inv_n = 1.0f / (float)pl.N;
  const float inv_tau = 1.0f / pl.tau;
  const int64_t es = (int64_t)sizeof(T);
  float* lse_eff = (float*)(ws + L.lse_eff);
  uint32_t* entries = (uint32_t*)(ws + L.entries);
  int* offsets = (int*)(ws + L.offsets);
  float* pw = (float*)(ws + L.pw);
  float* ew = (float*)(ws + L.ew);
  int* flags = (int*)(ws + L.flags);
  const int add_label = o.alpha > 0.f ? 1 : 0;
  const int kz = pl.K + add_label;   // weighted entries per row: the K cached ones, then the label
  if (o.labels) {
    // the scale g / (counted rows) is computed on the device and read in place of g
    KD_TRY(count_rows(pl, L, o, grad, true, ws, st));
    grad = (const float*)(ws + L.count + 8);
    inv_n = 1.0f;
  }
  const bool w_km = kKm && pl.N <= kWkmMaxTokens;
  if (!w_km) {
    // W^T [d][V_pad], zero past V
    KD_TRY(launch("transpose_w", 0.0, 2.0 * es * pl.V * pl.d, st, [&] {
      hipLaunchKernelGGL(transpose_pad_kernel<T>, dim3((unsigned)cdiv(pl.V_pad, 64), (unsigned)cdiv(pl.d, 64)),
                         dim3(256), 0, st, (const T*)w, pl.d, (int)pl.V, (int)pl.d, wt, pl.ld_v, (int)pl.V_pad);
    }));
  }
  for (int64_t r0 = 0; r0 < pl.N; r0 += pl.Nc) {
    const int nr = (int)std::min<int64_t>(pl.Nc, pl.N - r0);
    const int nr64 = (int)round_up(nr, 64);
    const T* hc = (const T*)h + r0 * pl.d;
    // H^T [d][Nc], zero past nr
    KD_TRY(launch("transpose_h", 0.0, 2.0 * es * nr * pl.d, st, [&] {
      hipLaunchKernelGGL(transpose_pad_kernel<T>, dim3((unsigned)cdiv(nr64, 64), (unsigned)cdiv(pl.d, 64)),
                         dim3(256), 0, st, hc, pl.d, nr, (int)pl.d, ht, pl.ld_t, nr64);
    }));
    // recompute logits, dZ = (g/N) softmax
    GemmArgs g = gemm_args(hc, pl.d, nr, w, pl.d, (int)pl.V, (int)pl.d);
    g.out = dz;
    g.ldo = pl.ld_v;
    g.out2 = dzt;
    g.ldo2 = pl.ld_t;
    g.out_rows = nr64;
    g.out_cols = (int)pl.V_pad;
    g.lse = lse + r0;
    g.grad = grad;
    g.inv_n = inv_n;
    if (o.labels) {
      KD_TRY(launch("mask_lse", 0.0, 12.0 * nr, st, [&] {
        hipLaunchKernelGGL(mask_lse_kernel, dim3((unsigned)cdiv(nr, 256)), dim3(256), 0, st, lse + r0,
                           o.labels + r0, nr, o.ignore, lse_eff);
      }));
      g.lse = lse_eff;
    }
    // the teacher's weight at every cached entry (and the label's), bucketed per
    // tile in a fixed order; the dZ epilogue subtracts them before its one rounding
    const int32_t* lab_c = o.labels ? o.labels + r0 : nullptr;
    const int nb = (int)cdiv(nr, RB_ROWS);
    KD_TRY(launch("teacher_weights", 0.0, (double)nr * (pl.K * (double)(pl.vdt == KD_BF16 ? 2 : 4) + 4.0 * kz), st,
                  [&] {
      if (pl.vdt == KD_BF16)
        hipLaunchKernelGGL(teacher_weights_kernel<bf16_t>, dim3(nb), dim3(256), 0, st, (const bf16_t*)val + r0 * pl.K,
                           nr, pl.K, kz, inv_tau, grad, inv_n, lab_c, o.ignore, o.alpha, pw);
      else
        hipLaunchKernelGGL(teacher_weights_kernel<float>, dim3(nb), dim3(256), 0, st, (const float*)val + r0 * pl.K,
                           nr, pl.K, kz, inv_tau, grad, inv_n, lab_c, o.ignore, o.alpha, pw);
    }));
    KD_TRY(run_bucket(pl, idx + r0 * pl.K, lab_c, o, add_label, nr, kz, true, pw, entries, ew, offsets, flags, st));
    g.entries = entries;
    g.offsets = offsets;
    g.ew = ew;
    g.kc = kz;
    KD_TRY((run_gemm<T, EPI_KL_DZ>("gemm_dz", g, (kKm ? 1 : 2) * es * nr * pl.V, st)));
    // dH = dZ W  (P[t][j] = sum_v dZ[t][v] W^T[j][v], or W read K-major)
    GemmArgs gh = w_km ? gemm_args(dz, pl.ld_v, nr, w, pl.d, (int)pl.d, (int)pl.V_pad)
                       : gemm_args(dz, pl.ld_v, nr, wt, pl.ld_v, (int)pl.d, (int)pl.V_pad);
    gh.krows_y = (int)pl.V;
    gh.out_rows = nr;
    gh.out_cols = (int)pl.d;
    gh.ldo = pl.d;
    const int S = dh_splits(pl, nr);
    if (S > 1) {
      // too few output tiles to fill the device: S partial sums over V, then their sum
      float* part = (float*)(ws + L.dhp);
      gh.out = part;
      gh.splits = S;
      gh.split_stride = (int64_t)nr * pl.d;
      KD_TRY((run_dh<T, EPI_STORE_F32>(gh, w_km, 4 * S * nr * pl.d, st)));
      const int64_t n4 = (int64_t)nr * pl.d / 4;
      const unsigned nb = (unsigned)std::min<int64_t>(4096, cdiv(n4, 256));
      KD_TRY(launch("dh_split_sum", 0.0, 4.0 * (S + 1) * nr * pl.d, st, [&] {
        if (pl.dhdt == KD_F32)
          hipLaunchKernelGGL(split_reduce_kernel<float>, dim3(nb), dim3(256), 0, st, part, S, gh.split_stride, n4,
                             (float*)dh + r0 * pl.d, 0);
        else
          hipLaunchKernelGGL(split_reduce_kernel<bf16_t>, dim3(nb), dim3(256), 0, st, part, S, gh.split_stride, n4,
                             (bf16_t*)dh + r0 * pl.d, 0);
      }));
    } else if (pl.dhdt == KD_F32) {
      gh.out = (float*)dh + r0 * pl.d;
      KD_TRY((run_dh<T, EPI_STORE_F32>(gh, w_km, 4 * nr * pl.d, st)));
    } else {
      gh.out = (bf16_t*)dh + r0 * pl.d;
      KD_TRY((run_dh<T, EPI_STORE_BF16>(gh, w_km, 2 * nr * pl.d, st)));
    }
    // dW (+)= dZ^T H  (P[v][j] = sum_t dZ[t][v] H^T[j][t]; bf16 reads X = dZ K-major)
    GemmArgs gw = kKm ? gemm_args(dz, pl.ld_v, (int)pl.V, ht, pl.ld_t, (int)pl.d, nr64)
                      : gemm_args(dzt, pl.ld_t, (int)pl.V, ht, pl.ld_t, (int)pl.d, nr64);
    gw.krows_x = nr;
    gw.out = dw;
    gw.ldo = pl.d;
    gw.out_rows = (int)pl.V;
    gw.out_cols = (int)pl.d;
    gw.accumulate = r0 > 0;
    int64_t txm = 0;
    const int SW = dw_splits(pl, nr64, &txm);
    if (SW > 1) {
      // the whole rounds of tiles, then the rest as SW partial sums over the chunk's
      // tokens, added to dW (or stored, for the first chunk) in split order
      const int64_t vm = txm * BX, vr = pl.V - vm;
      GemmArgs gm = gw;
      gm.nx = (int)vm;
      gm.n_tx = (int)txm;
      gm.out_rows = (int)vm;
      KD_TRY((run_gemm<T, EPI_STORE_F32, kKm, 0>("gemm_dw", gm, (r0 > 0 ? 8 : 4) * vm * pl.d, st)));
      float* part = (float*)(ws + L.dhp);
      GemmArgs gr = gw;
      // X rows vm.. : dZ columns (K-major) or dZ^T rows
      gr.X = (const char*)gw.X + (kKm ? vm * es : vm * gw.ldx * es);
      gr.nx = (int)vr;
      gr.n_tx = (int)cdiv(vr, BX);
      gr.out = part;
      gr.out_rows = (int)vr;
      gr.accumulate = 0;
      gr.splits = SW;
      gr.split_stride = vr * pl.d;
      KD_TRY((run_gemm<T, EPI_STORE_F32, kKm, 0>("gemm_dw_tail", gr, 4 * SW * vr * pl.d, st)));
      const int64_t n4 = vr * pl.d / 4;
      const unsigned nb = (unsigned)std::min<int64_t>(4096, cdiv(n4, 256));
      const int acc = r0 > 0;
      KD_TRY(launch("dw_split_sum", 0.0, 4.0 * (SW + 1 + acc) * vr * pl.d, st, [&] {
        hipLaunchKernelGGL(split_reduce_kernel<float>, dim3(nb), dim3(256), 0, st, part, SW, gr.split_stride, n4,
                           dw + vm * pl.d, acc);
      }));
    } else {
      KD_TRY((run_gemm<T, EPI_STORE_F32, kKm, 0>("gemm_dw", gw, (r0 > 0 ? 8 : 4) * pl.V * pl.d, st)));
    }
  }
  return KD_OK;
}

template <typename T, typename VT>
kd_status topk_impl(const Plan& pl, const Layout& L, const void* ht, const void* wt, int32_t* idx, void* val,
                    char* ws, hipStream_t st) {
  if (pl.N == 0) return KD_OK;
  bf16_t* S = (bf16_t*)(ws + L.s);
  double* bmax = (double*)(ws + L.bmax);
  double* wmax = (double*)(ws + L.wmax);
  int* overflow = (int*)(ws + L.overflow);
  float2* tops = (float2*)(ws + L.tops);
  int* todo = (int*)(ws + L.todo);
  const bool check = debug_checks();
  if (check) KD_TRY(zero_words(overflow, 4, st));
  const int64_t es = (int64_t)sizeof(T);
  const int nblk = (int)std::min<int64_t>(1024, cdiv(pl.V, 4));
  KD_TRY(launch("rownorm", 0.0, (double)es * pl.V * pl.d, st, [&] {
    hipLaunchKernelGGL(rownorm_max_kernel<T>, dim3(nblk), dim3(256), 0, st, (const T*)wt, (int)pl.V, (int)pl.d,
                       bmax);
  }));
  KD_TRY(launch("rownorm", 0.0, 8.0 * nblk, st, [&] {
    hipLaunchKernelGGL(max_reduce_kernel, dim3(1), dim3(256), 0, st, bmax, nblk, wmax);
  }));
  for (int64_t r0 = 0; r0 < pl.N; r0 += pl.Nc) {
    const int nr = (int)std::min<int64_t>(pl.Nc, pl.N - r0);
    const T* hc = (const T*)ht + r0 * pl.d;
    GemmArgs g = gemm_args(hc, pl.d, nr, wt, pl.d, (int)pl.V, (int)pl.d);
    g.out = S;
    g.ldo = pl.ld_v;
    g.out_rows = nr;
    g.out_cols = (int)pl.V_pad;
    g.partials = tops;
    g.ld_part = pl.Nc;
    KD_TRY((run_gemm<T, EPI_TOPK>("gemm_topk", g, 2 * nr * pl.V_pad, st)));
    // one pass over each row's logits from the tile pairs' bound; rows it cannot take
    // go to the general radix kernel
    KD_TRY(launch("topk_select", 0.0, 2.0 * nr * pl.V_pad + (double)nr * pl.K * (4 + sizeof(VT)), st, [&] {
      hipLaunchKernelGGL((topk_select_fast_kernel<T, VT>), dim3(nr), dim3(SEL_THREADS), 0, st, S, pl.ld_v,
                         (int)pl.V, pl.K, (const float2*)tops, pl.Nc, pl.n_ty, hc, (int)pl.d, (const T*)wt, wmax,
                         idx + r0 * pl.K, (VT*)val + r0 * pl.K, todo);
    }));
    KD_TRY(launch("topk_fallback", 0.0, 4.0 * nr, st, [&] {
      hipLaunchKernelGGL((topk_select_kernel<T, VT>), dim3(nr), dim3(SEL_THREADS), 0, st, S, pl.ld_v, (int)pl.V,
                         pl.K, hc, (int)pl.d, (const T*)wt, wmax, idx + r0 * pl.K, (VT*)val + r0 * pl.K, overflow,
                         (const int*)todo);
    }));
  }
  if (check) {
    int ov = 0;
    if (hipMemcpyAsync(&ov, overflow, sizeof(int), hipMemcpyDeviceToHost, st) != hipSuccess) return KD_ERR_LAUNCH;
    if (hipStreamSynchronize(st) != hipSuccess) return KD_ERR_LAUNCH;
    if (ov) return KD_ERR_TOPK_OVERFLOW;
  }
  return KD_OK;
}

}  // namespace

extern "C" {

kd_status kd_workspace_size(kd_op op_in, const kd_problem* p, size_t* bytes) {
  if (!bytes) return KD_ERR_NULL_POINTER;
  // a C caller may pass any int; it is read as one before it is used as a kd_op
  const int raw = enum_bits(op_in);
  if (raw != KD_OP_TOPK_BUILD && raw != KD_OP_KL_FWD && raw != KD_OP_KL_BWD) return KD_ERR_BAD_SHAPE;
  const kd_op op = (kd_op)raw;
  Plan pl;
  KD_TRY(validate(op, p, &pl));
  Layout L;
  *bytes = layout(op, pl, &L);
  return KD_OK;
}

kd_status kd_topk_cache_build(const kd_problem* p, const void* h_t, const void* w_t, int32_t* idx_out,
                              void* val_out, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  KD_TRY(validate(KD_OP_TOPK_BUILD, p, &pl));
  if (pl.N > 0 && (!h_t || !idx_out || !val_out)) return KD_ERR_NULL_POINTER;
  if (!w_t || !ws) return KD_ERR_NULL_POINTER;
  if (!aligned16(h_t) || !aligned16(w_t) || !aligned16(idx_out) || !aligned16(val_out) || !aligned16(ws))
    return KD_ERR_MISALIGNED;
  Layout L;
  if (ws_bytes < layout(KD_OP_TOPK_BUILD, pl, &L)) return KD_ERR_WORKSPACE_TOO_SMALL;
  KD_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (pl.xdt == KD_BF16) return topk_impl<bf16_t, bf16_t>(pl, L, h_t, w_t, idx_out, val_out, (char*)ws, st);
  return topk_impl<float, float>(pl, L, h_t, w_t, idx_out, val_out, (char*)ws, st);
}

}  // extern "C"

namespace {

// Options of the _ex calls: NULL, or labels NULL with no mix, is the plain loss.
kd_status read_opts(const kd_problem* p, const kd_loss_opts* opts, Opts* o) {
  *o = Opts{};
  if (!opts) return KD_OK;
  if (!(std::isfinite(opts->ce_weight) && opts->ce_weight >= 0.f && opts->ce_weight <= 1.f))
    return KD_ERR_BAD_OPTION;
  if (opts->student != KD_STUDENT_FULL && opts->student != KD_STUDENT_RENORM) return KD_ERR_BAD_OPTION;
  // the cross-entropy needs the full-vocabulary normaliser
  if (opts->student == KD_STUDENT_RENORM && opts->ce_weight > 0.f) return KD_ERR_BAD_OPTION;
  o->renorm = opts->student == KD_STUDENT_RENORM;
  if (!opts->labels) return opts->ce_weight > 0.f ? KD_ERR_BAD_OPTION : KD_OK;
  if ((reinterpret_cast<uintptr_t>(opts->labels) & 3u) != 0) return KD_ERR_MISALIGNED;
  if (p && p->n_tokens > 0) {
    o->labels = opts->labels;
    o->ignore = opts->ignore_index;
    o->alpha = opts->ce_weight;
  }
  return KD_OK;
}

kd_status fwd_entry(const kd_problem* p, const kd_loss_opts* opts, const void* h, const void* w,
                    const int32_t* idx, const void* val, float* loss_out, float* lse_out, float* kl_rows_out,
                    void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  KD_TRY(validate(KD_OP_KL_FWD, p, &pl));
  Opts o;
  KD_TRY(read_opts(p, opts, &o));
  if (!w || !loss_out || !ws) return KD_ERR_NULL_POINTER;
  if (pl.N > 0 && (!h || !idx || !val || !lse_out)) return KD_ERR_NULL_POINTER;
  if (!aligned16(h) || !aligned16(w) || !aligned16(idx) || !aligned16(val) || !aligned16(loss_out) ||
      !aligned16(lse_out) || !aligned16(kl_rows_out) || !aligned16(ws))
    return KD_ERR_MISALIGNED;
  Layout L;
  if (ws_bytes < layout(KD_OP_KL_FWD, pl, &L)) return KD_ERR_WORKSPACE_TOO_SMALL;
  KD_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (pl.xdt == KD_BF16)
    return fwd_impl<bf16_t>(pl, L, h, w, idx, val, loss_out, lse_out, kl_rows_out, (char*)ws, st, o);
  return fwd_impl<float>(pl, L, h, w, idx, val, loss_out, lse_out, kl_rows_out, (char*)ws, st, o);
}

kd_status bwd_entry(const kd_problem* p, const kd_loss_opts* opts, const void* h, const void* w,
                    const int32_t* idx, const void* val, const float* lse, const float* grad_loss, void* dh_out,
                    float* dw_out, void* ws, size_t ws_bytes, void* stream) {
  Plan pl;
  KD_TRY(validate(KD_OP_KL_BWD, p, &pl));
  Opts o;
  KD_TRY(read_opts(p, opts, &o));
  if (!w || !dw_out || !ws) return KD_ERR_NULL_POINTER;
  if (pl.N > 0 && (!h || !idx || !val || !lse || !dh_out)) return KD_ERR_NULL_POINTER;
  if (!aligned16(h) || !aligned16(w) || !aligned16(idx) || !aligned16(val) || !aligned16(lse) ||
      !aligned16(dh_out) || !aligned16(dw_out) || !aligned16(ws))
    return KD_ERR_MISALIGNED;
  Layout L;
  if (ws_bytes < layout(KD_OP_KL_BWD, pl, &L)) return KD_ERR_WORKSPACE_TOO_SMALL;
  KD_TRY(check_device());
  hipStream_t st = (hipStream_t)stream;
  if (pl.xdt == KD_BF16)
    return bwd_impl<bf16_t>(pl, L, h, w, idx, val, lse, grad_loss, dh_out, dw_out, (char*)ws, st, o);
  return bwd_impl<float>(pl, L, h, w, idx, val, lse, grad_loss, dh_out, dw_out, (char*)ws, st, o);
}

// ---- the allocation-free forward (kd_chunked_kl_fwd_noalloc)
//
// Its workspace is this file-scope device array: every device the library runs on
// holds its own copy from module load until the process ends.  In host code the
// name `scratch` is only a host-side stand-in; the device address of each device's
// copy comes from hipGetSymbolAddress, taken once per device with that device
// current, and only that address is handed to kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[256];   // per device; set once under g_scratch_mu

kd_status scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return KD_ERR_NO_DEVICE;
  if (dev >= 256) return KD_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KD_ERR_LAUNCH;
    g_scratch_ptr[dev] = ptr;
  }
  *out = (char*)g_scratch_ptr[dev];
  return KD_OK;
}

// The forward plan whose workspace fits the scratch array: the caller's chunk when
// one is given, else the largest multiple of 256 tokens up to the library default
// (the forward's results do not depend on the chunk).  KD_ERR_SCRATCH_TOO_SMALL
// when none fits.
kd_status noalloc_plan(const kd_problem* p, Plan* pl, Layout* L) {
  KD_TRY(validate(KD_OP_KL_FWD, p, pl));
  if (layout(KD_OP_KL_FWD, *pl, L) <= kScratchBytes) return KD_OK;
  if (p->chunk_tokens > 0) return KD_ERR_SCRATCH_TOO_SMALL;
  for (int64_t c = pl->Nc - BX; c >= BX; c -= BX) {
    pl->Nc = c;
    pl->ld_t = pad_ld(c, pl->esz);
    if (layout(KD_OP_KL_FWD, *pl, L) <= kScratchBytes) return KD_OK;
  }
  return KD_ERR_SCRATCH_TOO_SMALL;
}

}  // namespace

extern "C" {

kd_status kd_chunked_kl_fwd_noalloc(const kd_problem* p, const kd_loss_opts* opts, const void* h, const void* w,
                                    const int32_t* idx, const void* val, float* loss_out, float* lse_out,
                                    float* rows_out, void* stream) {
  Plan pl;
  Layout L;
  KD_TRY(noalloc_plan(p, &pl, &L));
  Opts o;
  KD_TRY(read_opts(p, opts, &o));
  if (!w || !loss_out) return KD_ERR_NULL_POINTER;
  if (pl.N > 0 && (!h || !idx || !val || !lse_out)) return KD_ERR_NULL_POINTER;
  if (!aligned16(h) || !aligned16(w) || !aligned16(idx) || !aligned16(val) || !aligned16(loss_out) ||
      !aligned16(lse_out) || !aligned16(rows_out))
    return KD_ERR_MISALIGNED;
  KD_TRY(check_device());
  char* ws = nullptr;
  KD_TRY(scratch_of_current_device(&ws));
  hipStream_t st = (hipStream_t)stream;
  if (pl.xdt == KD_BF16) return fwd_impl<bf16_t>(pl, L, h, w, idx, val, loss_out, lse_out, rows_out, ws, st, o);
  return fwd_impl<float>(pl, L, h, w, idx, val, loss_out, lse_out, rows_out, ws, st, o);
}

kd_status kd_chunked_kl_fwd(const kd_problem* p, const void* h, const void* w, const int32_t* idx,
                            const void* val, float* loss_out, float* lse_out, float* kl_rows_out, void* ws,
                            size_t ws_bytes, void* stream) {
  return fwd_entry(p, nullptr, h, w, idx, val, loss_out, lse_out, kl_rows_out, ws, ws_bytes, stream);
}

kd_status kd_chunked_kl_fwd_ex(const kd_problem* p, const kd_loss_opts* opts, const void* h, const void* w,
                               const int32_t* idx, const void* val, float* loss_out, float* lse_out,
                               float* rows_out, void* ws, size_t ws_bytes, void* stream) {
  return fwd_entry(p, opts, h, w, idx, val, loss_out, lse_out, rows_out, ws, ws_bytes, stream);
}

kd_status kd_chunked_kl_bwd(const kd_problem* p, const void* h, const void* w, const int32_t* idx,
                            const void* val, const float* lse, const float* grad_loss, void* dh_out, float* dw_out,
                            void* ws, size_t ws_bytes, void* stream) {
  return bwd_entry(p, nullptr, h, w, idx, val, lse, grad_loss, dh_out, dw_out, ws, ws_bytes, stream);
}

kd_status kd_chunked_kl_bwd_ex(const kd_problem* p, const kd_loss_opts* opts, const void* h, const void* w,
                               const int32_t* idx, const void* val, const float* lse, const float* grad_loss,
                               void* dh_out, float* dw_out, void* ws, size_t ws_bytes, void* stream) {
  return bwd_entry(p, opts, h, w, idx, val, lse, grad_loss, dh_out, dw_out, ws, ws_bytes, stream);
}

const char* kd_status_string(kd_status s_in) {
  switch (enum_bits(s_in)) {
    case KD_OK: return "ok";
    case KD_ERR_NULL_POINTER: return "a required pointer is NULL";
    case KD_ERR_BAD_SHAPE: return "a size is outside the supported domain";
    case KD_ERR_BAD_DTYPE: return "unsupported dtype or dtype combination";
    case KD_ERR_BAD_TAU: return "tau must be finite and > 0";
    case KD_ERR_MISALIGNED: return "a pointer is not 16-byte aligned";
    case KD_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than kd_workspace_size()";
    case KD_ERR_NO_DEVICE: return "no HIP device is current";
    case KD_ERR_UNSUPPORTED_ARCH: return "the current device is not gfx950 (MI355X)";
    case KD_ERR_LAUNCH: return "a kernel launch failed";
    case KD_ERR_IDX_OUT_OF_RANGE: return "a cached index (or a mixed-in label) is outside [0, V)";
    case KD_ERR_TOPK_OVERFLOW: return "too many near-ties at the K-th teacher logit";
    case KD_ERR_IO: return "a cache file could not be opened, read or written";
    case KD_ERR_BAD_FORMAT: return "a cache shard does not match the shard format";
    case KD_ERR_BAD_OPTION: return "a loss option is outside its domain";
    case KD_ERR_SCRATCH_TOO_SMALL: return "the problem needs more than the library's 64 MiB scratch array";
  }
  return "unknown status";
}

int kd_version(void) { return 102; }

kd_status kd_profile_begin(void) {
  Prof& p = prof();
  for (auto& r : p.recs) {
    p.pool.push_back(r.a);
    p.pool.push_back(r.b);
  }
  p.recs.clear();
  p.kinds.clear();
  p.failed = false;
  p.on = true;
  return KD_OK;
}

kd_status kd_profile_end(kd_kernel_stat* out, int max, int* n) {
  Prof& p = prof();
  p.on = false;
  kd_status st = p.failed ? KD_ERR_LAUNCH : KD_OK;
  std::vector<kd_kernel_stat> agg(p.kinds.size());
  for (size_t i = 0; i < p.kinds.size(); ++i) {
    std::memset(&agg[i], 0, sizeof(kd_kernel_stat));
    std::strncpy(agg[i].name, p.kinds[i].c_str(), sizeof(agg[i].name) - 1);
  }
  for (auto& r : p.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) st = KD_ERR_LAUNCH;
    kd_kernel_stat& a = agg[(size_t)r.kind];
    a.launches += 1;
    a.total_ms += ms;
    a.flops += r.flops;
    a.bytes += r.bytes;
    p.pool.push_back(r.a);
    p.pool.push_back(r.b);
  }
  p.recs.clear();
  if (n) *n = (int)agg.size();
  for (int i = 0; out && i < max && i < (int)agg.size(); ++i) out[i] = agg[(size_t)i];
  return st;
}

}  // extern "C"
