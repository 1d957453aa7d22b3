// Non-GEMM kernels of the chunked top-K KL loss and of the teacher-cache build.
#pragma once

#include "kd_common.hpp"
#include "kd_gemm.hpp"

namespace kd {

// ---------------------------------------------------------------------------
// Block-wide exclusive prefix sum of one int per thread (blockDim.x <= 1024).
__device__ __forceinline__ int block_excl_scan(int v, int* sh /* >= 32 ints */, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) { const int t = sh[w]; sh[w] = run; run += t; }
    sh[31] = run;
  }
  __syncthreads();
  const int r = sh[wave] + x - v;
  total = sh[31];
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Bucket the cache entries of one 256-token tile by 256-wide vocabulary tile, so
// the forward GEMM epilogue of tile (tx, ty) reads exactly the entries that fall
// inside it.  Entry = token (8 bits) | vocab within tile (8 bits) | k (16 bits).
// Out-of-range indices are skipped and flagged.  With labels, a row whose label
// equals `ignore` contributes no entry (its cache row is not read), and with
// add_label every other row's label is one more entry, k = kc.  Rows of entries
// are kz apart (kc, or kc + 1 with add_label).
__global__ void __launch_bounds__(1024) bucket_kernel(const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ labels, int ignore,
                                                      int add_label, int nr, int kc, int kz, int vocab, int n_ty,
                                                      uint32_t* __restrict__ entries, int* __restrict__ offsets,
                                                      int* __restrict__ bad) {
  extern __shared__ int hist[];   // n_ty + 64 ints
  __shared__ int lab[BX];
  int* sh = hist + n_ty + 1;
  const int tx = blockIdx.x;
  const int r0 = tx * BX;
  const int rows = min(BX, nr - r0);
  const int total = rows * kc;
  const int all = total + (add_label ? rows : 0);
  const bool masked = labels != nullptr;
  const int32_t* src = idx + (int64_t)r0 * kc;
  for (int b = threadIdx.x; b <= n_ty; b += blockDim.x) hist[b] = 0;
  if (masked)
    for (int t = threadIdx.x; t < rows; t += blockDim.x) lab[t] = labels[r0 + t];
  __syncthreads();
  // entry e: cache entry (t, k) for e < total, else the label of row e - total;
  // false for a row left out, else its vocabulary index in v
  auto entry = [&](int e, int& v, int& t, int& k) -> bool {
    if (e < total) {
      t = e / kc;
      k = e - t * kc;
    } else {
      t = e - total;
      k = kc;
    }
    if (masked && lab[t] == ignore) return false;
    v = e < total ? src[e] : lab[t];
    return true;
  };
  int nbad = 0;
  for (int e = threadIdx.x; e < all; e += blockDim.x) {
    int v, t, k;
    if (!entry(e, v, t, k)) continue;
    if ((unsigned)v < (unsigned)vocab) atomicAdd(&hist[v >> 8], 1);
    else ++nbad;
  }
  if (nbad) atomicAdd(bad, nbad);
  __syncthreads();
  // exclusive scan of hist[0..n_ty) in contiguous per-thread segments
  const int seg = (n_ty + blockDim.x - 1) / blockDim.x;
  const int b0 = min(n_ty, (int)threadIdx.x * seg), b1 = min(n_ty, b0 + seg);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += hist[b];
  int tot;
  int run = block_excl_scan(local, sh, tot);
  int* out = offsets + (int64_t)tx * (n_ty + 1);
  for (int b = b0; b < b1; ++b) {
    const int c = hist[b];
    hist[b] = run;
    out[b] = run;
    run += c;
  }
  if (threadIdx.x == 0) out[n_ty] = tot;
  __syncthreads();
  uint32_t* dst = entries + (int64_t)tx * BX * kz;
  for (int e = threadIdx.x; e < all; e += blockDim.x) {
    int v, t, k;
    if (entry(e, v, t, k) && (unsigned)v < (unsigned)vocab) {
      const int pos = atomicAdd(&hist[v >> 8], 1);
      dst[pos] = uint32_t(t) | (uint32_t(v & 255) << 8) | (uint32_t(k) << 16);
    }
  }
}

// ---------------------------------------------------------------------------
// float64 dot product of an h row and a w row of length d (a multiple of 8), by one
// wave: lane l sums the 16-byte chunks l, l + 64, ... in ascending order, then a
// butterfly over the wave, so every lane returns the same value and the order never
// depends on timing.  Up to 8 chunks per lane are loaded before any is used, which
// keeps 8 row segments per wave in flight (the w rows come from HBM at random).
template <typename T>
__device__ __forceinline__ double wave_dot_f64(const T* __restrict__ h, const T* __restrict__ w, int d, int lane) {
  constexpr int EPC = 16 / int(sizeof(T));
  constexpr int U = 8;
  double acc = 0.0;
  for (int j0 = lane * EPC; j0 < d; j0 += U * 64 * EPC) {
    u32x4 hv[U], wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * 64 * EPC;
      if (j < d) {
        hv[u] = *(const u32x4*)(h + j);
        wv[u] = *(const u32x4*)(w + j);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (j0 + u * 64 * EPC < d) {
        const T* hp = (const T*)&hv[u];
        const T* wp = (const T*)&wv[u];
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc = fma((double)to_f32<T>(hp[e]), (double)to_f32<T>(wp[e]), acc);
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  return acc;
}

// ---------------------------------------------------------------------------
// Block sum of one double per thread (256 threads), fixed order.
__device__ __forceinline__ double block_sum_256(double v, double* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  return sh[0];
}

// Rows per block and threads per row of the per-row kernels (merge, scatter).
constexpr int RB_ROWS = 16, RB_TPR = 16;

// Combine two (max, sum exp) pairs of one row.
__device__ __forceinline__ void lse_combine(float& M, float& S, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (M == -INFINITY) {
    M = m2;
    S = s2;
    return;
  }
  const float m = fmaxf(M, m2);
  S = S * exp2f((M - m) * kLog2e) + s2 * exp2f((m2 - m) * kLog2e);
  M = m;
}

// Reductions over the RB_TPR threads of one row: thread (r, q) is tid = r + RB_ROWS q,
// so a wave holds 4 values of q per row (shuffles over lanes 16, 32 apart) and the
// 4 waves meet in LDS.  Fixed order, so results are deterministic.
__device__ __forceinline__ float row_sum(float v, float* sh) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  const int r = threadIdx.x & (RB_ROWS - 1), w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) < RB_ROWS) sh[w * RB_ROWS + r] = v;
  __syncthreads();
  return (sh[r] + sh[RB_ROWS + r]) + (sh[2 * RB_ROWS + r] + sh[3 * RB_ROWS + r]);
}
__device__ __forceinline__ float row_max(float v, float* sh) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  const int r = threadIdx.x & (RB_ROWS - 1), w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) < RB_ROWS) sh[w * RB_ROWS + r] = v;
  __syncthreads();
  return fmaxf(fmaxf(sh[r], sh[RB_ROWS + r]), fmaxf(sh[2 * RB_ROWS + r], sh[3 * RB_ROWS + r]));
}

// Merge the per-tile (max, sum exp) partials of each row into lse, form the
// teacher softmax over the K cached logits and the row's KL, and sum the block's
// row losses (float64) for the deterministic loss reduction.  RB_ROWS rows per
// block, RB_TPR threads per row striding the vocabulary tiles (partials of
// consecutive rows are adjacent, so a wave's loads are coalesced over rows).
// With labels: a row whose label equals `ignore` gets lse only (loss term 0, its
// cache row unread); with alpha > 0 the row's term is (1 - alpha) KL + alpha CE,
// CE = lse - z[label], the label's logit gathered at k = kc (rows of zg are kz
// apart).
template <typename VT>
__global__ void __launch_bounds__(256) merge_kernel(const float2* __restrict__ partials, int64_t ld_part, int n_ty,
                                                    const int32_t* __restrict__ idx, const VT* __restrict__ val,
                                                    const float* __restrict__ zg, int nr, int kc, int kz, int vocab,
                                                    float inv_tau, const int32_t* __restrict__ labels, int ignore,
                                                    float alpha, float* __restrict__ lse_out,
                                                    float* __restrict__ kl_out, double* __restrict__ block_sums) {
  __shared__ float sh[4 * RB_ROWS];
  __shared__ float2 shp[4 * RB_ROWS];
  __shared__ float klrow[RB_ROWS];
  const int r = threadIdx.x & (RB_ROWS - 1), q = threadIdx.x / RB_ROWS;
  const int t = blockIdx.x * RB_ROWS + r;
  const bool valid = t < nr;
  const bool counted = valid && (labels == nullptr || labels[t] != ignore);
  // (1) log-sum-exp over the vocabulary tiles
  float M = -INFINITY, S = 0.f;
  if (valid)
    for (int y = q; y < n_ty; y += RB_TPR) {
      const float2 p = partials[(int64_t)y * ld_part + t];
      lse_combine(M, S, p.x, p.y);
    }
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) lse_combine(M, S, __shfl_xor(M, o), __shfl_xor(S, o));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) < RB_ROWS) shp[w * RB_ROWS + r] = make_float2(M, S);
  __syncthreads();
  M = shp[r].x;
  S = shp[r].y;
#pragma unroll
  for (int i = 1; i < 4; ++i) lse_combine(M, S, shp[i * RB_ROWS + r].x, shp[i * RB_ROWS + r].y);
  const float lse = M + logf(S);
  // (2) teacher softmax over the K cached logits and the row's KL
  const VT* vr = val + (int64_t)t * kc;
  const int32_t* ir = idx + (int64_t)t * kc;
  const float* zr = zg + (int64_t)t * kz;
  float vmax = -INFINITY;
  if (counted)
    for (int k = q; k < kc; k += RB_TPR) vmax = fmaxf(vmax, to_f32<VT>(vr[k]) * inv_tau);
  vmax = row_max(vmax, sh);
  float Z = 0.f;
  if (counted)
    for (int k = q; k < kc; k += RB_TPR) Z += expf(to_f32<VT>(vr[k]) * inv_tau - vmax);
  const float logZ = logf(row_sum(Z, sh));
  float kl = 0.f;
  if (counted)
    for (int k = q; k < kc; k += RB_TPR) {
      const float lp = to_f32<VT>(vr[k]) * inv_tau - vmax - logZ;
      const float p = expf(lp);
      if ((unsigned)ir[k] >= (unsigned)vocab) kl = NAN;
      else kl += (p > 0.f ? p * lp : 0.f) - p * (zr[k] - lse);
    }
  kl = row_sum(kl, sh);
  if (q == 0) {
    float l = 0.f;
    if (counted) {
      l = kl;
      if (alpha > 0.f) {
        const int y = labels[t];
        const float ce = (unsigned)y < (unsigned)vocab ? lse - zr[kc] : NAN;
        l = (1.f - alpha) * kl + alpha * ce;
      }
    }
    klrow[r] = l;
    if (valid) {
      lse_out[t] = lse;
      if (kl_out) kl_out[t] = l;
    }
  }
  __syncthreads();
  // (3) the block's KL sum over its rows, in row order (float64)
  if (threadIdx.x == 0) {
    double s = 0.0;
    for (int i = 0; i < RB_ROWS; ++i) s += (double)klrow[i];
    block_sums[blockIdx.x] = s;
  }
}

// loss = (sum of block sums) / N, summed in a fixed order; with `count` (the
// counted rows, from count_rows_kernel) the divisor is that count (loss 0 when
// it is 0).
__global__ void __launch_bounds__(256) loss_kernel(const double* __restrict__ block_sums, int nb, double inv_n,
                                                   const double* __restrict__ count, float* __restrict__ loss) {
  __shared__ double sh[256];
  double a = 0.0;
  for (int b = threadIdx.x; b < nb; b += 256) a += block_sums[b];
  const double s = block_sum_256(a, sh);
  if (threadIdx.x == 0) {
    const double inv = count ? (*count > 0.0 ? 1.0 / *count : 0.0) : inv_n;
    *loss = (float)(s * inv);
  }
}

// Number of rows whose label differs from `ignore` (one block, fixed order), and
// the gradient scale g / count that the backward applies to every counted row
// (0 when no row counts).
__global__ void __launch_bounds__(1024) count_rows_kernel(const int32_t* __restrict__ labels, int64_t n,
                                                          int ignore, const float* __restrict__ grad,
                                                          double* __restrict__ count_out,
                                                          float* __restrict__ scale_out) {
  __shared__ long long sh[1024];
  long long c = 0;
  for (int64_t i = threadIdx.x; i < n; i += 1024) c += labels[i] != ignore;
  sh[threadIdx.x] = c;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] += sh[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const long long tot = sh[0];
    *count_out = (double)tot;
    if (scale_out) scale_out[0] = tot > 0 ? (grad ? *grad : 1.0f) * (1.0f / (float)tot) : 0.0f;
  }
}

// lse of the counted rows, +inf for the ignored ones: the dZ epilogue's
// exp(z - lse) is then exactly 0 on an ignored row.
__global__ void __launch_bounds__(256) mask_lse_kernel(const float* __restrict__ lse,
                                                       const int32_t* __restrict__ labels, int nr, int ignore,
                                                       float* __restrict__ out) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t < nr) out[t] = labels[t] != ignore ? lse[t] : INFINITY;
}

// ---------------------------------------------------------------------------
// dst[c][r] = src[r][c] for r < rows, 0 for rows <= r < rows_pad; c < cols.
template <typename T>
__global__ void __launch_bounds__(256) transpose_pad_kernel(const T* __restrict__ src, int64_t ld_src, int rows,
                                                            int cols, T* __restrict__ dst, int64_t ld_dst,
                                                            int rows_pad) {
  __shared__ T tile[64][65];
  const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? src[(int64_t)r * ld_src + c] : T(0);
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows_pad) dst[(int64_t)c * ld_dst + r] = tile[tx][i];
  }
}

// ---------------------------------------------------------------------------
// Subtract the scaled teacher probabilities at the cached entries of each row
// from dZ (and from dZ^T when that copy exists).  RB_ROWS rows per block, RB_TPR
// threads per row.  Entries are applied in batches of RB_TPR in k order: within a
// batch, repeated indices are summed (in k order) by their first occurrence, and
// a block barrier orders the batches, so every element is updated by one thread
// at a time and repeated indices accumulate.  With labels, rows whose label
// equals `ignore` are left alone (their dZ row is 0 already), and with alpha > 0
// the teacher is weighted by 1 - alpha and the label is one more entry (k = kc)
// of weight alpha.
template <typename T, typename VT>
__global__ void __launch_bounds__(256) scatter_kernel(const int32_t* __restrict__ idx, const VT* __restrict__ val,
                                                      int nr, int kc, int vocab, float inv_tau,
                                                      const float* __restrict__ grad, float inv_n,
                                                      const int32_t* __restrict__ labels, int ignore, float alpha,
                                                      T* __restrict__ dz, int64_t ldz, T* __restrict__ dzt,
                                                      int64_t ldzt) {
  __shared__ float sh[4 * RB_ROWS];
  __shared__ int bidx[RB_ROWS][RB_TPR];
  __shared__ float bpe[RB_ROWS][RB_TPR];
  const int r = threadIdx.x & (RB_ROWS - 1), q = threadIdx.x / RB_ROWS;
  const int t = blockIdx.x * RB_ROWS + r;
  const bool counted = t < nr && (labels == nullptr || labels[t] != ignore);
  const float scale = (grad ? *grad : 1.0f) * inv_n;
  const float wt = scale * (1.0f - alpha);
  const int ke = kc + (alpha > 0.f ? 1 : 0);
  const VT* vr = val + (int64_t)t * kc;
  const int32_t* ir = idx + (int64_t)t * kc;
  float vmax = -INFINITY;
  if (counted)
    for (int k = q; k < kc; k += RB_TPR) vmax = fmaxf(vmax, to_f32<VT>(vr[k]) * inv_tau);
  vmax = row_max(vmax, sh);
  float Z = 0.f;
  if (counted)
    for (int k = q; k < kc; k += RB_TPR) Z += expf(to_f32<VT>(vr[k]) * inv_tau - vmax);
  const float logZ = logf(row_sum(Z, sh));
  for (int k0 = 0; k0 < ke; k0 += RB_TPR) {
    const int k = k0 + q;
    int v = -1;
    float pe = 0.f;
    if (counted && k < ke) {
      v = k < kc ? ir[k] : labels[t];
      if ((unsigned)v >= (unsigned)vocab) v = -1;
      else pe = k < kc ? wt * expf(to_f32<VT>(vr[k]) * inv_tau - vmax - logZ) : scale * alpha;
    }
    bidx[r][q] = v;
    bpe[r][q] = pe;
    __syncthreads();
    bool first = v >= 0;
    for (int j = 0; j < q && first; ++j) first = bidx[r][j] != v;
    if (first) {
      float sum = pe;
      for (int j = q + 1; j < RB_TPR; ++j)
        if (bidx[r][j] == v) sum += bpe[r][j];
      T* a = dz + (int64_t)t * ldz + v;
      *a = from_f32<T>(to_f32<T>(*a) - sum);
      if (dzt) {
        T* b = dzt + (int64_t)v * ldzt + t;
        *b = from_f32<T>(to_f32<T>(*b) - sum);
      }
    }
    __syncthreads();   // this batch's updates before the next batch's reads
  }
}

// out[i] = sum over s of part[s * stride + i], s in order (split-K partial sums).
template <typename OT>
__global__ void __launch_bounds__(256) split_reduce_kernel(const float* __restrict__ part, int splits,
                                                           int64_t stride, int64_t n4, OT* __restrict__ out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n4; i += (int64_t)gridDim.x * blockDim.x) {
    f32x4 a = *(const f32x4*)(part + 4 * i);
    for (int s = 1; s < splits; ++s) a += *(const f32x4*)(part + s * stride + 4 * i);
#pragma unroll
    for (int e = 0; e < 4; ++e) out[4 * i + e] = from_f32<OT>(a[e]);
  }
}

// Fill a float buffer (used for dW when there are no tokens).
__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// ---------------------------------------------------------------------------
// Teacher cache build.
// max over rows of the Euclidean norm of W_T (float64), per block then global.
template <typename T>
__global__ void __launch_bounds__(256) rownorm_max_kernel(const T* __restrict__ w, int rows, int d,
                                                          double* __restrict__ block_max) {
  __shared__ double sh[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double best = 0.0;
  for (int r = blockIdx.x * 4 + wave; r < rows; r += gridDim.x * 4) {
    const T* p = w + (int64_t)r * d;
    double s = 0.0;
    for (int j = lane; j < d; j += 64) {
      const double x = (double)to_f32<T>(p[j]);
      s += x * x;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    best = fmax(best, s);
  }
  if (lane == 0) sh[wave] = best;
  __syncthreads();
  if (threadIdx.x == 0) block_max[blockIdx.x] = sqrt(fmax(fmax(sh[0], sh[1]), fmax(sh[2], sh[3])));
}

__global__ void __launch_bounds__(256) max_reduce_kernel(const double* __restrict__ in, int n,
                                                         double* __restrict__ out) {
  __shared__ double sh[256];
  double m = 0.0;
  for (int i = threadIdx.x; i < n; i += 256) m = fmax(m, in[i]);
  sh[threadIdx.x] = m;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) sh[threadIdx.x] = fmax(sh[threadIdx.x], sh[threadIdx.x + s]);
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = sh[0];
}

constexpr int SEL_CAP = 6144;    // candidate capacity per row (K <= 4096)
constexpr int SEL_THREADS = 256;

// Finds the largest bin B of hist[4096] with count(bins >= B) >= need; writes B and
// count(bins > B) to res[0], res[1].  256 threads, 16 bins each.
__device__ __forceinline__ void select_bin(const uint32_t* hist, int need, int* sh, int* res) {
  const int t = threadIdx.x;
  int local = 0;
#pragma unroll
  for (int b = 0; b < 16; ++b) local += (int)hist[t * 16 + b];
  // count above this thread's bins = total - inclusive prefix
  int total;
  const int excl = block_excl_scan(local, sh, total);
  const int above = total - excl - local;
  if (above < need && above + local >= need) {
    int run = above;
    for (int b = 15; b >= 0; --b) {
      const int c = (int)hist[t * 16 + b];
      if (run + c >= need) {
        res[0] = t * 16 + b;
        res[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

// Exact top-K of one teacher row (general path; with rows_todo, only the rows the
// fast path below handed over).  s[V] holds the float32 MFMA logits.
//  1. Two 12-bit radix histograms of the order-preserving key locate a
//     sub-bin [lo, ...) that contains the K-th largest float32 value T_K.
//  2. Every value >= lo - 2*eps is a candidate, where eps bounds |fp32 - exact|
//     for any logit of the row (Higham's summation bound with Cauchy-Schwarz:
//     eps = 2 d 2^-23 ||h|| max_v ||w_v||).  Every exact top-K member is in the set.
//  3. Candidates are re-scored exactly-rounded in float64, ranked by (score desc,
//     index asc), and the first K are written.
template <typename T, typename VT>
__global__ void __launch_bounds__(SEL_THREADS) topk_select_kernel(
    const float* __restrict__ S, int64_t ld_s, int V, int K, const T* __restrict__ ht, int d,
    const T* __restrict__ wt, const double* __restrict__ wmax, int32_t* __restrict__ idx_out,
    VT* __restrict__ val_out, int* __restrict__ overflow, const int* __restrict__ rows_todo) {
  if (rows_todo && !rows_todo[blockIdx.x]) return;   // handled by topk_select_fast_kernel
  __shared__ uint32_t hist[4096];
  __shared__ int cidx[SEL_CAP];
  __shared__ double cscore[SEL_CAP];
  __shared__ int sh[40];
  __shared__ double shd[SEL_THREADS];
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* s = S + (int64_t)row * ld_s;
  const T* h = ht + (int64_t)row * d;

  // ||h||_2 in float64
  double hn = 0.0;
  for (int j = tid; j < d; j += SEL_THREADS) {
    const double x = (double)to_f32<T>(h[j]);
    hn += x * x;
  }
  hn = sqrt(block_sum_256(hn, shd));
  const double eps = 2.0 * (double)d * 0x1p-23 * hn * (*wmax);

  // pass 1: top 12 bits of the key
  for (int b = tid; b < 4096; b += SEL_THREADS) hist[b] = 0u;
  __syncthreads();
  for (int v = tid; v < V; v += SEL_THREADS) atomicAdd(&hist[float_key(s[v]) >> 20], 1u);
  __syncthreads();
  select_bin(hist, K, sh, sh + 34);
  const uint32_t B = (uint32_t)sh[34];
  const int above = sh[35];
  __syncthreads();
  // pass 2: next 12 bits inside bin B
  for (int b = tid; b < 4096; b += SEL_THREADS) hist[b] = 0u;
  __syncthreads();
  for (int v = tid; v < V; v += SEL_THREADS) {
    const uint32_t key = float_key(s[v]);
    if ((key >> 20) == B) atomicAdd(&hist[(key >> 8) & 0xfffu], 1u);
  }
  __syncthreads();
  select_bin(hist, K - above, sh, sh + 36);
  const uint32_t B2 = (uint32_t)sh[36];
  const float lo = key_float((B << 20) | (B2 << 8));
  const float thr = __double2float_rd((double)lo - 2.0 * eps);
  if (tid == 0) sh[38] = 0;
  __syncthreads();
  // pass 3: candidates
  for (int v = tid; v < V; v += SEL_THREADS) {
    if (s[v] >= thr) {
      const int pos = atomicAdd(&sh[38], 1);
      if (pos < SEL_CAP) cidx[pos] = v;
    }
  }
  __syncthreads();
  const int C = sh[38];
  if (C > SEL_CAP) {
    for (int k = tid; k < K; k += SEL_THREADS) {
      idx_out[(int64_t)row * K + k] = -1;
      val_out[(int64_t)row * K + k] = from_f32<VT>(NAN);
    }
    if (tid == 0) atomicAdd(overflow, 1);
    return;
  }
  // float64 re-scoring: one wave per candidate, lanes split d in 16-byte chunks
  for (int c = wave; c < C; c += SEL_THREADS / 64) {
    const double acc = wave_dot_f64<T>(h, wt + (int64_t)cidx[c] * d, d, lane);
    if (lane == 0) cscore[c] = acc;
  }
  __syncthreads();
  // rank by (score desc, index asc); write the first K
  for (int c = tid; c < C; c += SEL_THREADS) {
    const double sc = cscore[c];
    const int vi = cidx[c];
    int rank = 0;
    for (int o = 0; o < C; ++o) {
      const double so = cscore[o];
      rank += (so > sc) || (so == sc && cidx[o] < vi);
    }
    if (rank < K) {
      idx_out[(int64_t)row * K + rank] = vi;
      if constexpr (sizeof(VT) == 2) val_out[(int64_t)row * K + rank] = f64_to_bf16_rne(sc);
      else val_out[(int64_t)row * K + rank] = (float)sc;
    }
  }
}

// Exact top-K of one teacher row, fast path.  The GEMM epilogue left, for every
// 256-column vocabulary tile, the row's two largest float32 logits in the tile.
//  1. Those 2 n_ty values are distinct elements of the row, so their K-th largest
//     t is <= the row's K-th largest float32 logit (bitwise search over the
//     order-preserving keys, 32 block counts).
//  2. One pass over the row's tiles whose largest logit reaches t - 2 eps keeps
//     every logit >= t - 2 eps (eps as in the general path): the exact top-K are
//     all among them.
//  3. float64 re-scoring, ranking by (score desc, index asc), first K written.
// A row this path cannot take (2 n_ty < K, more tile values than TOPS_CAP, more
// candidates than FAST_CAP) is flagged in rows_todo for the general kernel.
constexpr int TOPS_CAP = 4096;
constexpr int FAST_CAP = 1536;
template <typename T, typename VT>
__global__ void __launch_bounds__(SEL_THREADS) topk_select_fast_kernel(
    const float* __restrict__ S, int64_t ld_s, int V, int K, const float2* __restrict__ tops, int64_t ld_tops,
    int n_ty, const T* __restrict__ ht, int d, const T* __restrict__ wt, const double* __restrict__ wmax,
    int32_t* __restrict__ idx_out, VT* __restrict__ val_out, int* __restrict__ rows_todo) {
  __shared__ uint32_t keys[TOPS_CAP];
  __shared__ int cidx[FAST_CAP];
  __shared__ double cscore[FAST_CAP];
  __shared__ double shd[SEL_THREADS];
  __shared__ int shc[SEL_THREADS / 64];
  __shared__ int ncand;
  const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = 2 * n_ty;
  if (M < K || M > TOPS_CAP) {
    if (tid == 0) rows_todo[row] = 1;
    return;
  }
  for (int q = tid; q < n_ty; q += SEL_THREADS) {
    const float2 t = tops[(int64_t)q * ld_tops + row];
    keys[2 * q] = float_key(t.x);
    keys[2 * q + 1] = float_key(t.y);
  }
  if (tid == 0) ncand = 0;
  __syncthreads();
  // 1. largest key t with #{keys >= t} >= K, i.e. the K-th largest key
  uint32_t t = 0;
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = t | (1u << b);
    int n = 0;
    for (int q = tid; q < M; q += SEL_THREADS) n += keys[q] >= c;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
    if (lane == 0) shc[wave] = n;
    __syncthreads();
    int tot = 0;
#pragma unroll
    for (int w = 0; w < SEL_THREADS / 64; ++w) tot += shc[w];
    __syncthreads();
    if (tot >= K) t = c;
  }
  const float* s = S + (int64_t)row * ld_s;
  const T* h = ht + (int64_t)row * d;
  double hn = 0.0;
  for (int j = tid; j < d; j += SEL_THREADS) {
    const double x = (double)to_f32<T>(h[j]);
    hn += x * x;
  }
  hn = sqrt(block_sum_256(hn, shd));
  const double eps = 2.0 * (double)d * 0x1p-23 * hn * (*wmax);
  const float thr = __double2float_rd((double)key_float(t) - 2.0 * eps);
  // 2. candidates.  A vocabulary tile whose largest logit is below the threshold
  // holds none, so only the other tiles are read (one wave per 256-column tile,
  // 16 bytes per lane; the index test covers the vocabulary tail).
  const uint32_t thr_key = float_key(thr);
  for (int q = wave; q < n_ty; q += SEL_THREADS / 64) {
    if (keys[2 * q] < thr_key) continue;
    const int v0 = 256 * q + 4 * lane;
    if (v0 >= V) continue;
    const f32x4 x = *(const f32x4*)(s + v0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int v = v0 + e;
      if (v < V && x[e] >= thr) {
        const int pos = atomicAdd(&ncand, 1);
        if (pos < FAST_CAP) cidx[pos] = v;
      }
    }
  }
  __syncthreads();
  const int C = ncand;
  if (C > FAST_CAP) {
    if (tid == 0) rows_todo[row] = 1;
    return;
  }
  // 3. float64 re-scoring: one wave per candidate, lanes split d in 16-byte chunks
  for (int c = wave; c < C; c += SEL_THREADS / 64) {
    const double acc = wave_dot_f64<T>(h, wt + (int64_t)cidx[c] * d, d, lane);
    if (lane == 0) cscore[c] = acc;
  }
  __syncthreads();
  for (int c = tid; c < C; c += SEL_THREADS) {
    const double sc = cscore[c];
    const int vi = cidx[c];
    int rank = 0;
    for (int o = 0; o < C; ++o) {
      const double so = cscore[o];
      rank += (so > sc) || (so == sc && cidx[o] < vi);
    }
    if (rank < K) {
      idx_out[(int64_t)row * K + rank] = vi;
      if constexpr (sizeof(VT) == 2) val_out[(int64_t)row * K + rank] = f64_to_bf16_rne(sc);
      else val_out[(int64_t)row * K + rank] = (float)sc;
    }
  }
  if (tid == 0) rows_todo[row] = 0;
}

}  // namespace kd
