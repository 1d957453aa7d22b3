// MFMA GEMM core with fused epilogues for the chunked top-K KL loss (gfx950).
//
// Every contraction of the loss has the form
//     P[n][m] = sum_k X[n][k] * Y[m][k]        (both operands K-contiguous)
// with P stored row-major, so one lane writes 4 consecutive m of one row n:
//   logits   Z[t][v]  : X = H rows (tokens),     Y = W rows (vocabulary), K = d
//   dH[t][j]          : X = dZ rows (tokens),    Y = W^T rows (hidden),   K = V
//   dW[v][j]          : X = dZ^T rows (vocab),   Y = H^T rows (hidden),   K = tokens
//   teacher S[t][v]   : X = H_T rows,            Y = W_T rows,            K = d
//
// Workgroup tile 256 (n) x 256 (m), 8 waves arranged 4 (n) x 2 (m), each wave
// owning 64 x 128 outputs as 4 x 8 MFMA 16x16 blocks (128 fp32 accumulators per
// lane).  K is staged 128 bytes per row per stage (64 bf16 / 32 fp32) through a
// double-buffered, row-padded LDS tile: the global loads of stage s+1 are in
// flight while stage s feeds the MFMAs.  bf16 uses v_mfma_f32_16x16x32_bf16; fp32
// uses four v_mfma_f32_16x16x4_f32 over the same 16-byte fragment.
//
// MFMA 16x16 lane layout used throughout: operand lane l supplies row (l % 16)
// and a 16-byte K slice (l / 16); the result lane l holds column n = l % 16 and
// rows m = 4 * (l / 16) + e, e = 0..3.  Here the Y fragment is the MFMA "A"
// operand (m) and the X fragment the "B" operand (n).
#pragma once

#include "kd_common.hpp"

namespace kd {

constexpr int BX = 256, BY = 256;
constexpr int KBYTES = 128;                 // K bytes per row per stage
constexpr int PITCH = KBYTES + 16;          // padded LDS row pitch (bytes)
constexpr int WAVES_X = 4, WAVES_Y = 2;
constexpr int NWAVES = WAVES_X * WAVES_Y;
constexpr int NTHREADS = 64 * NWAVES;       // 512
constexpr int WX = BX / WAVES_X;            // 64
constexpr int WY = BY / WAVES_Y;            // 128
constexpr int FX = WX / 16, FY = WY / 16;   // 4 x 8 MFMA blocks per wave
constexpr int STAGE_BYTES = (BX + BY) * PITCH;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;  // 147456 of the 160 KiB per CU

// Epilogue staging of the forward gather: per wave 64 tokens x 64 vocabulary
// floats (two rounds cover the wave's 128 vocabulary columns).
constexpr int SPITCH = 68;                                      // floats
constexpr int STAGE_WAVE_FLOATS = WX * SPITCH;
constexpr int STATS_OFF = NWAVES * STAGE_WAVE_FLOATS * 4;       // bytes
static_assert(STATS_OFF + WAVES_Y * BX * 8 <= LDS_BYTES, "epilogue LDS");

enum Epi : int {
  EPI_STORE_F32 = 0,   // P -> float out (optionally += existing)
  EPI_STORE_BF16 = 1,  // P -> bf16 out
  EPI_KL_FWD = 2,      // per-row online (max, sum exp) partials + cached-entry gather
  EPI_KL_DZ = 3,       // dZ = (g/N) exp(z - lse) -> dZ and dZ^T buffers
};

struct GemmArgs {
  const void* X; int64_t ldx;     // [nx][k], elements
  const void* Y; int64_t ldy;     // [ny][k]
  int nx, ny, k;                  // valid rows of X and Y; contraction length
  int n_tx, n_ty, group;          // tile grid and tile-order grouping
  // plain stores / dZ buffers
  void* out; int64_t ldo;         // P rows
  void* out2; int64_t ldo2;       // dZ^T rows (EPI_KL_DZ)
  int out_rows, out_cols;         // store bounds of `out` (cols multiple of 4)
  int accumulate;                 // EPI_STORE_F32: out += P
  // KL forward / backward
  const float* lse;               // per chunk row
  const float* grad;              // device scalar or null (= 1)
  float inv_n;                    // 1 / N (all tokens)
  const uint32_t* entries;        // bucketed cache entries of the chunk
  const int* offsets;             // [n_tx][n_ty + 1]
  int kc;                         // cache entries per row (K)
  float* zg;                      // [rows][K] gathered logits
  float2* partials;               // [n_ty][ld_part] per-row (max, sum exp)
  int64_t ld_part;
};

// Workgroup -> tile.  Each XCD receives one contiguous range of the logical
// order, and the logical order walks `group` X-tiles for every Y-tile, so the
// 32 tiles that one XCD runs at a time share X and Y strips in its L2.
__device__ __forceinline__ void tile_of(int bid, int n_tx, int n_ty, int group, int& tx, int& ty) {
  const int n = n_tx * n_ty;
  const int per = n / kXcds, rem = n % kXcds;
  const int xcd = bid % kXcds, i = bid / kXcds;
  const int lin = xcd * per + min(xcd, rem) + i;
  const int width = group * n_ty;
  const int g = lin / width;
  const int first = g * group;
  const int gx = min(group, n_tx - first);
  const int r = lin - g * width;
  tx = first + r % gx;
  ty = r / gx;
}

template <typename T> struct Mma;
template <> struct Mma<bf16_t> {
  __device__ __forceinline__ static void run(f32x4& c, const u32x4& a, const u32x4& b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                0, 0, 0);
  }
};
template <> struct Mma<float> {
  __device__ __forceinline__ static void run(f32x4& c, const u32x4& a, const u32x4& b) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[e]), __uint_as_float(b[e]), c, 0, 0, 0);
  }
};

template <typename T> __device__ __forceinline__ void store4(T* p, const f32x4& v);
template <> __device__ __forceinline__ void store4<float>(float* p, const f32x4& v) { *(f32x4*)p = v; }
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const f32x4& v) {
  u32x2 w;
  w[0] = uint32_t(f32_to_bf16(v[0])) | (uint32_t(f32_to_bf16(v[1])) << 16);
  w[1] = uint32_t(f32_to_bf16(v[2])) | (uint32_t(f32_to_bf16(v[3])) << 16);
  *(u32x2*)p = w;
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T, int EPI>
__global__ void __launch_bounds__(NTHREADS, 1) gemm_kernel(const GemmArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];
  constexpr int EPC = 16 / int(sizeof(T));      // elements per 16-byte chunk
  constexpr int KE = KBYTES / int(sizeof(T));   // elements per stage

  int tx, ty;
  tile_of(blockIdx.x, a.n_tx, a.n_ty, a.group, tx, ty);
  const int x0 = tx * BX, y0 = ty * BY;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wx = wave % WAVES_X, wy = wave / WAVES_X;

  // ---- loader: thread owns 16-byte chunk (row lrow + 64 j, column lq) of X and Y
  const T* Xb = (const T*)a.X + (int64_t)x0 * a.ldx;
  const T* Yb = (const T*)a.Y + (int64_t)y0 * a.ldy;
  const int xrows = min(BX, a.nx - x0), yrows = min(BY, a.ny - y0);
  const int lrow = tid >> 3, lq = tid & 7;
  const int kq = lq * EPC;
  uint32_t xoff[4], yoff[4];
  bool xok[4], yok[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = lrow + 64 * j;
    xok[j] = r < xrows;
    yok[j] = r < yrows;
    xoff[j] = uint32_t((xok[j] ? r : 0) * a.ldx + kq);
    yoff[j] = uint32_t((yok[j] ? r : 0) * a.ldy + kq);
  }
  const uint32_t lds_st = uint32_t(lrow * PITCH + lq * 16);

  u32x4 stg[8];
  auto gload = [&](int k0) {
    const bool kok = (k0 + kq) < a.k;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      stg[j] = (kok && xok[j]) ? *(const u32x4*)(Xb + xoff[j] + k0) : u32x4{0u, 0u, 0u, 0u};
      stg[4 + j] = (kok && yok[j]) ? *(const u32x4*)(Yb + yoff[j] + k0) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto lstore = [&](int s) {
    char* base = lds + s * STAGE_BYTES + lds_st;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      *(u32x4*)(base + 64 * j * PITCH) = stg[j];
      *(u32x4*)(base + (BX + 64 * j) * PITCH) = stg[4 + j];
    }
  };

  f32x4 acc[FX][FY];
#pragma unroll
  for (int i = 0; i < FX; ++i)
#pragma unroll
    for (int j = 0; j < FY; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t xs_off = uint32_t((wx * WX + (lane & 15)) * PITCH + (lane >> 4) * 16);
  const uint32_t ys_off = uint32_t((BX + wy * WY + (lane & 15)) * PITCH + (lane >> 4) * 16);
  auto compute = [&](int s) {
    const char* base = lds + s * STAGE_BYTES;
#pragma unroll
    for (int f = 0; f < KBYTES / 64; ++f) {
      u32x4 bx[FX], by[FY];
#pragma unroll
      for (int i = 0; i < FX; ++i) bx[i] = *(const u32x4*)(base + xs_off + i * 16 * PITCH + f * 64);
#pragma unroll
      for (int j = 0; j < FY; ++j) by[j] = *(const u32x4*)(base + ys_off + j * 16 * PITCH + f * 64);
#pragma unroll
      for (int i = 0; i < FX; ++i)
#pragma unroll
        for (int j = 0; j < FY; ++j) Mma<T>::run(acc[i][j], by[j], bx[i]);
    }
  };

  const int nk = (a.k + KE - 1) / KE;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload((kt + 1) * KE);
    compute(kt & 1);
    if (more) lstore((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogues.  Lane (i, j, e) holds P[n = x0 + wx*64 + i*16 + lane%16][m = mcol + j*16 + e].
  const int nrow0 = x0 + wx * WX + (lane & 15);
  const int mcol = y0 + wy * WY + (lane >> 4) * 4;

  if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_STORE_BF16) {
    typedef typename std::conditional<EPI == EPI_STORE_F32, float, bf16_t>::type OT;
#pragma unroll
    for (int i = 0; i < FX; ++i) {
      const int n = nrow0 + i * 16;
      if (n >= a.out_rows) continue;
      OT* orow = (OT*)a.out + (int64_t)n * a.ldo;
#pragma unroll
      for (int j = 0; j < FY; ++j) {
        const int m = mcol + j * 16;
        if (m >= a.out_cols) continue;
        f32x4 v = acc[i][j];
        if constexpr (EPI == EPI_STORE_F32) {
          if (a.accumulate) v += *(const f32x4*)(orow + m);
        }
        store4<OT>(orow + m, v);
      }
    }
  } else if constexpr (EPI == EPI_KL_FWD) {
    // (1) per-token max and sum of exp over this wave's 128 vocabulary columns.
    float tm[FX], ts[FX];
#pragma unroll
    for (int i = 0; i < FX; ++i) {
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < FY; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (mcol + j * 16 + e < a.ny) mx = fmaxf(mx, acc[i][j][e]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float s = 0.f;
      if (mx != -INFINITY) {
        const float mb = mx * kLog2e;
#pragma unroll
        for (int j = 0; j < FY; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (mcol + j * 16 + e < a.ny) s += fast_exp2(fmaf(acc[i][j][e], kLog2e, -mb));
      }
      s += __shfl_xor(s, 16);
      s += __shfl_xor(s, 32);
      tm[i] = mx;
      ts[i] = s;
    }
    // (2) merge the two waves that share these tokens; one partial per (row, vocab tile).
    float2* st = (float2*)(lds + STATS_OFF);
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int i = 0; i < FX; ++i) st[wy * BX + wx * WX + i * 16 + lane] = make_float2(tm[i], ts[i]);
    }
    // (3) gather the cached entries that fall in this tile (wave-private LDS staging).
    float* sw = (float*)lds + wave * STAGE_WAVE_FLOATS;
    const int* off = a.offsets + (int64_t)tx * (a.n_ty + 1) + ty;
    const int eb = off[0], ee = off[1];
    const uint32_t* ent = a.entries + (int64_t)tx * BX * a.kc;
#pragma unroll
    for (int rnd = 0; rnd < 2; ++rnd) {
#pragma unroll
      for (int i = 0; i < FX; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *(f32x4*)(sw + (i * 16 + (lane & 15)) * SPITCH + jj * 16 + (lane >> 4) * 4) = acc[i][rnd * 4 + jj];
      wave_sync_lds();
      const int tlo = wx * WX, vlo = wy * WY + rnd * 64;
      for (int e = eb + lane; e < ee; e += 64) {
        const uint32_t u = ent[e];
        const int t = int(u & 255u) - tlo, v = int((u >> 8) & 255u) - vlo, k = int(u >> 16);
        if (t >= 0 && t < WX && v >= 0 && v < 64)
          a.zg[(int64_t)(x0 + tlo + t) * a.kc + k] = sw[t * SPITCH + v];
      }
      wave_sync_lds();
    }
    __syncthreads();
    if (tid < BX) {
      const float2 p0 = st[tid], p1 = st[BX + tid];
      const float M = fmaxf(p0.x, p1.x);
      float S = 0.f;
      if (M != -INFINITY) S = p0.y * fast_exp2((p0.x - M) * kLog2e) + p1.y * fast_exp2((p1.x - M) * kLog2e);
      const int row = x0 + tid;
      if (row < a.nx) a.partials[(int64_t)ty * a.ld_part + row] = make_float2(M, S);
    }
  } else if constexpr (EPI == EPI_KL_DZ) {
    const float g = a.grad ? *a.grad : 1.0f;
    const float scale = g * a.inv_n;
    T* dz = (T*)a.out;
    T* dzt = (T*)a.out2;
#pragma unroll
    for (int i = 0; i < FX; ++i) {
      const int n = nrow0 + i * 16;
      if (n >= a.out_rows) continue;
      const bool rv = n < a.nx;
      const float nl = rv ? -a.lse[n] * kLog2e : 0.f;
#pragma unroll
      for (int j = 0; j < FY; ++j) {
        const int m = mcol + j * 16;
        if (m >= a.out_cols) continue;
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = (rv && m + e < a.ny) ? scale * fast_exp2(fmaf(acc[i][j][e], kLog2e, nl)) : 0.f;
        store4<T>(dz + (int64_t)n * a.ldo + m, v);
#pragma unroll
        for (int e = 0; e < 4; ++e) dzt[(int64_t)(m + e) * a.ldo2 + n] = from_f32<T>(v[e]);
      }
    }
  }
}

}  // namespace kd
