// MFMA GEMM core with fused epilogues for the chunked top-K KL loss (gfx950).
//
// Every contraction of the loss has the form
//     P[n][m] = sum_k X[n][k] * Y[m][k]        (both operands K-contiguous)
// with P stored row-major, so one lane writes 4 consecutive m of one row n:
//   logits   Z[t][v]  : X = H rows (tokens),     Y = W rows (vocabulary), K = d
//   dH[t][j]          : X = dZ rows (tokens),    Y = W^T rows (hidden),   K = V
//   dW[v][j]          : X = dZ read K-major (bf16) or dZ^T rows (fp32),
//                       Y = H^T rows (hidden),   K = tokens
//   teacher S[t][v]   : X = H_T rows,            Y = W_T rows,            K = d
//
// Main loop (one workgroup per BX x BY output tile, 8 waves of 64 x 128 outputs):
//  * operands reach LDS through wave-wide buffer loads that write LDS directly
//    (no staging registers, no ds_write), each lane 16 bytes, 8 lanes per 128-byte
//    row segment; rows past an operand's end and K past its end read as zero
//    (out-of-range buffer offsets), so tails need no branches;
//  * LDS holds 2 stages of 128 bytes of K per row (64 bf16 / 32 fp32); the load of
//    stage kt + 2 is issued right after the barrier that frees stage kt's buffer;
//  * each stage is two 64-byte MFMA fragments; in source order the fragments of the
//    next half are read from LDS before the MFMAs of the current half (one barrier
//    per stage, placed between the halves).  For row-major operands the compiler
//    then moves each read next to its first use (the two waves of a SIMD cover each
//    other's waits); with a K-major operand scheduling-group barriers keep the reads
//    spread over the MFMAs;
//  * the 16-byte chunks of each LDS row are XOR-swizzled by row % 8, which makes the
//    fragment reads (ds_read_b128, lane = row l % 16, chunk l / 16) free of bank
//    conflicts on gfx950 (measured: 4 LDS cycles per read, 256 B/clk);
//  * bf16 uses v_mfma_f32_16x16x32_bf16; fp32 uses four v_mfma_f32_16x16x4_f32 on
//    the same 16-byte fragment.
//  * K-major operands (bf16 only): an operand stored as [k][n] (n contiguous) is read
//    with ds_read_b64_tr_b16.  Within each 16-lane group, output lane j, element e
//    comes from input lane 4e + j/4, element j % 4 (measured), so input lane 4e + q
//    pointing at k-row k0 + e, columns n0 + 4q .. n0 + 4q + 3 delivers rows k0..k0+3 of
//    column n0 + j to lane j; two such reads (k0 and k0 + 4) make one MFMA fragment.
//    The stage is laid out in 256-byte blocks, each holding 8 k-rows x 32 bytes of
//    one 16-column fragment, so a read's bank position depends on the lane alone
//    (the 32 lanes of a half-wave cover all 32 eight-byte bank slots) and fragment,
//    k-half and row-half are immediate offsets (measured: 1.8x faster than 512-byte
//    XOR-swizzled k-rows).  The dW product reads dZ this way, so no N x V transposed
//    copy of dZ is ever written.
//
// MFMA 16x16 lane layout: operand lane l supplies row (l % 16) and the 16-byte K
// slice (l / 16); result lane l holds column n = l % 16 and rows m = 4(l/16)+e.
// The Y fragment is the MFMA "A" operand (m), the X fragment the "B" operand (n).
#pragma once

#include <type_traits>

#include "kd_common.hpp"

namespace kd {

template <int BX_, int BY_, int WAVES_X_, int WAVES_Y_>
struct GemmCfg {
  static constexpr int BX = BX_, BY = BY_;
  static constexpr int WAVES_X = WAVES_X_, WAVES_Y = WAVES_Y_;
  static constexpr int NWAVES = WAVES_X * WAVES_Y;
  static constexpr int NTHREADS = 64 * NWAVES;
  static constexpr int WX = BX / WAVES_X, WY = BY / WAVES_Y;
  static constexpr int FX = WX / 16, FY = WY / 16;
  static constexpr int KB = 128;                        // K bytes per row per stage
  static constexpr int CPR = KB / 16;                   // 16-byte chunks per row
  static constexpr int STAGE_BYTES = (BX + BY) * KB;
  static constexpr int MAIN_LDS = 2 * STAGE_BYTES;
  static constexpr int DMA_PER_WAVE = STAGE_BYTES / 1024 / NWAVES;   // 1 KB wave-wide loads per stage
  static_assert(STAGE_BYTES % (1024 * NWAVES) == 0 && (BX * KB) % 1024 == 0, "DMA blocks");
  static_assert((BX * KB / 1024) % DMA_PER_WAVE == 0, "a wave's blocks are all X or all Y");
  static_assert(WX % 16 == 0 && WY % 64 == 0, "wave tile");
  // chunk swizzle of LDS row r (conflict-free ds_read_b128 fragment reads)
  __device__ __forceinline__ static int swz(int r) { return r & 7; }
};

// The library's configuration: 256 x 256 tiles, 8 waves (4 along X, 2 along Y),
// 64 x 128 outputs per wave (2 x 64 KiB LDS stages).
typedef GemmCfg<256, 256, 4, 2> MainCfg;

constexpr int BX = MainCfg::BX, BY = MainCfg::BY;

// Epilogue staging of the forward gather: per wave WX tokens x 64 vocabulary floats.
constexpr int SPITCH = 68;   // floats per staged token row
template <class C> constexpr int stage_wave_floats() { return C::WX * SPITCH; }
template <class C> constexpr int stats_off() { return C::NWAVES * stage_wave_floats<C>() * 4; }
template <class C> constexpr int fwd_lds() { return stats_off<C>() + C::WAVES_Y * C::BX * 8; }
template <class C, int EPI> constexpr int kernel_lds() {
  return ((EPI == 2 || EPI == 3) && fwd_lds<C>() > C::MAIN_LDS) ? fwd_lds<C>() : C::MAIN_LDS;
}

enum Epi : int {
  EPI_STORE_F32 = 0,   // P -> float out (optionally += existing)
  EPI_STORE_BF16 = 1,  // P -> bf16 out
  EPI_KL_FWD = 2,      // per-row online (max, sum exp) partials + cached-entry gather
  EPI_KL_DZ = 3,       // dZ = (g/N) exp(z - lse) - (cached-entry weights) -> dZ (and, if given, dZ^T)
  EPI_TOPK = 4,        // P -> bf16 out, plus the two largest float32 values of each row in the tile
};

struct GemmArgs {
  const void* X; int64_t ldx;     // [nx][k], elements
  const void* Y; int64_t ldy;     // [ny][k]
  int nx, ny, k;                  // valid rows of X and Y; contraction length
  int n_tx, n_ty, group;          // tile grid and tile-order grouping
  int krows_x, krows_y;           // K-major operands: rows of k that exist (rows past them read as 0)
  // split-K (EPI_STORE_F32 only): n_tx * n_ty * splits workgroups; split s sums its
  // share of the K stages into out + s * split_stride
  int splits;
  int64_t split_stride;
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
  const float* ew;                // EPI_KL_DZ: weight of each bucketed entry (subtracted from dZ)
  const int* offsets;             // [n_tx][n_ty + 1]
  int kc;                         // cache entries per row (K)
  float* zg;                      // [rows][K] gathered logits
  float2* partials;               // [n_ty][ld_part] per row: (max, sum exp) or (1st, 2nd largest)
  int64_t ld_part;
};

// Workgroup -> tile.  Each XCD receives one contiguous range of the logical
// order, and the logical order walks `group` X-tiles for every Y-tile, so the
// tiles that one XCD runs at a time share X and Y strips in its L2.
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

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past any operand: loads return 0

// One wave-wide 16-byte-per-lane buffer load written straight into LDS: lane i's
// data lands at LDS byte address lds_addr + 16 i (lds_addr wave-uniform).  It has no
// destination register; completion is tracked with s_waitcnt vmcnt by the caller.
// Every offset that selects rows goes through voff or the descriptor (both are
// range-checked against the descriptor's size); the scalar offset stays 0.
__device__ __forceinline__ void dma16(uint32_t lds_addr, uint32_t voff, const u32x4& rsrc) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_addr), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Raw buffer descriptor (gfx9 layout) in scalar registers.
__device__ __forceinline__ u32x4 buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t b = (uint64_t)base;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = 0x00020000u;
  return r;
}

template <class C, typename T, int EPI, int XKM = 0, int YKM = 0>
__global__ void __launch_bounds__(C::NTHREADS, 1) gemm_kernel(const GemmArgs a) {
  static_assert(!(XKM || YKM) || (sizeof(T) == 2 && C::BX == 256 && C::BY == 256),
                "K-major operands: bf16, 512-byte k rows");
  __shared__ __attribute__((aligned(16))) char lds[kernel_lds<C, EPI>()];
  constexpr int ES = int(sizeof(T));
  constexpr int EPC = 16 / ES;            // elements per 16-byte chunk
  constexpr int KE = C::KB / ES;          // elements per stage
  constexpr int FX = C::FX, FY = C::FY, WX = C::WX, WY = C::WY, BXc = C::BX, BYc = C::BY;

  const int split = (int)blockIdx.x / (a.n_tx * a.n_ty);
  int tx, ty;
  tile_of((int)blockIdx.x - split * a.n_tx * a.n_ty, a.n_tx, a.n_ty, a.group, tx, ty);
  const int x0 = tx * BXc, y0 = ty * BYc;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wx = wave % C::WAVES_X, wy = wave / C::WAVES_X;

  const int xrows = min(BXc, a.nx - x0), yrows = min(BYc, a.ny - y0);

  f32x4 acc[FX][FY];
#pragma unroll
  for (int i = 0; i < FX; ++i)
#pragma unroll
    for (int j = 0; j < FY; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane fragment read offsets of the two 64-byte halves of a stage row
  // (fragment rows start at multiples of 16, so the swizzle depends on lane % 16)
  const int fr = lane & 15, fq = lane >> 4;
  uint32_t xs[2], ys[2];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int ch = (f * 4 + fq) ^ C::swz(fr);
    xs[f] = uint32_t((wx * WX + fr) * C::KB + ch * 16);
    ys[f] = uint32_t((BXc + wy * WY + fr) * C::KB + ch * 16);
  }
  const int nk_all = (a.k + KE - 1) / KE;
  const int k_per = (nk_all + a.splits - 1) / a.splits;
  const int st0 = split * k_per;                          // this workgroup's first stage
  const int nk = max(0, min(k_per, nk_all - st0));
  {
    // ---- LDS-DMA pipeline.  Stage kt lives in LDS buffer kt % 2.
    constexpr int DPW = C::DMA_PER_WAVE;
    constexpr int RPB = 1024 / C::KB;                    // rows per 1 KB DMA block
    constexpr int XBLK = BXc * C::KB / 1024;             // X blocks per stage
    const uint32_t lds_base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
    // block b of a stage: rows b*RPB .. of X (b < XBLK) or of Y
    const bool wave_x = wave * DPW < XBLK;               // a wave's blocks are all X or all Y
    const bool wave_km = wave_x ? (XKM != 0) : (YKM != 0);
    const int bl0 = wave * DPW - (wave_x ? 0 : XBLK);    // first block of this wave in its operand
    const int64_t ld = wave_x ? a.ldx : a.ldy;
    const uint32_t ldb = uint32_t(ld * ES);              // operand row stride in bytes
    const int col0 = wave_x ? x0 : y0;
    const char* opb = (const char*)(wave_x ? a.X : a.Y); // operand base
    const uint32_t op_rows = uint32_t(wave_x ? xrows : yrows);
    const int krows = wave_x ? a.krows_x : a.krows_y;
    // Row-major: block = RPB rows x 128 bytes; lane -> (row, swizzled 16-byte chunk),
    // one offset per block from the tile's descriptor (rows past the tile's valid
    // rows fall outside it and read as 0)
    const u32x4 od = buffer_desc(opb + (int64_t)col0 * ld * ES, op_rows * ldb);
    const int lrow = lane / C::CPR;
    const int lch = (lane % C::CPR) ^ C::swz(lrow);      // RPB = 8: the swizzle depends on the lane alone
    const int kq = lch * EPC;                            // first k element of this lane's chunk
    // K-major: a stage of an operand is 64 k-rows x 256 columns (32 KB).  LDS byte
    //   1024 m + 256 b + 128 r1 + 32 e + 16 c + 8 hf   holds k-row
    //   16 (m & 1) + 8 r1 + e + 4 ((m >> 3) & 1) + 32 (m >> 4),  columns
    //   16 (b + 4 ((m >> 1) & 3)) + 8 c + 4 hf + 0..3,
    // i.e. fragment G = b + 4 ((m >> 1) & 3) (16 columns), k-half f = m >> 4,
    // k-quad h = (m >> 3) & 1 and rows 8 g + e with g = 2 (m & 1) + r1.  DMA m writes
    // the 1 KB at 1024 m; its lane L covers b = L / 16, r1 = (L / 8) & 1,
    // e = (L / 2) & 3, c = L & 1, which in the operand is rows 8 r1 + e and bytes
    // 32 b + 16 c past the DMA's first row and column.
    // Per-block offsets, loop-invariant: row-major block q is rows (bl0 + q) RPB ..;
    // K-major block m = bl0 + q starts at k-row r0(m) and byte cb(m) of the row.
    const uint32_t voff_km = uint32_t((8 * ((lane >> 3) & 1) + ((lane >> 1) & 3)) * ldb +
                                      (2 * (lane >> 4) + (lane & 1)) * 16);
    uint32_t voff[DPW];
#pragma unroll
    for (int q = 0; q < DPW; ++q) {
      const int m = bl0 + q;
      const int r0 = 16 * (m & 1) + 4 * ((m >> 3) & 1) + 32 * (m >> 4);
      voff[q] = wave_km ? voff_km + uint32_t(r0) * ldb + uint32_t(col0 * ES + 128 * ((m >> 1) & 3))
                        : uint32_t((m * RPB + lrow) * ldb + lch * 16);
    }
    auto issue = [&](int stage, int buf) {
      const int k0 = (st0 + stage) * KE;
      const uint32_t ldsb = lds_base + uint32_t(buf * C::STAGE_BYTES + wave * DPW * 1024);
      if (wave_km) {
        // one descriptor per stage from k-row k0, column 0 of the operand's rows: rows
        // past krows, and bytes past the end of the last valid row, read as 0
        const int rows = krows - k0;
        const int64_t nb = (int64_t)rows * ldb;
        const u32x4 d = buffer_desc(opb + (int64_t)k0 * ldb,
                                    rows > 0 ? uint32_t(nb < 0xffffffffll ? nb : 0xffffffffll) : 0u);
#pragma unroll
        for (int q = 0; q < DPW; ++q) dma16(ldsb + q * 1024, voff[q], d);
      } else {
        // chunks at or past k read as 0
        const bool kin = k0 + kq < a.k;
#pragma unroll
        for (int q = 0; q < DPW; ++q) dma16(ldsb + q * 1024, kin ? voff[q] + uint32_t(k0 * ES) : kOOB, od);
      }
    };
    // K-major fragment G of k-half f: lane 16 g + 4 e + q reads k-rows 8 g + e (+4)
    // at columns 16 G + 4 q; lane part of the address, the rest are immediates
    const uint32_t trb = uint32_t(1024 * (lane >> 5) + 128 * ((lane >> 4) & 1) + 32 * ((lane >> 2) & 3) +
                                  8 * (lane & 3));
    auto trfrag = [&](const char* region, int G, int f) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      const char* p = region + trb + 256 * (G & 3) + 2048 * (G >> 2) + 16384 * f;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)p);
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 8192));
      const u32x2 a0 = __builtin_bit_cast(u32x2, lo), a1 = __builtin_bit_cast(u32x2, hi);
      return u32x4{a0[0], a0[1], a1[0], a1[1]};
    };
    auto rdfrag = [&](u32x4 (&bx)[FX], u32x4 (&by)[FY], int buf, int f) {
      const char* base = lds + buf * C::STAGE_BYTES;
#pragma unroll
      for (int i = 0; i < FX; ++i) {
        if constexpr (XKM) bx[i] = trfrag(base, (wx * WX) / 16 + i, f);
        else bx[i] = *(const u32x4*)(base + xs[f] + i * 16 * C::KB);
      }
#pragma unroll
      for (int j = 0; j < FY; ++j) {
        if constexpr (YKM) by[j] = trfrag(base + BXc * C::KB, (wy * WY) / 16 + j, f);
        else by[j] = *(const u32x4*)(base + ys[f] + j * 16 * C::KB);
      }
    };
    auto mma = [&](const u32x4 (&bx)[FX], const u32x4 (&by)[FY]) {
#pragma unroll
      for (int i = 0; i < FX; ++i)
#pragma unroll
        for (int j = 0; j < FY; ++j) Mma<T>::run(acc[i][j], by[j], bx[i]);
    };
    // With a K-major operand (twice the LDS reads: two transposing reads per fragment)
    // the next half's reads are spread over this half's MFMAs, one read per two MFMAs
    // (measured: dW 2.7 % faster).  Row-major operands keep the compiler's schedule,
    // which measured 3 % faster than this interleave for them.
    auto interleave = [&]() {
      if constexpr (XKM || YKM) {
        constexpr int NREAD = (XKM ? 2 : 1) * FX + (YKM ? 2 : 1) * FY;
        constexpr int NMMA = FX * FY;
        constexpr int PER = NMMA / NREAD > 0 ? NMMA / NREAD : 1;
#pragma unroll
        for (int r = 0; r < NREAD; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
          __builtin_amdgcn_sched_group_barrier(0x008, PER, 0); // then PER MFMAs
        }
        if constexpr (NMMA > PER * NREAD) __builtin_amdgcn_sched_group_barrier(0x008, NMMA - PER * NREAD, 0);
      }
    };
    // The waves of the second Y half (the ones that load Y) get the higher issue
    // priority, so they run ahead of the X loaders instead of behind them (measured:
    // dW 2.6 %, dZ 1.2 %, forward 0.9 % faster; the dH products 0.4 % slower, so they
    // keep equal priorities).
    if constexpr (XKM || EPI == EPI_KL_FWD || EPI == EPI_KL_DZ || EPI == EPI_TOPK) {
      if (wy == C::WAVES_Y - 1) __builtin_amdgcn_s_setprio(1);
    }
    issue(0, 0);
    wait_vmcnt<0>();
    __syncthreads();
    issue(1, 1);
    u32x4 h0x[FX], h0y[FY], h1x[FX], h1y[FY];
    rdfrag(h0x, h0y, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      rdfrag(h1x, h1y, cur, 1);          // second half of stage kt
      mma(h0x, h0y);                     // first half of stage kt
      interleave();
      wait_vmcnt<0>();                   // own loads of stage kt + 1 have landed
      __syncthreads();                   // everyone's; every read of stage kt is done
      issue(kt + 2, cur);                // stage kt + 2 into stage kt's buffer (past K: zeros;
                                         // past this split's stages: loaded, never read)
      rdfrag(h0x, h0y, cur ^ 1, 0);      // first half of stage kt + 1
      mma(h1x, h1y);                     // second half of stage kt
      interleave();
    }
    wait_vmcnt<0>();
    __syncthreads();
  }

  // ---- epilogues.  Lane (i, j, e) holds P[n = x0 + wx*WX + i*16 + lane%16][m = mcol + j*16 + e].
  const int nrow0 = x0 + wx * WX + (lane & 15);
  const int mcol = y0 + wy * WY + (lane >> 4) * 4;

  if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_STORE_BF16 || EPI == EPI_TOPK) {
    typedef typename std::conditional<EPI == EPI_STORE_BF16 || EPI == EPI_TOPK, bf16_t, float>::type OT;
#pragma unroll
    for (int i = 0; i < FX; ++i) {
      const int n = nrow0 + i * 16;
      if (n >= a.out_rows) continue;
      OT* orow = (OT*)a.out + split * a.split_stride + (int64_t)n * a.ldo;
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
    if constexpr (EPI == EPI_TOPK) {
      // The two largest values of each row among the tile's valid columns: in-lane,
      // then over the 4 lanes sharing the row, then over the waves along Y in LDS.
      // Distinct elements of the row, so the K-th largest over all tiles' pairs
      // bounds the row's K-th largest from below.
      float2* st = (float2*)lds;   // the main loop's buffers are free after its last barrier
#pragma unroll
      for (int i = 0; i < FX; ++i) {
        float a1 = -INFINITY, a2 = -INFINITY;
#pragma unroll
        for (int j = 0; j < FY; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float v = acc[i][j][e];
            if (mcol + j * 16 + e < a.ny) {
              a2 = fmaxf(a2, fminf(a1, v));
              a1 = fmaxf(a1, v);
            }
          }
#pragma unroll
        for (int o = 16; o <= 32; o <<= 1) {
          const float b1 = __shfl_xor(a1, o), b2 = __shfl_xor(a2, o);
          a2 = fmaxf(fminf(a1, b1), fmaxf(a2, b2));
          a1 = fmaxf(a1, b1);
        }
        if ((lane >> 4) == 0) st[wy * BXc + wx * WX + i * 16 + lane] = make_float2(a1, a2);
      }
      __syncthreads();
      if (tid < BXc) {
        float2 t = st[tid];
#pragma unroll
        for (int w = 1; w < C::WAVES_Y; ++w) {
          const float2 b = st[w * BXc + tid];
          t.y = fmaxf(fminf(t.x, b.x), fmaxf(t.y, b.y));
          t.x = fmaxf(t.x, b.x);
        }
        const int row = x0 + tid;
        if (row < a.nx) a.partials[(int64_t)ty * a.ld_part + row] = t;
      }
    }
  } else if constexpr (EPI == EPI_KL_FWD) {
    // (1) per-token max and sum of exp over this wave's WY vocabulary columns.
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
    // (2) merge the waves that share these tokens; one partial per (row, vocab tile).
    float2* st = (float2*)(lds + stats_off<C>());
    if ((lane >> 4) == 0) {
#pragma unroll
      for (int i = 0; i < FX; ++i) st[wy * BXc + wx * WX + i * 16 + lane] = make_float2(tm[i], ts[i]);
    }
    // (3) gather the cached entries that fall in this tile (wave-private LDS staging).
    float* sw = (float*)lds + wave * stage_wave_floats<C>();
    const int* off = a.offsets + (int64_t)tx * (a.n_ty + 1) + ty;
    const int eb = off[0], ee = off[1];
    const uint32_t* ent = a.entries + (int64_t)tx * BXc * a.kc;
#pragma unroll
    for (int rnd = 0; rnd < WY / 64; ++rnd) {
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
    if (tid < BXc) {
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < C::WAVES_Y; ++w) M = fmaxf(M, st[w * BXc + tid].x);
      float S = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < C::WAVES_Y; ++w) {
          const float2 p = st[w * BXc + tid];
          S += p.y * fast_exp2((p.x - M) * kLog2e);
        }
      }
      const int row = x0 + tid;
      if (row < a.nx) a.partials[(int64_t)ty * a.ld_part + row] = make_float2(M, S);
    }
  } else if constexpr (EPI == EPI_KL_DZ) {
    // dZ in 64 x 64 blocks (one wave's tokens x 64 vocabulary columns per round),
    // staged in the wave's LDS: (1) the softmax part, (2) minus the weights of the
    // tile's cached entries that fall in the block, (3) one rounding to T and a
    // row-contiguous store (and for float32 inputs a token-contiguous store of dZ^T).
    const float g = a.grad ? *a.grad : 1.0f;
    const float scale = g * a.inv_n;
    T* dz = (T*)a.out;
    T* dzt = (T*)a.out2;
    float* sw = (float*)lds + wave * stage_wave_floats<C>();
    const int tlo = wx * WX;
    const int* off = a.offsets + (int64_t)tx * (a.n_ty + 1) + ty;
    const int eb = off[0], ee = off[1];
    const uint32_t* ent = a.entries + (int64_t)tx * BXc * a.kc;
    const float* ewt = a.ew + (int64_t)tx * BXc * a.kc;
    float nl[FX];
    bool rv[FX];
#pragma unroll
    for (int i = 0; i < FX; ++i) {
      const int n = nrow0 + i * 16;
      rv[i] = n < a.nx;
      nl[i] = rv[i] ? -a.lse[n] * kLog2e : 0.f;
    }
    const int row0 = x0 + tlo;
#pragma unroll
    for (int rnd = 0; rnd < WY / 64; ++rnd) {
      const int vlo = wy * WY + rnd * 64;
      const int col0 = y0 + vlo;
#pragma unroll
      for (int i = 0; i < FX; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int m = mcol + (rnd * 4 + jj) * 16;
          f32x4 v;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = (rv[i] && m + e < a.ny) ? scale * fast_exp2(fmaf(acc[i][rnd * 4 + jj][e], kLog2e, nl[i])) : 0.f;
          *(f32x4*)(sw + (i * 16 + (lane & 15)) * SPITCH + jj * 16 + (lane >> 4) * 4) = v;
        }
      wave_sync_lds();
      // Entries of this block: lanes take 64 bucket entries at a time; lanes that hold
      // the same (token, column) form a group whose lowest lane subtracts the group's
      // summed weights, added in lane order (the bucket's order, which is k order for
      // one token and column), so repeated indices accumulate in a fixed order.
      for (int e0 = eb; e0 < ee; e0 += 64) {
        const int e = e0 + lane;
        int key = -1;
        float wgt = 0.f;
        if (e < ee) {
          const uint32_t u = ent[e];
          const int t = int(u & 255u) - tlo, v = int((u >> 8) & 255u) - vlo;
          if (t >= 0 && t < WX && v >= 0 && v < 64) {
            key = t * SPITCH + v;
            wgt = ewt[e];
          }
        }
        uint64_t todo = __ballot(key >= 0);
        while (todo) {
          const int l = __builtin_ctzll(todo);
          const int kl = __builtin_amdgcn_readlane(key, l);
          const uint64_t m = __ballot(key == kl);
          float sum = 0.f;
          for (uint64_t mm = m; mm; mm &= mm - 1)
            sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), __builtin_ctzll(mm)));
          if (lane == l) sw[kl] -= sum;
          todo &= ~m;
        }
      }
      wave_sync_lds();
      if (row0 < a.out_rows && col0 < a.out_cols) {
        if constexpr (sizeof(T) == 2) {
          // 8 rows per store instruction, 8 lanes x 16 bytes per 64-column row segment:
          // each segment is one whole, aligned 128-byte line, written non-temporally
          // (L2 has nothing to merge, and the chunk's 4 GB of dZ does not displace the
          // operand strips there; measured 0.5-0.8 % faster.  The other epilogues write
          // parts of lines and measured slower with non-temporal stores.)
#pragma unroll
          for (int r8 = 0; r8 < 64; r8 += 8) {
            const int r = r8 + (lane >> 3), c = (lane & 7) * 8;
            const float* q = sw + r * SPITCH + c;
            const f32x4 lo = *(const f32x4*)q, hi = *(const f32x4*)(q + 4);
            u32x4 w;
            w[0] = uint32_t(f32_to_bf16(lo[0])) | (uint32_t(f32_to_bf16(lo[1])) << 16);
            w[1] = uint32_t(f32_to_bf16(lo[2])) | (uint32_t(f32_to_bf16(lo[3])) << 16);
            w[2] = uint32_t(f32_to_bf16(hi[0])) | (uint32_t(f32_to_bf16(hi[1])) << 16);
            w[3] = uint32_t(f32_to_bf16(hi[2])) | (uint32_t(f32_to_bf16(hi[3])) << 16);
            if (row0 + r < a.out_rows) __builtin_nontemporal_store(w, (u32x4*)(dz + (int64_t)(row0 + r) * a.ldo + col0 + c));
          }
        } else {
          // 4 rows per store instruction, 16 lanes x 16 bytes per row segment
#pragma unroll
          for (int r4 = 0; r4 < 64; r4 += 4) {
            const int r = r4 + (lane >> 4), c = (lane & 15) * 4;
            if (row0 + r < a.out_rows) *(f32x4*)(dz + (int64_t)(row0 + r) * a.ldo + col0 + c) = *(const f32x4*)(sw + r * SPITCH + c);
          }
          if (dzt && row0 + lane < a.out_rows) {
            // dZ^T: lane = token, so each store covers 64 consecutive tokens of one column
            for (int c = 0; c < 64; ++c) dzt[(int64_t)(col0 + c) * a.ldo2 + row0 + lane] = sw[lane * SPITCH + c];
          }
        }
      }
      wave_sync_lds();
    }
  }
}

}  // namespace kd
