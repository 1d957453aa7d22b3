// Device-side helpers shared by the kdkl kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bfloat16 values are stored and moved as their 16-bit patterns.
typedef uint16_t bf16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(bf16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// float32 -> bfloat16, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return bf16_t(0x7fc0);
  u += 0x7fffu + ((u >> 16) & 1u);
  return bf16_t(u >> 16);
}

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Order-preserving map float -> uint32 (larger float <-> larger key).
__device__ __forceinline__ uint32_t float_key(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// float64 -> bfloat16 bits, a single rounding to nearest even (no float32 step).
__device__ __forceinline__ bf16_t f64_to_bf16_rne(double x) {
  if (x != x) return bf16_t(0x7fc0);
  const double ax = fabs(x);
  double r;
  if (ax < 0x1p-126) {
    r = rint(ax * 0x1p133) * 0x1p-133;           // bf16 subnormal spacing 2^-133
  } else {
    uint64_t b = (uint64_t)__double_as_longlong(ax);
    b += 0xfffffffffffull + ((b >> 45) & 1ull);  // keep 7 explicit mantissa bits, ties to even
    b &= ~((1ull << 45) - 1ull);
    r = __longlong_as_double((long long)b);
  }
  const float f = (float)r;                      // exact, or +inf past the bf16 range
  bf16_t h = bf16_t(__float_as_uint(f) >> 16);
  if (x < 0) h |= 0x8000;
  return h;
}

// Hardware dispatches workgroup b to XCD (b % 8) on MI355X.
constexpr int kXcds = 8;

}  // namespace kd
