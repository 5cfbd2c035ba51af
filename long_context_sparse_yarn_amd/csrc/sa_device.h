// Device-side helpers shared by the gfx950 kernels of the sink-attention
// library: vector types for the matrix-core operands, bf16 conversions and
// wave-level reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

#define SA_LOG2E 1.4426950408889634f

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (inputs are finite here).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two fp32 -> packed bf16 pair with the hardware conversion
// (v_cvt_pk_bf16_f32, round to nearest even).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

// acc + lo(w) + hi(w) for a packed bf16 pair (v_dot2c_f32_bf16 against 1, 1).
__device__ __forceinline__ float sum_bf16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
}

// fp64 -> bf16 with one rounding (to nearest, ties to even).  First round
// to fp32 to nearest (hardware).  A bf16 rounding midpoint is itself an fp32
// value, so that first step can only land ON a midpoint, never across one;
// when it lands on one (low 16 bits 0x8000) without being exact, the fp64
// value says which side it came from and the bf16 rounding goes that way.
// Otherwise rounding the fp32 value to bf16 to nearest even is exact.
// Both candidates are computed and one is selected, so a wave takes no
// branch per element.
__device__ __forceinline__ uint32_t f64_to_bf16_bits(double x) {
  const float t = (float)x;
  const uint32_t u = __float_as_uint(t);
  const uint32_t nearest = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const double td = (double)t;
  const uint32_t side = (fabs(x) > fabs(td) ? u + 0x8000u : u) >> 16;
  const bool on_mid = ((u & 0xFFFFu) == 0x8000u) & (td != x);
  return on_mid ? side : nearest;
}

// ---------------------------------------------------------------- loads
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// ---------------------------------------------------------------- MFMA
// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).  Lane l supplies
// row l%16 of A and column l%16 of B, each as the 8 contraction elements
// 8*(l/16) .. 8*(l/16)+7; it receives D rows 4*(l/16) .. +3 of column l%16.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------- wave ops
__device__ __forceinline__ float xor_max(float v, int m) {
  return fmaxf(v, __shfl_xor(v, m, 64));
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// max over the four lanes l, l^16, l^32, l^48 (one query column of a
// 16x16 MFMA result), with the gfx950 lane-swap instructions.
__device__ __forceinline__ float max_over_col(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_col(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
