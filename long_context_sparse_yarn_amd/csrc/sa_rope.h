// Angle and rotation arithmetic shared by the RoPE kernels (yarn_rope and
// the rotate-and-append path), so that both produce the same bits.
//
// "MoE-Xtend" README, ROPE + SCALING: pair i = coordinates (i, i + d/2) at
// position p is rotated by the angle p * inv_freq_i, with cos and sin both
// scaled by the YaRN concentration c.
//
// Angles: a = p * inv_freq_i is formed in fp64 (it reaches 1.3e5 rad at 128K
// context, where fp32 would lose ~1e-2 rad) and reduced modulo pi/2 in fp64
// with a two-part pi/2 (Cody and Waite's method); sin and cos of the reduced
// angle |r| <= pi/4 come from their Taylor series to degree 17/18 (the first
// dropped terms are below 1e-19), evaluated in fp64.
#pragma once

#include "sa_device.h"

namespace sa_rope {

// (cos a, sin a) for an fp64 angle a >= 0.
__device__ __forceinline__ void sincos_reduced(double a, double* s_out, double* c_out) {
  constexpr double kTwoOverPi = 0.63661977236758134308;
  constexpr double kPio2Hi = 1.5707963267948966192;       // fp64 nearest pi/2
  constexpr double kPio2Lo = 6.123233995736766036e-17;    // pi/2 - kPio2Hi
  const double k = rint(a * kTwoOverPi);
  double r = fma(-k, kPio2Hi, a);
  r = fma(-k, kPio2Lo, r);
  const double z = r * r;
  // 1/n! by recurrence
  constexpr double f3 = 1.0 / 6.0, f5 = f3 / 20.0, f7 = f5 / 42.0, f9 = f7 / 72.0,
                   f11 = f9 / 110.0, f13 = f11 / 156.0, f15 = f13 / 210.0, f17 = f15 / 272.0;
  constexpr double f2 = 0.5, f4 = f2 / 12.0, f6 = f4 / 30.0, f8 = f6 / 56.0, f10 = f8 / 90.0,
                   f12 = f10 / 132.0, f14 = f12 / 182.0, f16 = f14 / 240.0, f18 = f16 / 306.0;
  double sp = fma(z, -f17, f15);
  sp = fma(z, sp, -f13);
  sp = fma(z, sp, f11);
  sp = fma(z, sp, -f9);
  sp = fma(z, sp, f7);
  sp = fma(z, sp, -f5);
  sp = fma(z, sp, f3);
  const double sr = fma(-r * z, sp, r);                    // r - r^3/3! + ...
  double cp = fma(z, f18, -f16);
  cp = fma(z, cp, f14);
  cp = fma(z, cp, -f12);
  cp = fma(z, cp, f10);
  cp = fma(z, cp, -f8);
  cp = fma(z, cp, f6);
  cp = fma(z, cp, -f4);
  cp = fma(z, cp, f2);
  const double cr = fma(-z, cp, 1.0);                      // 1 - r^2/2! + ...
  const int q = (int)((int64_t)k & 3);
  const double s = (q & 1) ? cr : sr;
  const double c = (q & 1) ? sr : cr;
  *s_out = (q & 2) ? -s : s;
  *c_out = ((q + 1) & 2) ? -c : c;
}


// The two outputs of a pair (u, v) = (x_i, x_{i+d/2}) under (c*cos, c*sin):
// u' = u*cc - v*ss and v' = v*cc + u*ss, each with one fused multiply-add so
// that every kernel computing them gets the same fp64 value.
__device__ __forceinline__ double rot_first(double u, double v, double cc, double ss) {
  return fma(u, cc, -(v * ss));
}
__device__ __forceinline__ double rot_second(double u, double v, double cc, double ss) {
  return fma(v, cc, u * ss);
}

// ---- bf16 rows: the same bits from fp32 arithmetic where that is provably
// safe.  For a pair (u, v) of bf16 values and the fp64 entries (cc, ss),
// |cc|, |ss| <= c (the concentration), the fp32 evaluation
//     y32 = fmaf(u, cc32, -(v*ss32)),   cc32, ss32 = fp32 roundings of cc, ss,
// differs from the fp64 value y64 = rot_first(u, v, cc, ss) by at most
// 1.5 * 2^-23 (|u cc| + |v ss|) (two representation errors and two
// roundings of 2^-24; the fp64 errors are 2^-29 times smaller), so by less
// than E = 2^-22 c (|u| + |v|).  Rounding to bf16 changes only at midpoints
// of bf16 intervals.  y32 lies in its interval at distance dist <= ulp/2
// from the interval's midpoint, and the nearest other midpoint is at least
// ulp/4 away (ulp/4 where the interval starts a binade).  So if
//     dist > 2E
// then E < ulp/4 and E < dist: y64 lies on y32's side of every midpoint and
// both round to the same bf16.  Then the fp32 value is used (packed to bf16
// by the hardware conversion, round to nearest even); otherwise -- near-ties,
// strong cancellation, NaN or infinity, |u| + |v| below 2^-100 where fp32
// products may underflow -- the fp64 rotation is evaluated.  Likewise for
// rot_second (same E).  k2 = 2 * 2^-22 * c, rounded up with room for the
// rounding of |u| + |v| (bf16_rot_k2).
__device__ __forceinline__ float bf16_rot_k2(double conc) {
  return (float)(conc * 0x1p-21 * (1.0 + 0x1p-12));
}
__device__ __forceinline__ float bf16_mid(float y) {
  return __uint_as_float((__float_as_uint(y) & 0xFFFF0000u) | 0x8000u);
}

// Rotate 8 pairs: a holds coordinates i..i+7 (bf16), b coordinates
// i+d/2..i+d/2+7; fe / de the fp32 / fp64 (c*cos, c*sin) of pairs i..i+7.
// Writes the rotated halves to *wa, *wb with the bits of the fp64 rotation
// rounded once (f64_to_bf16_bits).
__device__ __forceinline__ void rot8_bf16(u32x4 a, u32x4 b, const float2* fe,
                                          const double2* de, float k2, u32x4* wa, u32x4* wb) {
  // fp32 values of pair i; the three conditions for using them go into wave
  // masks (scalar ANDs), not into per-lane bits
  auto fast = [&](int i, float* f1, float* f2, uint64_t* okm) {
    const float u = (i & 1) ? bf16_hi(a[i >> 1]) : bf16_lo(a[i >> 1]);
    const float v = (i & 1) ? bf16_hi(b[i >> 1]) : bf16_lo(b[i >> 1]);
    const float2 e = fe[i];
    *f1 = fmaf(u, e.x, -(v * e.y));
    *f2 = fmaf(v, e.x, u * e.y);
    const float sum = fabsf(u) + fabsf(v);
    const float tol = sum * k2;
    *okm &= __builtin_amdgcn_ballot_w64(sum >= 0x1p-100f) &
            __builtin_amdgcn_ballot_w64(fabsf(*f1 - bf16_mid(*f1)) > tol) &
            __builtin_amdgcn_ballot_w64(fabsf(*f2 - bf16_mid(*f2)) > tol);
  };
  const uint64_t live = __builtin_amdgcn_ballot_w64(true);
  float y1[8], y2[8];
  uint64_t okm[8];                    // per pair: the lanes whose fp32 values stand (wave-uniform)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    okm[i] = live;
    fast(i, &y1[i], &y2[i], &okm[i]);
  }
  u32x4 ra, rb;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    ra[j] = pack_bf16x2(y1[2 * j], y1[2 * j + 1]);
    rb[j] = pack_bf16x2(y2[2 * j], y2[2 * j + 1]);
  }
  // rare: the pairs some lane could not decide take the fp64 rotation on
  // those lanes (no recomputation of the others)
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (okm[i] != live && !((okm[i] >> __lane_id()) & 1)) {
      const double u = (double)((i & 1) ? bf16_hi(a[i >> 1]) : bf16_lo(a[i >> 1]));
      const double v = (double)((i & 1) ? bf16_hi(b[i >> 1]) : bf16_lo(b[i >> 1]));
      const double2 e = de[i];
      const uint32_t r1 = f64_to_bf16_bits(rot_first(u, v, e.x, e.y));
      const uint32_t r2 = f64_to_bf16_bits(rot_second(u, v, e.x, e.y));
      const int j = i >> 1;
      if (i & 1) {
        ra[j] = (ra[j] & 0xFFFFu) | (r1 << 16);
        rb[j] = (rb[j] & 0xFFFFu) | (r2 << 16);
      } else {
        ra[j] = (ra[j] & 0xFFFF0000u) | r1;
        rb[j] = (rb[j] & 0xFFFF0000u) | r2;
      }
    }
  }
  *wa = ra;
  *wb = rb;
}

}  // namespace sa_rope
