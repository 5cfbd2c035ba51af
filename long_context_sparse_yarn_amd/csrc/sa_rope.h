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

}  // namespace sa_rope
