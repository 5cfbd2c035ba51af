// yarn_rope / yarn_rope_apply: rotate head rows at global positions, from a
// source buffer into a destination (the same buffer for the in-place form).
//
// "MoE-Xtend" README, ROPE + SCALING: cos/sin of (position * inv_freq_i),
// both scaled by the YaRN concentration c; DESIGN CONTRACTS: the position is
// the global index offset + t and never resets.  Pair i is coordinates
// (i, i + d/2).
//
// Angles: a = p * inv_freq_i is formed in fp64 (it reaches 1.3e5 rad at 128K
// context, where fp32 would lose ~1e-2 rad) and reduced modulo pi/2 in fp64
// with a two-part pi/2 (Cody and Waite's method); sin and cos of the reduced
// angle |r| <= pi/4 come from their Taylor series to degree 17/18 (the first
// dropped terms are below 1e-19), evaluated in fp64.
//
// One workgroup takes `rows` consecutive (b, t) rows.  Each thread first
// issues the 16-byte loads of its (row, head, 8-pair chunk) tasks; the
// workgroup then builds the (c*cos, c*sin) table of its rows once in LDS, so
// that work overlaps the memory latency and is shared by all heads.  Pairs
// are rotated in fp64 and rounded once to the storage type (an fp32 rotation
// would lose many bf16 ulps where the two products nearly cancel).  The
// kernel is HBM-bound: each element is read and written once.
#include "sa_device.h"
#include "sa_kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTasks = 2;            // 8-pair chunks per thread
constexpr int kMaxTable = 1024;      // rows * d/2 table entries in LDS (16 KB)

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

template <int ELT>
struct Rot;
template <>
struct Rot<2> {                      // bf16: 8 values in one 16-byte vector, fp64 math
  typedef double2 Entry;
  u32x4 w;
  __device__ __forceinline__ void load(const char* p) { w = ld16(p); }
  __device__ __forceinline__ double get(int i) const {
    const uint32_t u = w[i >> 1];
    return (double)((i & 1) ? bf16_hi(u) : bf16_lo(u));
  }
  __device__ __forceinline__ static Entry entry(double c, double s) { return make_double2(c, s); }
  __device__ __forceinline__ static void rotate(const Rot& a, const Rot& b, const Entry* e,
                                                char* pa, char* pb) {
    uint32_t y1[8], y2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double u = a.get(i), v = b.get(i);
      y1[i] = f64_to_bf16_bits(u * e[i].x - v * e[i].y);
      y2[i] = f64_to_bf16_bits(v * e[i].x + u * e[i].y);
    }
    st16(pa, u32x4{y1[0] | (y1[1] << 16), y1[2] | (y1[3] << 16), y1[4] | (y1[5] << 16),
                   y1[6] | (y1[7] << 16)});
    st16(pb, u32x4{y2[0] | (y2[1] << 16), y2[2] | (y2[3] << 16), y2[4] | (y2[5] << 16),
                   y2[6] | (y2[7] << 16)});
  }
};
template <>
struct Rot<4> {                      // fp32: 8 values in two 16-byte vectors, fp64 math
  typedef double2 Entry;
  f32x4 w0, w1;
  __device__ __forceinline__ void load(const char* p) {
    w0 = *reinterpret_cast<const f32x4*>(p);
    w1 = *reinterpret_cast<const f32x4*>(p + 16);
  }
  __device__ __forceinline__ double get(int i) const { return (double)(i < 4 ? w0[i] : w1[i - 4]); }
  __device__ __forceinline__ static Entry entry(double c, double s) { return make_double2(c, s); }
  __device__ __forceinline__ static void rotate(const Rot& a, const Rot& b, const Entry* e,
                                                char* pa, char* pb) {
    f32x4 o[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double u = a.get(i), v = b.get(i);
      o[i >> 2][i & 3] = (float)(u * e[i].x - v * e[i].y);
      o[2 + (i >> 2)][i & 3] = (float)(v * e[i].x + u * e[i].y);
    }
    *reinterpret_cast<f32x4*>(pa) = o[0];
    *reinterpret_cast<f32x4*>(pa + 16) = o[1];
    *reinterpret_cast<f32x4*>(pb) = o[2];
    *reinterpret_cast<f32x4*>(pb + 16) = o[3];
  }
};

template <int ELT>
__global__ __launch_bounds__(kThreads) void rope_kernel(RopeArgs a, int rows) {
  typedef typename Rot<ELT>::Entry Entry;
  __shared__ Entry cs[kMaxTable];
  const int half = a.d >> 1;
  const int cpr = half >> 3;               // 8-pair chunks per head
  const int per_row = a.H * cpr;
  const int row0 = blockIdx.x * rows;
  const int nrows = min(rows, a.BT - row0);
  const int ntask = nrows * per_row;
  const char* src = reinterpret_cast<const char*>(a.src);
  char* base = reinterpret_cast<char*>(a.x);

  Rot<ELT> x1[kTasks], x2[kTasks];
  char* ptr[kTasks];
  int tab[kTasks];
#pragma unroll
  for (int k = 0; k < kTasks; ++k) {
    const int e = threadIdx.x + k * kThreads;
    ptr[k] = nullptr;
    tab[k] = 0;
    if (e < ntask) {
      const int r = e / per_row;
      const int rem = e - r * per_row;
      const int h = rem / cpr, ch = rem - h * cpr;
      const int64_t off = (((int64_t)(row0 + r) * a.H + h) * a.d + 8 * ch) * ELT;
      ptr[k] = base + off;
      tab[k] = r * half + 8 * ch;
      x1[k].load(src + off);
      x2[k].load(src + off + half * ELT);
    }
  }
  for (int e = threadIdx.x; e < nrows * half; e += kThreads) {
    const int r = e / half, i = e - r * half;
    const int t = (row0 + r) % a.T;
    double sn, cn;
    sincos_reduced((double)(a.offset + t) * a.inv_freq[i], &sn, &cn);
    cs[e] = Rot<ELT>::entry(cn * a.conc, sn * a.conc);
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kTasks; ++k)
    if (ptr[k]) Rot<ELT>::rotate(x1[k], x2[k], &cs[tab[k]], ptr[k], ptr[k] + half * ELT);
}

// Fallback for d/2 not a multiple of 8 (d in {8, 24, 40, ...}) or rows
// wider than one workgroup's tasks: one pair per thread and step, fp64.
template <int ELT>
__global__ __launch_bounds__(kThreads) void rope_pairs_kernel(RopeArgs a) {
  const int half = a.d >> 1;
  const int64_t n = (int64_t)a.BT * a.H * half;
  for (int64_t e = blockIdx.x * (int64_t)kThreads + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * kThreads) {
    const int i = (int)(e % half);
    const int64_t rh = e / half;                     // row * H + h
    const int t = (int)((rh / a.H) % a.T);
    double sn, cn;
    sincos_reduced((double)(a.offset + t) * a.inv_freq[i], &sn, &cn);
    const double cc = cn * a.conc, ss = sn * a.conc;
    const int64_t off = (rh * a.d + i) * ELT;
    const char* sp = reinterpret_cast<const char*>(a.src) + off;
    const char* sq = sp + half * ELT;
    char* p = reinterpret_cast<char*>(a.x) + off;
    char* q = p + half * ELT;
    if (ELT == 2) {
      const double u = bf16_to_f32(*reinterpret_cast<const uint16_t*>(sp));
      const double v = bf16_to_f32(*reinterpret_cast<const uint16_t*>(sq));
      *reinterpret_cast<uint16_t*>(p) = (uint16_t)f64_to_bf16_bits(u * cc - v * ss);
      *reinterpret_cast<uint16_t*>(q) = (uint16_t)f64_to_bf16_bits(v * cc + u * ss);
    } else {
      const double u = *reinterpret_cast<const float*>(sp), v = *reinterpret_cast<const float*>(sq);
      *reinterpret_cast<float*>(p) = (float)(u * cc - v * ss);
      *reinterpret_cast<float*>(q) = (float)(v * cc + u * ss);
    }
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, int elt_bytes, hipStream_t s) {
  const int half = a.d / 2;
  if (half % 8 || a.H * (half / 8) > kThreads * kTasks) {
    const int64_t n = (int64_t)a.BT * a.H * half;
    const int64_t blocks = (n + kThreads - 1) / kThreads;
    const int grid = (int)(blocks < 65536 ? blocks : 65536);
    if (elt_bytes == 2)
      hipLaunchKernelGGL(rope_pairs_kernel<2>, dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(rope_pairs_kernel<4>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  const int per_row = a.H * (half / 8);
  int rows = (kThreads * kTasks) / per_row;
  if (rows < 1) rows = 1;
  while (rows > 1 && rows * half > kMaxTable) --rows;
  const int grid = (a.BT + rows - 1) / rows;
  if (elt_bytes == 2)
    hipLaunchKernelGGL(rope_kernel<2>, dim3(grid), dim3(kThreads), 0, s, a, rows);
  else
    hipLaunchKernelGGL(rope_kernel<4>, dim3(grid), dim3(kThreads), 0, s, a, rows);
  return hipGetLastError();
}
