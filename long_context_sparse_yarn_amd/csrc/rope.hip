// yarn_rope / yarn_rope_apply: rotate head rows at global positions, from a
// source buffer into a destination (the same buffer for the in-place form).
//
// "MoE-Xtend" README, ROPE + SCALING: cos/sin of (position * inv_freq_i),
// both scaled by the YaRN concentration c; DESIGN CONTRACTS: the position is
// the global index offset + t and never resets.  Pair i is coordinates
// (i, i + d/2).
//
// Angles and the pair rotation: sa_rope.h.
//
// A workgroup takes a block of consecutive (b, t) rows (up to 32, about four
// per thread) and all their heads.  Its threads build the block's (c*cos, c*sin) table in LDS
// once (shared by every head) while their first loads are in flight; each
// thread then owns one (head, 8-pair chunk) column and walks the rows two
// at a time, loading both halves of the chunk and writing both rotated
// halves.  Pairs are rotated in fp64 and rounded once to the storage type
// (an fp32 rotation would lose many bf16 ulps where the two products nearly
// cancel).  The kernel is HBM-bound: each element is read and written once.
#include "sa_device.h"
#include "sa_kernels.h"
#include "sa_rope.h"

namespace {

using sa_rope::rot_first;
using sa_rope::rot_second;
using sa_rope::sincos_reduced;

constexpr int kThreads = 256;
constexpr int kRows = 32;            // most rows per workgroup
constexpr int kRowsPerThread = 4;    // aim: each thread walks about this many rows

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
      y1[i] = f64_to_bf16_bits(rot_first(u, v, e[i].x, e[i].y));
      y2[i] = f64_to_bf16_bits(rot_second(u, v, e[i].x, e[i].y));
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
      o[i >> 2][i & 3] = (float)rot_first(u, v, e[i].x, e[i].y);
      o[2 + (i >> 2)][i & 3] = (float)rot_second(u, v, e[i].x, e[i].y);
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
  extern __shared__ __attribute__((aligned(16))) char smem[];
  Entry* cs = reinterpret_cast<Entry*>(smem);            // [rows][half]
  const int half = a.d >> 1;
  const int cpr = half >> 3;                             // 8-pair chunks per head
  const int per_row = a.H * cpr;                         // <= kThreads (launcher)
  const int rstep = kThreads / per_row;
  const int row0 = blockIdx.x * rows;
  const int nrows = min(rows, a.BT - row0);
  const int q = threadIdx.x % per_row, r0 = threadIdx.x / per_row;
  const int h = q / cpr, ch = q - h * cpr;
  const bool active = r0 < rstep;
  const int64_t rowbytes = (int64_t)a.H * a.d * ELT;
  const int64_t col = ((int64_t)h * a.d + 8 * ch) * ELT;
  const char* src = reinterpret_cast<const char*>(a.src) + (int64_t)row0 * rowbytes + col;
  char* dst = reinterpret_cast<char*>(a.x) + (int64_t)row0 * rowbytes + col;
  const int hb = half * ELT;

  Rot<ELT> x1[2], x2[2];
  auto load = [&](int r, int k) {
    if (active && r < nrows) {
      x1[k].load(src + r * rowbytes);
      x2[k].load(src + r * rowbytes + hb);
    }
  };
  load(r0, 0);
  load(r0 + rstep, 1);
  for (int e = threadIdx.x; e < nrows * half; e += kThreads) {
    const int r = e / half, i = e - r * half;
    const int t = (row0 + r) % a.T;
    double sn, cn;
    sincos_reduced((double)(a.offset + t) * a.inv_freq[i], &sn, &cn);
    cs[e] = Rot<ELT>::entry(cn * a.conc, sn * a.conc);
  }
  __syncthreads();
  if (!active) return;
  for (int r = r0; r < nrows; r += 2 * rstep) {
    Rot<ELT>::rotate(x1[0], x2[0], &cs[r * half + 8 * ch], dst + r * rowbytes,
                     dst + r * rowbytes + hb);
    load(r + 2 * rstep, 0);
    const int r1 = r + rstep;
    if (r1 < nrows)
      Rot<ELT>::rotate(x1[1], x2[1], &cs[r1 * half + 8 * ch], dst + r1 * rowbytes,
                       dst + r1 * rowbytes + hb);
    load(r1 + 2 * rstep, 1);
  }
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
      *reinterpret_cast<uint16_t*>(p) = (uint16_t)f64_to_bf16_bits(rot_first(u, v, cc, ss));
      *reinterpret_cast<uint16_t*>(q) = (uint16_t)f64_to_bf16_bits(rot_second(u, v, cc, ss));
    } else {
      const double u = *reinterpret_cast<const float*>(sp), v = *reinterpret_cast<const float*>(sq);
      *reinterpret_cast<float*>(p) = (float)rot_first(u, v, cc, ss);
      *reinterpret_cast<float*>(q) = (float)rot_second(u, v, cc, ss);
    }
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, int elt_bytes, hipStream_t s) {
  const int half = a.d / 2;
  if (half % 8 || a.H * (half / 8) > kThreads) {
    const int64_t n = (int64_t)a.BT * a.H * half;
    const int64_t blocks = (n + kThreads - 1) / kThreads;
    const int grid = (int)(blocks < 65536 ? blocks : 65536);
    if (elt_bytes == 2)
      hipLaunchKernelGGL(rope_pairs_kernel<2>, dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL(rope_pairs_kernel<4>, dim3(grid), dim3(kThreads), 0, s, a);
    return hipGetLastError();
  }
  const int rstep = kThreads / (a.H * (half / 8));
  const int rows = rstep * kRowsPerThread < kRows ? rstep * kRowsPerThread : kRows;
  const int grid = (a.BT + rows - 1) / rows;
  const size_t lds = (size_t)rows * half * 16;
  if (elt_bytes == 2)
    hipLaunchKernelGGL(rope_kernel<2>, dim3(grid), dim3(kThreads), lds, s, a, rows);
  else
    hipLaunchKernelGGL(rope_kernel<4>, dim3(grid), dim3(kThreads), lds, s, a, rows);
  return hipGetLastError();
}
