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
// A workgroup takes a block of positions t and a group of sequences b (up
// to 32 rows (b, t), one per thread and head column) and all their heads.  Its
// threads build the (c*cos, c*sin) table of the block's positions in LDS
// once -- shared by every head and every sequence of the group -- while
// their first loads are in flight; each thread then owns one (head, 8-pair
// chunk) column and walks its rows, loading both halves of the chunk and
// writing both rotated halves.  Every output carries the bits of the pair's fp64 rotation rounded
// once to the storage type; for bf16 rows they come from fp32 arithmetic
// where an error bound shows that it rounds the same way, and from fp64
// otherwise (sa_rope.h), since a plain fp32 rotation would lose bf16 ulps
// where the two products nearly cancel.
#include "sa_device.h"
#include "sa_kernels.h"
#include "sa_rope.h"

namespace {

using sa_rope::rot_first;
using sa_rope::rot_second;
using sa_rope::sincos_reduced;

constexpr int kThreads = 256;
constexpr int kRows = 32;            // most rows per workgroup
// rows a thread rotates: one (more workgroups, each table still shared by
// the group's sequences) measured 10% faster than four (GPT-OSS-Lite Q:
// 13.2 against 14.6 us; gpt-oss Q 24.1 against 26.8) and 2-4% faster than two
constexpr int kRowsPerThread = 1;

template <int ELT>
struct Rot;
template <>
struct Rot<2> {                      // bf16: 8 values in one 16-byte vector
  u32x4 w;
  __device__ __forceinline__ void load(const char* p) { w = ld16(p); }
  static constexpr bool kF32Table = true;
  // fp32 arithmetic where it provably rounds like the fp64 rotation (sa_rope.h)
  __device__ __forceinline__ static void rotate(const Rot& a, const Rot& b, const float2* fe,
                                                const double2* de, float k2, char* pa, char* pb) {
    u32x4 wa, wb;
    sa_rope::rot8_bf16(a.w, b.w, fe, de, k2, &wa, &wb);
    st16(pa, wa);
    st16(pb, wb);
  }
};
template <>
struct Rot<4> {                      // fp32: 8 values in two 16-byte vectors, fp64 math
  f32x4 w0, w1;
  static constexpr bool kF32Table = false;
  __device__ __forceinline__ void load(const char* p) {
    w0 = *reinterpret_cast<const f32x4*>(p);
    w1 = *reinterpret_cast<const f32x4*>(p + 16);
  }
  __device__ __forceinline__ double get(int i) const { return (double)(i < 4 ? w0[i] : w1[i - 4]); }
  __device__ __forceinline__ static void rotate(const Rot& a, const Rot& b, const float2*,
                                                const double2* e, float, char* pa, char* pb) {
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

// Rows of a workgroup: sequences [b0, b0 + bg) x positions [t0, t0 + tb),
// row r = (b0 + r / tb, t0 + r % tb); the table has tb rows.
template <int ELT>
__global__ __launch_bounds__(kThreads) void rope_kernel(RopeArgs a, int tb, int bg) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int half = a.d >> 1;
  double2* cs = reinterpret_cast<double2*>(smem);          // [tb][half] fp64
  float2* cs32 = reinterpret_cast<float2*>(cs + tb * half);   // [tb][half] fp32 (bf16 rows)
  const int cpr = half >> 3;                             // 8-pair chunks per head
  const int per_row = a.H * cpr;                         // <= kThreads (launcher)
  const int rstep = kThreads / per_row;
  const int B = a.BT / a.T;
  const int n_tb = (a.T + tb - 1) / tb;
  const int t0 = (blockIdx.x % n_tb) * tb;
  const int b0 = (blockIdx.x / n_tb) * bg;
  const int ntb = min(tb, a.T - t0);                     // positions in this block
  const int q = threadIdx.x % per_row, r0 = threadIdx.x / per_row;
  const int h = q / cpr, ch = q - h * cpr;
  const bool active = r0 < rstep;
  const int64_t rowbytes = (int64_t)a.H * a.d * ELT;
  const int64_t col = ((int64_t)h * a.d + 8 * ch) * ELT;
  const char* src = reinterpret_cast<const char*>(a.src) + col;
  char* dst = reinterpret_cast<char*>(a.x) + col;
  const int hb = half * ELT;
  const int rows = tb * bg;
  auto row_of = [&](int r) -> int64_t {                  // global (b, t) row, or -1
    const int b = b0 + r / tb, t = r - (r / tb) * tb;
    return (b < B && t < ntb) ? (int64_t)b * a.T + t0 + t : -1;
  };

  // every row of this thread (at most kRowsPerThread) is loaded up front, so
  // that all of the workgroup's reads are in flight while the table is built
  Rot<ELT> x1[kRowsPerThread], x2[kRowsPerThread];
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int r = r0 + k * rstep;
    const int64_t gr = r < rows ? row_of(r) : -1;
    if (active && gr >= 0) {
      x1[k].load(src + gr * rowbytes);
      x2[k].load(src + gr * rowbytes + hb);
    }
  }
  for (int e = threadIdx.x; e < ntb * half; e += kThreads) {
    const int t = e / half, i = e - t * half;
    double sn, cn;
    sincos_reduced((double)(a.offset + t0 + t) * a.inv_freq[i], &sn, &cn);
    const double cc = cn * a.conc, ss = sn * a.conc;
    cs[e] = make_double2(cc, ss);
    if (Rot<ELT>::kF32Table) cs32[e] = make_float2((float)cc, (float)ss);
  }
  __syncthreads();
  if (!active) return;
  const float k2 = sa_rope::bf16_rot_k2(a.conc);
#pragma unroll
  for (int k = 0; k < kRowsPerThread; ++k) {
    const int r = r0 + k * rstep;
    const int64_t gr = r < rows ? row_of(r) : -1;
    if (gr >= 0) {
      const int t = r % tb;
      Rot<ELT>::rotate(x1[k], x2[k], &cs32[t * half + 8 * ch], &cs[t * half + 8 * ch], k2,
                       dst + gr * rowbytes, dst + gr * rowbytes + hb);
    }
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
  // rows per workgroup: at most kRowsPerThread per thread (all loaded at once),
  // as a group of sequences times a block of positions that share one table
  const int rows = rstep * kRowsPerThread < kRows ? rstep * kRowsPerThread : kRows;
  const int B = a.BT / a.T;
  const int bg = B < rows ? B : rows;
  const int tb = rows / bg;
  const int grid = ((a.T + tb - 1) / tb) * ((B + bg - 1) / bg);
  const size_t lds = (size_t)tb * half * (elt_bytes == 2 ? 24 : 16);
  if (elt_bytes == 2)
    hipLaunchKernelGGL(rope_kernel<2>, dim3(grid), dim3(kThreads), lds, s, a, tb, bg);
  else
    hipLaunchKernelGGL(rope_kernel<4>, dim3(grid), dim3(kThreads), lds, s, a, tb, bg);
  return hipGetLastError();
}
