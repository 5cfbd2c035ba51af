// yarn_rope_apply: rotate head rows in place at global positions.
//
// "MoE-Xtend" README, ROPE + SCALING: cos/sin of (position * inv_freq_i),
// both scaled by the YaRN concentration c; DESIGN CONTRACTS: the position is
// the global index offset + t and never resets.  Pair i is coordinates
// (i, i + d/2).
//
// One workgroup takes `rows` consecutive (b, t) rows.  It first evaluates
// the d/2 angles of each of its rows once, in fp64 (p * inv_freq_i reaches
// 1.3e5 rad at 128K context, where fp32 would lose ~1e-2 rad), and keeps
// (c*cos, c*sin) in LDS; then every (row, head, 4-pair chunk) task rotates
// in fp64 and rounds once to the storage type.  The kernel is HBM-bound:
// each element is read and written once.
#include "sa_device.h"
#include "sa_kernels.h"

namespace {

constexpr int kThreads = 256;
constexpr int kMaxTable = 2048;  // rows * d/2 entries of double2 in LDS (32 KB)

template <int ELT>
struct Vec4;
template <>
struct Vec4<2> {  // 4 bf16 = 8 bytes
  static __device__ __forceinline__ void load(const void* p, double* v) {
    u32x2 w = *reinterpret_cast<const u32x2*>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  }
  static __device__ __forceinline__ void store(void* p, const double* v) {
    u32x2 w;
    w.x = f64_to_bf16_bits(v[0]) | (f64_to_bf16_bits(v[1]) << 16);
    w.y = f64_to_bf16_bits(v[2]) | (f64_to_bf16_bits(v[3]) << 16);
    *reinterpret_cast<u32x2*>(p) = w;
  }
};
template <>
struct Vec4<4> {  // 4 fp32 = 16 bytes
  static __device__ __forceinline__ void load(const void* p, double* v) {
    f32x4 w = *reinterpret_cast<const f32x4*>(p);
    v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
  }
  static __device__ __forceinline__ void store(void* p, const double* v) {
    f32x4 w;
    w.x = (float)v[0]; w.y = (float)v[1]; w.z = (float)v[2]; w.w = (float)v[3];
    *reinterpret_cast<f32x4*>(p) = w;
  }
};

template <int ELT>
__global__ __launch_bounds__(kThreads) void rope_kernel(RopeArgs a, int rows) {
  __shared__ double2 cs[kMaxTable];
  const int half = a.d >> 1;
  const int row0 = blockIdx.x * rows;
  const int nrows = min(rows, a.BT - row0);

  for (int e = threadIdx.x; e < nrows * half; e += kThreads) {
    const int r = e / half, i = e - r * half;
    const int t = (row0 + r) % a.T;
    const double ang = (double)(a.offset + t) * a.inv_freq[i];
    double sn, cn;
    sincos(ang, &sn, &cn);
    cs[e] = make_double2(cn * a.conc, sn * a.conc);
  }
  __syncthreads();

  const int cpr = half >> 2;            // 4-pair chunks per head
  const int per_row = a.H * cpr;
  char* base = reinterpret_cast<char*>(a.x);
  for (int e = threadIdx.x; e < nrows * per_row; e += kThreads) {
    const int r = e / per_row;
    const int rem = e - r * per_row;
    const int h = rem / cpr, ch = rem - h * cpr;
    char* rowp = base + (((int64_t)(row0 + r) * a.H + h) * a.d) * ELT;
    double x1[4], x2[4], y1[4], y2[4];
    Vec4<ELT>::load(rowp + (4 * ch) * ELT, x1);
    Vec4<ELT>::load(rowp + (half + 4 * ch) * ELT, x2);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double2 c = cs[r * half + 4 * ch + k];
      y1[k] = x1[k] * c.x - x2[k] * c.y;
      y2[k] = x2[k] * c.x + x1[k] * c.y;
    }
    Vec4<ELT>::store(rowp + (4 * ch) * ELT, y1);
    Vec4<ELT>::store(rowp + (half + 4 * ch) * ELT, y2);
  }
}

}  // namespace

hipError_t launch_rope(const RopeArgs& a, int elt_bytes, hipStream_t s) {
  const int half = a.d / 2;
  const int per_row = a.H * (half / 4);
  int rows = 1024 / (per_row > 0 ? per_row : 1);
  rows = rows < 1 ? 1 : (rows > 64 ? 64 : rows);
  while (rows > 1 && rows * half > kMaxTable) --rows;
  const int grid = (a.BT + rows - 1) / rows;
  if (elt_bytes == 2)
    hipLaunchKernelGGL(rope_kernel<2>, dim3(grid), dim3(kThreads), 0, s, a, rows);
  else
    hipLaunchKernelGGL(rope_kernel<4>, dim3(grid), dim3(kThreads), 0, s, a, rows);
  return hipGetLastError();
}
