// kv_cache_append: copy T_new rotated K rows and unrotated V rows into the
// cache at rows [o, o + T_new) ("MoE-Xtend" README, KV CACHE: extend writes
// [offset:offset+t]; DESIGN CONTRACTS: append-only).
//
// K keeps the row layout [B, C, n_kv, d].  V goes to the blocked layout
// [B, C/32, n_kv, d, 32] (keys contiguous per coordinate).  One workgroup
// owns one (b, g, 32-key block) and copies only the rows of that block that
// fall in [o, o + T_new), so rows outside the range keep their bits.
// K rows move as 16-byte vectors.  V rows are staged through LDS and written
// transposed: a full block as 16-byte vectors of 8 keys of one coordinate, a
// partial block (at either end of the range) element by element.
#include "sa_device.h"
#include "sa_kernels.h"

#include <type_traits>

namespace {

constexpr int kThreads = 256;

template <int ELT>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a, int64_t kb0, int nblk) {
  typedef typename std::conditional<ELT == 2, uint16_t, uint32_t>::type E;
  constexpr int VEC = 16 / ELT;                 // elements per 16-byte vector
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int d = a.d;
  const int pitch = d + 1;                      // odd pitch: transposed reads spread banks
  const int blk = blockIdx.x % nblk;
  const int rest = blockIdx.x / nblk;
  const int g = rest % a.n_kv;
  const int b = rest / a.n_kv;
  const int64_t kb = kb0 + blk;
  const int64_t key_lo = max(kb * 32, a.o);
  const int64_t key_hi = min(kb * 32 + 32, a.o + a.T_new);
  const int nk = (int)(key_hi - key_lo);
  const int kk0 = (int)(key_lo - kb * 32);      // first slot in the block

  E* tile = reinterpret_cast<E*>(smem);
  const E* ksrc = reinterpret_cast<const E*>(a.k_src);
  const E* vsrc = reinterpret_cast<const E*>(a.v_src);
  E* kc = reinterpret_cast<E*>(a.kc);
  E* vc = reinterpret_cast<E*>(a.vc);
  const int64_t src_row0 = ((int64_t)b * a.T_new + (key_lo - a.o)) * a.n_kv + g;   // in rows of d
  const int64_t dst_row0 = ((int64_t)b * a.C + key_lo) * a.n_kv + g;
  const int vpr = d / VEC;                      // vectors per row

  // K rows and V rows (into LDS), 16 bytes at a time
  for (int e = threadIdx.x; e < nk * vpr; e += kThreads) {
    const int r = e / vpr, c = (e - r * vpr) * VEC;
    const int64_t so = (src_row0 + (int64_t)r * a.n_kv) * d + c;
    st16(kc + (dst_row0 + (int64_t)r * a.n_kv) * d + c, ld16(ksrc + so));
    const u32x4 v = ld16(vsrc + so);
    const E* ve = reinterpret_cast<const E*>(&v);
#pragma unroll
    for (int i = 0; i < VEC; ++i) tile[r * pitch + c + i] = ve[i];
  }
  __syncthreads();
  E* vblk = vc + (((int64_t)b * (a.C / 32) + kb) * a.n_kv + g) * (int64_t)d * 32;
  if (nk == 32) {
    // full block: coordinate c, keys 8k .. 8k+7 (bf16) / 4k .. 4k+3 (fp32)
    constexpr int KV = VEC;
    for (int e = threadIdx.x; e < d * (32 / KV); e += kThreads) {
      const int c = e / (32 / KV), k = (e - c * (32 / KV)) * KV;
      u32x4 w;
      E* we = reinterpret_cast<E*>(&w);
#pragma unroll
      for (int i = 0; i < KV; ++i) we[i] = tile[(k + i) * pitch + c];
      st16(vblk + c * 32 + k, w);
    }
  } else {
    for (int e = threadIdx.x; e < nk * d; e += kThreads) {
      const int c = e / nk, r = e - c * nk;
      vblk[c * 32 + kk0 + r] = tile[r * pitch + c];
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int elt_bytes, hipStream_t s) {
  const int64_t kb0 = a.o / 32;
  const int64_t kb1 = (a.o + a.T_new - 1) / 32;
  const int nblk = (int)(kb1 - kb0 + 1);
  const int64_t grid = (int64_t)nblk * a.n_kv * a.B;
  const size_t lds = (size_t)32 * (a.d + 1) * elt_bytes;
  if (elt_bytes == 2)
    hipLaunchKernelGGL(append_kernel<2>, dim3((unsigned)grid), dim3(kThreads), lds, s, a, kb0, nblk);
  else
    hipLaunchKernelGGL(append_kernel<4>, dim3((unsigned)grid), dim3(kThreads), lds, s, a, kb0, nblk);
  return hipGetLastError();
}
