// kv_cache_append: copy T_new rotated K rows and unrotated V rows into the
// cache at rows [o, o + T_new) ("MoE-Xtend" README, KV CACHE: extend writes
// [offset:offset+t]; DESIGN CONTRACTS: append-only).
//
// K keeps the row layout [B, C, n_kv, d].  V goes to the blocked layout
// [B, C/32, n_kv, d, 32] (keys contiguous per coordinate).  One workgroup
// owns one (b, g, 32-key block) and copies only the rows of that block that
// fall in [o, o + T_new), so rows outside the range keep their bits.  The
// V rows are staged through LDS and written transposed, 32 keys of one
// coordinate side by side.
#include "sa_device.h"
#include "sa_kernels.h"
#include <type_traits>

namespace {

constexpr int kThreads = 256;

template <int ELT>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a, int64_t kb0, int nblk) {
  // LDS tile of V: 32 keys x d elements (+1 element pad per row)
  extern __shared__ char smem[];
  const int d = a.d;
  const int pitch = d + 1;
  int blk = blockIdx.x % nblk;
  int rest = blockIdx.x / nblk;
  const int g = rest % a.n_kv;
  const int b = rest / a.n_kv;
  const int64_t kb = kb0 + blk;
  const int64_t key_lo = max(kb * 32, a.o);
  const int64_t key_hi = min(kb * 32 + 32, a.o + a.T_new);
  const int nk = (int)(key_hi - key_lo);
  const int kk0 = (int)(key_lo - kb * 32);     // first slot in the block

  typedef typename std::conditional<ELT == 2, uint16_t, uint32_t>::type E;
  E* tile = reinterpret_cast<E*>(smem);
  const E* ksrc = reinterpret_cast<const E*>(a.k_src);
  const E* vsrc = reinterpret_cast<const E*>(a.v_src);
  E* kc = reinterpret_cast<E*>(a.kc);
  E* vc = reinterpret_cast<E*>(a.vc);

  // K rows: plain copy of d elements per key; V rows into LDS.
  for (int e = threadIdx.x; e < nk * d; e += kThreads) {
    const int r = e / d, c = e - r * d;
    const int64_t key = key_lo + r;
    const int64_t t = key - a.o;
    const int64_t src = (((int64_t)b * a.T_new + t) * a.n_kv + g) * d + c;
    kc[(((int64_t)b * a.C + key) * a.n_kv + g) * d + c] = ksrc[src];
    tile[r * pitch + c] = vsrc[src];
  }
  __syncthreads();
  // V out: for each coordinate c, slots kk0 .. kk0+nk of the 32-key block.
  E* vblk = vc + (((int64_t)b * (a.C / 32) + kb) * a.n_kv + g) * (int64_t)d * 32;
  for (int e = threadIdx.x; e < nk * d; e += kThreads) {
    const int c = e / nk, r = e - c * nk;
    vblk[c * 32 + kk0 + r] = tile[r * pitch + c];
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
