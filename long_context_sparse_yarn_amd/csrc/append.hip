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
//
// kv_cache_append_rope does the same with unrotated K: each K row is rotated
// at its cache row index, which is its global position (DESIGN CONTRACTS),
// with the arithmetic of yarn_rope (sa_rope.h), so the cache receives the
// bits that yarn_rope followed by kv_cache_append would write.  A workgroup
// owns one (b, 32-key block, group of heads): it stages V through LDS as
// above and builds the block's (c*cos, c*sin) table once in LDS for all its
// heads; each thread then takes a (row, head, 8-pair chunk), loads both
// halves of the chunk, and writes both rotated halves.  Optionally the same
// workgroups rotate the layer's Q rows, which sit at the same positions, out
// of place with the same table (kv_cache_append_rope_qk).
#include "sa_device.h"
#include "sa_kernels.h"
#include "sa_rope.h"

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

template <int ELT>
__global__ __launch_bounds__(kThreads) void append_rope_kernel(AppendRopeArgs ar, int64_t kb0,
                                                               int nblk, int hc) {
  typedef typename std::conditional<ELT == 2, uint16_t, uint32_t>::type E;
  constexpr int VEC = 16 / ELT;                 // elements per 16-byte vector
  const AppendArgs& a = ar.ap;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int d = a.d, half = d / 2;
  const int pitch = d + 1;
  const int nhc = (a.n_kv + hc - 1) / hc;
  const int blk = blockIdx.x % nblk;
  const int rest = blockIdx.x / nblk;
  const int h0 = (rest % nhc) * hc;
  const int b = rest / nhc;
  const int nh = min(hc, a.n_kv - h0);
  const int64_t kb = kb0 + blk;
  const int64_t key_lo = max(kb * 32, a.o);
  const int64_t key_hi = min(kb * 32 + 32, a.o + a.T_new);
  const int nk = (int)(key_hi - key_lo);
  const int kk0 = (int)(key_lo - kb * 32);

  double2* tab = reinterpret_cast<double2*>(smem);                      // [32][half]
  E* vtile = reinterpret_cast<E*>(smem + (size_t)32 * half * sizeof(double2));   // [nh][32][d+1]
  const E* ksrc = reinterpret_cast<const E*>(a.k_src);
  const E* vsrc = reinterpret_cast<const E*>(a.v_src);
  E* kc = reinterpret_cast<E*>(a.kc);
  E* vc = reinterpret_cast<E*>(a.vc);
  // element offsets of row 0, head h0 in the source and in the cache; rows
  // step by n_kv heads in both
  const E* src0 = ksrc + (((int64_t)b * a.T_new + (key_lo - a.o)) * a.n_kv + h0) * d;
  const E* vsrc0 = vsrc + (((int64_t)b * a.T_new + (key_lo - a.o)) * a.n_kv + h0) * d;
  E* dst0 = kc + (((int64_t)b * a.C + key_lo) * a.n_kv + h0) * d;
  const int rstride = a.n_kv * d;

  // V rows into LDS: thread -> vector column q of a row (nh*d/VEC per row),
  // rows stepping by the threads per row
  {
    const int per_row = nh * (d / VEC);
    const int rstep = kThreads / per_row;
    const int q = threadIdx.x % per_row, r0 = threadIdx.x / per_row;
    const int hh = q / (d / VEC), c = (q - hh * (d / VEC)) * VEC;
    if (r0 < rstep)
      for (int r = r0; r < nk; r += rstep) {
        const u32x4 v = ld16(vsrc0 + r * rstride + hh * d + c);
        const E* ve = reinterpret_cast<const E*>(&v);
#pragma unroll
        for (int i = 0; i < VEC; ++i) vtile[(hh * 32 + r) * pitch + c + i] = ve[i];
      }
  }
  // (c*cos, c*sin) of the block's rows: thread -> pair i, rows stepping
  {
    const int rstep = kThreads / half;
    const int i = threadIdx.x % half, r0 = threadIdx.x / half;
    if (r0 < rstep)
      for (int r = r0; r < nk; r += rstep) {
        double sn, cn;
        sa_rope::sincos_reduced((double)(key_lo + r) * ar.inv_freq[i], &sn, &cn);
        tab[r * half + i] = make_double2(cn * ar.conc, sn * ar.conc);
      }
  }
  __syncthreads();
  // Rotation of nheads heads of each of the nk rows: thread -> (head,
  // 8-pair chunk) column; both halves of the chunk in, both rotated halves
  // out (reads finish before writes, so src may equal dst).
  auto rotate_rows = [&](const E* src, int src_rstride, E* dst, int dst_rstride, int nheads) {
    const int cpr = half / VEC;                 // chunks per head
    const int per_row = nheads * cpr;
    auto one = [&](int r, int hh, int c) {
      const E* row = src + r * src_rstride + hh * d;
      const u32x4 uv = ld16(row + c), vv = ld16(row + c + half);
      const E* ue = reinterpret_cast<const E*>(&uv);
      const E* ve = reinterpret_cast<const E*>(&vv);
      const double2* t = &tab[r * half + c];
      u32x4 w1, w2;
      E* o1 = reinterpret_cast<E*>(&w1);
      E* o2 = reinterpret_cast<E*>(&w2);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        double u, v;
        if constexpr (ELT == 2) {
          u = (double)bf16_to_f32(ue[i]);
          v = (double)bf16_to_f32(ve[i]);
        } else {
          u = (double)__uint_as_float(ue[i]);
          v = (double)__uint_as_float(ve[i]);
        }
        const double2 cs = t[i];
        const double y1 = sa_rope::rot_first(u, v, cs.x, cs.y);
        const double y2 = sa_rope::rot_second(u, v, cs.x, cs.y);
        if constexpr (ELT == 2) {
          o1[i] = (E)f64_to_bf16_bits(y1);
          o2[i] = (E)f64_to_bf16_bits(y2);
        } else {
          o1[i] = __float_as_uint((float)y1);
          o2[i] = __float_as_uint((float)y2);
        }
      }
      E* out = dst + r * dst_rstride + hh * d;
      st16(out + c, w1);
      st16(out + c + half, w2);
    };
    if (per_row <= kThreads) {                  // fixed column, rows stepping
      const int rstep = kThreads / per_row;
      const int q = threadIdx.x % per_row, r0 = threadIdx.x / per_row;
      const int hh = q / cpr, c = (q - hh * cpr) * VEC;
      if (r0 < rstep)
        for (int r = r0; r < nk; r += rstep) one(r, hh, c);
    } else {
      for (int e = threadIdx.x; e < nk * per_row; e += kThreads) {
        const int r = e / per_row, q = e - r * per_row;
        const int hh = q / cpr;
        one(r, hh, (q - hh * cpr) * VEC);
      }
    }
  };
  rotate_rows(src0, rstride, dst0, rstride, nh);
  if (ar.q_src) {
    // this head group's share of the Q heads, rotated at the same rows
    const int qpg = (ar.n_q + nhc - 1) / nhc;
    const int qh0 = (rest % nhc) * qpg;
    const int nq = min(qpg, ar.n_q - qh0);
    if (nq > 0) {
      const int64_t qoff = (((int64_t)b * a.T_new + (key_lo - a.o)) * ar.n_q + qh0) * d;
      rotate_rows(reinterpret_cast<const E*>(ar.q_src) + qoff, ar.n_q * d,
                  reinterpret_cast<E*>(ar.q_dst) + qoff, ar.n_q * d, nq);
    }
  }
  // V: transposed into the blocked layout, one head after another
  for (int hh = 0; hh < nh; ++hh) {
    E* vblk = vc + (((int64_t)b * (a.C / 32) + kb) * a.n_kv + h0 + hh) * (int64_t)d * 32;
    const E* vt = vtile + hh * 32 * pitch;
    if (nk == 32) {
      for (int e = threadIdx.x; e < d * (32 / VEC); e += kThreads) {
        const int c = e / (32 / VEC), k = (e - c * (32 / VEC)) * VEC;
        u32x4 w;
        E* we = reinterpret_cast<E*>(&w);
#pragma unroll
        for (int i = 0; i < VEC; ++i) we[i] = vt[(k + i) * pitch + c];
        st16(vblk + c * 32 + k, w);
      }
    } else {
      for (int e = threadIdx.x; e < nk * d; e += kThreads) {
        const int c = e / nk, r = e - c * nk;
        vblk[c * 32 + kk0 + r] = vt[r * pitch + c];
      }
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

// Heads per workgroup: as many as keep its LDS (table + V tiles) within
// kAppendRopeLds, so that at least two workgroups share a CU.
constexpr size_t kAppendRopeLds = 64 * 1024;

hipError_t launch_append_rope(const AppendRopeArgs& ar, int elt_bytes, hipStream_t s) {
  const AppendArgs& a = ar.ap;
  const int64_t kb0 = a.o / 32;
  const int64_t kb1 = (a.o + a.T_new - 1) / 32;
  const int nblk = (int)(kb1 - kb0 + 1);
  const size_t tab = (size_t)32 * (a.d / 2) * sizeof(double2);
  const size_t per_head = (size_t)32 * (a.d + 1) * elt_bytes;
  int hc = tab + per_head >= kAppendRopeLds ? 1 : (int)((kAppendRopeLds - tab) / per_head);
  if (hc > a.n_kv) hc = a.n_kv;
  const int nhc = (a.n_kv + hc - 1) / hc;
  const int64_t grid = (int64_t)nblk * nhc * a.B;
  const size_t lds = tab + (size_t)hc * per_head;
  if (elt_bytes == 2)
    hipLaunchKernelGGL(append_rope_kernel<2>, dim3((unsigned)grid), dim3(kThreads), lds, s, ar, kb0, nblk, hc);
  else
    hipLaunchKernelGGL(append_rope_kernel<4>, dim3((unsigned)grid), dim3(kThreads), lds, s, ar, kb0, nblk, hc);
  return hipGetLastError();
}
