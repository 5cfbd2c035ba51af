// kv_cache_append: copy T_new rotated K rows and unrotated V rows into the
// cache at rows [o, o + T_new) ("MoE-Xtend" README, KV CACHE: extend writes
// [offset:offset+t]; DESIGN CONTRACTS: append-only).
//
// K keeps the row layout [B, C, n_kv, d].  V goes to the blocked layout
// [B, C/32, n_kv, d, 32] (keys contiguous per coordinate).  One workgroup
// owns one (b, g, 32-key block) and copies only the rows of that block that
// fall in [o, o + T_new), so rows outside the range keep their bits.
// K rows move as 16-byte vectors.  V goes through registers: for a full
// block a thread transposes an 8-key x 8-coordinate tile (bf16) and writes
// 16-byte vectors of 8 keys of one coordinate; a partial block (at either
// end of the range) moves element by element.
//
// A launch writes one contiguous run of cache rows; a ring cache (a band
// layer's W rows, position p in row p mod W) is written in at most two runs
// by the caller.
//
// kv_cache_append_rope does the same with unrotated K: each K row is rotated
// at its global position (DESIGN CONTRACTS; pos0 is the position of the
// launch's first cache row),
// with the arithmetic of yarn_rope (sa_rope.h), so the cache receives the
// bits that yarn_rope followed by kv_cache_append would write.  A workgroup
// owns one (b, 32-key block, group of heads): it moves V as above and builds
// the block's (c*cos, c*sin) table once in LDS for all its heads; each
// thread then takes a (row, head, 8-pair chunk), loads both halves of the
// chunk, and writes both rotated halves.  Optionally the same
// workgroups rotate the layer's Q rows, which sit at the same positions, out
// of place with the same table (kv_cache_append_rope_qk).
#include "sa_device.h"
#include "sa_kernels.h"
#include "sa_rope.h"

#include <type_traits>

// Rows of its column a thread loads before the V copy and the table.
#ifndef SA_APPEND_PREFETCH
#define SA_APPEND_PREFETCH 1
#endif

namespace {

constexpr int kThreads = 256;

// Rows [key_lo, key_lo + nk) of nheads V heads, all in one 32-key block, into
// the blocked layout [.., d, 32].  src: row key_lo of the first head (rows
// rstride elements apart, heads d apart); dst: the block of the first head
// (heads d*32 apart); kk0: slot of key_lo in the block.  A full block moves
// as register-transposed tiles: a thread loads 8 keys x 8 coordinates
// (bf16; 4 x 4 for fp32) as 16-byte row vectors and stores the 8 (4)
// coordinate vectors of 8 (4) keys; partial blocks go element by element.
template <int ELT>
__device__ __forceinline__ void v_to_blocked(
    const typename std::conditional<ELT == 2, uint16_t, uint32_t>::type* src, int rstride,
    typename std::conditional<ELT == 2, uint16_t, uint32_t>::type* dst, int nheads, int d, int nk,
    int kk0) {
  constexpr int VEC = 16 / ELT;                 // keys (= coordinates) per tile side
  if (nk == 32) {
    const int cgs = d / VEC;                    // coordinate groups per head
    const int ntask = nheads * cgs * (32 / VEC);
    for (int tk = threadIdx.x; tk < ntask; tk += kThreads) {
      const int kg = tk % (32 / VEC), rest = tk / (32 / VEC);
      const int hh = rest / cgs, cg = rest - hh * cgs;
      u32x4 R[VEC];
#pragma unroll
      for (int k = 0; k < VEC; ++k) R[k] = ld16(src + (kg * VEC + k) * rstride + hh * d + cg * VEC);
      auto* out = dst + (int64_t)hh * d * 32 + (cg * VEC) * 32 + kg * VEC;
#pragma unroll
      for (int c = 0; c < VEC; ++c) {
        u32x4 w;
        if constexpr (ELT == 2) {
          // keys 2m, 2m+1 of coordinate c: halves c&1 of word c/2 of rows 2m, 2m+1
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
          for (int m = 0; m < 4; ++m) w[m] = __builtin_amdgcn_perm(R[2 * m + 1][c >> 1], R[2 * m][c >> 1], sel);
        } else {
#pragma unroll
          for (int m = 0; m < 4; ++m) w[m] = R[m][c];
        }
        st16(out + c * 32, w);
      }
    }
  } else {
    for (int e = threadIdx.x; e < nheads * d * nk; e += kThreads) {
      const int r = e % nk, hc = e / nk;        // hc = head * d + coordinate
      const int hh = hc / d, c = hc - hh * d;
      dst[(int64_t)hh * d * 32 + c * 32 + kk0 + r] = src[r * rstride + hc];
    }
  }
}

template <int ELT>
__global__ __launch_bounds__(kThreads) void append_kernel(AppendArgs a, int64_t kb0, int nblk) {
  typedef typename std::conditional<ELT == 2, uint16_t, uint32_t>::type E;
  constexpr int VEC = 16 / ELT;                 // elements per 16-byte vector
  const int d = a.d;
  const int blk = blockIdx.x % nblk;
  const int rest = blockIdx.x / nblk;
  const int g = rest % a.n_kv;
  const int b = rest / a.n_kv;
  const int64_t kb = kb0 + blk;
  const int64_t key_lo = max(kb * 32, a.o);
  const int64_t key_hi = min(kb * 32 + 32, a.o + a.T_new);
  const int nk = (int)(key_hi - key_lo);
  const int kk0 = (int)(key_lo - kb * 32);      // first slot in the block

  const E* ksrc = reinterpret_cast<const E*>(a.k_src);
  const E* vsrc = reinterpret_cast<const E*>(a.v_src);
  E* kc = reinterpret_cast<E*>(a.kc);
  E* vc = reinterpret_cast<E*>(a.vc);
  const int64_t src_row0 = ((int64_t)b * a.src_T + a.src_t0 + (key_lo - a.o)) * a.n_kv + g;   // in rows of d
  const int64_t dst_row0 = ((int64_t)b * a.C + key_lo) * a.n_kv + g;
  const int vpr = d / VEC;                      // vectors per row
  const int rstride = a.n_kv * d;

  // K rows, 16 bytes at a time
  for (int e = threadIdx.x; e < nk * vpr; e += kThreads) {
    const int r = e / vpr, c = (e - r * vpr) * VEC;
    st16(kc + dst_row0 * d + (int64_t)r * rstride + c, ld16(ksrc + src_row0 * d + (int64_t)r * rstride + c));
  }
  v_to_blocked<ELT>(vsrc + src_row0 * d, rstride,
                    vc + (((int64_t)b * (a.C / 32) + kb) * a.n_kv + g) * (int64_t)d * 32, 1, d, nk,
                    kk0);
}

template <int ELT, int BATCH>
__global__ __launch_bounds__(kThreads) void append_rope_kernel(AppendRopeArgs ar, int64_t kb0,
                                                               int nblk, int hc, int ngr, int qpg) {
  typedef typename std::conditional<ELT == 2, uint16_t, uint32_t>::type E;
  constexpr int VEC = 16 / ELT;                 // elements per 16-byte vector
  const AppendArgs& a = ar.ap;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int d = a.d, half = d / 2;
  // head group grp of ngr: K heads [h0, h0 + nh) (possibly none) and Q heads
  // [grp * qpg, ...)
  const int blk = blockIdx.x % nblk;
  const int rest = blockIdx.x / nblk;
  const int grp = rest % ngr;
  const int b = rest / ngr;
  const int h0 = min(grp * hc, a.n_kv);
  const int nh = min(hc, a.n_kv - h0);
  const int64_t kb = kb0 + blk;
  const int64_t key_lo = max(kb * 32, a.o);
  const int64_t key_hi = min(kb * 32 + 32, a.o + a.T_new);
  const int nk = (int)(key_hi - key_lo);
  const int kk0 = (int)(key_lo - kb * 32);

  double2* tab = reinterpret_cast<double2*>(smem);                      // [32][half] fp64
  float2* tab32 = reinterpret_cast<float2*>(tab + 32 * half);           // [32][half] fp32 (bf16)
  const E* ksrc = reinterpret_cast<const E*>(a.k_src);
  const E* vsrc = reinterpret_cast<const E*>(a.v_src);
  E* kc = reinterpret_cast<E*>(a.kc);
  E* vc = reinterpret_cast<E*>(a.vc);
  // element offsets of row 0, head h0 in the source and in the cache; rows
  // step by n_kv heads in both
  const int64_t srow = (int64_t)b * a.src_T + a.src_t0 + (key_lo - a.o);   // source row of key_lo
  const E* src0 = ksrc + (srow * a.n_kv + h0) * d;
  const E* vsrc0 = vsrc + (srow * a.n_kv + h0) * d;
  E* dst0 = kc + (((int64_t)b * a.C + key_lo) * a.n_kv + h0) * d;
  const int rstride = a.n_kv * d;
  // this head group's share of the Q heads, rotated at the same rows
  const int qh0 = grp * qpg;
  const int nq = ar.q_src ? max(0, min(qpg, ar.n_q - qh0)) : 0;
  const int64_t qoff = (srow * ar.n_q + qh0) * d;

  // bf16: one column space over the group's K and Q heads (column = head,
  // 8-pair chunk); a thread keeps one column and steps over rows.  Its first
  // row is loaded here, before the V copy and the table, so that those reads
  // are in flight while the table is built (deeper prefetch measured slower:
  // the registers it holds cost occupancy).
  constexpr int kMaxRows = SA_APPEND_PREFETCH;
  const int cpr = half / VEC;
  const int ncols = (nh + nq) * cpr;
  const bool pre = ELT == 2 && ncols > 0 && ncols <= kThreads;
  const int crstep = pre ? kThreads / ncols : 1;
  const int ccol = pre ? threadIdx.x % ncols : 0, cr0 = pre ? threadIdx.x / ncols : 0;
  const bool cact = pre && cr0 < crstep;
  const int chh = ccol / cpr, cc0 = (ccol - chh * cpr) * VEC;
  const bool cq = chh >= nh;
  const E* csrc = cq ? reinterpret_cast<const E*>(ar.q_src) + qoff + (chh - nh) * d : src0 + chh * d;
  E* cdst = cq ? reinterpret_cast<E*>(ar.q_dst) + qoff + (chh - nh) * d : dst0 + chh * d;
  const int cs_stride = cq ? ar.n_q * d : rstride;          // source row stride
  const int cd_stride = cq ? ar.n_q * d : rstride;          // destination row stride
  u32x4 pu[kMaxRows], pv[kMaxRows];
#pragma unroll
  for (int k = 0; k < kMaxRows; ++k) {
    const int r = cr0 + k * crstep;
    if (cact && r < nk) {
      pu[k] = ld16(csrc + r * cs_stride + cc0);
      pv[k] = ld16(csrc + r * cs_stride + cc0 + half);
    }
  }

  // V: straight into the blocked layout (no LDS)
  if (nh > 0)
    v_to_blocked<ELT>(vsrc0, rstride,
                      vc + (((int64_t)b * (a.C / 32) + kb) * a.n_kv + h0) * (int64_t)d * 32, nh, d,
                      nk, kk0);
  // (c*cos, c*sin) of the block's rows: thread -> pair i, rows stepping
  {
    const int rstep = kThreads / half;
    const int i = threadIdx.x % half, r0 = threadIdx.x / half;
    if (r0 < rstep)
      for (int r = r0; r < nk; r += rstep) {
        double sn, cn;
        sa_rope::sincos_reduced((double)(a.pos0 + (key_lo - a.o) + r) * ar.inv_freq[i], &sn, &cn);
        const double cc = cn * ar.conc, ss = sn * ar.conc;
        tab[r * half + i] = make_double2(cc, ss);
        if constexpr (ELT == 2) tab32[r * half + i] = make_float2((float)cc, (float)ss);
      }
  }
  __syncthreads();
  // Rotation of nheads heads of each of the nk rows: thread -> (head,
  // 8-pair chunk) column; both halves of the chunk in, both rotated halves
  // out (reads finish before writes, so src may equal dst).
  const float k2 = sa_rope::bf16_rot_k2(ar.conc);
  auto rotate_rows = [&](const E* src, int src_rstride, E* dst, int dst_rstride, int nheads) {
    const int cpr = half / VEC;                 // chunks per head
    const int per_row = nheads * cpr;
    auto one = [&](int r, int hh, int c) {
      const E* row = src + r * src_rstride + hh * d;
      const u32x4 uv = ld16(row + c), vv = ld16(row + c + half);
      E* out = dst + r * dst_rstride + hh * d;
      if constexpr (ELT == 2) {   // fp32 where it rounds like fp64 (sa_rope.h)
        u32x4 w1, w2;
        sa_rope::rot8_bf16(uv, vv, &tab32[r * half + c], &tab[r * half + c], k2, &w1, &w2);
        st16(out + c, w1);
        st16(out + c + half, w2);
      } else {                    // fp32 rows: the fp64 rotation rounded to fp32
        const double2* t = &tab[r * half + c];
        f32x4 o1, o2;
#pragma unroll
        for (int i = 0; i < VEC; ++i) {
          const double u = (double)__uint_as_float(uv[i]);
          const double v = (double)__uint_as_float(vv[i]);
          const double2 cs = t[i];
          o1[i] = (float)sa_rope::rot_first(u, v, cs.x, cs.y);
          o2[i] = (float)sa_rope::rot_second(u, v, cs.x, cs.y);
        }
        *reinterpret_cast<f32x4*>(out + c) = o1;
        *reinterpret_cast<f32x4*>(out + c + half) = o2;
      }
    };
    if (per_row <= kThreads) {                  // fixed column, rows stepping
      const int rstep = kThreads / per_row;
      const int q = threadIdx.x % per_row, r0 = threadIdx.x / per_row;
      const int hh = q / cpr, c = (q - hh * cpr) * VEC;
      if (r0 < rstep)
        for (int r = r0; r < nk; r += 2 * rstep) {
          one(r, hh, c);
          if (r + rstep < nk) one(r + rstep, hh, c);
        }
    } else {
      for (int e = threadIdx.x; e < nk * per_row; e += kThreads) {
        const int r = e / per_row, q = e - r * per_row;
        const int hh = q / cpr;
        one(r, hh, (q - hh * cpr) * VEC);
      }
    }
  };
  if (pre) {
    if (cact) {
      // the prefetched rows, then any further ones (more than kMaxRows per thread)
#pragma unroll
      for (int k = 0; k < kMaxRows; ++k) {
        const int r = cr0 + k * crstep;
        if (r < nk) {
          u32x4 w1, w2;
          sa_rope::rot8_bf16(pu[k], pv[k], &tab32[r * half + cc0], &tab[r * half + cc0], k2,
                             &w1, &w2);
          st16(cdst + r * cd_stride + cc0, w1);
          st16(cdst + r * cd_stride + cc0 + half, w2);
        }
      }
      // in batches of BATCH rows whose loads are all issued before the first
      // is used (see the launcher)
      constexpr int kBatch = BATCH;
      for (int r = cr0 + kMaxRows * crstep; r < nk; r += kBatch * crstep) {
        u32x4 u[kBatch], v[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int rr = min(r + k * crstep, nk - 1);   // past the block: a repeat, not stored
          u[k] = ld16(csrc + rr * cs_stride + cc0);
          v[k] = ld16(csrc + rr * cs_stride + cc0 + half);
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
          const int rr = r + k * crstep;
          if (rr < nk) {
            u32x4 w1, w2;
            sa_rope::rot8_bf16(u[k], v[k], &tab32[rr * half + cc0], &tab[rr * half + cc0], k2, &w1,
                               &w2);
            st16(cdst + rr * cd_stride + cc0, w1);
            st16(cdst + rr * cd_stride + cc0 + half, w2);
          }
        }
      }
    }
    return;
  }
  if (nh > 0) rotate_rows(src0, rstride, dst0, rstride, nh);
  if (nq > 0)
    rotate_rows(reinterpret_cast<const E*>(ar.q_src) + qoff, ar.n_q * d,
                reinterpret_cast<E*>(ar.q_dst) + qoff, ar.n_q * d, nq);
}

// Rows of positions [p0, p0 + n) from one cache to another; a workgroup owns
// one (b, g, run of up to 32 positions).  Source and destination rows come
// from each side's own mapping (ring: p mod C; linear: p - base), so a run
// may cross a 32-row V block or the ring's end on either side: K moves as
// 16-byte row vectors, V element by element with consecutive threads on
// consecutive keys of one coordinate (runs of 2-byte accesses).
template <int ELT>
__global__ __launch_bounds__(kThreads) void copy_rows_kernel(CopyRowsArgs a, int nrun) {
  typedef typename std::conditional<ELT == 2, uint16_t, uint32_t>::type E;
  constexpr int VEC = 16 / ELT;
  const int d = a.d;
  const int run = blockIdx.x % nrun;
  const int rest = blockIdx.x / nrun;
  const int g = rest % a.n_kv;
  const int b = rest / a.n_kv;
  const int64_t p_lo = a.p0 + (int64_t)run * 32;
  const int nk = (int)min((int64_t)32, a.p0 + a.n - p_lo);
  // rows of p_lo on both sides (one modulo per workgroup); row p_lo + r is
  // then a step with at most one wrap
  const int64_t rs0 = a.ring_s ? p_lo % a.Cs : p_lo - a.base_s;
  const int64_t rd0 = a.ring_d ? p_lo % a.Cd : p_lo - a.base_d;
  auto row_s = [&](int r) { const int64_t x = rs0 + r; return (a.ring_s && x >= a.Cs) ? x - a.Cs : x; };
  auto row_d = [&](int r) { const int64_t x = rd0 + r; return (a.ring_d && x >= a.Cd) ? x - a.Cd : x; };
  const E* ks = reinterpret_cast<const E*>(a.ks);
  const E* vs = reinterpret_cast<const E*>(a.vs);
  E* kd = reinterpret_cast<E*>(a.kd);
  E* vd = reinterpret_cast<E*>(a.vd);
  const int vpr = d / VEC;
  for (int e = threadIdx.x; e < nk * vpr; e += kThreads) {
    const int r = e / vpr, c = (e - r * vpr) * VEC;
    st16(kd + (((int64_t)b * a.Cd + row_d(r)) * a.n_kv + g) * d + c,
         ld16(ks + (((int64_t)b * a.Cs + row_s(r)) * a.n_kv + g) * d + c));
  }
  // V: consecutive threads on consecutive keys of one coordinate
  const E* vsb = vs + (((int64_t)b * (a.Cs / 32)) * a.n_kv + g) * (int64_t)d * 32;
  E* vdb = vd + (((int64_t)b * (a.Cd / 32)) * a.n_kv + g) * (int64_t)d * 32;
  const int64_t blk_s = (int64_t)a.n_kv * d * 32, blk_d = blk_s;   // elements per 32-row block
  for (int e = threadIdx.x; e < 32 * d; e += kThreads) {
    const int r = e & 31, c = e >> 5;
    if (r >= nk) continue;
    const int64_t rs = row_s(r), rd = row_d(r);
    vdb[(rd >> 5) * blk_d + c * 32 + (rd & 31)] = vsb[(rs >> 5) * blk_s + c * 32 + (rs & 31)];
  }
}

}  // namespace

hipError_t launch_copy_rows(const CopyRowsArgs& a, int elt_bytes, hipStream_t s) {
  const int nrun = (a.n + 31) / 32;
  const int64_t grid = (int64_t)nrun * a.n_kv * a.B;
  if (elt_bytes == 2)
    hipLaunchKernelGGL(copy_rows_kernel<2>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, nrun);
  else
    hipLaunchKernelGGL(copy_rows_kernel<4>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, nrun);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int elt_bytes, hipStream_t s) {
  const int64_t kb0 = a.o / 32;
  const int64_t kb1 = (a.o + a.T_new - 1) / 32;
  const int nblk = (int)(kb1 - kb0 + 1);
  const int64_t grid = (int64_t)nblk * a.n_kv * a.B;
  if (elt_bytes == 2)
    hipLaunchKernelGGL(append_kernel<2>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, kb0, nblk);
  else
    hipLaunchKernelGGL(append_kernel<4>, dim3((unsigned)grid), dim3(kThreads), 0, s, a, kb0, nblk);
  return hipGetLastError();
}

// Head groups: a workgroup rotates at most about kGroupCols (head, chunk)
// columns per row, so that many workgroups share the work (each builds the
// block's angle table, its only LDS).
#ifndef SA_GROUP_COLS
#define SA_GROUP_COLS 64
#endif
constexpr int kGroupCols = SA_GROUP_COLS;

hipError_t launch_append_rope(const AppendRopeArgs& ar, int elt_bytes, hipStream_t s) {
  const AppendArgs& a = ar.ap;
  const int64_t kb0 = a.o / 32;
  const int64_t kb1 = (a.o + a.T_new - 1) / 32;
  const int nblk = (int)(kb1 - kb0 + 1);
  const size_t tab = (size_t)32 * (a.d / 2) * (sizeof(double2) + (elt_bytes == 2 ? sizeof(float2) : 0));
  const int cpr = a.d / 2 / (16 / elt_bytes);
  const int n_q = ar.q_src ? ar.n_q : 0;
  const int cols = (a.n_kv + n_q) * cpr;
  int ngr = (cols + kGroupCols - 1) / kGroupCols;
  if (ngr > a.n_kv + n_q) ngr = a.n_kv + n_q;
  const int hc = (a.n_kv + ngr - 1) / ngr;                  // K heads per group
  const int qpg = n_q ? (n_q + ngr - 1) / ngr : 0;
  const int64_t grid = (int64_t)nblk * ngr * a.B;
  const size_t lds = tab;
  // With few workgroups (under two per CU) each thread has several rows and
  // nothing else hides their loads' latency: batches of four rows, loaded
  // together (one sequence's 2048-row chunk, 64/8 heads, d 64: 320
  // workgroups, 13.2 against 15.0 us).  With more workgroups the batch's
  // registers cost a wave per SIMD and one row at a time is faster (the
  // same heads over 8192 rows: 29.8 against 33.3 us).
  const bool batch = grid < 2 * 256;
  if (elt_bytes == 2) {
    if (batch)
      hipLaunchKernelGGL((append_rope_kernel<2, 4>), dim3((unsigned)grid), dim3(kThreads), lds, s, ar,
                         kb0, nblk, hc, ngr, qpg);
    else
      hipLaunchKernelGGL((append_rope_kernel<2, 1>), dim3((unsigned)grid), dim3(kThreads), lds, s, ar,
                         kb0, nblk, hc, ngr, qpg);
  } else {
    hipLaunchKernelGGL((append_rope_kernel<4, 1>), dim3((unsigned)grid), dim3(kThreads), lds, s, ar,
                       kb0, nblk, hc, ngr, qpg);
  }
  return hipGetLastError();
}
