// sinkattn_decode (bf16): one query token per sequence against the cache.
//
// What is computed: as prefill, for the single query at position p = o - 1
// whose own K/V row was appended just before ("MoE-Xtend" README,
// ARCHITECTURE: append KV at offset = t, then t++; per-step cost O(T) on
// full layers and O(W) on band layers).
//
// How (gfx950 design): decode is a stream over the cache, so the kernel is
// built to keep HBM busy.
//  * Split-KV: each wave owns one (b, g) pair and one contiguous run of
//    32-key blocks of the allowed range; the pairs x splits give thousands
//    of independent waves for 256 CUs.  Consecutive waves take the KV heads
//    of one (b, split), so the waves in flight together read whole cache
//    rows (the heads of a row are contiguous) and whole V blocks.
//  * Matrix cores on 8 of 16 columns: the q_mult query heads of the group
//    form the N side of S^T = K Q^T (v_mfma_f32_16x16x32_bf16), so one K row
//    load serves all heads of the group.  K operands load straight from HBM
//    in the row layout; V^T operands load straight from the blocked V
//    layout (8 consecutive keys of one coordinate = one 16-byte load); no
//    LDS round trip.  A wave works on 64 keys at a time while the loads of
//    the next 64 keys are in flight.
//  * Lazy running max, as in prefill: the cross-lane max and the rescale of
//    the accumulators happen only when a score passes the running max by
//    more than 2^8.
//  * Each wave writes a partial (m, l, acc) in base-2 units to the
//    workspace; a merge kernel folds the partials of a head in a fixed order
//    and adds the sink exactly once:
//      M = max(sigma', max_c m_c), L = 2^(sigma'-M) + sum_c l_c 2^(m_c-M),
//      out = sum_c acc_c 2^(m_c-M) / L        (sigma' = sigma * log2 e).
//    Splits with no allowed key carry m = -inf, l = 0 and drop out.  With
//    few (b, g) pairs (at most 8) a workgroup's four waves take four pieces
//    of one (b, g)'s run instead and fold their partials in LDS into one
//    (same formula, no sink), so the merge gathers a quarter as many.  A span
//    of at most 256 rows (a band layer) runs in one launch instead: a
//    workgroup of four waves per (b, g), each wave one or two 32-key blocks
//    of a 128-row band, folding their partials in LDS in the same fixed way,
//    so a band step costs a block's memory latency or two rather than a
//    chain of them.
//  * A whole step in the same launch (launch_decode_step_bf16): the kernels
//    take the token's unrotated Q, K and V.  Each wave (the workgroup, in the
//    short kernel) rotates the group's Q heads in LDS with the RoPE kernels'
//    arithmetic (sa_rope.h, same bits), and the one wave whose run of blocks
//    holds the token's cache row also rotates K, writes the K and V row to
//    the cache and, when it reaches that block, puts the row into its
//    operands in registers (the block's loads may predate the stores).  The
//    row's raw loads go out before the first block's, the table and the
//    rotation run while the block loads are in flight.
#include "sa_device.h"
#include "sa_kernels.h"
#include "sa_rope.h"

#include <type_traits>

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// Split-KV waves to aim for: 2048 (8 per CU) keep HBM busy; with at most 8
// (b, g) pairs, 1024 do as well and halve the merge's partials (B = 1,
// 67.6k rows, 64/8 heads: split + merge 27.7 against 29.1 us; at B = 8 the
// 2048 target is 0.7% faster; 512 and fewer lose the memory parallelism).
constexpr int kTargetWaves = 2048;
constexpr int kTargetWavesFewPairs = 1024;
constexpr int kFewPairs = 8;
constexpr int kMaxSplits = 256;                 // waves (partials) per (b, g) at most
constexpr int64_t kSingleSplitRows = 256;   // spans this short run as one short launch
constexpr float kSlack = 8.0f;
// With at most kFewPairs (b, g) pairs each split workgroup folds its waves'
// partials into one (see decode_split_body).
__host__ __device__ constexpr bool fold_splits(int pairs) { return pairs <= kFewPairs; }

template <int D>
struct BlockOps {
  static constexpr int KS = D / 32;
  static constexpr int DT = D / 16;
  u32x4 k[2][KS];
  u32x4 v[DT];
};

template <int D>
__device__ __forceinline__ void load_block(BlockOps<D>& o, const uint16_t* kbase,
                                           const uint16_t* vblk, int kstride, int j, int g4) {
  // K: M tile mt, row i = j -> key 8*(j>>2) + 4*mt + (j&3) of the block
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    const int key = 8 * (j >> 2) + 4 * mt + (j & 3);
#pragma unroll
    for (int ks = 0; ks < BlockOps<D>::KS; ++ks)
      o.k[mt][ks] = ld16(kbase + (int64_t)key * kstride + 32 * ks + 8 * g4);
  }
  // V^T: coordinate 16*dt + j, keys 8*g4 .. 8*g4+7
#pragma unroll
  for (int dt = 0; dt < BlockOps<D>::DT; ++dt)
    o.v[dt] = ld16(vblk + (16 * dt + j) * 32 + 8 * g4);
}

// One wave's pass over cache blocks [b0, b1) of sequence b, KV head g (keys
// of the allowed range [lo, hi) only): lane (j, g4) ends with the running
// reference m_run (base-2 units; -inf while nothing is allowed), its share
// l_run of the sum of weights (the column's four lanes add up to the sum)
// and O^T[16 dt + 4 g4 + r][head j] against that reference.  No sink.
//
// Hooks (NoStep, or StepHooks for a fused step): pre() before the first
// block loads, post(qop) after them (fills qop if the hooks own Q), and
// subst(kb, ops) on each block's operands before they are used.
template <int D, bool SHORT, class Hooks>
__device__ __forceinline__ void decode_blocks(const AttnArgs& a, int b, int g, int b0,
                                              int b1, int64_t lo, int64_t hi,
                                              u32x4 (&qop)[D / 32], float& m_run,
                                              float& l_run, f32x4 (&O)[D / 16], Hooks& hk) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g4 = lane >> 4;
  const int64_t C = a.C;
  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.kc);
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.vc);
  const float scale = a.sm_scale * SA_LOG2E;
  m_run = -INFINITY;
  l_run = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kstride = a.n_kv * D;
  const uint16_t* kpair = kc + ((int64_t)b * C * a.n_kv + g) * D;        // row 0 of (b, g)
  const uint16_t* vpair = vc + ((int64_t)b * (C / 32) * a.n_kv + g) * (int64_t)(D * 32);
  const int64_t vbstride = (int64_t)a.n_kv * D * 32;                      // per 32-key block

  // Loads are never skipped: a block past the run repeats the run's last
  // block (block 0 for an empty run; a cache holds at least one), whose
  // values go unused.  With every load issued, the compiler knows how many
  // are in flight and waits for exactly the block it is about to use, not
  // for the prefetched ones behind it.
  // nu (1 or 2): how many of the two operand sets to fill and use
  auto loadn = [&](auto nu, BlockOps<D>(&ops)[2], int kb) {
#pragma unroll
    for (int u = 0; u < decltype(nu)::value; ++u) {
      const int kbu = max(0, min(kb + u, b1 - 1));
      load_block<D>(ops[u], kpair + kbu * 32 * kstride, vpair + kbu * vbstride, kstride, j, g4);
    }
  };
  // blocks kb, kb + 1 from the operands in cur.  A block at or past b1 (the
  // repeat load2 made) goes through the same instructions with every key
  // masked and V zeroed, so that every loaded register is consumed on every
  // path and the compiler never has to drain the loads in flight.
  auto processn = [&](auto nu, BlockOps<D>(&cur)[2], int kb) __attribute__((always_inline)) {
    constexpr int NU = decltype(nu)::value;
    f32x4 Sc[2][2];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      Sc[u][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      Sc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      hk.subst(kb + u, cur[u]);
      const int64_t k0 = (int64_t)(kb + u) * 32;
      const int64_t top = kb + u < b1 ? hi : k0;     // keys from top on are masked
      if (k0 + 32 > top) {   // zero V of masked keys (unwritten rows; the repeat)
        const int valid = (int)max((int64_t)-1, top - (k0 + 8 * g4));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t keep = (2 * w + 1 < valid) ? 0xFFFFFFFFu : (2 * w < valid ? 0x0000FFFFu : 0u);
            cur[u].v[dt][w] &= keep;
          }
      }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) Sc[u][mt] = mfma16x16x32(cur[u].k[mt][ks], qop[ks], Sc[u][mt]);
      // lane (j, g4), element (mt, r): key k0 + 8*g4 + 4*mt + r
      if (k0 < lo || k0 + 32 > top) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t key = k0 + 8 * g4 + 4 * mt + r;
            if (key < lo || key >= top) Sc[u][mt][r] = -INFINITY;
          }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < NU; ++u)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, Sc[u][mt][r]);
    if (__builtin_amdgcn_ballot_w64(mx * scale > m_run + kSlack) != 0) {
      const float m_new = fmaxf(m_run, max_over_col(mx) * scale);
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const int e = 2 * e2;
        const float p0 = fast_exp2(fmaf(Sc[u][e >> 2][e & 3], scale, -m_use));
        const float p1 = fast_exp2(fmaf(Sc[u][(e + 1) >> 2][(e + 1) & 3], scale, -m_use));
        w[e2] = pack_bf16x2(p0, p1);
        l_run = sum_bf16x2(w[e2], l_run);
      }
      const u32x4 Pk = {w[0], w[1], w[2], w[3]};
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt] = mfma16x16x32(cur[u].v[dt], Pk, O[dt]);
    }
  };
  // Two operand sets in turn (no register copies, which would wait for the
  // loads in flight): the loads of one pair of blocks run while the other
  // pair is computed.
  using One = std::integral_constant<int, 1>;
  using Two = std::integral_constant<int, 2>;
  auto load2 = [&](BlockOps<D>(&ops)[2], int kb) { loadn(Two{}, ops, kb); };
  auto process = [&](BlockOps<D>(&cur)[2], int kb) __attribute__((always_inline)) {
    processn(Two{}, cur, kb);
  };
  BlockOps<D> A[2], Bo[2];
  // A short span's waves (one or two blocks each, none for an empty run)
  // load and multiply only their own blocks: no repeat of the last one and
  // no prefetch behind it.
  if (SHORT && b1 - b0 <= 2) {
    hk.pre();
    if (b1 - b0 == 2) {
      loadn(Two{}, A, b0);
      hk.post(qop);
      processn(Two{}, A, b0);
    } else {
      loadn(One{}, A, b0);
      hk.post(qop);
      processn(One{}, A, b0);
    }
    return;
  }
  hk.pre();
  load2(A, b0);
  hk.post(qop);
  // One exit, at the top: a break between the two halves gave the loop a
  // second way back to its head on which the compiler could not tell the
  // loads still in flight, so it drained every load at the head of each pass.
  int kb = b0;
  for (; kb + 2 < b1; kb += 4) {
    load2(Bo, kb + 2);
    process(A, kb);
    load2(A, kb + 4);
    process(Bo, kb + 2);
  }
  if (kb < b1) process(A, kb);     // the run's last pair, in A
}

// The Q^T operand of (b, g): column j = head g*q_mult + j (zero past q_mult).
template <int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int b, int g, u32x4 (&qop)[D / 32]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g4 = lane >> 4;
  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  const bool qv = j < a.q_mult;
  const uint16_t* qrow = q + ((int64_t)b * a.n_q + g * a.q_mult + (qv ? j : 0)) * D;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) qop[ks] = qv ? ld16(qrow + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0};
}

// Plain decode: the cache already holds the token's row, q its rotated Q.
struct NoStep {
  __device__ __forceinline__ void pre() {}
  template <class Q>
  __device__ __forceinline__ void post(Q&) {}
  template <class Ops>
  __device__ __forceinline__ void subst(int64_t, Ops&) {}
};

// LDS of one fused step for group (b, g): the (c cos, c sin) table of the
// token's position (fp64 and fp32, as the RoPE kernels keep it), the rotated
// rows (the group's q_mult Q heads, then the K row) and the raw V row.
template <int D>
struct StepStage {
  static constexpr int H = D / 2;
  __host__ __device__ static constexpr size_t bytes(int q_mult) {
    return (size_t)H * 24 + (size_t)(q_mult + 1) * D * 2 + (size_t)D * 2;
  }
  double2* tab;
  float2* tab32;
  uint16_t* rows;
  uint16_t* vrow;
  __device__ __forceinline__ StepStage(char* p, int q_mult)
      : tab(reinterpret_cast<double2*>(p)),
        tab32(reinterpret_cast<float2*>(p + H * 16)),
        rows(reinterpret_cast<uint16_t*>(p + H * 24)),
        vrow(reinterpret_cast<uint16_t*>(p + H * 24 + (q_mult + 1) * D * 2)) {}
};

// Ordering of a stage's LDS between the threads that share it: one wave
// (its LDS operations run in order; the clobber keeps the compiler's order)
// or a whole workgroup.
struct WaveSync {
  __device__ __forceinline__ void operator()() const {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
};
struct GroupSync {
  __device__ __forceinline__ void operator()() const { __syncthreads(); }
};

// A fused step's hooks for group (b, g), run by NTHR threads (tid = 0 ..
// NTHR-1) that share one stage.
//   pre:   raw loads -- one (row, 8-pair chunk) item per thread and pass:
//          both halves of the chunk; the V row (16 bytes per thread).
//   post:  the table (thread i: pair i, sincos in fp64 as the RoPE kernels),
//          the rotation of every item (sa_rope::rot8_bf16: the RoPE
//          kernels' bits) into the stage; the owner also stores the K row,
//          the V row (blocked layout) and the rotated Q; then every wave
//          reads its Q^T operand from the stage.
//   subst: on the block that holds the token's row, the K operand lanes of
//          that key and the V^T operand lanes of that key take the new row.
template <int D, int NTHR, class Sync>
struct StepHooks {
  static constexpr int H = D / 2;
  static constexpr int CPR = H / 8;                        // 8-pair chunks per row
  static constexpr int MAXI = (17 * CPR + NTHR - 1) / NTHR;  // items per thread (q_mult <= 16)
  const AttnArgs& a;
  const StepArgs& st;
  StepStage<D> sg;
  int b, g, tid;
  bool owner;         // holds the token's block: rotates K, writes the row
  int n_items;
  int64_t kb_new;
  // the group's rows: Q heads g*q_mult .. (b, g*q_mult + r), the K and V row of (b, g)
  const uint16_t* qsrc;
  const uint16_t* ksrc;
  const uint16_t* vsrc;
  u32x4 ru[MAXI], rv[MAXI], rvrow;
  double invf;        // inv_freq of pair tid (tid < H)

  __device__ __forceinline__ StepHooks(const AttnArgs& a_, const StepArgs& st_, char* lds, int b_,
                                       int g_, int tid_, bool owner_)
      : a(a_), st(st_), sg(lds, a_.q_mult), b(b_), g(g_), tid(tid_), owner(owner_) {
    n_items = (a.q_mult + (owner ? 1 : 0)) * CPR;
    kb_new = st.row / 32;
    qsrc = reinterpret_cast<const uint16_t*>(st.q_raw) + ((int64_t)b * a.n_q + g * a.q_mult) * D;
    ksrc = reinterpret_cast<const uint16_t*>(st.k_raw) + ((int64_t)b * a.n_kv + g) * D;
    vsrc = reinterpret_cast<const uint16_t*>(st.v_raw) + ((int64_t)b * a.n_kv + g) * D;
  }
  __device__ __forceinline__ void pre() {
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int it = tid + i * NTHR;
      if (it < n_items) {
        const int r = it / CPR, c = (it - r * CPR) * 8;
        const uint16_t* src = r < a.q_mult ? qsrc + r * D : ksrc;
        ru[i] = ld16(src + c);
        rv[i] = ld16(src + c + H);
      }
    }
    if (owner && tid < D / 8) rvrow = ld16(vsrc + 8 * tid);
    static_assert(H <= NTHR, "one pair of the table per thread");
    if (tid < H) invf = st.inv_freq[tid];
  }
  template <class Q>
  __device__ __forceinline__ void post(Q& qop) {
    const Sync sync;
    if (tid < H) {
      double sn, cn;
      sa_rope::sincos_reduced((double)st.pos * invf, &sn, &cn);
      const double cc = cn * st.conc, ss = sn * st.conc;
      sg.tab[tid] = make_double2(cc, ss);
      sg.tab32[tid] = make_float2((float)cc, (float)ss);
    }
    if (owner && tid < D / 8) st16(sg.vrow + 8 * tid, rvrow);
    sync();
    const float k2 = sa_rope::bf16_rot_k2(st.conc);
    uint16_t* krow = reinterpret_cast<uint16_t*>(const_cast<void*>(a.kc)) +
                     (((int64_t)b * a.C + st.row) * a.n_kv + g) * D;
    uint16_t* qrot = reinterpret_cast<uint16_t*>(st.q_rot) +
                     ((int64_t)b * a.n_q + g * a.q_mult) * D;
#pragma unroll
    for (int i = 0; i < MAXI; ++i) {
      const int it = tid + i * NTHR;
      if (it < n_items) {
        const int r = it / CPR, c = (it - r * CPR) * 8;
        u32x4 wa, wb;
        sa_rope::rot8_bf16(ru[i], rv[i], &sg.tab32[c], &sg.tab[c], k2, &wa, &wb);
        st16(sg.rows + r * D + c, wa);
        st16(sg.rows + r * D + c + H, wb);
        if (owner) {
          if (r == a.q_mult) {
            st16(krow + c, wa);
            st16(krow + c + H, wb);
          } else if (st.q_rot) {
            st16(qrot + r * D + c, wa);
            st16(qrot + r * D + c + H, wb);
          }
        }
      }
    }
    if (owner) {
      uint16_t* vblk = reinterpret_cast<uint16_t*>(const_cast<void*>(a.vc)) +
                       (((int64_t)b * (a.C / 32) + kb_new) * a.n_kv + g) * (int64_t)(D * 32) +
                       (st.row & 31);
      for (int i = tid; i < D; i += NTHR) vblk[i * 32] = sg.vrow[i];
    }
    sync();
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qop[ks] = j < a.q_mult ? *reinterpret_cast<const u32x4*>(sg.rows + j * D + 32 * ks + 8 * g4)
                             : u32x4{0, 0, 0, 0};
  }
  template <class Ops>
  __device__ __forceinline__ void subst(int64_t kb, Ops& ops) {
    if (kb != kb_new) return;
    const int lane = threadIdx.x & 63;
    const int j = lane & 15, g4 = lane >> 4;
    const int kk = (int)(st.row & 31);
    // K operand: row i = j of M tile mt holds key 8*(j>>2) + 4*mt + (j&3)
    if (j == 4 * (kk >> 3) + (kk & 3)) {
      const int mtn = (kk >> 2) & 1;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(sg.rows + a.q_mult * D + 32 * ks + 8 * g4);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          if (mt == mtn) ops.k[mt][ks] = kv;
      }
    }
    // V^T operand: lane (j, g4) holds keys 8*g4 .. 8*g4+7 of coordinate 16*dt + j
    if (g4 == (kk >> 3)) {
      const int wn = (kk & 7) >> 1;
      const bool hi16 = kk & 1;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const uint32_t nv = sg.vrow[16 * dt + j];
#pragma unroll
        for (int w = 0; w < 4; ++w)
          if (w == wn)
            ops.v[dt][w] = hi16 ? ((ops.v[dt][w] & 0xFFFFu) | (nv << 16))
                                : ((ops.v[dt][w] & 0xFFFF0000u) | nv);
      }
    }
  }
};

// The partials of a workgroup's waves (one run each of the same (b, g))
// meet in LDS and are folded in wave order into the workgroup's one partial
// (no sink: the merge adds it once).
template <int D>
__device__ __forceinline__ void fold_partial(const DecodeArgs& da, int pair, int split, int wave,
                                             float m_run, float l_run, const f32x4 (&O)[D / 16]) {
  constexpr int DT = D / 16;
  __shared__ __attribute__((aligned(16))) float acc_s[kWaves][16][D];
  __shared__ float m_s[kWaves][16], l_s[kWaves][16];
  const AttnArgs& a = da.at;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g4 = lane >> 4;
  const int S = da.n_splits;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4*>(&acc_s[wave][j][16 * dt + 4 * g4]) = O[dt];
  if (g4 == 0) {
    m_s[wave][j] = m_run;
    l_s[wave][j] = l_run;
  }
  __syncthreads();
  constexpr int CPH = D / 4;
  float* ml = da.ws + (int64_t)a.B * a.n_kv * S * a.q_mult * D;
  for (int i = threadIdx.x; i < a.q_mult * CPH; i += kThreads) {
    const int jq = i / CPH, c = i - jq * CPH;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_s[w][jq]);
    float L = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = m_s[w][jq];
      const float sc = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      L += l_s[w][jq] * sc;
      o += *reinterpret_cast<const f32x4*>(&acc_s[w][jq][4 * c]) * sc;
    }
    const int64_t slot = ((int64_t)pair * S + split) * a.q_mult + jq;
    *reinterpret_cast<f32x4*>(da.ws + slot * D + 4 * c) = o;
    if (c == 0) {
      ml[2 * slot] = M;
      ml[2 * slot + 1] = L;
    }
  }
}

// FOLD false: one wave per (b, g, split), KV head fastest, so that the waves
// running side by side read whole cache rows (all heads of a row are
// contiguous) and whole 32-key V blocks; each wave writes its partial.
// FOLD true (few (b, g) pairs): one workgroup per (b, g, split), (b, g)
// fastest, its run cut into one contiguous piece per wave and the waves'
// partials folded into one, so the merge reads a quarter of the partials.
// With many pairs the per-wave layout streams the cache faster (B = 8,
// 131k rows, 64/8 heads: 357 us against 392), with 8 pairs the fold wins
// (B = 1, 67.6k rows: split + merge 27.1 against 27.9 us).
template <int D, bool STEP, bool FOLD>
__device__ __forceinline__ void decode_split_body(const DecodeArgs& da, const StepArgs* st) {
  constexpr int DT = D / 16;
  const AttnArgs& a = da.at;
  const int lane = threadIdx.x & 63;
  // the wave index is uniform: scalar, so that the block loop runs on scalars
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g4 = lane >> 4;
  const int S = da.n_splits;               // partials per (b, g)
  const int pairs = a.B * a.n_kv;
  int b, g, split;
  if constexpr (FOLD) {
    const int pr = blockIdx.x % pairs;
    split = blockIdx.x / pairs;
    b = pr / a.n_kv;
    g = pr - b * a.n_kv;
  } else {
    const int wid = blockIdx.x * kWaves + wave;
    if (wid >= pairs * S) return;
    g = wid % a.n_kv;
    split = (wid / a.n_kv) % S;
    b = wid / (a.n_kv * S);
  }
  const int pair = b * a.n_kv + g;

  const int64_t P = a.q_offset;                         // query position
  const int64_t lo = a.window > 0 ? max((int64_t)0, P - a.window + 1) : 0;
  const int64_t hi = P + 1;
  const int64_t kb_lo = lo / 32, nblk = (hi + 31) / 32 - kb_lo;
  const int64_t pc = FOLD ? (int64_t)split * kWaves + wave : split;   // this wave's piece
  const int64_t np = FOLD ? (int64_t)S * kWaves : S;                  // pieces per (b, g)
  // block indices fit 32 bits (bf16 caches hold fewer than 2^31 rows); the
  // bounds are uniform, and kept in scalar registers, so the block loop's
  // compares and clamps are scalar
  const int b0 = __builtin_amdgcn_readfirstlane((int)(kb_lo + (pc * nblk) / np));
  const int b1 = __builtin_amdgcn_readfirstlane((int)(kb_lo + ((pc + 1) * nblk) / np));

  u32x4 qop[D / 32];
  float m_run, l_run;
  f32x4 O[DT];
  if constexpr (STEP) {
    extern __shared__ __attribute__((aligned(16))) char step_lds[];
    const int64_t kb_new = st->row / 32;
    StepHooks<D, 64, WaveSync> hk(a, *st, step_lds + wave * StepStage<D>::bytes(a.q_mult),
                                  b, g, lane, b0 <= kb_new && kb_new < b1);
    decode_blocks<D, false>(a, b, g, b0, b1, lo, hi, qop, m_run, l_run, O, hk);
  } else {
    load_q<D>(a, b, g, qop);
    NoStep hk;
    decode_blocks<D, false>(a, b, g, b0, b1, lo, hi, qop, m_run, l_run, O, hk);
  }
  l_run = sum_over_col(l_run);
  if constexpr (FOLD) {
    fold_partial<D>(da, pair, split, wave, m_run, l_run, O);
  } else if (j < a.q_mult) {
    const int64_t slot = ((int64_t)pair * S + split) * a.q_mult + j;
    float* acc = da.ws + slot * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<f32x4*>(acc + 16 * dt + 4 * g4) = O[dt];
    if (g4 == 0) {
      float* ml = da.ws + (int64_t)pairs * S * a.q_mult * D + 2 * slot;
      ml[0] = m_run;
      ml[1] = l_run;
    }
  }
}

// Split-KV partials (per wave, or folded per workgroup), written to the
// workspace for the merge.
template <int D, bool FOLD>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(DecodeArgs da) {
  decode_split_body<D, false, FOLD>(da, nullptr);
}
// The same with the step's rotation and append (per-wave stages in dynamic LDS).
template <int D, bool FOLD>
__global__ __launch_bounds__(kThreads) void decode_step_bf16_kernel(DecodeArgs da, StepArgs st) {
  decode_split_body<D, true, FOLD>(da, &st);
}

// A span of at most kShortRows rows (a band layer, or the first steps of a
// sequence) in one launch with no workspace: a workgroup per (b, g) whose
// waves take one or two 32-key blocks each; the partials meet in LDS and are
// folded in wave order, with the sink added once, by all of the workgroup's
// threads.
// Four waves: a 128-row band is four or five 32-key blocks, so each wave
// takes one or two, and the fold has four partials to add (the fused step
// at d = 64, B = 1 and 8: 6.8-7.0 us per launch against 8.1-8.4 with eight
// waves; two waves 6.6-6.8, but they would walk four blocks each on a
// 256-row span).
template <int D>
constexpr int short_waves() { return 4; }

template <int D, bool STEP>
__device__ __forceinline__ void decode_short_body(const AttnArgs& a, const StepArgs* st) {
  constexpr int DT = D / 16;
  constexpr int kShortWaves = short_waves<D>();
  constexpr int kShortThreads = kShortWaves * 64;
  __shared__ __attribute__((aligned(16))) float acc_s[kShortWaves][16][D];
  __shared__ float m_s[kShortWaves][16], l_s[kShortWaves][16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 15, g4 = lane >> 4;
  const int pair = blockIdx.x;
  const int b = pair / a.n_kv, g = pair - (pair / a.n_kv) * a.n_kv;

  const int64_t P = a.q_offset;
  const int64_t lo = a.window > 0 ? max((int64_t)0, P - a.window + 1) : 0;
  const int64_t hi = P + 1;
  const int64_t kb_lo = lo / 32, nblk = (hi + 31) / 32 - kb_lo;
  const int b0 = __builtin_amdgcn_readfirstlane((int)(kb_lo + (wave * nblk) / kShortWaves));
  const int b1 = __builtin_amdgcn_readfirstlane((int)(kb_lo + ((wave + 1) * nblk) / kShortWaves));

  u32x4 qop[D / 32];
  float m_run, l_run;
  f32x4 O[DT];
  if constexpr (STEP) {   // one stage for the workgroup; every thread takes part
    extern __shared__ __attribute__((aligned(16))) char step_lds[];
    StepHooks<D, kShortThreads, GroupSync> hk(a, *st, step_lds, b, g, threadIdx.x, true);
    decode_blocks<D, true>(a, b, g, b0, b1, lo, hi, qop, m_run, l_run, O, hk);
  } else {
    load_q<D>(a, b, g, qop);
    NoStep hk;
    decode_blocks<D, true>(a, b, g, b0, b1, lo, hi, qop, m_run, l_run, O, hk);
  }
  l_run = sum_over_col(l_run);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *reinterpret_cast<f32x4*>(&acc_s[wave][j][16 * dt + 4 * g4]) = O[dt];
  if (g4 == 0) {
    m_s[wave][j] = m_run;
    l_s[wave][j] = l_run;
  }
  __syncthreads();
  // fold: thread -> (head jq, 4 coordinates)
  constexpr int CPH = D / 4;
  for (int i = threadIdx.x; i < a.q_mult * CPH; i += kShortThreads) {
    const int jq = i / CPH, c = i - jq * CPH;
    const int h = g * a.q_mult + jq;
    const float sg = a.sinks[h] * SA_LOG2E;
    float M = sg;
#pragma unroll
    for (int w = 0; w < kShortWaves; ++w) M = fmaxf(M, m_s[w][jq]);
    float L = (sg == -INFINITY) ? 0.f : fast_exp2(sg - M);
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kShortWaves; ++w) {
      const float mw = m_s[w][jq];
      const float sc = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
      L += l_s[w][jq] * sc;
      o += *reinterpret_cast<const f32x4*>(&acc_s[w][jq][4 * c]) * sc;
    }
    o *= 1.0f / L;
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.n_q + h) * D + 4 * c;
    *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
  }
}

template <int D>
__global__ __launch_bounds__(short_waves<D>() * 64) void decode_short_bf16_kernel(AttnArgs a) {
  decode_short_body<D, false>(a, nullptr);
}
// The same with the step's rotation and append (one stage in dynamic LDS).
template <int D>
__global__ __launch_bounds__(short_waves<D>() * 64) void decode_short_step_bf16_kernel(AttnArgs a,
                                                                                      StepArgs st) {
  decode_short_body<D, true>(a, &st);
}

// One workgroup per (b, h).  Every global load is issued first: thread s < S
// takes split s's (m, l), and the accumulators are dealt round-robin over the
// splits to groups of threads (16-byte loads, held in registers); then the
// maximum and the weights, the weighted sums per group, and the groups added
// in group order.  Every sum has a fixed order, so the result is
// deterministic.
constexpr int kMergeThreads = 256;

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kMergeThreads / 64; ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
  return r;
}

template <int D, int MAXS>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs da) {
  constexpr int CPS = D / 4;                        // f32x4 vectors per split
  constexpr int G = kMergeThreads / CPS;            // split groups
  constexpr int KMAX = (MAXS + G - 1) / G;          // partials per group at most
  __shared__ float wsh[MAXS];
  __shared__ float red[kMergeThreads / 64];
  __shared__ f32x4 part[G][CPS];
  const AttnArgs& a = da.at;
  const int tid = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.n_q, h = bh - b * a.n_q;
  const int g = h / a.q_mult, jq = h - g * a.q_mult;
  const int S = da.n_splits;
  const int pairs = a.B * a.n_kv;
  const int pair = b * a.n_kv + g;
  const float* ml = da.ws + (int64_t)pairs * S * a.q_mult * D;
  const int64_t slot0 = ((int64_t)pair * S) * a.q_mult + jq;   // slot of split 0
  const int64_t sstride = a.q_mult;                            // slots between splits

  const int grp = tid / CPS, c = tid - grp * CPS;
  f32x4 accs[KMAX];
  const float* src = da.ws + slot0 * D + 4 * c;
#pragma unroll
  for (int k = 0; k < KMAX; ++k) {
    const int sp = grp + k * G;
    accs[k] = (grp < G && sp < S) ? *reinterpret_cast<const f32x4*>(src + sp * sstride * D)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float m = tid < S ? ml[2 * (slot0 + tid * sstride)] : -INFINITY;
  const float lv = tid < S ? ml[2 * (slot0 + tid * sstride) + 1] : 0.f;
  const float sg = a.sinks[h] * SA_LOG2E;

  const float M = fmaxf(sg, block_reduce(m, red, true));
  const float w = (tid < S && m != -INFINITY) ? fast_exp2(m - M) : 0.f;
  if (tid < S) wsh[tid] = w;
  const float L = block_reduce(lv * w, red, false) + ((sg == -INFINITY) ? 0.f : fast_exp2(sg - M));
  // block_reduce's barriers made wsh visible
  if (grp < G) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
      const int sp = grp + k * G;
      if (sp < S) acc += accs[k] * wsh[sp];
    }
    part[grp][c] = acc;
  }
  __syncthreads();
  if (tid < CPS) {
    f32x4 o = part[0][tid];
#pragma unroll
    for (int i = 1; i < G; ++i) o += part[i][tid];
    o *= 1.0f / L;
    uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.n_q + h) * D + 4 * tid;
    *reinterpret_cast<u32x2*>(out) = u32x2{pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
  }
}

// The merge, built for 64 partials at most where they fit (fewer loads in
// the unrolled gather than with the 256 bound: B = 1, 32 partials per
// (b, g): split + merge 27.1 against 27.7 us; a 32 bound measured 27.5).
template <int D>
void launch_merge(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid(a.at.B * a.at.n_q), block(kMergeThreads);
  if (a.n_splits <= 64)
    hipLaunchKernelGGL((decode_merge_kernel<D, 64>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, kMaxSplits>), grid, block, 0, s, a);
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  if (a.n_splits == 1) {
    hipLaunchKernelGGL(decode_short_bf16_kernel<D>, dim3(a.at.B * a.at.n_kv),
                       dim3(short_waves<D>() * 64), 0, s, a.at);
    return hipGetLastError();
  }
  const int pairs = a.at.B * a.at.n_kv;
  if (fold_splits(pairs))
    hipLaunchKernelGGL((decode_bf16_kernel<D, true>), dim3(pairs * a.n_splits), dim3(kThreads), 0,
                       s, a);
  else
    hipLaunchKernelGGL((decode_bf16_kernel<D, false>), dim3((pairs * a.n_splits + kWaves - 1) / kWaves),
                       dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_merge<D>(a, s);
  return hipGetLastError();
}

template <int D>
hipError_t launch_step_d(const DecodeArgs& a, const StepArgs& st, hipStream_t s) {
  const size_t stage = StepStage<D>::bytes(a.at.q_mult);
  if (a.n_splits == 1) {
    hipLaunchKernelGGL(decode_short_step_bf16_kernel<D>, dim3(a.at.B * a.at.n_kv),
                       dim3(short_waves<D>() * 64), stage, s, a.at, st);
    return hipGetLastError();
  }
  const int pairs = a.at.B * a.at.n_kv;
  if (fold_splits(pairs))
    hipLaunchKernelGGL((decode_step_bf16_kernel<D, true>), dim3(pairs * a.n_splits), dim3(kThreads),
                       kWaves * stage, s, a, st);
  else
    hipLaunchKernelGGL((decode_step_bf16_kernel<D, false>),
                       dim3((pairs * a.n_splits + kWaves - 1) / kWaves), dim3(kThreads),
                       kWaves * stage, s, a, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_merge<D>(a, s);
  return hipGetLastError();
}

}  // namespace

int decode_splits(int B, int n_kv, int64_t span_rows) {
  if (span_rows <= kSingleSplitRows) return 1;       // short span: one workgroup per (b, g)
  const int64_t nblk = (span_rows + 31) / 32 + 1;   // a span may straddle one more block
  const int64_t pairs = (int64_t)B * n_kv;
  const int64_t target = pairs <= kFewPairs ? kTargetWavesFewPairs : kTargetWaves;
  int64_t w = (target + pairs - 1) / pairs;          // waves per pair
  if (w > nblk) w = nblk;
  if (w > kMaxSplits) w = kMaxSplits;
  const int64_t s = fold_splits((int)pairs) ? w / kWaves : w;   // partials per pair
  return (int)(s < 1 ? 1 : s);
}

int decode_max_splits(int B, int n_kv, int64_t capacity) {
  return decode_splits(B, n_kv, capacity);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s) {
  switch (a.at.d) {
    case 64: return launch_d<64>(a, s);
    case 96: return launch_d<96>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_step_bf16(const DecodeArgs& a, const StepArgs& st, hipStream_t s) {
  switch (a.at.d) {
    case 64: return launch_step_d<64>(a, st, s);
    case 96: return launch_step_d<96>(a, st, s);
    case 128: return launch_step_d<128>(a, st, s);
    default: return hipErrorInvalidValue;
  }
}
