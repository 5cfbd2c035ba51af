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
//    Splits with no allowed key carry m = -inf, l = 0 and drop out.  A span
//    of at most 256 rows (a band layer) runs in one launch instead: a
//    workgroup per (b, g) whose waves take one or two 32-key blocks each and
//    fold their partials in LDS in the same fixed way, so a band step costs
//    one block's memory latency rather than a chain of them.
#include "sa_device.h"
#include "sa_kernels.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
#ifndef SA_DEC_WAVES
#define SA_DEC_WAVES 2048
#endif
constexpr int kTargetWaves = SA_DEC_WAVES;
constexpr int kMaxSplits = 256;
constexpr int64_t kSingleSplitRows = 256;   // spans this short run as one short launch
constexpr float kSlack = 8.0f;

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
template <int D>
__device__ __forceinline__ void decode_blocks(const AttnArgs& a, int b, int g, int64_t b0,
                                              int64_t b1, int64_t lo, int64_t hi,
                                              const u32x4 (&qop)[D / 32], float& m_run,
                                              float& l_run, f32x4 (&O)[D / 16]) {
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

  BlockOps<D> cur[2], nxt[2];
  auto load2 = [&](BlockOps<D>(&ops)[2], int64_t kb) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      if (kb + u < b1)
        load_block<D>(ops[u], kpair + (kb + u) * 32 * kstride, vpair + (kb + u) * vbstride,
                      kstride, j, g4);
  };
  if (b0 < b1) load2(cur, b0);
  for (int64_t kb = b0; kb < b1; kb += 2) {
    if (kb + 2 < b1) load2(nxt, kb + 2);
    const bool two = kb + 1 < b1;
    f32x4 Sc[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      Sc[u][0] = f32x4{0.f, 0.f, 0.f, 0.f};
      Sc[u][1] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (u == 1 && !two) break;
      const int64_t k0 = (kb + u) * 32;
      if (k0 + 32 > hi) {    // zero V of keys past the query (unwritten rows)
        const int valid = (int)(hi - (k0 + 8 * g4));
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
      if (k0 < lo || k0 + 32 > hi) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t key = k0 + 8 * g4 + 4 * mt + r;
            if (key < lo || key >= hi) Sc[u][mt][r] = -INFINITY;
          }
      }
    }
    if (!two) {
      Sc[1][0] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      Sc[1][1] = Sc[1][0];
    }
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 2; ++u)
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
    for (int u = 0; u < 2; ++u) {
      if (u == 1 && !two) break;
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
    if (kb + 2 < b1) {
      cur[0] = nxt[0];
      cur[1] = nxt[1];
    }
  }
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

// Split-KV partials: one wave per (b, g, split) over its run of the allowed
// blocks, written to the workspace for the merge.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(DecodeArgs da) {
  constexpr int DT = D / 16;
  const AttnArgs& a = da.at;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g4 = lane >> 4;
  const int wid = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int S = da.n_splits;
  const int pairs = a.B * a.n_kv;
  if (wid >= pairs * S) return;
  // KV head fastest: waves running side by side read whole cache rows
  // (all heads of a row are contiguous) and whole 32-key V blocks.
  const int g = wid % a.n_kv;
  const int split = (wid / a.n_kv) % S;
  const int b = wid / (a.n_kv * S);
  const int pair = b * a.n_kv + g;

  const int64_t P = a.q_offset;                         // query position
  const int64_t lo = a.window > 0 ? max((int64_t)0, P - a.window + 1) : 0;
  const int64_t hi = P + 1;
  const int64_t kb_lo = lo / 32, nblk = (hi + 31) / 32 - kb_lo;
  const int64_t b0 = kb_lo + (split * nblk) / S;
  const int64_t b1 = kb_lo + ((split + 1) * nblk) / S;

  u32x4 qop[D / 32];
  load_q<D>(a, b, g, qop);
  float m_run, l_run;
  f32x4 O[DT];
  decode_blocks<D>(a, b, g, b0, b1, lo, hi, qop, m_run, l_run, O);
  l_run = sum_over_col(l_run);
  if (j < a.q_mult) {
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

// A span of at most kShortRows rows (a band layer, or the first steps of a
// sequence) in one launch with no workspace: a workgroup per (b, g) whose
// waves take one or two 32-key blocks each; the partials meet in LDS and are
// folded in wave order, with the sink added once, by all of the workgroup's
// threads.
// Eight waves at d = 64; four at d = 96 and 128, whose per-wave pass needs
// more registers than two waves per SIMD leave it.
template <int D>
constexpr int short_waves() { return D == 64 ? 8 : 4; }

template <int D>
__global__ __launch_bounds__(short_waves<D>() * 64) void decode_short_bf16_kernel(AttnArgs a) {
  constexpr int DT = D / 16;
  constexpr int kShortWaves = short_waves<D>();
  constexpr int kShortThreads = kShortWaves * 64;
  __shared__ __attribute__((aligned(16))) float acc_s[kShortWaves][16][D];
  __shared__ float m_s[kShortWaves][16], l_s[kShortWaves][16];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15, g4 = lane >> 4;
  const int pair = blockIdx.x;
  const int b = pair / a.n_kv, g = pair - (pair / a.n_kv) * a.n_kv;

  const int64_t P = a.q_offset;
  const int64_t lo = a.window > 0 ? max((int64_t)0, P - a.window + 1) : 0;
  const int64_t hi = P + 1;
  const int64_t kb_lo = lo / 32, nblk = (hi + 31) / 32 - kb_lo;
  const int64_t b0 = kb_lo + (wave * nblk) / kShortWaves;
  const int64_t b1 = kb_lo + ((wave + 1) * nblk) / kShortWaves;

  u32x4 qop[D / 32];
  load_q<D>(a, b, g, qop);
  float m_run, l_run;
  f32x4 O[DT];
  decode_blocks<D>(a, b, g, b0, b1, lo, hi, qop, m_run, l_run, O);
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

template <int D>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(DecodeArgs da) {
  constexpr int CPS = D / 4;                        // f32x4 vectors per split
  constexpr int G = kMergeThreads / CPS;            // split groups
  constexpr int KMAX = (kMaxSplits + G - 1) / G;    // splits per group at most
  __shared__ float wsh[kMaxSplits];
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

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  if (a.n_splits == 1) {
    hipLaunchKernelGGL(decode_short_bf16_kernel<D>, dim3(a.at.B * a.at.n_kv),
                       dim3(short_waves<D>() * 64), 0, s, a.at);
    return hipGetLastError();
  }
  const int waves = a.at.B * a.at.n_kv * a.n_splits;
  const int grid = (waves + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(decode_bf16_kernel<D>, dim3(grid), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(a.at.B * a.at.n_q), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int decode_splits(int B, int n_kv, int64_t span_rows) {
  if (span_rows <= kSingleSplitRows) return 1;       // short span: one workgroup per (b, g)
  const int64_t nblk = (span_rows + 31) / 32 + 1;   // a span may straddle one more block
  int64_t s = (kTargetWaves + (int64_t)B * n_kv - 1) / ((int64_t)B * n_kv);
  if (s > nblk) s = nblk;
  if (s > kMaxSplits) s = kMaxSplits;
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
