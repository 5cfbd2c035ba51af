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
//    of independent waves for 256 CUs.
//  * Matrix cores on 8 of 16 columns: the q_mult query heads of the group
//    form the N side of S^T = K Q^T (v_mfma_f32_16x16x32_bf16), so one K row
//    load serves all heads of the group.  K operands load straight from HBM
//    in the row layout; V^T operands load straight from the blocked V
//    layout (8 consecutive keys of one coordinate = one 16-byte load); no
//    LDS round trip.  The next block's loads are issued before the current
//    block is multiplied.
//  * Each wave writes a partial (m, l, acc) in base-2 units to the
//    workspace; a merge kernel folds the partials of a head in a fixed order
//    and adds the sink exactly once:
//      M = max(sigma', max_c m_c), L = 2^(sigma'-M) + sum_c l_c 2^(m_c-M),
//      out = sum_c acc_c 2^(m_c-M) / L        (sigma' = sigma * log2 e).
//    Splits with no allowed key carry m = -inf, l = 0 and drop out.
#include "sa_device.h"
#include "sa_kernels.h"

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kTargetWaves = 4096;
constexpr int kMaxSplits = 256;

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

template <int D>
__global__ __launch_bounds__(kThreads) void decode_bf16_kernel(DecodeArgs da) {
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  const AttnArgs& a = da.at;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, g4 = lane >> 4;
  const int wid = blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int S = da.n_splits;
  const int pairs = a.B * a.n_kv;
  if (wid >= pairs * S) return;
  const int split = wid % S;
  const int pair = wid / S;
  const int b = pair / a.n_kv, g = pair - b * a.n_kv;
  const int64_t C = a.C;

  const int64_t P = a.q_offset;                         // query position
  const int64_t lo = a.window > 0 ? max((int64_t)0, P - a.window + 1) : 0;
  const int64_t hi = P + 1;
  const int64_t kb_lo = lo / 32, nblk = (hi + 31) / 32 - kb_lo;
  const int64_t b0 = kb_lo + (split * nblk) / S;
  const int64_t b1 = kb_lo + ((split + 1) * nblk) / S;

  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);
  const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.kc);
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.vc);

  // Q^T operand: column j = head g*q_mult + j (zero past q_mult)
  u32x4 qop[KS];
  const bool qv = j < a.q_mult;
  const uint16_t* qrow = q + ((int64_t)b * a.n_q + g * a.q_mult + (qv ? j : 0)) * D;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qop[ks] = qv ? ld16(qrow + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0};

  const float scale = a.sm_scale * SA_LOG2E;
  float m_run = -INFINITY, l_run = 0.f;
  f32x4 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) O[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kstride = a.n_kv * D;
  const uint16_t* kpair = kc + ((int64_t)b * C * a.n_kv + g) * D;        // row 0 of (b, g)
  const uint16_t* vpair = vc + ((int64_t)b * (C / 32) * a.n_kv + g) * (int64_t)(D * 32);
  const int64_t vbstride = (int64_t)a.n_kv * D * 32;                      // per 32-key block

  BlockOps<D> cur, nxt;
  if (b0 < b1) load_block<D>(cur, kpair + b0 * 32 * kstride, vpair + b0 * vbstride, kstride, j, g4);
  for (int64_t kb = b0; kb < b1; ++kb) {
    if (kb + 1 < b1)
      load_block<D>(nxt, kpair + (kb + 1) * 32 * kstride, vpair + (kb + 1) * vbstride, kstride, j, g4);
    const int64_t k0 = kb * 32;
    const bool partial = (k0 < lo) || (k0 + 32 > hi);
    if (k0 + 32 > hi) {    // zero V of keys past the query (unwritten rows)
      const int valid = (int)(hi - (k0 + 8 * g4));
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t keep = (2 * w + 1 < valid) ? 0xFFFFFFFFu : (2 * w < valid ? 0x0000FFFFu : 0u);
          cur.v[dt][w] &= keep;
        }
    }
    f32x4 S[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) S[mt] = mfma16x16x32(cur.k[mt][ks], qop[ks], S[mt]);
    // lane (j, g4), element (mt, r): key k0 + 8*g4 + 4*mt + r
    if (partial) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t key = k0 + 8 * g4 + 4 * mt + r;
          if (key < lo || key >= hi) S[mt][r] = -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S[mt][r]);
    mx = xor_max(mx, 16);
    mx = xor_max(mx, 32);
    const float m_new = fmaxf(m_run, mx * scale);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float p[8], ls = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      p[e] = fast_exp2(fmaf(S[e >> 2][e & 3], scale, -m_use));
      ls += p[e];
    }
    const u32x4 Pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                      pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])};
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt] = mfma16x16x32(cur.v[dt], Pk, O[dt] * alpha);
    if (kb + 1 < b1) cur = nxt;
  }

  // ---- partial of this split: lanes (j < q_mult)
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
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

// One wave per (b, h): fold the partials of its splits in split order.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(DecodeArgs da) {
  const AttnArgs& a = da.at;
  const int lane = threadIdx.x;
  const int bh = blockIdx.x;
  const int b = bh / a.n_q, h = bh - b * a.n_q;
  const int g = h / a.q_mult, jq = h - g * a.q_mult;
  const int S = da.n_splits;
  const int pairs = a.B * a.n_kv;
  const int pair = b * a.n_kv + g;
  const float* ml = da.ws + (int64_t)pairs * S * a.q_mult * D;
  const float sg = a.sinks[h] * SA_LOG2E;

  float M = sg;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * (((int64_t)pair * S + s) * a.q_mult + jq)]);
  float L = (sg == -INFINITY) ? 0.f : fast_exp2(sg - M);
  constexpr int PER = (D + 63) / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;
  for (int s = 0; s < S; ++s) {
    const int64_t slot = ((int64_t)pair * S + s) * a.q_mult + jq;
    const float m = ml[2 * slot];
    if (m == -INFINITY) continue;
    const float w = fast_exp2(m - M);
    L += ml[2 * slot + 1] * w;
    const float* src = da.ws + slot * D;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int dd = lane + 64 * i;
      if (dd < D) acc[i] += src[dd] * w;
    }
  }
  const float inv = 1.0f / L;
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out) + ((int64_t)b * a.n_q + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int dd = lane + 64 * i;
    if (dd < D) out[dd] = (uint16_t)f32_to_bf16_bits(acc[i] * inv);
  }
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  const int waves = a.at.B * a.at.n_kv * a.n_splits;
  const int grid = (waves + kWaves - 1) / kWaves;
  hipLaunchKernelGGL(decode_bf16_kernel<D>, dim3(grid), dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel<D>, dim3(a.at.B * a.at.n_q), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int decode_splits(int B, int n_kv, int64_t span_rows) {
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
