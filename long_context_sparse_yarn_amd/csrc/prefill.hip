// sinkattn_prefill (bf16): sink-augmented grouped-query attention of a chunk
// of queries against the KV cache, on the gfx950 matrix cores.
//
// What is computed ("MoE-Xtend" README, ATTENTION STACK; "GQA Attention"
// study note, How it works): for query head h of KV group g = h / q_mult at
// global position p, softmax over the allowed scores sm_scale*<q, K_j>
// (j <= p, and j > p - W for a band of W keys) together with one extra
// column holding the head's sink logit; the sink column is dropped after
// normalisation and the remaining weights mix V.
//
// How (gfx950 design):
//  * A workgroup (4 waves) owns one (b, g) pair and a block of query
//    positions.  All q_mult heads of the group are stacked, so every 64-key
//    K/V tile staged in LDS feeds 128 (or 256) query rows at once.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16:
//    each lane then owns one query column and 16 of the tile's keys, so the
//    softmax state (running max m, partial sum l) is per lane.  K rows are
//    read from LDS in a permuted order chosen so that each lane's keys are 8
//    consecutive keys per 32-key half; its exp'd scores packed to bf16 are
//    directly the B operand of O^T += V^T P^T, and V^T comes from the
//    blocked V cache layout (32 keys contiguous per coordinate).
//  * Online softmax in base 2 (log2 e folded into the scale and the sink),
//    seeded with the sink: m = sigma*log2e, l = 1 (sigma = -inf: m = -inf,
//    l = 0).  The reference is lazy: it moves to the running max (with a
//    cross-lane max and a rescale of O and l) only when a lane's tile sum
//    passes 2^64 or a query has no reference yet, in a slow path outside the
//    steady-state loop; so most tiles need no max, no cross-lane traffic and
//    no accumulator rescale, and nothing comes near overflow.  Probabilities are rounded
//    to bf16 once (v_cvt_pk_bf16_f32) and the row sums accumulate those same
//    rounded values (v_dot2c_f32_bf16), so numerator and denominator agree.
//  * Masks are computed from positions, only on tiles that cross the
//    diagonal or the band edge; rows past the last query position are
//    zero-filled in LDS, so unwritten cache rows are never read.
//  * K/V tiles are double-buffered: the next tile's global loads are in
//    flight while the current tile is multiplied.
//  * Workgroups of the same (b, g) are spread so that, when B*n_kv is a
//    multiple of 8, every XCD serves fixed KV heads and their K/V stays in
//    that XCD's L2; the longest (latest) query blocks start first.
#include "sa_device.h"
#include "sa_kernels.h"

#include <type_traits>

namespace {

constexpr int kTile = 64;  // keys per tile
constexpr float kHeadroom = 18446744073709551616.0f;   // 2^64: largest tile sum kept

// LDS placement of K row r, 16-byte chunk k (in elements).  Rows are not
// padded (d = 96 rows take 256 bytes so that the swizzle below stays a
// permutation of the row's slots); chunk k of row r sits in slot
// k ^ f(r), f(r) = (r&3) | ((r>>1)&4) | ((r>>1)&8) (the top bit only where a
// row has 16 slots).  The operand reads take rows 32h + 8q + 4t + r'
// (q, r' < 4) across 16 lanes and a chunk per lane group; with this swizzle a
// wave's 16-byte reads hit no bank twice (timed at the conflict-free rate of
// a linear read, against twice that for a padded pitch).
template <int D>
constexpr int k_pitch() { return D == 96 ? 128 : D; }
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  constexpr int mask = k_pitch<D>() / 8 - 1;
  return ((r & 3) | ((r >> 1) & 4) | ((r >> 1) & 8)) & mask;
}
template <int D>
__device__ __forceinline__ int k_lds(int r, int k) {
  return r * k_pitch<D>() + 8 * (k ^ k_swz<D>(r));
}
// V^T rows (one per coordinate and 32-key half, 64 bytes each) are not
// padded either; chunk c of row r sits in slot c ^ ((r>>1)&3), which keeps
// the 16-lane V^T operand reads conflict-free.
__device__ __forceinline__ int v_lds(int r, int c) { return r * 32 + 8 * (c ^ ((r >> 1) & 3)); }

template <int D, int NT, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(AttnArgs a, int BQ, int n_qb) {
  constexpr int kThreads = NW * 64;
  constexpr int KS = D / 32;          // contraction steps of S^T = K Q^T
  constexpr int DT = D / 16;          // coordinate tiles of O^T
  constexpr int KTOT = kTile * D / 8; // 16-byte K chunks per tile
  constexpr int VTOT = 2 * D * 4;     // 16-byte V chunks per tile
  constexpr int KCH = (KTOT + kThreads - 1) / kThreads;   // per thread
  constexpr int VCH = (VTOT + kThreads - 1) / kThreads;
  constexpr int KBUF = kTile * k_pitch<D>();

  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][2 * D * 32];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int j = lane & 15;
  const int g4 = lane >> 4;

  const int pairs = a.B * a.n_kv;
  const int pair = blockIdx.x % pairs;
  const int qb = n_qb - 1 - (int)(blockIdx.x / pairs);
  const int b = pair / a.n_kv;
  const int g = pair - b * a.n_kv;
  const int p0 = qb * BQ;
  const int t_end = min(p0 + BQ, a.T_q);
  const int64_t C = a.C;

  const uint16_t* q = reinterpret_cast<const uint16_t*>(a.q);

  // ---- this lane's query rows (one per 16-wide N tile)
  int tpos[NT], head[NT];
  bool rvalid[NT];
  u32x4 qop[NT][KS];
  float m_run[NT], l_run[NT];
  f32x4 O[DT][NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int r = (wave * NT + n) * 16 + j;
    const int m = r % a.q_mult;
    int tp = p0 + r / a.q_mult;
    rvalid[n] = (r < BQ * a.q_mult) && (tp < a.T_q);
    if (!rvalid[n]) tp = t_end - 1;
    tpos[n] = tp;
    head[n] = g * a.q_mult + m;
    const uint16_t* qrow = q + (((int64_t)b * a.T_q + tp) * a.n_q + head[n]) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qop[n][ks] = rvalid[n] ? ld16(qrow + 32 * ks + 8 * g4) : u32x4{0, 0, 0, 0};
    const float sg = a.sinks[head[n]] * SA_LOG2E;
    m_run[n] = sg;                                   // -inf when the sink is off
    l_run[n] = (g4 == 0 && sg != -INFINITY) ? 1.0f : 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const float scale = a.sm_scale * SA_LOG2E;
  const int64_t P_min = a.q_offset + p0;
  const int64_t P_max = a.q_offset + t_end - 1;
  const int64_t lo = a.window > 0 ? max((int64_t)0, P_min - a.window + 1) : 0;
  const int64_t hi = P_max + 1;   // keys >= hi are masked for every row here
  const int64_t t_first = lo / kTile, t_last = (hi - 1) / kTile;

  // ---- per-thread load slots: K chunk (row, ch) and V chunk (blk, dd, ch)
  const int64_t krow_stride = (int64_t)a.n_kv * D;                  // elements per cache row
  const int64_t vblk_stride = (int64_t)a.n_kv * D * 32;             // elements per 32-key block
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.kc) + ((int64_t)b * C * a.n_kv + g) * D;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.vc) +
                          ((int64_t)b * (C / 32) * a.n_kv + g) * (int64_t)(D * 32);
  int k_row[KCH], k_off[KCH], k_lds_off[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int c = min((int)threadIdx.x + i * kThreads, KTOT - 1);   // excess slots repeat the last
    k_row[i] = c / (D / 8);
    const int ch = c - k_row[i] * (D / 8);
    k_off[i] = 8 * ch;
    k_lds_off[i] = k_lds<D>(k_row[i], ch);
  }
  int v_key[VCH], v_off[VCH], v_lds_off[VCH];
#pragma unroll
  for (int i = 0; i < VCH; ++i) {
    const int c = min((int)threadIdx.x + i * kThreads, VTOT - 1);
    const int blk = c / (D * 4);
    const int rem = c - blk * (D * 4);
    const int dd = rem >> 2, ch = rem & 3;
    v_key[i] = 32 * blk + 8 * ch;                                  // first key of the chunk
    v_off[i] = (int)(blk * vblk_stride) + dd * 32 + 8 * ch;
    v_lds_off[i] = v_lds(blk * D + dd, ch);
  }

  u32x4 kreg[KCH], vreg[VCH];
  auto load_tile = [&](int64_t t) {
    const int64_t k0 = t * kTile;
    const uint16_t* kt = kbase + k0 * krow_stride;
    const uint16_t* vt = vbase + (k0 / 32) * vblk_stride;
    if (k0 + kTile <= hi) {                // whole tile below the last query
#pragma unroll
      for (int i = 0; i < KCH; ++i) kreg[i] = ld16(kt + k_row[i] * krow_stride + k_off[i]);
#pragma unroll
      for (int i = 0; i < VCH; ++i) vreg[i] = ld16(vt + v_off[i]);
      return;
    }
#pragma unroll
    for (int i = 0; i < KCH; ++i)
      kreg[i] = k0 + k_row[i] < hi ? ld16(kt + k_row[i] * krow_stride + k_off[i])
                                   : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int64_t key0 = k0 + v_key[i];
      u32x4 v = {0, 0, 0, 0};
      if (key0 < hi) {
        v = ld16(vt + v_off[i]);
        if (key0 + 8 > hi) {       // zero the keys past the last query
          const int valid = (int)(hi - key0);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t keep = (2 * w + 1 < valid) ? 0xFFFFFFFFu : (2 * w < valid ? 0x0000FFFFu : 0u);
            v[w] &= keep;
          }
        }
      }
      vreg[i] = v;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) st16(&Ks[buf][k_lds_off[i]], kreg[i]);
#pragma unroll
    for (int i = 0; i < VCH; ++i) st16(&Vs[buf][v_lds_off[i]], vreg[i]);
  };

  // LDS read offsets of this lane's operands: K chunk g4 + 4*ks of row
  // krow(mt) sits at ka_row[mt] + 32*(ks ^ ka_hi[mt]) (the swizzle's low two
  // bits act on g4, its high bits on ks); V^T reads add uniform offsets.
  int ka_row[4], ka_hi[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int krow = 32 * (mt >> 1) + 8 * (j >> 2) + 4 * (mt & 1) + (j & 3);
    const int f = k_swz<D>(krow);
    ka_row[mt] = krow * k_pitch<D>() + 8 * (g4 ^ (f & 3));
    ka_hi[mt] = f >> 2;
  }
  const int va_off = v_lds(j, g4);

  // ---- one tile of keys, in three parts: scores S^T = K Q^T (masked on
  // tiles that cross the diagonal or the band edge), probabilities against
  // the current reference m_run, and O^T += V^T P^T.
  struct Scores { f32x4 v[4][NT]; };
  auto scores = [&](int buf, int64_t k0, auto masked) {
    Scores S;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int n = 0; n < NT; ++n) S.v[mt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const u32x4 A = ld16(&Ks[buf][ka_row[mt] + 32 * (ks ^ ka_hi[mt])]);
#pragma unroll
        for (int n = 0; n < NT; ++n) S.v[mt][n] = mfma16x16x32(A, qop[n][ks], S.v[mt][n]);
      }
    }
    // lane (j, g4) holds, for M tile mt and element r, the score of key
    // k0 + 32*(mt>>1) + 8*g4 + 4*(mt&1) + r.
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int rel0 = (int)(k0 - (a.q_offset + tpos[n]));   // key - p at (mt, r) = 0
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rel = rel0 + 32 * (mt >> 1) + 8 * g4 + 4 * (mt & 1) + r;
            const bool ok = rel <= 0 && (a.window <= 0 || rel > -a.window);
            if (!ok) S.v[mt][n][r] = -INFINITY;
          }
      }
    }
    return S;
  };
  // p = 2^(s*scale - m_run), rounded to bf16 once; ls = this lane's sum of
  // those rounded values (v_dot2 against 1).
  auto probs = [&](const Scores& S, u32x4 (&Pk)[2][NT], float (&ls)[NT]) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float m_use = (m_run[n] == -INFINITY) ? 0.f : m_run[n];
      float acc = 0.f;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          const int e = 2 * e2;
          const float p0 = fast_exp2(fmaf(S.v[2 * h + (e >> 2)][n][e & 3], scale, -m_use));
          const float p1 = fast_exp2(fmaf(S.v[2 * h + ((e + 1) >> 2)][n][(e + 1) & 3], scale, -m_use));
          w[e2] = pack_bf16x2(p0, p1);
          acc = sum_bf16x2(w[e2], acc);
        }
        Pk[h][n] = u32x4{w[0], w[1], w[2], w[3]};
      }
      ls[n] = acc;
    }
  };
  auto pv = [&](int buf, const u32x4 (&Pk)[2][NT]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x4 A = ld16(&Vs[buf][va_off + (h * D + 16 * dt) * 32]);
#pragma unroll
        for (int n = 0; n < NT; ++n) O[dt][n] = mfma16x16x32(A, Pk[h][n], O[dt][n]);
      }
  };
  // Move the reference to the true running max (column max across the four
  // lanes of a query) and rescale what has been accumulated.
  auto rescale = [&](const Scores& S) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, S.v[mt][n][r]);
      const float m_new = fmaxf(m_run[n], max_over_col(mx) * scale);
      // m_run == -inf: nothing accumulated yet (and m_new may be -inf too)
      const float alpha = (m_run[n] == -INFINITY) ? 0.f : fast_exp2(m_run[n] - m_new);
      l_run[n] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt][n] *= alpha;
      m_run[n] = m_new;
    }
  };

  load_tile(t_first);
  store_tile(0);
  __syncthreads();

  // Steady state: the reference m_run stays put while every lane's tile sum
  // stays below 2^64 (so no exponential, partial sum or accumulator can come
  // near fp32/bf16 overflow); a tile that breaks that, or a query with no
  // reference yet (no sink and nothing seen), leaves the loop for the slow
  // path, which moves the reference, redoes that tile and comes back.  The
  // fast loop never rewrites O outside the matrix cores.
  int buf = 0;
  int64_t t = t_first;
  for (;;) {
    bool slow = false;
    Scores S;
    u32x4 Pk[2][NT];
    float ls[NT];
    for (; t <= t_last; ++t) {
      const bool more = t < t_last;
      if (more) load_tile(t + 1);
      const int64_t k0 = t * kTile;
      const bool need_mask = (k0 + kTile - 1 > P_min) ||
                             (a.window > 0 && k0 < P_max - a.window + 1);
      if (need_mask)
        S = scores(buf, k0, std::true_type{});
      else
        S = scores(buf, k0, std::false_type{});
      probs(S, Pk, ls);
      bool bad = false;
#pragma unroll
      for (int n = 0; n < NT; ++n) bad |= !(ls[n] <= kHeadroom) || m_run[n] == -INFINITY;
      if (__builtin_amdgcn_ballot_w64(bad) != 0) {
        slow = true;
        break;
      }
#pragma unroll
      for (int n = 0; n < NT; ++n) l_run[n] += ls[n];
      pv(buf, Pk);
      if (more) store_tile(buf ^ 1);
      __syncthreads();
      buf ^= 1;
    }
    if (!slow) break;
    rescale(S);
    probs(S, Pk, ls);
#pragma unroll
    for (int n = 0; n < NT; ++n) l_run[n] += ls[n];
    pv(buf, Pk);
    if (t < t_last) store_tile(buf ^ 1);
    __syncthreads();
    buf ^= 1;
    ++t;
  }

  // ---- normalise and store: lane holds O^T[16*dt + 4*g4 + r][query]
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float inv = 1.0f / sum_over_col(l_run[n]);
    if (!rvalid[n]) continue;
    uint16_t* orow = out + (((int64_t)b * a.T_q + tpos[n]) * a.n_q + head[n]) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const f32x4 o = O[dt][n] * inv;
      u32x2 w = {pack_bf16x2(o.x, o.y), pack_bf16x2(o.z, o.w)};
      *reinterpret_cast<u32x2*>(orow + 16 * dt + 4 * g4) = w;
    }
  }
}

template <int D, int NT, int NW>
hipError_t launch_d(const AttnArgs& a, hipStream_t s) {
  const int rows = NW * NT * 16;
  if (a.q_mult > rows) return hipErrorInvalidValue;
  const int BQ = rows / a.q_mult;
  const int n_qb = (a.T_q + BQ - 1) / BQ;
  const int64_t grid = (int64_t)n_qb * a.B * a.n_kv;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, NT, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s,
                     a, BQ, n_qb);
  return hipGetLastError();
}

}  // namespace

// Tile shape per head dimension: N tiles (16 queries each) per wave and
// waves per workgroup, for full-causal layers and for band layers (whose
// workgroups re-read a window of K/V per query block, so taller query blocks
// cut traffic).  Overridable at build time for tuning sweeps.
#ifndef SA_PF64
#define SA_PF64 2, 4
#endif
#ifndef SA_PF96
#define SA_PF96 2, 8
#endif
#ifndef SA_PF128
#define SA_PF128 2, 4
#endif
#ifndef SA_PFB64
#define SA_PFB64 2, 4
#endif
#ifndef SA_PFB96
#define SA_PFB96 2, 8
#endif
#ifndef SA_PFB128
#define SA_PFB128 2, 4
#endif
constexpr int kBandWindowMax = 512;   // windows up to this use the band shape

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t s) {
  const bool band = a.window > 0 && a.window <= kBandWindowMax;
  switch (a.d) {
    case 64: return band ? launch_d<64, SA_PFB64>(a, s) : launch_d<64, SA_PF64>(a, s);
    case 96: return band ? launch_d<96, SA_PFB96>(a, s) : launch_d<96, SA_PF96>(a, s);
    case 128: return band ? launch_d<128, SA_PFB128>(a, s) : launch_d<128, SA_PF128>(a, s);
    default: return hipErrorInvalidValue;
  }
}
