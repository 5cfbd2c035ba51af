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
//    no accumulator rescale, and nothing comes near overflow.  Probabilities
//    are rounded to bf16 once (v_cvt_pk_bf16_f32); their row sums come from
//    the matrix cores (an all-ones A operand times the same P^T the PV product
//    uses), so numerator and denominator agree and the vector units, which
//    bound the unit, do no summing.
//  * Masks are computed from positions, only on tiles that cross the
//    diagonal or the band edge; rows past the last query position are
//    zero-filled in LDS, so unwritten cache rows are never read.
//  * K/V tiles are double-buffered: the next tile's global loads are in
//    flight while the current tile is multiplied.
//  * Workgroups of the same (b, g) are spread so that, when B*n_kv is a
//    multiple of 8, every XCD serves fixed KV heads and their K/V stays in
//    that XCD's L2; the longest (latest) query blocks start first.
#include "sa_device.h"
#include "sa_attn.h"
#include "sa_rope.h"


// 1: where it pays (d = 96 with two N tiles per wave), each unit's LDS
// operands (K for its scores, V for its PV) are read during the previous
// unit's vector work; 0: always at the start of the unit.
#ifndef SA_OPS_AHEAD
#define SA_OPS_AHEAD 1
#endif


namespace {

constexpr int kTile = 64;  // keys per tile
constexpr float kHeadroom = 18446744073709551616.0f;   // 2^64: largest tile sum kept
// neg_ref of a query with no reference yet: every allowed score then gives
// p = 2^(s*scale + 2^100) = inf, so the unit's sum fails the headroom test
// and the slow path sets a reference, with no test of its own per unit;
// masked scores (-inf) still give p = 0.
constexpr float kNoRef = 1267650600228229401496703205376.0f;   // 2^100

// 16 bytes from global memory straight into LDS: lane l of the wave writes
// LDS bytes [16 l, 16 l + 16) of the block at lds_block (uniform per wave).
__device__ __forceinline__ void lds_direct16(const void* src, const uint16_t* lds_block) {
  __builtin_amdgcn_global_load_lds(
      src, (__attribute__((address_space(3))) void*)(const_cast<uint16_t*>(lds_block)), 16, 0, 0);
}
// Wait for this wave's global loads (including those into LDS).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// LDS placement of K: rows are not padded (d/8 sixteen-byte slots each) and
// chunk k of row r sits in slot k ^ f(r).  The operand reads take rows
// 32h + 8q + 4t + r' (q, r' < 4) across 16 lanes and chunk g4 + 4*ks in lane
// group g4; with f(r) = (r&3) | ((r>>1)&4) | ((r>>1)&8) (bits above the row's
// slot count dropped) for d = 64 and 128, and f(r) = 2*(bit1(r) ^ bit4(r)) for
// the 12-slot rows of d = 96, a wave's 16-byte reads time at the rate of a
// linear read (a padded pitch measured twice that).  f uses row bits 0, 1, 3
// and 4 only, so it is the same for the four M tiles a lane reads.
template <int D>
constexpr int k_pitch() { return D; }
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  if constexpr (D == 96) return (((r >> 1) ^ (r >> 4)) & 1) << 1;
  constexpr int mask = D / 8 - 1;
  return ((r & 3) | ((r >> 1) & 4) | ((r >> 1) & 8)) & mask;
}
// V^T rows (one per coordinate and 32-key half, 64 bytes each) are not
// padded either; chunk c of row r sits in slot c ^ ((r>>1)&3), which keeps
// the 16-lane V^T operand reads conflict-free.
__device__ __forceinline__ int v_lds(int r, int c) { return r * 32 + 8 * (c ^ ((r >> 1) & 3)); }

// Full-causal walks at d = 64 take whole tiles in threes (LONG): that shape
// is held to three waves per SIMD (168 VGPRs), which its walk in threes
// would otherwise take to 178 (two waves); the few values this spills live
// outside the walk (set-up and epilogue).  Band layers (walks of three
// tiles or fewer) keep the plain walk and no spills.
template <int D, int NT, int NW, bool LONG>
constexpr int prefill_min_waves() { return (LONG && D == 64 && NT == 2 && NW == 4) ? 3 : 1; }

template <int D, int NT, int NW, bool ROPE, bool LONG>
__global__ __launch_bounds__(NW * 64, (prefill_min_waves<D, NT, NW, LONG>())) void prefill_bf16_kernel(
    AttnArgs a, int BQ, int n_qb, RopeTab rt) {
  constexpr int kThreads = NW * 64;
  constexpr int KS = D / 32;          // contraction steps of S^T = K Q^T
  constexpr int DT = D / 16;          // coordinate tiles of O^T
  constexpr int KBUF = kTile * k_pitch<D>();
  constexpr bool kPhaseSplit = D != 64;
  // Reading a unit's operands one unit ahead costs registers: 3% faster for
  // d = 96 full-causal blocks (212 VGPRs, still two waves per SIMD); d = 64
  // would drop from three waves per SIMD to two (12% slower) and the d = 96
  // band shape loses its third wave (20% slower).
  constexpr bool kOpsAhead = SA_OPS_AHEAD && D == 96 && NT >= 2;

  constexpr int VBUF = 2 * D * 32;
  // one LDS arena: three K tiles, three V^T tiles (and, before the first
  // tile arrives, the Q rotation table)
  __shared__ __attribute__((aligned(16))) uint16_t lds[3 * KBUF + 3 * VBUF];
  auto Kb = [&](int buf) __attribute__((always_inline)) { return lds + buf * KBUF; };
  auto Vb = [&](int buf) __attribute__((always_inline)) { return lds + 3 * KBUF + buf * VBUF; };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar
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
  // Row sums of the probabilities: on the matrix cores at d = 64, where the
  // vector units bound the unit (4% faster); at d = 96 and 128, where the
  // matrix cores have more to do per unit, by v_dot2 on the vector units
  // (the matrix-core sums cost d = 96 8%).
  constexpr bool kMfmaSums = D == 64;
  // Softmax state per query column: the reference is -neg_ref (m_ref on the
  // v_dot2 path, -inf while there is none), l_run the sum of the weights
  // against it, the sink's included (with matrix-core sums every lane of the
  // column holds the whole sum; with v_dot2 sums each lane holds the sum over
  // its own keys).  No reference (no sink and no allowed key seen yet):
  // l_run == 0 (matrix-core sums) or m_ref == -inf, and neg_ref = kNoRef
  // until the slow path sets one.
  float l_run[NT], m_ref[NT];
  float neg_ref[NT];
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
    neg_ref[n] = sg == -INFINITY ? kNoRef : -sg;
    m_ref[n] = sg;
    l_run[n] = (sg != -INFINITY && (kMfmaSums || g4 == 0)) ? 1.0f : 0.0f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) O[dt][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  if constexpr (ROPE) {
    // Rotate this lane's Q operands at their positions with yarn_rope's
    // arithmetic (so they carry exactly the bits yarn_rope would write): the
    // workgroup builds the (c*cos, c*sin) table of its positions in LDS, in
    // chunks of positions if it does not fit, and each lane rotates its
    // 8-coordinate chunks against their partner halves (loaded again; the
    // rows are in cache).
    constexpr int HALF = D / 2;
    constexpr int kTabRows = (int)(sizeof(lds) / (HALF * sizeof(double2)));
    double2* tab = reinterpret_cast<double2*>(lds);
    const int npos = t_end - p0;
    for (int c0 = 0; c0 < npos; c0 += kTabRows) {
      const int nc = min(kTabRows, npos - c0);
      if (c0 > 0) __syncthreads();              // readers of the previous chunk are done
      for (int e = threadIdx.x; e < nc * HALF; e += kThreads) {
        const int r = e / HALF, i = e - r * HALF;
        double sn, cn;
        sa_rope::sincos_reduced((double)(rt.pos_base + a.q_offset + p0 + c0 + r) * rt.inv_freq[i], &sn, &cn);
        tab[e] = make_double2(cn * rt.conc, sn * rt.conc);
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const int row = tpos[n] - p0 - c0;
        if (!rvalid[n] || row < 0 || row >= nc) continue;
        const uint16_t* qrow = q + (((int64_t)b * a.T_q + tpos[n]) * a.n_q + head[n]) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = 32 * ks + 8 * g4;       // the chunk's 8 coordinates lie in one half
          const bool first = c < HALF;
          const u32x4 pv = ld16(qrow + (first ? c + HALF : c - HALF));
          const double2* t = &tab[row * HALF + (first ? c : c - HALF)];
          uint32_t w[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t out[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const double x = (double)(h ? bf16_hi(qop[n][ks][e2]) : bf16_lo(qop[n][ks][e2]));
              const double y = (double)(h ? bf16_hi(pv[e2]) : bf16_lo(pv[e2]));
              const double2 cs = t[2 * e2 + h];
              const double o = first ? sa_rope::rot_first(x, y, cs.x, cs.y)
                                     : sa_rope::rot_second(y, x, cs.x, cs.y);
              out[h] = f64_to_bf16_bits(o);
            }
            w[e2] = out[0] | (out[1] << 16);
          }
          qop[n][ks] = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
    }
    __syncthreads();                            // the table area becomes tile buffers
  }

  const float scale = a.sm_scale * SA_LOG2E;
  // Positions fit in 32 bits (the launcher rejects caches of 2^31 rows or more).
  const int P_min = (int)a.q_offset + p0;
  const int P_max = (int)a.q_offset + t_end - 1;
  const int lo = a.window > 0 ? max(0, P_min - a.window + 1) : 0;
  const int hi = P_max + 1;   // keys >= hi are masked for every row here
  const int t_first = lo / kTile, t_last = (hi - 1) / kTile;

  // ---- tile loads.  Tiles go global -> LDS directly (16 bytes per lane,
  // lane l of a wave writing LDS slot l of a 1 KB block), each lane
  // fetching the chunk that the swizzled layout puts in its slot.  Keys at
  // or past hi (after the block's last query) are masked; the rows below
  // wr (the chunk's end: the caller appended the chunk before attending)
  // hold written values, so a tile that ends at or below wr loads whole.
  // Only a tile that crosses wr (the chunk's last query block) is
  // different: its K rows at or past hi are fetched from row hi-1 and its
  // V goes through registers with the keys at or past hi zeroed, so that
  // unwritten cache rows are never read (a probability is exactly 0 there,
  // but 0 * NaN would not be).
  const int wr = (int)a.q_offset + a.T_q;
  const int krow_stride = a.n_kv * D;                  // elements per cache row
  const int vblk_stride = a.n_kv * D * 32;             // elements per 32-key block
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(a.kc) + ((int64_t)b * C * a.n_kv + g) * D;
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(a.vc) +
                          ((int64_t)b * (C / 32) * a.n_kv + g) * (int64_t)(D * 32);
  constexpr int NSK = k_pitch<D>() / 8;           // 16-byte slots per K row
  constexpr int KBLK = NSK;                       // 1 KB blocks per K tile (64 rows)
  constexpr int VBLK = D / 8;                     // 1 KB blocks per V tile (2D rows of 4 slots)
  constexpr int KBW = (KBLK + NW - 1) / NW;       // blocks per wave
  constexpr int VBW = (VBLK + NW - 1) / NW;
  // K slot of block wave + i*NW: row k_r, chunk k_c, byte offset k_goff
  // within the tile (byte offsets from a uniform base: the loads take a
  // scalar base and a 32-bit vector offset, no 64-bit address arithmetic).
  int k_r[KBW], k_c[KBW];
  uint32_t k_goff[KBW], v_goff[VBW];
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    const int s = 64 * (wave + i * NW) + lane;
    const int r = (s / NSK) & 63;
    k_r[i] = r;
    k_c[i] = (s % NSK) ^ k_swz<D>(r);
    k_goff[i] = (uint32_t)(2 * (r * krow_stride + 8 * k_c[i]));
  }
#pragma unroll
  for (int i = 0; i < VBW; ++i) {
    const int s = 64 * (wave + i * NW) + lane;
    const int r = (s >> 2) % (2 * D);
    const int c = (s & 3) ^ ((r >> 1) & 3);
    v_goff[i] = (uint32_t)(2 * ((r >= D ? vblk_stride : 0) + (r % D) * 32 + 8 * c));
  }
  auto load_k = [&](int buf, int t) __attribute__((always_inline)) {
    const int k0 = t * kTile;
    const uint16_t* kt = kbase + (int64_t)k0 * krow_stride;     // uniform
    const bool full = k0 + kTile <= wr;
    const int last_row = hi - 1 - k0;
#pragma unroll
    for (int i = 0; i < KBW; ++i) {
      const int blk = wave + i * NW;
      if (KBLK % NW == 0 || blk < KBLK) {
        const uint32_t off = full ? k_goff[i]
                                  : (uint32_t)(2 * (min(k_r[i], last_row) * krow_stride + 8 * k_c[i]));
        lds_direct16(reinterpret_cast<const char*>(kt) + off, &Kb(buf)[512 * blk]);
      }
    }
  };
  auto load_v_full = [&](int buf, int t) __attribute__((always_inline)) {
    const uint16_t* vt = vbase + (int64_t)(t * (kTile / 32)) * vblk_stride;   // uniform
#pragma unroll
    for (int i = 0; i < VBW; ++i) {
      const int blk = wave + i * NW;
      if (VBLK % NW == 0 || blk < VBLK)
        lds_direct16(reinterpret_cast<const char*>(vt) + v_goff[i], &Vb(buf)[512 * blk]);
    }
  };
  // Register path: thread c of the workgroup moves chunks c, c + kThreads,
  // ... of the V^T tile (row = 32-key half * D + coordinate, chunk of 8
  // keys); zero = true writes zeros.
  auto store_v_regs = [&](int buf, int t, bool zero) __attribute__((always_inline)) {
    const int k0 = t * kTile;
    const uint16_t* vt = vbase + (int64_t)(k0 / 32) * vblk_stride;
    for (int cidx = threadIdx.x; cidx < 8 * D; cidx += kThreads) {
      const int r = cidx >> 2, ch = cidx & 3;
      const int half = r >= D ? 1 : 0, dd = r - half * D;
      const int key0 = k0 + 32 * half + 8 * ch;
      u32x4 v = {0, 0, 0, 0};
      if (!zero && key0 < hi) {
        v = ld16(vt + half * vblk_stride + dd * 32 + 8 * ch);
        if (key0 + 8 > hi) {
          const int valid = hi - key0;
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uint32_t keep = (2 * w + 1 < valid) ? 0xFFFFFFFFu : (2 * w < valid ? 0x0000FFFFu : 0u);
            v[w] &= keep;
          }
        }
      }
      st16(&Vb(buf)[v_lds(r, ch)], v);
    }
  };
  auto load_v = [&](int buf, int t) __attribute__((always_inline)) {
    if (t * kTile + kTile <= wr)
      load_v_full(buf, t);
    else
      store_v_regs(buf, t, false);
  };

  // LDS read offsets of this lane's operands.  The K rows of M tile mt are
  // krow0 + 4*(mt&1) + 32*(mt>>1) with krow0 = 8*(j>>2) + (j&3); the
  // swizzle f depends only on row bits 0, 1, 3 and 4, i.e. on j alone, so
  // chunk g4 + 4*ks of every M tile sits at ka[ks] plus a fixed offset
  // (the swizzle's low two bits act on g4, its high bits on ks).  V^T reads
  // add uniform offsets to va_off.
  int ka[KS];
  {
    const int krow0 = 8 * (j >> 2) + (j & 3);
    const int f = k_swz<D>(krow0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      ka[ks] = krow0 * k_pitch<D>() + 8 * (g4 ^ (f & 3)) + 32 * (ks ^ (f >> 2));
  }
  const int va_off = v_lds(j, g4);

  // ---- the parts of a unit of 32 keys (half a tile; key half h of tile t
  // holds keys 64t + 32h + [0, 32)): scores S^T = K Q^T (masked on units
  // that cross the diagonal or the band edge), probabilities against the
  // current reference, and O^T += V^T P^T.
  struct Scores { f32x4 v[2][NT]; };
  auto scores = [&](Scores& S, int buf, int h) __attribute__((always_inline)) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int n = 0; n < NT; ++n) S.v[mm][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int mt = 2 * h + mm;
        const u32x4 A = ld16(&Kb(buf)[ka[ks] + k_pitch<D>() * (4 * (mt & 1) + 32 * (mt >> 1))]);
#pragma unroll
        for (int n = 0; n < NT; ++n) S.v[mm][n] = mfma16x16x32(A, qop[n][ks], S.v[mm][n]);
      }
    }
  };
  // Lane (j, g4) holds, for M tile mm and element r, the score of key
  // k0h + 8*g4 + 4*mm + r; keys after the query or outside its band get -inf.
  // A key is allowed when d = p - key >= 0 and, in a band, d < W; with
  // d >= 0 the second test is an unsigned compare, and without a band its
  // limit passes every d.  Both tests are evaluated (no short circuit), so
  // the compiler keeps them as two compares and a select per score rather
  // than branching around the second.
  const uint32_t wlim = a.window > 0 ? (uint32_t)a.window : 0xFFFFFFF0u;
  auto apply_mask = [&](Scores& S, int k0h) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      if constexpr (LONG) {
        // (the full-causal instance, whose masked units are the diagonal's
        // few, keeps this form: the other costs it spilled registers)
        const int rel0 = k0h + 8 * g4 - ((int)a.q_offset + tpos[n]);   // key - p at (mm, r) = 0
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rel = rel0 + 4 * mm + r;
            const bool ok = rel <= 0 && (a.window <= 0 || rel > -a.window);
            S.v[mm][n][r] = ok ? S.v[mm][n][r] : -INFINITY;
          }
      } else {
        const int d0 = (int)a.q_offset + tpos[n] - (k0h + 8 * g4);   // p - key at (mm, r) = 0
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int c = 4 * mm + r;
            const bool ok = (d0 >= c) & ((uint32_t)d0 < wlim + (uint32_t)c);
            S.v[mm][n][r] = ok ? S.v[mm][n][r] : -INFINITY;
          }
      }
    }
  };
  // p = 2^(s*scale + neg_ref), rounded to bf16 once; on the v_dot2 path ls
  // receives this lane's sum of those rounded values.
  auto probs = [&](const Scores& S, u32x4 (&Pk)[NT], float (&ls)[NT]) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float acc = 0.f;
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const float p0 = fast_exp2(fmaf(S.v[e2 >> 1][n][2 * (e2 & 1)], scale, neg_ref[n]));
        const float p1 = fast_exp2(fmaf(S.v[e2 >> 1][n][2 * (e2 & 1) + 1], scale, neg_ref[n]));
        w[e2] = pack_bf16x2(p0, p1);
        if constexpr (!kMfmaSums) acc = sum_bf16x2(w[e2], acc);
      }
      Pk[n] = u32x4{w[0], w[1], w[2], w[3]};
      if constexpr (!kMfmaSums) ls[n] = acc;
    }
  };
  // A unit's row sums on the matrix cores (d = 64): with A all ones, every
  // row of ONES P^T is the column sum, so each lane receives its query's sum
  // over the unit's 32 keys, of the same rounded values the PV product uses.
  auto unit_sums = [&](const u32x4 (&Pk)[NT], float (&ls)[NT]) {
    if constexpr (kMfmaSums) {
      const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
#pragma unroll
      for (int n = 0; n < NT; ++n) ls[n] = mfma16x16x32(ones, Pk[n], f32x4{0.f, 0.f, 0.f, 0.f})[0];
    }
  };
  auto pv = [&](int buf, int h, const u32x4 (&Pk)[NT]) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const u32x4 A = ld16(&Vb(buf)[va_off + (h * D + 16 * dt) * 32]);
#pragma unroll
      for (int n = 0; n < NT; ++n) O[dt][n] = mfma16x16x32(A, Pk[n], O[dt][n]);
    }
  };
  // A unit's LDS operands held in registers: the K rows of its scores (KS
  // steps x 2 M tiles, from K buffer kb, half kh) and the V^T rows of its PV
  // (DT tiles, from V buffer vb, half vh).  Read one unit ahead, their LDS
  // latency hides behind the previous unit's vector work.
  struct Ops { u32x4 k[KS][2]; u32x4 v[DT]; };
  auto load_ops = [&](Ops& o, int kb, int kh, int vb, int vh) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int mt = 2 * kh + mm;
        o.k[ks][mm] = ld16(&Kb(kb)[ka[ks] + k_pitch<D>() * (4 * (mt & 1) + 32 * (mt >> 1))]);
      }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o.v[dt] = ld16(&Vb(vb)[va_off + (vh * D + 16 * dt) * 32]);
  };
  auto scores_ops = [&](Scores& S, const Ops& o) __attribute__((always_inline)) {
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int n = 0; n < NT; ++n) S.v[mm][n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int n = 0; n < NT; ++n) S.v[mm][n] = mfma16x16x32(o.k[ks][mm], qop[n][ks], S.v[mm][n]);
  };
  auto pv_ops = [&](const Ops& o, const u32x4 (&Pk)[NT]) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int n = 0; n < NT; ++n) O[dt][n] = mfma16x16x32(o.v[dt], Pk[n], O[dt][n]);
  };
  // Move the reference to the true running max over the scores of Sa and
  // Sb (column max across the four lanes of a query) and rescale what has
  // been accumulated.
  auto rescale = [&](const Scores& Sa, const Scores& Sb) __attribute__((always_inline)) {
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      float mx = -INFINITY;
#pragma unroll
      for (int mm = 0; mm < 2; ++mm)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fmaxf(Sa.v[mm][n][r], Sb.v[mm][n][r]));
      const bool none = kMfmaSums ? l_run[n] == 0.f : m_ref[n] == -INFINITY;   // O is 0 too
      const float m_cur = none ? -INFINITY : -neg_ref[n];
      const float m_new = fmaxf(m_cur, max_over_col(mx) * scale);
      const float alpha = none ? 0.f : fast_exp2(m_cur - m_new);
      l_run[n] *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) O[dt][n] *= alpha;
      m_ref[n] = m_new;
      neg_ref[n] = m_new == -INFINITY ? kNoRef : -m_new;
    }
  };
  // Does the unit starting at key k0h need masking?
  auto need_mask = [&](int k0h) __attribute__((always_inline)) {
    return (k0h + 31 > P_min) || (a.window > 0 && k0h < P_max - a.window + 1);
  };

  // ---- software pipeline over units.  Unit u computes S(u+1) and
  // O += V(u-1) P(u-1) on the matrix cores while the vector units turn S(u)
  // into P(u), all in one stretch of straight-line code; the row sums of
  // P(u) then go to the matrix cores too.  Tile t (units 2t and 2t+1) first
  // starts the loads of K(t+2) and V(t+1) into LDS and ends with one
  // barrier.  K and V have three LDS buffers each; with (b0, b1, b2)
  // rotating one place per tile, K(t), K(t+1), K(t+2) sit in b0, b1, b2 and
  // V(t-1), V(t), V(t+1) in b2, b0, b1.  After each unit, P(u) is checked:
  // the reference stays put while every lane's unit sum stays below 2^64
  // (so no exponential, partial sum or accumulator comes near fp32/bf16
  // overflow); a unit that breaks that, or a query with no reference yet
  // (no sink and nothing seen), recomputes S(u) from K (still in LDS), moves
  // the reference to the running max, rescales O (which then holds units up
  // to u-1) and recomputes P(u) and its sums.
  // The walk starts and stops on 32-key units (where the loop is peeled,
  // below): when the first allowed key
  // lies in the second half of the first tile, unit 2 t_first is skipped
  // (the pipeline starts at unit 2 t_first + 1 with a zero P before it);
  // when the last query lies in the first half of the last tile, unit
  // 2 t_last + 1 is skipped (only P(2 t_last) still enters O).
  // The loop is peeled (head and tail tiles outside it) only for the shapes
  // whose registers allow the extra copies of the unit: at d = 96 with two
  // N tiles per wave (and at d = 128) it would cost a wave per SIMD, so those
  // walk whole tiles.
  constexpr bool kPeel = D == 64 || (D == 96 && NT == 1);
  const int t0 = t_first;
  const bool skip_head = kPeel && (lo & (kTile - 1)) >= 32;
  const bool skip_tail = kPeel && ((hi - 1) & (kTile - 1)) < 32;
  int b0 = 0, b1 = 1, b2 = 2;
  load_k(0, t0);
  if (t0 + 1 <= t_last) load_k(1, t0 + 1);
  load_v(0, t0);
  store_v_regs(2, t0, true);     // "V(t0-1)", multiplied by P = 0 in unit 2*t0
  wait_vmem();
  __syncthreads();
  Scores S0, S1;
  u32x4 P0[NT], P1[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    P0[n] = u32x4{0, 0, 0, 0};
    P1[n] = u32x4{0, 0, 0, 0};
  }
  if (skip_head) {
    scores(S1, 0, 1);
    if (need_mask(t0 * kTile + 32)) apply_mask(S1, t0 * kTile + 32);
  } else {
    scores(S0, 0, 0);
    if (need_mask(t0 * kTile)) apply_mask(S0, t0 * kTile);
  }

  // One unit: Sc = S(u) in, Sn = S(u+1) out (from K buffer kbn, half hn,
  // first key k0n); Pp = P(u-1) in (V buffer vbp, half hp), Pc = P(u) out;
  // S(u) can be recomputed from K buffer kbc, half hc, first key k0c.  The
  // mask of S(u+1), where it needs one, is applied in place after the main
  // stretch.
  // oc: this unit's operands (read ahead); on: filled here with the next
  // unit's, from K buffer kbx half hx and V buffer vbx half vx.
  auto unit = [&](const Scores& Sc, Scores& Sn, const u32x4 (&Pp)[NT], u32x4 (&Pc)[NT],
                  const Ops& oc, Ops& on, int kbx, int hx, int vbx, int vx,
                  int kbn, int hn, int k0n, int vbp, int hp, int kbc, int hc, int k0c,
                  bool mask_next) __attribute__((always_inline)) {
    float ls[NT];
    if constexpr (kOpsAhead) {
      scores_ops(Sn, oc);
      pv_ops(oc, Pp);
    } else {
      scores(Sn, kbn, hn);
      pv(vbp, hp, Pp);
    }
    // d = 96 and 128 run two waves per SIMD: keeping each unit's MFMAs ahead
    // of its vector work (measured 5% faster at d = 96; d = 64, with three
    // waves per SIMD, is faster mixed).
    if constexpr (kPhaseSplit) __builtin_amdgcn_sched_barrier(0);
    if constexpr (kOpsAhead) load_ops(on, kbx, hx, vbx, vx);
    probs(Sc, Pc, ls);
    unit_sums(Pc, ls);
    // a query without a reference gets p = inf here (kNoRef), so this one
    // test also catches it
    bool bad = false;
#pragma unroll
    for (int n = 0; n < NT; ++n) bad |= !(ls[n] <= kHeadroom);
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      // The compiler may not hoist this recomputation onto the fast path
      // (LDS reads can be speculated): the clobber pins it here.
      asm volatile("" ::: "memory");
      Scores Sr;
      scores(Sr, kbc, hc);
      if (need_mask(k0c)) apply_mask(Sr, k0c);
      rescale(Sr, Sr);
      probs(Sr, Pc, ls);
      unit_sums(Pc, ls);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) l_run[n] += ls[n];
    if (mask_next) apply_mask(Sn, k0n);
  };
  // operands of unit 2 t0: K(t0) half 1, V(t0-1) half 1 (zeros); or, when
  // that unit is skipped, those of unit 2 t0 + 1: K(t0+1) half 0, V(t0) half 0
  Ops OA, OB;
  if constexpr (kOpsAhead) {
    if (skip_head)
      load_ops(OB, 1, 0, 0, 0);
    else
      load_ops(OA, 0, 1, 2, 1);
  }
  // unit 2t: S(2t+1) from K(t) half 1; P(2t-1) with V(t-1) half 1.  It reads
  // ahead the operands of unit 2t+1: K(t+1) half 0, V(t) half 0.
  // (c0, c1, c2: the buffers b0, b1, b2 of tile t)
  auto first_unit_at = [&](int t, int c0, int c1, int c2) __attribute__((always_inline)) {
    const int k0 = t * kTile;
    unit(S0, S1, P1, P0, OA, OB, c1, 0, c0, 0, c0, 1, k0 + 32, c2, 1, c0, 0, k0,
         need_mask(k0 + 32));
  };
  auto first_unit = [&](int t) __attribute__((always_inline)) { first_unit_at(t, b0, b1, b2); };
  // unit 2t+1: S(2t+2) from K(t+1) half 0 (a throw-away after the last tile);
  // P(2t) with V(t) half 0.  It reads ahead the operands of unit 2t+2:
  // K(t+1) half 1 and V(t) half 1, which the loads of tile t+1 (into the
  // buffers of K(t) and V(t-1)) leave in place; after the last tile they are
  // stale and unused.
  auto second_unit_at = [&](int t, int c0, int c1) __attribute__((always_inline)) {
    const int k0 = t * kTile;
    unit(S1, S0, P0, P1, OB, OA, c1, 1, c0, 1, c1, 0, k0 + kTile, c0, 0, c0, 1, k0 + 32,
         t < t_last && need_mask(k0 + kTile));
  };
  auto second_unit = [&](int t) __attribute__((always_inline)) { second_unit_at(t, b0, b1); };
  auto tile_loads_at = [&](int t, int c1, int c2) __attribute__((always_inline)) {
    if (t + 2 <= t_last) load_k(c2, t + 2);
    if (t + 1 <= t_last) load_v(c1, t + 1);
  };
  auto tile_loads = [&](int t) __attribute__((always_inline)) { tile_loads_at(t, b1, b2); };
  // A whole tile with its buffers as constants: three in a row bring the
  // rotation back to where it started, and with constant buffers the LDS
  // addresses of the unit's reads fold into the instructions' offsets (no
  // vector address arithmetic per unit).
  auto whole_tile_at = [&](int t, int c0, int c1, int c2) __attribute__((always_inline)) {
    tile_loads_at(t, c1, c2);
    first_unit_at(t, c0, c1, c2);
    second_unit_at(t, c0, c1);
    wait_vmem();
    __syncthreads();
  };
  auto tile_end = [&]() __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    const int k = b0;
    b0 = b1;
    b1 = b2;
    b2 = k;
  };
  if constexpr (kPeel) {
    int t = t0;
    if (skip_head) {             // tile t0: its second unit only
      tile_loads(t);
      second_unit(t);
      tile_end();
      ++t;
    }
    if (LONG && !skip_head) {    // buffers (0, 1, 2) at tile t: whole tiles in threes
      for (; t + 3 <= t_last; t += 3) {
        whole_tile_at(t, 0, 1, 2);
        whole_tile_at(t + 1, 1, 2, 0);
        whole_tile_at(t + 2, 2, 0, 1);
      }
    }
    for (; t < t_last; ++t) {    // whole tiles
      tile_loads(t);
      first_unit(t);
      second_unit(t);
      tile_end();
    }
    if (t == t_last) {           // the last tile (not reached when it was the skipped head's)
      first_unit(t);
      if (skip_tail) {
        pv(b0, 0, P0);           // P(2 t_last) with V(t_last) half 0
      } else {
        second_unit(t);
        pv(b0, 1, P1);           // P(2 t_last + 1) with V(t_last) half 1
      }
    } else {
      pv(b2, 1, P1);             // P(2 t0 + 1) with V(t0) half 1 (rotated to b2)
    }
  } else {
    for (int t = t0; t <= t_last; ++t) {
      tile_loads(t);
      first_unit(t);
      second_unit(t);
      tile_end();
    }
    pv(b2, 1, P1);               // P(2 t_last + 1) with V(t_last) half 1
  }

  // ---- normalise and store: lane holds O^T[16*dt + 4*g4 + r][query]
  uint16_t* out = reinterpret_cast<uint16_t*>(a.out);
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float inv = 1.0f / (kMfmaSums ? l_run[n] : sum_over_col(l_run[n]));
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

template <int D, int NT, int NW, bool LONG>
hipError_t launch_d(const AttnArgs& a, const RopeTab* rope, hipStream_t s) {
  const int rows = NW * NT * 16;
  if (a.q_mult > rows) return hipErrorInvalidValue;
  const int BQ = rows / a.q_mult;
  const int n_qb = (a.T_q + BQ - 1) / BQ;
  const int64_t grid = (int64_t)n_qb * a.B * a.n_kv;
  RopeTab rt;
  if (rope) {
    rt = *rope;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, NT, NW, true, LONG>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, s, a, BQ, n_qb, rt);
  } else {
    rt.conc = 0.0;
    rt.pos_base = 0;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, NT, NW, false, LONG>), dim3((unsigned)grid),
                       dim3(NW * 64), 0, s, a, BQ, n_qb, rt);
  }
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
#define SA_PF96 2, 4
#endif
#ifndef SA_PF128
#define SA_PF128 2, 8
#endif
#ifndef SA_PFB64
#define SA_PFB64 2, 4
#endif
#ifndef SA_PFB96
#define SA_PFB96 1, 8
#endif
#ifndef SA_PFB128
#define SA_PFB128 2, 8
#endif
constexpr int kBandWindowMax = 512;   // windows up to this use the band shape

hipError_t launch_prefill_bf16(const AttnArgs& a, const RopeTab* rope, hipStream_t s) {
  const bool band = a.window > 0 && a.window <= kBandWindowMax;
  switch (a.d) {
    case 64:
      return band ? launch_d<64, SA_PFB64, false>(a, rope, s) : launch_d<64, SA_PF64, true>(a, rope, s);
    case 96:
      return band ? launch_d<96, SA_PFB96, false>(a, rope, s) : launch_d<96, SA_PF96, true>(a, rope, s);
    case 128:
      return band ? launch_d<128, SA_PFB128, false>(a, rope, s)
                  : launch_d<128, SA_PF128, true>(a, rope, s);
    default: return hipErrorInvalidValue;
  }
}
