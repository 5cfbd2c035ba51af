// Sampling controls on gfx950: processed logits, top-k / top-p / min-p and
// the draw.
//
// "MoE-Xtend" README, SAMPLING CONTROLS: p = softmax(z / T); top-k, top-p
// and min-p truncations after logit bias and the repetition, presence and
// frequency penalties; T = 0 is greedy.  The project summary page: sampling
// is deterministic.
//
// Every truncation is a threshold on an order-preserving 32-bit key of the
// processed logit z': top-k the largest key whose count at or above it
// reaches k, top-p the largest key whose mass at or above it reaches
// ceil(top_p * top-k mass), min-p the smallest key whose weight reaches
// min_p (weights are monotone in the key, so a search finds it).  Masses
// are integers, q = floor(e * 2^40) with e = 2^((z' - m) log2(e) / T) <= 1,
// so every sum is exact and the result does not depend on scheduling.
//
// Four launches per call:
//  1. prep (grid chunks of 4096 x rows, the whole chip): z' stored once,
//     per-chunk maximum and its lowest id; clears the row's histogram and
//     candidate counter.  The only pass over the inputs in HBM.
//  2. histogram (chunks x rows): a 4096-bucket histogram (counts, masses) of
//     the key's top 12 bits in LDS, added into the row's global one with
//     integer atomics, plus 64 sums of 64 buckets and each chunk's mass;
//     when min-p is on, the tokens at or above the min-p key are gathered
//     into the row's candidate list.
//  3. gather (chunks x rows), rows with top-k or top-p and no min-p: one
//     wave reads the bucket of the k-th token or of the top-p crossing off
//     the histogram; when at most 4096 tokens lie at or above it, every
//     chunk adds its share to the candidate list.  Otherwise, with one rule
//     on and at most 4096 tokens in that bucket (edge mode), every chunk
//     adds the bucket's tokens and writes its mass above the bucket.
//  4. select (one 1024-thread workgroup per row): greedy rows take the
//     merged argmax.  Candidates (a prefix of the ranking that holds the
//     kept set) are sorted by key then id (one wave in registers up to 256,
//     a bitonic sort in LDS beyond), the thresholds read off their prefix
//     masses, and the kept ones re-sorted by id for the draw.  Without any
//     truncation the chunk masses locate the draw.  In edge mode two radix
//     levels over the bucket's tokens (in LDS) place the threshold, and the
//     per-chunk masses above the bucket plus the bucket's kept tokens
//     locate the draw.  Other large kept sets take two more radix levels
//     (12 + 8 bits, one pass each over z') per threshold, then per-chunk
//     kept masses and one scan of the chunk that holds the target.
#pragma clang fp contract(off)

#include "sa_device.h"
#include "sa_sample.h"

namespace {

// The histogram launch has one workgroup per chunk at small batches (one
// per CU at 8 rows), so it runs more threads per chunk to hide its loads
// and its contended LDS atomics (1024 against 256: 2 us less per call at
// 8 x 128,000, 3 us at 64 rows; 512 in between).
#ifndef SA_HIST_THREADS
#define SA_HIST_THREADS 1024
#endif
constexpr int kHistThreads = SA_HIST_THREADS;
constexpr int kHistPer = kSampleChunk / kHistThreads;
// The prep launch likewise: 512 threads per chunk were 1 us faster per call
// than 256 at 8 rows and even at 64; 1024 lost 3 us at 64 rows.
#ifndef SA_PREP_THREADS
#define SA_PREP_THREADS 512
#endif
constexpr int kPrepOnlyThreads = SA_PREP_THREADS;     // the prep launch
constexpr int kPrepOnlyPer = kSampleChunk / kPrepOnlyThreads;
// And the gather launch: 512 threads were 1.3 us (top-k 50) and 1.5 us
// (flat top-p) faster per call than 256; 1024 lost 2.5 us at 64 rows.
#ifndef SA_GATHER_THREADS
#define SA_GATHER_THREADS 512
#endif
constexpr int kGatherThreads = SA_GATHER_THREADS;     // the gather launch
constexpr int kGatherPer = kSampleChunk / kGatherThreads;
constexpr int kNB = kSampleBuckets;
constexpr int kHist = kSampleHist;                  // 4096 buckets, then 64 sums of 64 buckets
constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelPer = 4;                          // 16-byte loads in flight per thread in a select pass
constexpr int kCap = kSampleCap;
constexpr float kFltMax = 3.4028235e38f;
typedef unsigned long long u64;

// Order-preserving key: a larger float gets a larger key; -0 and +0 share one.
__device__ __forceinline__ uint32_t fkey(float z) {
  const uint32_t u = __float_as_uint(z + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fval(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ float temp_coef(float T) { return SA_LOG2E / T; }
// exp((z - m) / T) as 2^((z - m) c), c = log2(e) / T; exactly 1 at the maximum
__device__ __forceinline__ float rel_weight(float z, float m, float c) {
  const float d = z - m;
  return fast_exp2(d == 0.f ? 0.f : d * c);
}
__device__ __forceinline__ u64 fixed_mass(float e) { return (u64)(e * 1099511627776.0f); }  // 2^40
__device__ __forceinline__ u64 mass_of_key(uint32_t k, float m, float c) {
  return fixed_mass(rel_weight(fval(k), m, c));
}

// The smallest key whose weight reaches min_p (0 < min_p <= 1): the
// maximum's weight is 1 and -inf's is 0; weights rise with the key, so a
// search between them: each round the 64 lanes of a wave test 64 evenly
// spaced keys of (lo, hi] and keep the sub-interval where the test first
// passes (about six rounds for 32-bit keys).  Every wave that calls it gets
// the same key.  Call from one whole wave.
__device__ __forceinline__ uint32_t minp_key(float m, float c, float min_p) {
  const uint32_t lane = threadIdx.x & 63;
  uint32_t lo = fkey(-INFINITY), hi = fkey(m);     // weight(lo) < min_p <= weight(hi)
  while (hi - lo > 1) {
    const uint32_t step = (hi - lo + 63) / 64;
    const uint32_t k = min(hi, lo + step * (lane + 1));
    const u64 pass = __ballot(rel_weight(fval(k), m, c) >= min_p);
    const int f = pass ? (int)(__ffsll((long long)pass) - 1) : 63;
    const uint32_t nhi = min(hi, lo + step * (uint32_t)(f + 1));
    lo = f == 0 ? lo : lo + step * (uint32_t)f;
    hi = nhi;
  }
  return hi;
}

__device__ __forceinline__ bool params_ok(const sa_sample_params& p, float u) {
  const bool base = p.temperature >= 0.f && p.temperature <= kFltMax && p.top_k >= 0 && p.top_p > 0.f &&
                    p.top_p <= 1.f && p.min_p >= 0.f && p.min_p <= 1.f && p.repetition > 0.f &&
                    p.repetition <= kFltMax && fabsf(p.presence) <= kFltMax && fabsf(p.frequency) <= kFltMax;
  return base && (p.temperature == 0.f || (u >= 0.f && u < 1.f));
}

// (v, a) beats (bv, ba): larger value, or equal value and lower id; -1 is no entry
__device__ __forceinline__ bool better(float v, int a, float bv, int ba) {
  return a >= 0 && (ba < 0 || v > bv || (v == bv && a < ba));
}

__device__ __forceinline__ u64 wave_sum_u64(u64 x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
  return x;
}

__device__ __forceinline__ u64 wave_incl_scan(u64 x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const u64 y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Appends to the row's candidate list the entries (key << 32 | ~id) of this
// thread's PER ids whose take bit is set.  Same-address atomics serialize
// in L2, so the workgroup reserves all of its slots with one atomic: each
// wave counts its ids by ballot, thread 0 adds the waves' counts to the
// row's counter, and each wave writes from its offset.  Call from the whole
// workgroup (THREADS threads, PER ids each); s holds THREADS / 64 + 1 words.
template <int PER, int THREADS>
__device__ __forceinline__ void append_candidates(const SampleArgs& a, int b, const uint32_t (&key)[PER],
                                                  const int (&id)[PER], const bool (&take)[PER], uint32_t* s) {
  constexpr int kWaves = THREADS / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const u64 below = (1ull << lane) - 1ull;
  u64 mask[PER];
  uint32_t n = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    mask[j] = __ballot(take[j]);
    n += (uint32_t)__popcll(mask[j]);
  }
  if (lane == 0) s[w] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tot = 0;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) tot += s[i];
    s[kWaves] = tot ? atomicAdd(&a.ncand[b], tot) : 0u;
  }
  __syncthreads();
  if (n == 0) return;                                 // wave-uniform
  uint32_t base = s[kWaves];
  for (int i = 0; i < w; ++i) base += s[i];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const uint32_t slot = base + (uint32_t)__popcll(mask[j] & below);
    if (take[j] && slot < (uint32_t)kCap) a.cand[(int64_t)b * kCap + slot] = ((u64)key[j] << 32) | (uint32_t)~(uint32_t)id[j];
    base += (uint32_t)__popcll(mask[j]);
  }
}

// Row maximum and its lowest id from the per-chunk results: wave 0 loads
// them (C <= 64) and reduces; every thread gets the result through LDS.
__device__ __forceinline__ void row_max(const SampleArgs& a, int b, float* m, int* arg, float* sv, int* si) {
  if (threadIdx.x < 64) {
    const int c = threadIdx.x;
    float bv = c < a.C ? a.chunk_max[(int64_t)b * a.C + c] : 0.f;
    int ba = c < a.C ? a.chunk_arg[(int64_t)b * a.C + c] : -1;
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      const float ov = __shfl_xor(bv, s, 64);
      const int oa = __shfl_xor(ba, s, 64);
      if (better(ov, oa, bv, ba)) {
        bv = ov;
        ba = oa;
      }
    }
    if (c == 0) {
      *sv = bv;
      *si = ba;
    }
  }
  __syncthreads();
  *arg = *si;
  *m = *arg >= 0 ? *sv : -INFINITY;
}

// ------------------------------------------------------------------ prep
__global__ __launch_bounds__(kPrepOnlyThreads) void sample_prep_kernel(SampleArgs a) {
  const int b = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const sa_sample_params P = a.params[b];
  const bool pen = a.counts && (P.repetition != 1.f || P.presence != 0.f || P.frequency != 0.f);
  const float* L = a.logits + (int64_t)b * a.logits_stride;
  const float* Bi = a.bias ? a.bias + (int64_t)b * a.bias_stride : nullptr;
  const int32_t* Cn = pen ? a.counts + (int64_t)b * a.V : nullptr;
  const int v0 = c * kSampleChunk + tid;
  float z[kPrepOnlyPer];
#pragma unroll
  for (int j = 0; j < kPrepOnlyPer; ++j) {
    const int v = v0 + j * kPrepOnlyThreads;
    z[j] = v < a.V ? L[v] : 0.f;
  }
  if (Bi) {
#pragma unroll
    for (int j = 0; j < kPrepOnlyPer; ++j) {
      const int v = v0 + j * kPrepOnlyThreads;
      if (v < a.V) z[j] = z[j] + Bi[v];
    }
  }
  if (pen) {
    int n[kPrepOnlyPer];
#pragma unroll
    for (int j = 0; j < kPrepOnlyPer; ++j) {
      const int v = v0 + j * kPrepOnlyThreads;
      n[j] = v < a.V ? Cn[v] : 0;
    }
#pragma unroll
    for (int j = 0; j < kPrepOnlyPer; ++j) {
      if (n[j] > 0) {
        float t = z[j] > 0.f ? z[j] / P.repetition : z[j] * P.repetition;
        t = t - P.presence;
        z[j] = t - P.frequency * (float)n[j];
      }
    }
  }
  float* Z = a.zp + (int64_t)b * a.zs;
  float* O = a.processed ? a.processed + (int64_t)b * a.V : nullptr;
  float best = 0.f;
  int arg = -1;
#pragma unroll
  for (int j = 0; j < kPrepOnlyPer; ++j) {
    const int v = v0 + j * kPrepOnlyThreads;
    if (v < a.V) {
      Z[v] = z[j];
      if (O) O[v] = z[j];
      if (z[j] > -INFINITY && (arg < 0 || z[j] > best)) {   // NaN never wins
        best = z[j];
        arg = v;
      }
    }
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(best, m, 64);
    const int oa = __shfl_xor(arg, m, 64);
    if (better(ov, oa, best, arg)) {
      best = ov;
      arg = oa;
    }
  }
  __shared__ float wv[kPrepOnlyThreads / 64];
  __shared__ int wa[kPrepOnlyThreads / 64];
  if ((tid & 63) == 0) {
    wv[tid >> 6] = best;
    wa[tid >> 6] = arg;
  }
  // clear this chunk's share of the row's histogram (filled by the next launch)
  const int share = (kHist + a.C - 1) / a.C;
  for (int i = c * share + tid; i < min(kHist, (c + 1) * share); i += kPrepOnlyThreads) {
    a.hist_count[(int64_t)b * kHist + i] = 0u;
    a.hist_mass[(int64_t)b * kHist + i] = 0ull;
  }
  if (c == 0 && tid == 0) a.ncand[b] = 0u;
  __syncthreads();
  if (tid == 0) {
    float bv = wv[0];
    int ba = wa[0];
    for (int w = 1; w < kPrepOnlyThreads / 64; ++w)
      if (better(wv[w], wa[w], bv, ba)) {
        bv = wv[w];
        ba = wa[w];
      }
    a.chunk_max[(int64_t)b * a.C + c] = ba >= 0 ? bv : -INFINITY;
    a.chunk_arg[(int64_t)b * a.C + c] = ba;
  }
}

// ------------------------------------------------------------- histogram
__global__ __launch_bounds__(kHistThreads) void sample_hist_kernel(SampleArgs a) {
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63;
  const sa_sample_params P = a.params[b];
  if (!params_ok(P, a.u[b]) || P.temperature == 0.f) return;
  __shared__ float rmv;
  __shared__ int rmi;
  float m;
  int arg;
  row_max(a, b, &m, &arg, &rmv, &rmi);
  if (!(fabsf(m) <= kFltMax)) return;               // no finite maximum: the row has no token
  const float cT = temp_coef(P.temperature);
  const bool gather = P.min_p > 0.f;
  const uint32_t km = gather ? minp_key(m, cT, P.min_p) : 0u;
  __shared__ uint32_t hc[kNB];
  __shared__ u64 hm[kNB];
  __shared__ u64 wq[2][kHistThreads / 64];
  __shared__ uint32_t s_app[kHistThreads / 64 + 1];
  for (int i = tid; i < kNB; i += kHistThreads) {
    hc[i] = 0u;
    hm[i] = 0ull;
  }
  __syncthreads();
  const float* Z = a.zp + (int64_t)b * a.zs;
  // this workgroup's chunks: hist_cpw consecutive chunks of the row (one
  // histogram in LDS and one flush for all of them)
  const int c_end = min(a.C, ((int)blockIdx.x + 1) * a.hist_cpw);
  for (int c = (int)blockIdx.x * a.hist_cpw; c < c_end; ++c) {
    const int v0 = c * kSampleChunk + tid;
    float z[kHistPer];
#pragma unroll
    for (int j = 0; j < kHistPer; ++j) {
      const int v = v0 + j * kHistThreads;
      z[j] = v < a.V ? Z[v] : 0.f;
    }
    u64 qsum = 0;
    uint32_t key[kHistPer];
    int id[kHistPer];
    bool take[kHistPer];
#pragma unroll
    for (int j = 0; j < kHistPer; ++j) {
      const int v = v0 + j * kHistThreads;
      const uint32_t k = fkey(z[j]);
      key[j] = k;
      id[j] = v;
      take[j] = gather && v < a.V && k >= km;
      if (v < a.V) {
        atomicAdd(&hc[k >> 20], 1u);
        const u64 q = fixed_mass(rel_weight(z[j], m, cT));
        qsum += q;
        if (q) atomicAdd(&hm[k >> 20], q);
      }
    }
    if (gather) append_candidates<kHistPer, kHistThreads>(a, b, key, id, take, s_app);
    // the chunk's mass (two buffers: a wave may start the next chunk while
    // thread 0 still reads this one's)
    qsum = wave_sum_u64(qsum);
    if (lane == 0) wq[c & 1][tid >> 6] = qsum;
    __syncthreads();
    if (tid == 0) {
      u64 t = 0;
#pragma unroll
      for (int w = 0; w < kHistThreads / 64; ++w) t += wq[c & 1][w];
      a.chunk_mass[(int64_t)b * a.C + c] = t;
    }
  }
  for (int i = tid; i < kNB; i += kHistThreads) {
    if (hc[i]) atomicAdd(&a.hist_count[(int64_t)b * kHist + i], hc[i]);
    if (hm[i]) atomicAdd(&a.hist_mass[(int64_t)b * kHist + i], hm[i]);
  }
  if (tid < 64) {                                   // the sums of 64 buckets
    uint32_t sc = 0;
    u64 sm = 0;
#pragma unroll 4
    for (int i = 0; i < 64; ++i) {
      const int k = 64 * tid + ((i + tid) & 63);      // staggered: no bank conflicts
      sc += hc[k];
      sm += hm[k];
    }
    if (sc) atomicAdd(&a.hist_count[(int64_t)b * kHist + kNB + tid], sc);
    if (sm) atomicAdd(&a.hist_mass[(int64_t)b * kHist + kNB + tid], sm);
  }
}

// ---------------------------------------------------------- bucket bound
// The first-level histogram (counts c1, masses m1, 4096 buckets by the key's
// top 12 bits) tells in which bucket each threshold falls.  One wave does
// it, lane l holding the 64 buckets 4095 - 64 l - 63 .. 4095 - 64 l, so the
// gather launch (256 threads) and the select launch (1024) get the same
// integers.

struct Pick {
  uint32_t digit;             // bucket at which the running weight reaches the target
  u64 cnt_above, mass_above;  // counts and masses of the buckets above it
  u64 cnt_at;                 // count of the bucket itself
};

__device__ __forceinline__ void wave_scan3(u64& w, u64& c, u64& m) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const u64 yw = __shfl_up(w, d, 64), yc = __shfl_up(c, d, 64), ym = __shfl_up(m, d, 64);
    if (lane >= d) {
      w += yw;
      c += yc;
      m += ym;
    }
  }
}

// Scanning the row's buckets (cnt, mass: 4096 buckets then 64 sums of 64)
// from the top down, the bucket at which the running count (by_mass: mass)
// first reaches target (target <= the total): first over the 64 sums, then
// over the 64 buckets of the one that reaches it.  Call from one whole wave.
__device__ __forceinline__ Pick wave_pick(const uint32_t* cnt, const u64* mass, bool by_mass, u64 target) {
  const int lane = threadIdx.x & 63;
  const u64 cc = cnt[kNB + 63 - lane], cm = mass[kNB + 63 - lane], cw = by_mass ? cm : cc;
  u64 iw = cw, ic = cc, im = cm;
  wave_scan3(iw, ic, im);
  const u64 h1 = __ballot(iw - cw < target && iw >= target);
  const int L1 = h1 ? (int)(__ffsll((long long)h1) - 1) : 63;
  const int sup = 63 - L1;
  const u64 aw = __shfl(iw - cw, L1, 64), ac = __shfl(ic - cc, L1, 64), am = __shfl(im - cm, L1, 64);
  const int bk = 64 * sup + 63 - lane;
  const u64 fc = cnt[bk], fm = mass[bk], fw = by_mass ? fm : fc;
  u64 jw = fw, jc = fc, jm = fm;
  wave_scan3(jw, jc, jm);
  const u64 h2 = __ballot(aw + jw - fw < target && aw + jw >= target);
  const int L2 = h2 ? (int)(__ffsll((long long)h2) - 1) : 63;
  Pick p;
  p.digit = (uint32_t)(64 * sup + 63 - L2);
  p.cnt_above = ac + __shfl(jc - fc, L2, 64);
  p.mass_above = am + __shfl(jm - fm, L2, 64);
  p.cnt_at = __shfl(fc, L2, 64);
  return p;
}

// Lower bound (bucket) on the keys of the kept set when top-k or top-p is on
// and min-p is off: top-k's bucket, or top-p's bucket on the whole mass;
// with both on, top-k's bucket (the top-k mass needs every token above the
// k-th).  nb counts the tokens at or above the bucket; cnt_above and
// mass_above those above it, cnt_at those in it.
struct Bound {
  uint32_t blb;
  u64 nb, cnt_above, mass_above, cnt_at;
};

// Call from one whole wave.
__device__ __forceinline__ Bound wave_bound(const uint32_t* cnt, const u64* mass, const sa_sample_params& P, int V, u64 q_all) {
  const bool kA = P.top_k > 0 && P.top_k < V, pA = P.top_p < 1.f;
  Bound bd;
  if (!kA && !pA) {
    bd.blb = 0;
    bd.nb = (u64)V;
    bd.cnt_above = bd.mass_above = bd.cnt_at = 0;
    return bd;
  }
  const u64 tau = max(1ull, (u64)ceil((double)P.top_p * (double)q_all));
  const Pick p = wave_pick(cnt, mass, !kA, kA ? (u64)P.top_k : tau);
  bd.blb = p.digit;
  bd.nb = p.cnt_above + p.cnt_at;
  bd.cnt_above = p.cnt_above;
  bd.mass_above = p.mass_above;
  bd.cnt_at = p.cnt_at;
  return bd;
}

// Min-p off, exactly one of top-k and top-p on, too many tokens at or above
// the bound for the candidate list but few enough in the bound's bucket:
// the list holds that bucket only (the edge of the kept set), the
// histogram gives what lies above it.
__device__ __forceinline__ bool edge_mode(const sa_sample_params& P, int V, const Bound& bd) {
  const bool kA = P.top_k > 0 && P.top_k < V, pA = P.top_p < 1.f;
  return !(P.min_p > 0.f) && kA != pA && bd.nb > (u64)kCap && bd.cnt_at <= (u64)kCap;
}

// The row's total mass from the per-chunk sums (one whole wave).
__device__ __forceinline__ u64 wave_row_mass(const SampleArgs& a, int b) {
  const int lane = threadIdx.x & 63;
  return wave_sum_u64(lane < a.C ? a.chunk_mass[(int64_t)b * a.C + lane] : 0ull);
}

// ---------------------------------------------------------------- gather
// Rows with top-k or top-p on and min-p off: the tokens at or above the
// bucket bound, when there are at most 4096 of them, go to the row's
// candidate list; in edge mode the tokens in the bound's bucket do, and
// each chunk's mass above the bucket goes to chunk_kmass.  Every chunk in
// its own workgroup.
__global__ __launch_bounds__(kGatherThreads) void sample_gather_kernel(SampleArgs a) {
  const int b = blockIdx.y, c = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const sa_sample_params P = a.params[b];
  if (!params_ok(P, a.u[b]) || P.temperature == 0.f || P.min_p > 0.f) return;
  if (!(P.top_k > 0 && P.top_k < a.V) && !(P.top_p < 1.f)) return;
  // (a row without a finite maximum has no histogram; whatever is gathered
  // for it, the select launch does not read it)
  __shared__ Bound s_bd;
  __shared__ float s_m;
  __shared__ u64 s_q[kGatherThreads / 64];
  const float* Z = a.zp + (int64_t)b * a.zs;
  const int v0 = c * kSampleChunk + tid;
  float z[kGatherPer];                                     // in flight while the bound is found
#pragma unroll
  for (int j = 0; j < kGatherPer; ++j) {
    const int v = v0 + j * kGatherThreads;
    z[j] = v < a.V ? Z[v] : 0.f;
  }
  if (tid < 64) {
    const bool in = lane < a.C;
    const u64 cm = in ? a.chunk_mass[(int64_t)b * a.C + lane] : 0ull;
    float mx = in ? a.chunk_max[(int64_t)b * a.C + lane] : -INFINITY;
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sft, 64));
    const Bound bd =
        wave_bound(a.hist_count + (int64_t)b * kHist, a.hist_mass + (int64_t)b * kHist, P, a.V, wave_sum_u64(cm));
    if (tid == 0) {
      s_bd = bd;
      s_m = mx;
    }
  }
  __syncthreads();
  const Bound bd = s_bd;
  const bool edge = edge_mode(P, a.V, bd);
  if (bd.nb > (u64)kCap && !edge) return;           // the select launch takes the radix path
  uint32_t key[kGatherPer];
  int id[kGatherPer];
  bool take[kGatherPer];
  u64 q = 0;
  const float m = s_m, cT = temp_coef(P.temperature);
#pragma unroll
  for (int j = 0; j < kGatherPer; ++j) {
    const int v = v0 + j * kGatherThreads;
    key[j] = fkey(z[j]);
    id[j] = v;
    const uint32_t d = key[j] >> 20;
    take[j] = v < a.V && (edge ? d == bd.blb : d >= bd.blb);
    if (edge && v < a.V && d > bd.blb) q += fixed_mass(rel_weight(z[j], m, cT));
  }
  __shared__ uint32_t s_app[kGatherThreads / 64 + 1];
  if (edge) {
    q = wave_sum_u64(q);
    if (lane == 0) s_q[tid >> 6] = q;              // read after append's barriers
  }
  append_candidates<kGatherPer, kGatherThreads>(a, b, key, id, take, s_app);
  if (edge && tid == 0) {
    u64 t = 0;
#pragma unroll
    for (int i = 0; i < kGatherThreads / 64; ++i) t += s_q[i];
    a.chunk_kmass[(int64_t)b * a.C + c] = t;
  }
}

// ---------------------------------------------------------------- select
struct SelShared {
  uint32_t c1[kNB];                       // first-level histogram (from the global one)
  u64 m1[kNB];
  union {
    struct {
      uint32_t c[kNB];
      u64 m[kNB];
    } h;                                  // deeper radix levels
    struct {
      u64 key[kCap];
      u64 cum[kCap];
    } cand;                               // candidates
    u64 grp[kSampleMaxV / 64];            // kept mass per run of 64 ids
  } u;
  u64 cm[kSampleMaxV / kSampleChunk];     // kept mass per chunk
  u64 wtot[3][kSelWaves];
  uint32_t digit;
  u64 add_cnt, add_mass;
  int idx;
  u64 val;
  float rmv;
  int rmi;
  uint32_t nlisted;
  Bound bd;
  int res_token, res_kept;
};

// Exclusive prefix sums over the workgroup's threads of three values, and totals.
__device__ __forceinline__ void block_scan3(SelShared& S, const u64 (&x)[3], u64 (&excl)[3], u64 (&tot)[3]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  u64 inc[3] = {x[0], x[1], x[2]};
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const u64 y = __shfl_up(inc[i], d, 64);
      if (lane >= d) inc[i] += y;
    }
  }
  if (lane == 63)
    for (int i = 0; i < 3; ++i) S.wtot[i][w] = inc[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    u64 base = 0, t = 0;
    for (int k = 0; k < kSelWaves; ++k) {
      const u64 v = S.wtot[i][k];
      if (k < w) base += v;
      t += v;
    }
    excl[i] = base + inc[i] - x[i];
    tot[i] = t;
  }
  __syncthreads();
}

// f(j, v, z) over ids [lo, hi) (lo a multiple of 4) in 16-byte loads, z
// holding ids v .. v+3 (those >= hi are not ids: callers test v + e < hi);
// kSelPer loads in flight per thread; every lane of every wave calls f the
// same number of times (ballots and wave reductions allowed).  Thread t
// sees v = v0 + 4 (j * 1024 + t): the lanes of a wave hold 256 consecutive
// ids and the workgroup 4096 (one chunk) per j.  Rows of z' are padded to a
// multiple of 64 floats, so a load that starts below hi stays in the row.
template <class F>
__device__ __forceinline__ void row_pass(const float* Z, int lo, int hi, F f) {
  for (int v0 = lo; v0 < hi; v0 += kSelPer * 4 * kSelThreads) {
    f32x4 z[kSelPer];
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
      const int v = v0 + 4 * (j * kSelThreads + (int)threadIdx.x);
      z[j] = v < hi ? *reinterpret_cast<const f32x4*>(Z + v) : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) f(j, v0 + 4 * (j * kSelThreads + (int)threadIdx.x), z[j]);
  }
}

// Scanning buckets from the top digit down: the digit at which above_w plus
// the weight (count or mass) of the buckets at and above it first reaches
// target.  S.digit gets it; S.add_cnt / S.add_mass the counts and masses of
// the buckets above it.  The caller guarantees that the target is reached.
__device__ __forceinline__ void pick_digit(SelShared& S, const uint32_t* cnt, const u64* mass, int NB, bool by_mass,
                           u64 target, u64 above_w) {
  const int t = threadIdx.x;
  uint32_t cc[4];
  u64 cm[4];
  u64 x[3] = {0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pos = 4 * t + i;
    cc[i] = pos < NB ? cnt[NB - 1 - pos] : 0u;
    cm[i] = pos < NB ? mass[NB - 1 - pos] : 0ull;
    x[1] += cc[i];
    x[2] += cm[i];
  }
  x[0] = by_mass ? x[2] : x[1];
  u64 ex[3], tot[3];
  if (t == 0) S.digit = 0;
  block_scan3(S, x, ex, tot);
  u64 run = above_w + ex[0], rc = ex[1], rm = ex[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u64 w = by_mass ? cm[i] : (u64)cc[i];
    if (run < target && run + w >= target) {
      S.digit = (uint32_t)(NB - 1 - (4 * t + i));
      S.add_cnt = rc;
      S.add_mass = rm;
    }
    run += w;
    rc += cc[i];
    rm += cm[i];
  }
  __syncthreads();
}

// One pass over z': histogram of (key >> digit_shift) & digit_mask over the
// keys with key >> prefix_shift == prefix.
__device__ __forceinline__ void level_pass(SelShared& S, const float* Z, int V, float m, float cT, uint32_t prefix,
                           int prefix_shift, int digit_shift, uint32_t digit_mask) {
  for (int i = threadIdx.x; i < kNB; i += kSelThreads) {
    S.u.h.c[i] = 0u;
    S.u.h.m[i] = 0ull;
  }
  __syncthreads();
  row_pass(Z, 0, V, [&](int, int v, f32x4 z4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t k = fkey(z4[e]);
      if (v + e < V && (k >> prefix_shift) == prefix) {
        const uint32_t d = (k >> digit_shift) & digit_mask;
        atomicAdd(&S.u.h.c[d], 1u);
        const u64 q = fixed_mass(rel_weight(z4[e], m, cT));
        if (q) atomicAdd(&S.u.h.m[d], q);
      }
    }
  });
  __syncthreads();
}

// The largest key K whose tokens at or above it have count (by_mass: mass)
// >= target (target <= the row's total), with the mass at or above K.
// Level 1 from S.c1/m1; levels 2 (12 bits) and 3 (8 bits) by passes over z'.
__device__ __forceinline__ void descend(SelShared& S, const float* Z, int V, float m, float cT, bool by_mass, u64 target,
                        uint32_t* K, u64* mass_ge) {
  pick_digit(S, S.c1, S.m1, kNB, by_mass, target, 0);
  const uint32_t d1 = S.digit;
  u64 ac = S.add_cnt, am = S.add_mass;
  __syncthreads();
  level_pass(S, Z, V, m, cT, d1, 20, 8, 0xFFFu);
  pick_digit(S, S.u.h.c, S.u.h.m, kNB, by_mass, target, by_mass ? am : ac);
  const uint32_t d2 = S.digit;
  ac += S.add_cnt;
  am += S.add_mass;
  __syncthreads();
  level_pass(S, Z, V, m, cT, (d1 << 12) | d2, 8, 0, 0xFFu);
  pick_digit(S, S.u.h.c, S.u.h.m, 256, by_mass, target, by_mass ? am : ac);
  const uint32_t d3 = S.digit;
  am += S.add_mass;
  *K = (d1 << 20) | (d2 << 8) | d3;
  *mass_ge = am + S.u.h.m[d3];
  __syncthreads();
}

// The draw inside ids [lo, hi) (lo a multiple of 4, hi - lo <= 4096 * 256):
// the first id whose key is >= Ks and whose cumulative kept mass from lo
// exceeds t (t below the range's kept mass).  Kept masses per run of 256
// ids (one wave's load), a scan over the runs, then one wave's scan of the
// run holding t.  Returns the id (-1 if t is not below the range's kept
// mass); *kept gets the range's kept count.
__device__ __forceinline__ int draw_range(SelShared& S, const float* Z, int lo, int hi, uint32_t Ks, float m, float cT, u64 t,
                          int* kept) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ng = (hi - lo + 255) / 256;
  uint32_t nk = 0;
  row_pass(Z, lo, hi, [&](int, int v, f32x4 z4) {
    u64 q = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = v + e < hi && fkey(z4[e]) >= Ks;
      nk += in ? 1u : 0u;
      q += in ? fixed_mass(rel_weight(z4[e], m, cT)) : 0ull;
    }
    const u64 s = wave_sum_u64(q);
    if (lane == 0 && v < hi) S.u.grp[(v - lo) >> 8] = s;
  });
  if (tid == 0) {
    S.idx = -1;
    S.val = 0;
  }
  __syncthreads();
  u64 gq[4];
  u64 x[3] = {0, (u64)nk, 0}, ex[3], tot[3];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * tid + i;
    gq[i] = g < ng ? S.u.grp[g] : 0ull;
    x[0] += gq[i];
  }
  block_scan3(S, x, ex, tot);
  *kept = (int)tot[1];
  u64 run = ex[0];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = 4 * tid + i;
    if (g < ng && run <= t && t < run + gq[i]) {
      S.idx = g;
      S.val = run;
    }
    run += gq[i];
  }
  __syncthreads();
  if (wave == 0 && S.idx >= 0) {
    const int v = lo + 256 * S.idx + 4 * lane;
    const f32x4 z4 = v < hi ? *reinterpret_cast<const f32x4*>(Z + v) : f32x4{0.f, 0.f, 0.f, 0.f};
    u64 q[4], own = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = v + e < hi && fkey(z4[e]) >= Ks;
      q[e] = in ? fixed_mass(rel_weight(z4[e], m, cT)) : 0ull;
      own += q[e];
    }
    const u64 inc = wave_incl_scan(own);
    u64 c = S.val + inc - own;                    // kept mass before this lane's ids
    int first = 3;
#pragma unroll
    for (int e = 3; e >= 0; --e) {
      u64 ce = c;
      for (int f = 0; f <= e; ++f) ce += q[f];
      if (ce > t) first = e;
    }
    const u64 over = __ballot(S.val + inc > t);
    const int L = over ? (int)(__ffsll((long long)over) - 1) : 0;
    const int id = __shfl(v + first, L, 64);
    if (lane == 0) S.res_token = over ? id : -1;
  }
  if (tid == 0 && S.idx < 0) S.res_token = -1;
  __syncthreads();
  const int r = S.res_token;
  __syncthreads();
  return r;
}

// In-place bitonic sort, descending, of S.u.cand.key[0, n), n a power of two.
__device__ __forceinline__ void sort_desc(SelShared& S, int n) {
  for (int k = 2; k <= n; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n; i += kSelThreads) {
        const int p = i ^ j;
        if (p > i) {
          const u64 x = S.u.cand.key[i], y = S.u.cand.key[p];
          const bool desc = (i & k) == 0;
          if (desc ? x < y : x > y) {
            S.u.cand.key[i] = y;
            S.u.cand.key[p] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Pads S.u.cand.key[n, 2^ceil(log2 n)) with 0 (sorts last) and sorts.
__device__ __forceinline__ void pad_sort(SelShared& S, int n) {
  const int np = pow2_at_least(max(n, 2));
  for (int i = n + (int)threadIdx.x; i < np; i += kSelThreads) S.u.cand.key[i] = 0ull;
  __syncthreads();
  sort_desc(S, np);
}

// Inclusive prefix over the first n candidates of mass_of(e) into S.u.cand.cum.
template <class F>
__device__ __forceinline__ void cand_prefix(SelShared& S, int n, F mass_of) {
  u64 q[4];
  u64 x[3] = {0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * (int)threadIdx.x + i;
    q[i] = e < n ? mass_of(e) : 0;
    x[0] += q[i];
  }
  u64 ex[3], tot[3];
  block_scan3(S, x, ex, tot);
  u64 run = ex[0];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = 4 * (int)threadIdx.x + i;
    run += q[i];
    if (e < n) S.u.cand.cum[e] = run;
  }
  __syncthreads();
}

// Bitonic sort, descending, of the 64 R values a wave holds, element
// i = 64 r + lane in x[r]: partners 64 or more apart sit in one lane,
// nearer ones are a shuffle away.
template <int R>
__device__ __forceinline__ void wave_sort_desc(u64 (&x)[R]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= 64 * R; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 64) {
        const int rj = j / 64;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int p = r ^ rj;
          if (p > r) {
            const bool desc = ((64 * r + lane) & k) == 0;
            const u64 lo = x[r], hi = x[p];
            const bool swap = desc ? lo < hi : lo > hi;
            x[r] = swap ? hi : lo;
            x[p] = swap ? lo : hi;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const u64 y = __shfl_xor(x[r], j, 64);
          const bool desc = ((64 * r + lane) & k) == 0, lower = (lane & j) == 0;
          x[r] = (desc == lower) ? (x[r] > y ? x[r] : y) : (x[r] < y ? x[r] : y);
        }
      }
    }
  }
}
// Element e (wave-uniform) of a wave-held array.
template <int R>
__device__ __forceinline__ u64 wave_at(const u64 (&x)[R], int e) {
  u64 v = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const u64 y = __shfl(x[r], e & 63, 64);
    if (r == (e >> 6)) v = y;
  }
  return v;
}
// Inclusive prefix over elements 0..n-1 in order of the masses of the keys
// in key_of(x[r]).
template <int R, class K>
__device__ __forceinline__ void wave_prefix(const u64 (&x)[R], int n, u64 (&cum)[R], float m, float cT, K key_of) {
  const int lane = threadIdx.x & 63;
  u64 base = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const u64 q = 64 * r + lane < n ? mass_of_key(key_of(x[r]), m, cT) : 0ull;
    const u64 inc = wave_incl_scan(q);
    cum[r] = base + inc;
    base += __shfl(inc, 63, 64);
  }
}
// The first element (in order) for which pred holds, or -1.
template <int R, class F>
__device__ __forceinline__ int wave_first(F pred) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const u64 h = __ballot(pred(r, 64 * r + lane));
    if (h) return 64 * r + (int)(__ffsll((long long)h) - 1);
  }
  return -1;
}
// How many elements pred holds for.
template <int R, class F>
__device__ __forceinline__ int wave_count(F pred) {
  const int lane = threadIdx.x & 63;
  int c = 0;
#pragma unroll
  for (int r = 0; r < R; ++r) c += __popcll(__ballot(pred(r, 64 * r + lane)));
  return c;
}

// At most 64 R candidates (key << 32 | ~id) in S.u.cand.key[0, n): one wave
// sorts, thresholds and draws in registers, with no barrier.  Call from one
// whole wave.
template <int R>
__device__ __forceinline__ int finish_in_wave(SelShared& S, int n, bool kA, bool pA, const sa_sample_params& P, float u,
                              float m, float cT, u64 q_all, uint32_t Km, int* kept) {
  const int lane = threadIdx.x & 63;
  u64 x[R], cum[R];
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = 64 * r + lane < n ? S.u.cand.key[64 * r + lane] : 0ull;
  wave_sort_desc<R>(x);
  auto hi_key = [](u64 v) { return (uint32_t)(v >> 32); };
  wave_prefix<R>(x, n, cum, m, cT, hi_key);
  uint32_t Kk = 0, Kp = 0;
  u64 qk = q_all;
  if (kA && n >= P.top_k) {
    Kk = hi_key(wave_at<R>(x, P.top_k - 1));
    const int c = wave_count<R>([&](int r, int e) { return e < n && hi_key(x[r]) >= Kk; });
    qk = wave_at<R>(cum, c - 1);
  }
  if (pA) {
    const u64 tau = max(1ull, (u64)ceil((double)P.top_p * (double)qk));
    const int e = wave_first<R>([&](int r, int i) { return i < n && cum[r] >= tau; });
    if (e >= 0) Kp = hi_key(wave_at<R>(x, e));
  }
  const uint32_t Ks = max(max(Kk, Kp), Km);
  const int nk = wave_count<R>([&](int r, int e) { return e < n && hi_key(x[r]) >= Ks; });
  if (nk == 0) return -1;
  const u64 qn = wave_at<R>(cum, nk - 1);
  u64 t = (u64)((double)u * (double)qn);
  if (t >= qn) t = qn - 1;
  // the kept ones by increasing id: (~id << 32 | key), descending
#pragma unroll
  for (int r = 0; r < R; ++r) x[r] = 64 * r + lane < nk ? (((u64)(uint32_t)x[r] << 32) | (x[r] >> 32)) : 0ull;
  wave_sort_desc<R>(x);
  wave_prefix<R>(x, nk, cum, m, cT, [](u64 v) { return (uint32_t)v; });
  int at = wave_first<R>([&](int r, int i) { return i < nk && cum[r] > t; });
  if (at < 0) at = nk - 1;
  *kept = nk;
  return (int)~(uint32_t)(wave_at<R>(x, at) >> 32);
}

// The candidates S.u.cand.key[0, n) (key << 32 | ~id) are every token at or
// above some key, a prefix of the ranking that holds the kept set.  Returns
// the token (and the kept count in *kept), or -1.
__device__ __forceinline__ int finish_in_lds(SelShared& S, int n, bool kA, bool pA, const sa_sample_params& P, float u,
                             float m, float cT, u64 q_all, uint32_t Km, int* kept) {
  if (n <= 256) {                    // one wave, in registers (64, 128 or 256 slots)
    if (threadIdx.x < 64) {
      int k = 0;
      const int t = n <= 64    ? finish_in_wave<1>(S, n, kA, pA, P, u, m, cT, q_all, Km, &k)
                    : n <= 128 ? finish_in_wave<2>(S, n, kA, pA, P, u, m, cT, q_all, Km, &k)
                               : finish_in_wave<4>(S, n, kA, pA, P, u, m, cT, q_all, Km, &k);
      if (threadIdx.x == 0) {
        S.res_token = t;
        S.res_kept = k;
      }
    }
    __syncthreads();
    *kept = S.res_kept;
    return S.res_token;
  }
  pad_sort(S, n);
  cand_prefix(S, n, [&](int e) { return mass_of_key((uint32_t)(S.u.cand.key[e] >> 32), m, cT); });
  auto key_at = [&](int e) { return (uint32_t)(S.u.cand.key[e] >> 32); };
  // the last candidate whose key is >= K, plus one (0: none)
  auto count_ge = [&](uint32_t K) {
    if (threadIdx.x == 0) S.idx = 0;
    __syncthreads();
    for (int e = (int)threadIdx.x; e < n; e += kSelThreads)
      if (key_at(e) >= K && (e + 1 == n || key_at(e + 1) < K)) S.idx = e + 1;
    __syncthreads();
    const int r = S.idx;
    __syncthreads();
    return r;
  };
  uint32_t Kk = 0, Kp = 0;
  u64 qk = q_all;
  if (kA && n >= P.top_k) {
    Kk = key_at(P.top_k - 1);
    qk = S.u.cand.cum[count_ge(Kk) - 1];
  }
  if (pA) {
    const u64 tau = max(1ull, (u64)ceil((double)P.top_p * (double)qk));
    if (threadIdx.x == 0) S.idx = -1;
    __syncthreads();
    for (int e = (int)threadIdx.x; e < n; e += kSelThreads)
      if (S.u.cand.cum[e] >= tau && (e == 0 || S.u.cand.cum[e - 1] < tau)) S.idx = e;
    __syncthreads();
    if (S.idx >= 0) Kp = key_at(S.idx);
    __syncthreads();
  }
  const uint32_t Ks = max(max(Kk, Kp), Km);
  const int nk = count_ge(Ks);
  if (nk == 0) return -1;
  const u64 qn = S.u.cand.cum[nk - 1];
  u64 t = (u64)((double)u * (double)qn);
  if (t >= qn) t = qn - 1;
  __syncthreads();
  // the kept tokens by increasing id: (~id << 32 | key), descending
  for (int e = (int)threadIdx.x; e < nk; e += kSelThreads) {
    const u64 x = S.u.cand.key[e];
    S.u.cand.key[e] = ((u64)(uint32_t)x << 32) | (x >> 32);
  }
  __syncthreads();
  pad_sort(S, nk);
  cand_prefix(S, nk, [&](int e) { return mass_of_key((uint32_t)S.u.cand.key[e], m, cT); });
  if (threadIdx.x == 0) S.idx = nk - 1;
  __syncthreads();
  for (int e = (int)threadIdx.x; e < nk; e += kSelThreads)
    if (S.u.cand.cum[e] > t && (e == 0 || S.u.cand.cum[e - 1] <= t)) S.idx = e;
  __syncthreads();
  *kept = nk;
  return (int)~(uint32_t)(S.u.cand.key[S.idx] >> 32);
}

// Candidates from the row's list in the workspace into LDS, then finish.
__device__ __forceinline__ int finish_from_list(SelShared& S, const SampleArgs& a, int b, int n, bool kA, bool pA,
                                const sa_sample_params& P, float u, float m, float cT, u64 q_all, uint32_t Km,
                                int* kept) {
  for (int i = threadIdx.x; i < n; i += kSelThreads) S.u.cand.key[i] = a.cand[(int64_t)b * kCap + i];
  __syncthreads();
  return finish_in_lds(S, n, kA, pA, P, u, m, cT, q_all, Km, kept);
}

// The chunk that holds the draw, from lane c's kept mass cmv of chunk c
// (c < C): t = floor(u * total), below the total; S.idx gets the first
// chunk whose running mass exceeds t and S.val t minus the mass before it.
// Call from wave 0 (the whole wave).
__device__ __forceinline__ void pick_chunk(SelShared& S, u64 cmv, int C, float u) {
  const int lane = threadIdx.x & 63;
  const u64 inc = wave_incl_scan(cmv);
  const u64 qn = __shfl(inc, 63, 64);
  u64 t = (u64)((double)u * (double)qn);
  if (t >= qn) t = qn - 1;
  const u64 hit = __ballot(lane < C && inc > t);
  const int c = hit ? (int)(__ffsll((long long)hit) - 1) : 0;
  const u64 before = __shfl(inc, c, 64) - __shfl(cmv, c, 64);
  if (lane == 0) {
    S.idx = c;
    S.val = t - before;
  }
}

// The draw over the whole row for kept = key >= Ks: kept mass per chunk of
// 4096 ids (one wave sum per chunk per wave), the chunk that holds the
// target, then draw_range inside it.
__device__ __forceinline__ int draw_row(SelShared& S, const SampleArgs& a, const float* Z, int V, uint32_t Ks, float m, float cT,
                        float u, int* kept) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int C = a.C;
  if (tid < C) S.cm[tid] = 0ull;
  __syncthreads();
  uint32_t nk = 0;
  row_pass(Z, 0, V, [&](int j, int v, f32x4 z4) {
    u64 q = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool in = v + e < V && fkey(z4[e]) >= Ks;
      nk += in ? 1u : 0u;
      q += in ? fixed_mass(rel_weight(z4[e], m, cT)) : 0ull;
    }
    const u64 s = wave_sum_u64(q);
    const int c = v / kSampleChunk;             // one j of the workgroup is one chunk
    if (lane == 0 && s && c < C) atomicAdd(&S.cm[c], s);
  });
  u64 x[3] = {0, (u64)nk, 0}, ex[3], tot[3];
  block_scan3(S, x, ex, tot);
  const int kept_all = (int)tot[1];
  if (tid < 64) pick_chunk(S, tid < C ? S.cm[tid] : 0ull, C, u);
  __syncthreads();
  const int c = S.idx;
  const u64 t_in = S.val;
  __syncthreads();
  int k_unused;
  const int token = draw_range(S, Z, c * kSampleChunk, min(V, (c + 1) * kSampleChunk), Ks, m, cT, t_in, &k_unused);
  *kept = kept_all;
  return token;
}

// Edge mode: the row's list holds every token of the bound's bucket bd.blb
// (n <= 4096, four per thread, kept in registers); the histogram gives the
// count and mass above the bucket and the gather launch each chunk's mass
// above it.  Two radix levels over the bucket's low 20 key bits (10 + 10,
// bins in c1 / m1, unused here) place the threshold exactly: the k-th key,
// or the key at which the running mass reaches top-p's share.  The kept
// tokens of the bucket add their masses to their chunks, and the draw runs
// inside the chunk that holds it.
__device__ __forceinline__ int finish_edge(SelShared& S, const SampleArgs& a, int b, int n, const Bound& bd, bool kA,
                           const sa_sample_params& P, float u, float m, float cT, u64 q_all, const float* Z, int V,
                           int* kept) {
  constexpr int R = kCap / kSelThreads;
  constexpr int kLow = 1024;                        // bins per level
  const int tid = threadIdx.x, C = a.C;
  if (n <= 0) {                                     // the bound's bucket always holds a token
    *kept = 0;
    return -1;
  }
  const u64* x = S.u.cand.key;                      // masses recomputed where needed
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int e = tid + r * kSelThreads;
    if (e < n) S.u.cand.key[e] = a.cand[(int64_t)b * kCap + e];
  }
  for (int i = tid; i < kLow; i += kSelThreads) {
    S.c1[i] = 0u;
    S.m1[i] = 0ull;
  }
  if (tid < C) S.cm[tid] = a.chunk_kmass[(int64_t)b * C + tid];
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t k = (uint32_t)(x[tid + r * kSelThreads] >> 32);
    if (tid + r * kSelThreads < n) {
      const uint32_t d = (k >> 10) & (kLow - 1);
      const u64 q = mass_of_key(k, m, cT);
      atomicAdd(&S.c1[d], 1u);
      if (q) atomicAdd(&S.m1[d], q);
    }
  }
  __syncthreads();
  const bool by_mass = !kA;
  const u64 target = kA ? (u64)P.top_k : max(1ull, (u64)ceil((double)P.top_p * (double)q_all));
  const u64 above = by_mass ? bd.mass_above : bd.cnt_above;
  pick_digit(S, S.c1, S.m1, kLow, by_mass, target, above);
  const uint32_t d1 = S.digit;
  u64 ac = S.add_cnt, am = S.add_mass;
  __syncthreads();
  for (int i = tid; i < kLow; i += kSelThreads) {
    S.c1[i] = 0u;
    S.m1[i] = 0ull;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t k = (uint32_t)(x[tid + r * kSelThreads] >> 32);
    if (tid + r * kSelThreads < n && ((k >> 10) & (kLow - 1)) == d1) {
      const u64 q = mass_of_key(k, m, cT);
      atomicAdd(&S.c1[k & (kLow - 1)], 1u);
      if (q) atomicAdd(&S.m1[k & (kLow - 1)], q);
    }
  }
  __syncthreads();
  pick_digit(S, S.c1, S.m1, kLow, by_mass, target, above + (by_mass ? am : ac));
  const uint32_t d2 = S.digit;
  ac += S.add_cnt + S.c1[d2];                       // the bucket's kept count
  const uint32_t Ks = (bd.blb << 20) | (d1 << 10) | d2;
  __syncthreads();
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t k = (uint32_t)(x[tid + r * kSelThreads] >> 32);
    if (tid + r * kSelThreads < n && k >= Ks) {
      const u64 q = mass_of_key(k, m, cT);
      if (q) atomicAdd(&S.cm[(int)~(uint32_t)x[tid + r * kSelThreads] / kSampleChunk], q);
    }
  }
  __syncthreads();
  if (tid < 64) pick_chunk(S, tid < C ? S.cm[tid] : 0ull, C, u);
  __syncthreads();
  const int c = S.idx;
  const u64 t_in = S.val;
  __syncthreads();
  int k_unused;
  const int token = draw_range(S, Z, c * kSampleChunk, min(V, (c + 1) * kSampleChunk), Ks, m, cT, t_in, &k_unused);
  *kept = (int)(bd.cnt_above + ac);
  return token;
}

__global__ __launch_bounds__(kSelThreads) void sample_select_kernel(SampleArgs a) {
  __shared__ SelShared S;
  const int b = blockIdx.x, tid = threadIdx.x;
  const sa_sample_params P = a.params[b];
  const float u = a.u[b];
  // the row maximum and its lowest id, the row's total mass and its listed
  // candidates, in one round trip by wave 0 (the mass is meaningful only for
  // rows the histogram launch processed)
  if (tid < 64) {
    float bv = tid < a.C ? a.chunk_max[(int64_t)b * a.C + tid] : 0.f;
    int ba = tid < a.C ? a.chunk_arg[(int64_t)b * a.C + tid] : -1;
    const u64 cm = tid < a.C ? a.chunk_mass[(int64_t)b * a.C + tid] : 0ull;
    const uint32_t nl = a.ncand[b];
#pragma unroll
    for (int sft = 32; sft >= 1; sft >>= 1) {
      const float ov = __shfl_xor(bv, sft, 64);
      const int oa = __shfl_xor(ba, sft, 64);
      if (better(ov, oa, bv, ba)) {
        bv = ov;
        ba = oa;
      }
    }
    const u64 total = wave_sum_u64(cm);
    if (tid == 0) {
      S.rmv = bv;
      S.rmi = ba;
      S.val = total;
      S.nlisted = nl;
    }
  }
  __syncthreads();
  const int arg = S.rmi;
  const float m = arg >= 0 ? S.rmv : -INFINITY;
  const u64 q_all = S.val;             // the row's total mass
  const uint32_t listed = S.nlisted;
  __syncthreads();
  // each path stores its result as soon as it has it (nothing stays live
  // across the other paths' code)
  auto emit = [&](int token, int kept) {
    if (tid == 0) {
      a.tokens[b] = token;
      if (a.n_kept) a.n_kept[b] = token >= 0 ? kept : 0;
      if (a.update_counts && a.counts && token >= 0) a.counts[(int64_t)b * a.V + token] += 1;
    }
  };
  const bool ok = params_ok(P, u);
  if (ok && P.temperature == 0.f) {                 // greedy
    emit(arg, 1);
    return;
  }
  if (!ok || !(fabsf(m) <= kFltMax)) {
    emit(-1, 0);
    return;
  }
  const int V = a.V;
  const float* Z = a.zp + (int64_t)b * a.zs;
  const float cT = temp_coef(P.temperature);
  const bool kA = P.top_k > 0 && P.top_k < V, pA = P.top_p < 1.f, mA = P.min_p > 0.f;
  const uint32_t Km = mA ? minp_key(m, cT, P.min_p) : 0u;
  int kept;
  // one call site per finish (each inlines a large body)
  int n_list = -1;
  if (mA && listed <= (uint32_t)kCap && !(kA && pA && (int)listed < P.top_k)) {
    n_list = (int)listed;                           // the min-p candidates of the histogram launch
  } else if (!mA && !kA && !pA) {
    // ---- no truncation: the chunk masses locate the draw
    if (tid < 64) pick_chunk(S, tid < a.C ? a.chunk_mass[(int64_t)b * a.C + tid] : 0ull, a.C, u);
    __syncthreads();
    const int c = S.idx;
    const u64 t_in = S.val;
    __syncthreads();
    int k_unused;
    emit(draw_range(S, Z, c * kSampleChunk, min(V, (c + 1) * kSampleChunk), 0u, m, cT, t_in, &k_unused), V);
    return;
  } else if (!mA) {
    if (tid < 64) {
      const Bound bd = wave_bound(a.hist_count + (int64_t)b * kHist, a.hist_mass + (int64_t)b * kHist, P, V, q_all);
      if (tid == 0) S.bd = bd;
    }
    __syncthreads();
    const Bound& bd = S.bd;                         // read from LDS where needed
    if (bd.nb <= (u64)kCap) {
      n_list = (int)min(listed, (uint32_t)kCap);    // every token at or above the bound
    } else if (edge_mode(P, V, bd)) {
      // ---- gathered by the gather launch: the bound's bucket
      const int token = finish_edge(S, a, b, (int)min(listed, (uint32_t)kCap), bd, kA, P, u, m, cT, q_all, Z, V,
                                    &kept);
      emit(token, kept);
      return;
    }
  }
  if (n_list >= 0) {
    // ---- a candidate list that holds the whole kept set
    const int token = finish_from_list(S, a, b, n_list, kA, pA, P, u, m, cT, q_all, Km, &kept);
    emit(token, kept);
    return;
  }
  // ---- large kept set: radix levels over z' (top-k's key, then top-p's
  // on the top-k mass), then the draw
  for (int i = tid; i < kNB; i += kSelThreads) {
    S.c1[i] = a.hist_count[(int64_t)b * kHist + i];
    S.m1[i] = a.hist_mass[(int64_t)b * kHist + i];
  }
  __syncthreads();
  uint32_t Kk = 0, Kp = 0;
  u64 qk = q_all;
  if (kA) descend(S, Z, V, m, cT, false, (u64)P.top_k, &Kk, &qk);
  if (pA) {
    const u64 tau = max(1ull, (u64)ceil((double)P.top_p * (double)qk));
    u64 unused;
    descend(S, Z, V, m, cT, true, tau, &Kp, &unused);
  }
  const int token = draw_row(S, a, Z, V, max(max(Kk, Kp), Km), m, cT, u, &kept);
  emit(token, kept);
}

__global__ __launch_bounds__(256) void sample_count_kernel(const int32_t* ids, int H, int64_t stride,
                                                           int32_t* counts, int V) {
  const int b = blockIdx.y, j = blockIdx.x * 256 + threadIdx.x;
  if (j >= H) return;
  const int id = ids[(int64_t)b * stride + j];
  if (id >= 0 && id < V) atomicAdd(&counts[(int64_t)b * V + id], 1);
}

}  // namespace

#ifndef SA_HIST_WGS
#define SA_HIST_WGS 384
#endif
hipError_t launch_sample(const SampleArgs& args, hipStream_t s) {
  SampleArgs a = args;
  // several chunks per histogram workgroup once the batch gives more than
  // SA_HIST_WGS workgroups (one and a half per CU; swept 128-768), up to 8
  a.hist_cpw = max(1, min(8, (a.B * a.C) / SA_HIST_WGS));
  const dim3 grid(a.C, a.B);
  hipLaunchKernelGGL(sample_prep_kernel, grid, dim3(kPrepOnlyThreads), 0, s, a);
  hipLaunchKernelGGL(sample_hist_kernel, dim3((a.C + a.hist_cpw - 1) / a.hist_cpw, a.B), dim3(kHistThreads), 0, s,
                     a);
  hipLaunchKernelGGL(sample_gather_kernel, grid, dim3(kGatherThreads), 0, s, a);
  hipLaunchKernelGGL(sample_select_kernel, dim3(a.B), dim3(kSelThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_sample_count(const int32_t* ids, int B, int H, int64_t ids_stride, int32_t* counts,
                               int V, hipStream_t s) {
  hipLaunchKernelGGL(sample_count_kernel, dim3((H + 255) / 256, B), dim3(256), 0, s, ids, H, ids_stride,
                     counts, V);
  return hipGetLastError();
}
