// MoE layer on the gfx950 matrix cores: router with top-k, dispatch by
// expert, the selected SwiGLU experts, and the weighted combine.
//
// What is computed ("MoE-Xtend" README, MOE ROUTING; "GPT-OSS-Lite" visual
// guide, Architecture Specifications): logits = x W_r^T (a bf16 linear,
// rounded once), the k largest per token (equal logits: lower expert id
// first), weights = softmax over those k logits; each token's row goes to
// its k experts only; expert e computes W2_e (silu(W1_e x) * (W3_e x)) with
// every linear rounded once to bf16 and the gated product rounded to bf16;
// y = sum_slots w * expert output (+ an optional shared SwiGLU expert with
// weight 1), summed in fp32 in slot order and rounded once to bf16.
//
// How:
//  * router: one wave per 16 tokens, C^T = W_r x^T by MFMA with operands
//    straight from global memory (W_r is small and cached); the wave's
//    logits go through LDS to 16 lanes that each run the top-k and softmax
//    of one token.
//  * dispatch, deterministic: per block of 256 tokens a count per expert
//    (LDS integer atomics), one pass that turns counts into per-(block,
//    expert) offsets and expert starts, then a scatter in which each
//    (token, slot) takes the rank of its token among the block's tokens
//    routed to the same expert (wave ballots + popcount): rows are listed
//    by expert, then token.
//  * experts: the shared GEMM core (sa_gemm.h) over 256 rows of one expert
//    per workgroup.  Up: the rows are gathered through the dispatch list;
//    each wave's 128 weight rows are 64 gate rows and the 64 matching up
//    rows, so a lane holds both factors of its features and applies
//    silu(a) * b in registers.  Down: the expert's rows are contiguous; the
//    epilogue scales by the token's routing weight and writes an fp32 row
//    per (token, slot).  The slots are summed in order by the shared
//    expert's down pass when there is one, else by a combine pass.
#include "sa_device.h"
#include "sa_gemm.h"
#include "sa_kernels.h"

namespace {

constexpr int kThreads = sa_gemm::kThreads;
constexpr int kTM = sa_gemm::kTM;
constexpr int kBlock = 256;            // tokens per dispatch block

__device__ __forceinline__ float round_bf16(float x) {
  return __uint_as_float(pack_bf16x2(x, 0.f) << 16);
}

// ---------------------------------------------------------------- router
template <int ET>
__global__ __launch_bounds__(256) void moe_router_kernel(MoeArgs a) {
  __shared__ float lg[4][16][16 * ET];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g4 = lane >> 4;
  const int t0 = (blockIdx.x * 4 + wave) * 16;
  const int dm = a.d_model;
  const uint16_t* x = reinterpret_cast<const uint16_t*>(a.x);
  const uint16_t* wr = reinterpret_cast<const uint16_t*>(a.w_router);
  const int tok = min(t0 + j, a.N - 1);
  f32x4 acc[ET];
#pragma unroll
  for (int e = 0; e < ET; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < dm; k0 += 32) {
    const u32x4 B = ld16(x + (int64_t)tok * dm + k0 + 8 * g4);
#pragma unroll
    for (int e = 0; e < ET; ++e) {
      const int er = min(16 * e + j, a.E - 1);
      acc[e] = mfma16x16x32(ld16(wr + (int64_t)er * dm + k0 + 8 * g4), B, acc[e]);
    }
  }
  // lane: experts 16e + 4 g4 + r of token t0 + j
  uint16_t* lo = reinterpret_cast<uint16_t*>(a.logits);
#pragma unroll
  for (int e = 0; e < ET; ++e)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ex = 16 * e + 4 * g4 + r;
      const float v = round_bf16(acc[e][r]);
      lg[wave][j][ex] = v;
      if (ex < a.E && t0 + j < a.N)
        lo[(int64_t)(t0 + j) * a.E + ex] = (uint16_t)(__float_as_uint(v) >> 16);
    }
  __syncthreads();
  if (g4 != 0 || t0 + j >= a.N) return;
  // top-k, largest first, equal logits in increasing expert id
  const float* v = lg[wave][j];
  uint64_t taken = 0;
  int sel[8];
  float sv[8];
  for (int s = 0; s < a.k; ++s) {
    int bi = -1;
    float best = 0.f;
    for (int e = 0; e < a.E; ++e) {
      if ((taken >> e) & 1) continue;
      if (bi < 0 || v[e] > best) {
        bi = e;
        best = v[e];
      }
    }
    taken |= 1ull << bi;
    sel[s] = bi;
    sv[s] = best;
  }
  float z = 0.f, ex[8];
  for (int s = 0; s < a.k; ++s) {
    ex[s] = __expf(sv[s] - sv[0]);
    z += ex[s];
  }
  const float inv = 1.0f / z;
  for (int s = 0; s < a.k; ++s) {
    a.ids[(int64_t)(t0 + j) * a.k + s] = sel[s];
    a.weights[(int64_t)(t0 + j) * a.k + s] = ex[s] * inv;
  }
}

// ---------------------------------------------------------------- dispatch
__global__ __launch_bounds__(kBlock) void moe_count_kernel(MoeArgs a) {
  __shared__ int cnt[64];
  if (threadIdx.x < 64) cnt[threadIdx.x] = 0;
  __syncthreads();
  const int t = blockIdx.x * kBlock + threadIdx.x;
  if (t < a.N)
    for (int s = 0; s < a.k; ++s) {
      const int id = a.ids[(int64_t)t * a.k + s];
      if (id >= 0 && id < a.E) atomicAdd(&cnt[id], 1);   // ids outside [0, E) are skipped
    }
  __syncthreads();
  if (threadIdx.x < a.E) a.counts[blockIdx.x * a.E + threadIdx.x] = cnt[threadIdx.x];
}

// one workgroup: thread e turns expert e's per-block counts into offsets
__global__ __launch_bounds__(64) void moe_scan_kernel(MoeArgs a, int nblk) {
  __shared__ int tot[64], first[64];
  extern __shared__ int cnt[];                    // [nblk][E], loaded in parallel
  const int e = threadIdx.x;
  for (int i = threadIdx.x; i < nblk * a.E; i += 64) cnt[i] = a.counts[i];
  __syncthreads();
  int run = 0;
  if (e < a.E)
    for (int b = 0; b < nblk; ++b) {
      const int c = cnt[b * a.E + e];
      cnt[b * a.E + e] = run;
      run += c;
    }
  tot[e] = e < a.E ? run : 0;
  __syncthreads();
  if (e == 0) {
    int s = 0, ts = 0;
    for (int i = 0; i < a.E; ++i) {
      first[i] = s;
      a.expert_start[i] = s;
      a.tile_start[i] = ts;
      s += tot[i];
      ts += (tot[i] + kTM - 1) / kTM;
    }
    a.expert_start[a.E] = s;
    a.tile_start[a.E] = ts;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nblk * a.E; i += 64) a.offsets[i] = cnt[i] + first[i % a.E];
}

__global__ __launch_bounds__(kBlock) void moe_scatter_kernel(MoeArgs a) {
  __shared__ int wave_tot[kBlock / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * kBlock + threadIdx.x;
  const bool live = t < a.N;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int e = 0; e < a.E; ++e) {
    int slot = -1;
    if (live)
      for (int s = 0; s < a.k; ++s)
        if (a.ids[(int64_t)t * a.k + s] == e) slot = s;
    const uint64_t ball = __builtin_amdgcn_ballot_w64(slot >= 0);
    if (lane == 0) wave_tot[wave] = __popcll(ball);
    __syncthreads();
    int pre = __popcll(ball & below);
    for (int w = 0; w < wave; ++w) pre += wave_tot[w];
    if (slot >= 0) a.rows[a.offsets[blockIdx.x * a.E + e] + pre] = t * a.k + slot;
    __syncthreads();
  }
}

// ---------------------------------------------------------------- experts
// Which expert and which 256-row tile of it a workgroup's tile index names;
// false past the last tile.
__device__ __forceinline__ bool find_tile(const MoeArgs& a, const MoeGroup& g, int tile, int* e,
                                          int* r0, int* nrows) {
  if (g.shared) {
    *e = 0;
    *r0 = tile * kTM;
    *nrows = min(kTM, a.N - *r0);
    return *r0 < a.N;
  }
  if (tile >= a.tile_start[a.E]) return false;
  int ex = 0;
  while (a.tile_start[ex + 1] <= tile) ++ex;
  *e = ex;
  *r0 = a.expert_start[ex] + (tile - a.tile_start[ex]) * kTM;
  *nrows = min(kTM, a.expert_start[ex + 1] - *r0);
  return true;
}

// h = silu(x W1^T) * (x W3^T) for 256 rows of one expert x 128 features
__global__ __launch_bounds__(kThreads) void moe_up_kernel(MoeArgs a, MoeGroup g, int n_ft) {
  using G = sa_gemm::Gemm<256>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[G::LDS_ELEMS];
  const int tile = blockIdx.x / n_ft, ft = blockIdx.x % n_ft;
  int e, r0, nrows;
  if (!find_tile(a, g, tile, &e, &r0, &nrows)) return;
  const int f0 = ft * 128, ffn = g.ffn, dm = a.d_model;
  const uint16_t* w13 = reinterpret_cast<const uint16_t*>(g.w13) + (int64_t)e * 2 * ffn * dm;
  uint32_t w_off[G::WBW], x_off[G::XBW];
#pragma unroll
  for (int i = 0; i < G::WBW; ++i) {
    int r, c;
    G::w_slot(i, &r, &c);
    // LDS row r: wave half r / 128; its first 64 rows are gate rows, the
    // next 64 the up rows of the same features
    const int half = r >> 7, q = r & 127;
    const int wrow = (q < 64 ? 0 : ffn) + f0 + 64 * half + (q & 63);
    w_off[i] = (uint32_t)wrow * (uint32_t)dm + 8 * c;
  }
#pragma unroll
  for (int i = 0; i < G::XBW; ++i) {
    int r, c;
    G::x_slot(i, &r, &c);
    const int gr = r0 + min(r, nrows - 1);
    const int tok = g.shared ? gr : a.rows[gr] / a.k;
    x_off[i] = (uint32_t)tok * (uint32_t)dm + 8 * c;
  }
  f32x4 acc[G::FT][G::TT];
  G::run(w13, w_off, reinterpret_cast<const uint16_t*>(a.x), x_off, dm, lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g4 = lane >> 4, wf = wave & 1, wt = wave >> 1;
  uint16_t* h = reinterpret_cast<uint16_t*>(g.h);
#pragma unroll
  for (int t = 0; t < G::TT; ++t) {
    const int r = 64 * wt + 16 * t + j;
    if (r >= nrows) continue;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float av = round_bf16(acc[f][t][q]), bv = round_bf16(acc[f + 4][t][q]);
        o[q] = __float_as_uint(round_bf16(av / (1.0f + __expf(-av)) * bv)) >> 16;
      }
      *reinterpret_cast<u32x2*>(h + (int64_t)(r0 + r) * ffn + f0 + 64 * wf + 16 * f + 4 * g4) =
          u32x2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
    }
  }
}

// out = w * (h W2^T) for 256 rows of one expert x 256 output features
// combine: the shared expert, run last, adds the k routed slots of its rows
// in slot order and writes y (the same sums, in the same order, as
// moe_combine_kernel over k + 1 slots)
__global__ __launch_bounds__(kThreads) void moe_down_kernel(MoeArgs a, MoeGroup g, int n_ft,
                                                            int combine) {
  using G = sa_gemm::Gemm<256>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[G::LDS_ELEMS];
  const int tile = blockIdx.x / n_ft, ft = blockIdx.x % n_ft;
  int e, r0, nrows;
  if (!find_tile(a, g, tile, &e, &r0, &nrows)) return;
  const int f0 = ft * 256, ffn = g.ffn, dm = a.d_model;
  const uint16_t* w2 = reinterpret_cast<const uint16_t*>(g.w2) + (int64_t)e * dm * ffn;
  uint32_t w_off[G::WBW], x_off[G::XBW];
#pragma unroll
  for (int i = 0; i < G::WBW; ++i) {
    int r, c;
    G::w_slot(i, &r, &c);
    w_off[i] = (uint32_t)min(f0 + r, dm - 1) * (uint32_t)ffn + 8 * c;
  }
#pragma unroll
  for (int i = 0; i < G::XBW; ++i) {
    int r, c;
    G::x_slot(i, &r, &c);
    x_off[i] = (uint32_t)(r0 + min(r, nrows - 1)) * (uint32_t)ffn + 8 * c;
  }
  f32x4 acc[G::FT][G::TT];
  G::run(w2, w_off, reinterpret_cast<const uint16_t*>(g.h), x_off, ffn, lds, acc);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g4 = lane >> 4, wf = wave & 1, wt = wave >> 1;
  const int S = a.k + 1;                          // slots per token row of the output
#pragma unroll
  for (int t = 0; t < G::TT; ++t) {
    const int r = 64 * wt + 16 * t + j;
    if (r >= nrows) continue;
    int tok, slot;
    float wgt;
    if (g.shared) {
      tok = r0 + r;
      slot = a.k;
      wgt = 1.f;
    } else {
      const int code = a.rows[r0 + r];
      tok = code / a.k;
      slot = code - tok * a.k;
      wgt = a.weights[code];
    }
    float* orow = a.out_slots + ((int64_t)tok * S + slot) * dm;
    const float* trow = a.out_slots + (int64_t)tok * S * dm;
#pragma unroll
    for (int f = 0; f < G::FT; ++f) {
      const int feat = f0 + 128 * wf + 16 * f + 4 * g4;
      if (feat >= dm) continue;
      f32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = wgt * round_bf16(acc[f][t][q]);
      if (combine) {
        f32x4 sum = *reinterpret_cast<const f32x4*>(trow + feat);
        for (int sl = 1; sl < a.k; ++sl) sum += *reinterpret_cast<const f32x4*>(trow + sl * dm + feat);
        sum += o;
        *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.y) + (int64_t)tok * dm + feat) =
            u32x2{pack_bf16x2(sum[0], sum[1]), pack_bf16x2(sum[2], sum[3])};
      } else {
        *reinterpret_cast<f32x4*>(orow + feat) = o;
      }
    }
  }
}

// y = bf16(sum over the slots in order)
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs a, int nslots) {
  const int64_t n4 = (int64_t)a.N * a.d_model / 4;
  const int S = a.k + 1;
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    const int64_t tok = i / (a.d_model / 4);
    const int f = (int)(i - tok * (a.d_model / 4)) * 4;
    const float* src = a.out_slots + tok * S * a.d_model + f;
    f32x4 s = *reinterpret_cast<const f32x4*>(src);
    for (int sl = 1; sl < nslots; ++sl) s += *reinterpret_cast<const f32x4*>(src + sl * a.d_model);
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.y) + tok * a.d_model + f) =
        u32x2{pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3])};
  }
}

}  // namespace

hipError_t launch_moe_route(const MoeArgs& a, hipStream_t s) {
  const int grid = (a.N + 63) / 64;
  switch ((a.E + 15) / 16) {
    case 1: hipLaunchKernelGGL(moe_router_kernel<1>, dim3(grid), dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL(moe_router_kernel<2>, dim3(grid), dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL(moe_router_kernel<3>, dim3(grid), dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL(moe_router_kernel<4>, dim3(grid), dim3(256), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_moe_dispatch(const MoeArgs& a, hipStream_t s) {
  const int nblk = (a.N + kBlock - 1) / kBlock;
  hipLaunchKernelGGL(moe_count_kernel, dim3(nblk), dim3(kBlock), 0, s, a);
  hipLaunchKernelGGL(moe_scan_kernel, dim3(1), dim3(64), (size_t)nblk * a.E * sizeof(int), s, a,
                     nblk);
  hipLaunchKernelGGL(moe_scatter_kernel, dim3(nblk), dim3(kBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_moe_experts(const MoeArgs& a, const MoeGroup& g, bool combine, hipStream_t s) {
  // tiles: an upper bound (one partial tile per expert at most); workgroups
  // past the last tile return at once
  const int tiles = g.shared ? (a.N + kTM - 1) / kTM : (a.N * a.k + kTM - 1) / kTM + a.E;
  const int n_up = g.ffn / 128, n_down = (a.d_model + 255) / 256;
  hipLaunchKernelGGL(moe_up_kernel, dim3(tiles * n_up), dim3(kThreads), 0, s, a, g, n_up);
  hipLaunchKernelGGL(moe_down_kernel, dim3(tiles * n_down), dim3(kThreads), 0, s, a, g, n_down,
                     combine ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_moe_combine(const MoeArgs& a, int nslots, hipStream_t s) {
  const int64_t n4 = (int64_t)a.N * a.d_model / 4;
  const int64_t blocks = (n4 + 255) / 256;
  hipLaunchKernelGGL(moe_combine_kernel, dim3((unsigned)(blocks < 8192 ? blocks : 8192)), dim3(256),
                     0, s, a, nslots);
  return hipGetLastError();
}
