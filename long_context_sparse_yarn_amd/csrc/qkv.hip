// sinkattn_qkv_rope_append: the layer's fused qkv projection with the RoPE
// and cache append as its epilogue, on the gfx950 matrix cores.
//
// What is computed ("GQA Attention" study note on gpt-oss, How it works;
// "MoE-Xtend" README, ROPE + SCALING and KV CACHE): qkv = x W^T + b for the
// hidden states x [B*T, d_model] and the fused weight W [d_qkv, d_model],
// d_qkv = d (n_q + 2 n_kv), rounded once to bf16 as a bf16 linear layer
// returns it; split [Q | K | V], each head-major; Q rotated at positions
// pos0 + t into q_rot, K rotated into the cache rows, V appended unrotated.
// Every rotated value carries the bits of yarn_rope applied to the bf16
// projection (the fp64 rotation rounded once, sa_rope.h).
//
// How:
//  * C^T = W x^T with v_mfma_f32_16x16x32_bf16: a workgroup (8 waves) owns
//    256 tokens x 256 features (4 heads at d = 64, 2 at d = 128; 2 heads,
//    192 features at d = 96), so each byte staged from L2 feeds >= 110
//    flops; wave (wf, wt) owns half of the features (whole heads) and 64 of
//    the tokens, so each lane ends with 4 consecutive features of one token
//    per 16x16 tile, and the two halves of a RoPE pair (e, e + d/2) sit in
//    the same lane (d/2 is a multiple of 16).
//  * Both operands are contiguous along d_model (W is the linear layer's
//    [out, in] matrix); the contraction is the shared GEMM core (sa_gemm.h).
//  * Epilogue in registers: + bias (fp32), one rounding to bf16, rotation
//    against a per-position table of fp64 (c cos, c sin) built by a small
//    kernel first (the same sincos_reduced as every RoPE path), fp32 where
//    the error bound proves the same rounding and fp64 otherwise; Q and K
//    leave as 8-byte rows (4 features), V as 2-byte stores into the blocked
//    layout (16 lanes = 16 consecutive keys of one coordinate).
#include "sa_device.h"
#include "sa_kernels.h"
#include "sa_gemm.h"
#include "sa_rope.h"

namespace {

constexpr int kThreads = sa_gemm::kThreads;   // 8 waves: 2 feature halves x 4 token quarters
// Tokens per workgroup by head dimension (256 or 128; overridable for tuning).
#ifndef SA_QKV_TM64
#define SA_QKV_TM64 256
#endif
#ifndef SA_QKV_TM96
#define SA_QKV_TM96 128
#endif
#ifndef SA_QKV_TM128
#define SA_QKV_TM128 256
#endif

// tab[t][i] = (c cos, c sin)(pos0 + t) * inv_freq_i), fp64
__global__ __launch_bounds__(kThreads) void rope_table_kernel(QkvArgs a) {
  const int half = a.d / 2;
  const int64_t n = (int64_t)a.T * half;
  for (int64_t e = blockIdx.x * (int64_t)kThreads + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * kThreads) {
    const int t = (int)(e / half), i = (int)(e - (int64_t)t * half);
    double sn, cn;
    sa_rope::sincos_reduced((double)(a.pos0 + t) * a.inv_freq[i], &sn, &cn);
    a.tab[e] = make_double2(cn * a.conc, sn * a.conc);
  }
}

// bf16 value (as fp32) of fp32 x, round to nearest even
__device__ __forceinline__ float round_bf16(float x) {
  return __uint_as_float(pack_bf16x2(x, 0.f) << 16);
}

// 128-token tiles take half the LDS, so two workgroups can share a CU when
// the registers fit (<= 128 per lane): ask for that occupancy.
template <int D, int TM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(TM == 128 ? 4 : 1)))
void qkv_rope_append_kernel(QkvArgs a, int n_mt) {
  constexpr int HPW = D == 64 ? 4 : 2;  // heads per workgroup
  constexpr int F = HPW * D;            // features per workgroup (256, 192, 256)
  constexpr int HW = HPW / 2;           // heads per wave
  using G = sa_gemm::Gemm<F, TM>;
  constexpr int TT = G::TT;
  __shared__ __attribute__((aligned(16))) uint16_t lds[G::LDS_ELEMS];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 15, g4 = lane >> 4;
  const int wf = wave & 1, wt = wave >> 1;       // feature half, 64-token quarter
  const int mt = blockIdx.x % n_mt, nt = blockIdx.x / n_mt;
  const int M = a.B * a.T;
  const int H = a.n_q + 2 * a.n_kv;             // heads of the fused width
  const int dqkv = H * D;
  const int m0 = mt * TM, f0 = nt * F;

  // element offsets of the chunks this lane stages; rows past the ends are
  // clamped (their results are never stored)
  uint32_t w_off[G::WBW], x_off[G::XBW];
#pragma unroll
  for (int i = 0; i < G::WBW; ++i) {
    int r, c;
    G::w_slot(i, &r, &c);
    w_off[i] = (uint32_t)min(f0 + r, dqkv - 1) * (uint32_t)a.d_model + 8 * c;
  }
#pragma unroll
  for (int i = 0; i < G::XBW; ++i) {
    int r, c;
    G::x_slot(i, &r, &c);
    x_off[i] = (uint32_t)min(m0 + r, M - 1) * (uint32_t)a.d_model + 8 * c;
  }
  f32x4 acc[G::FT][TT];
  G::run(reinterpret_cast<const uint16_t*>(a.w), w_off, reinterpret_cast<const uint16_t*>(a.x),
         x_off, a.d_model, lds, acc);

  // ---- epilogue: lane holds features 16f + 4*g4 + r (of the wave's FW) of
  // token 16t + j (of its 64); the wave's features are HW whole heads
  const float k2 = sa_rope::bf16_rot_k2(a.conc);
  uint16_t* qo = reinterpret_cast<uint16_t*>(a.q_rot);
  uint16_t* kc = reinterpret_cast<uint16_t*>(a.kc);
  uint16_t* vc = reinterpret_cast<uint16_t*>(a.vc);
  constexpr int FH = D / 16;                      // feature tiles per head
#pragma unroll
  for (int hw = 0; hw < HW; ++hw) {
    const int hd = HPW * nt + HW * wf + hw;       // head in the fused width
    if (hd >= H) break;
    const int kind = hd < a.n_q ? 0 : (hd < a.n_q + a.n_kv ? 1 : 2);   // Q, K, V
    const int hh = kind == 0 ? hd : (kind == 1 ? hd - a.n_q : hd - a.n_q - a.n_kv);
    const uint16_t* bg = reinterpret_cast<const uint16_t*>(a.bias) + (int64_t)hd * D;
    float val[FH][TT][4];
#pragma unroll
    for (int f = 0; f < FH; ++f) {
      const u32x2 bb = *reinterpret_cast<const u32x2*>(bg + 16 * f + 4 * g4);
      const float bv[4] = {bf16_lo(bb.x), bf16_hi(bb.x), bf16_lo(bb.y), bf16_hi(bb.y)};
#pragma unroll
      for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) val[f][t][r] = round_bf16(acc[FH * hw + f][t][r] + bv[r]);
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const int m = m0 + G::TQ * wt + 16 * t + j;
      if (m >= M) continue;
      const int b = m / a.T, tt = m - b * a.T;
      const int64_t crow = a.row0 + tt;             // cache row of this token
      if (kind == 2) {
        uint16_t* vp = vc + (((int64_t)b * (a.C / 32) + crow / 32) * a.n_kv + hh) * (int64_t)D * 32 +
                       crow % 32;
#pragma unroll
        for (int f = 0; f < FH; ++f)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            vp[(16 * f + 4 * g4 + r) * 32] = (uint16_t)(__float_as_uint(val[f][t][r]) >> 16);
        continue;
      }
      uint16_t* row = kind == 0 ? qo + (((int64_t)b * a.T + tt) * a.n_q + hh) * D
                                : kc + (((int64_t)b * a.C + crow) * a.n_kv + hh) * D;
      const double2* tb = a.tab + (int64_t)tt * (D / 2);
#pragma unroll
      for (int f = 0; f < FH / 2; ++f) {
        const int e = 16 * f + 4 * g4;              // pair index of r = 0
        uint32_t y1[4], y2[4];
        bool ok = true;
        double2 cs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          cs[r] = tb[e + r];
          const float u = val[f][t][r], v = val[f + FH / 2][t][r];
          const float cc = (float)cs[r].x, ss = (float)cs[r].y;
          const float f1 = fmaf(u, cc, -(v * ss)), f2 = fmaf(v, cc, u * ss);
          const float sum = fabsf(u) + fabsf(v), tol = sum * k2;
          ok = ok & (sum >= 0x1p-100f) & (fabsf(f1 - sa_rope::bf16_mid(f1)) > tol) &
               (fabsf(f2 - sa_rope::bf16_mid(f2)) > tol);
          y1[r] = __float_as_uint(round_bf16(f1)) >> 16;
          y2[r] = __float_as_uint(round_bf16(f2)) >> 16;
        }
        if (__builtin_amdgcn_ballot_w64(!ok) != 0) {   // rare: the fp64 rotation
          if (!ok) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const double u = val[f][t][r], v = val[f + FH / 2][t][r];
              y1[r] = f64_to_bf16_bits(sa_rope::rot_first(u, v, cs[r].x, cs[r].y));
              y2[r] = f64_to_bf16_bits(sa_rope::rot_second(u, v, cs[r].x, cs[r].y));
            }
          }
        }
        *reinterpret_cast<u32x2*>(row + e) = u32x2{y1[0] | (y1[1] << 16), y1[2] | (y1[3] << 16)};
        *reinterpret_cast<u32x2*>(row + e + D / 2) =
            u32x2{y2[0] | (y2[1] << 16), y2[2] | (y2[3] << 16)};
      }
    }
  }
}

template <int D, int TM>
hipError_t launch_d(const QkvArgs& a, hipStream_t s) {
  constexpr int HPW = D == 64 ? 4 : 2;
  const int M = a.B * a.T;
  const int n_mt = (M + TM - 1) / TM;
  const int H = a.n_q + 2 * a.n_kv;
  const int n_nt = (H + HPW - 1) / HPW;
  hipLaunchKernelGGL((qkv_rope_append_kernel<D, TM>), dim3((unsigned)(n_mt * n_nt)), dim3(kThreads), 0,
                     s, a, n_mt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qkv_rope_append(const QkvArgs& a, hipStream_t s) {
  const int64_t n = (int64_t)a.T * (a.d / 2);
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                     dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.d) {
    case 64: return launch_d<64, SA_QKV_TM64>(a, s);
    case 96: return launch_d<96, SA_QKV_TM96>(a, s);
    case 128: return launch_d<128, SA_QKV_TM128>(a, s);
    default: return hipErrorInvalidValue;
  }
}
