// fp32 sink attention (prefill and decode): the full-precision variant on
// the vector ALUs, for fp32 activations and caches.
//
// Same definition as the bf16 kernels ("MoE-Xtend" README, ATTENTION STACK;
// "GQA Attention" study note, How it works).  One wave owns one
// (b, t, h) query row: lanes take 64 keys at a time, each forming one score;
// an online softmax in natural-exp units, seeded with the sink (m = sigma,
// l = 1; sigma = -inf gives m = -inf, l = 0), folds the chunks; each lane
// accumulates the output coordinates lane, lane+64, ...  Decode uses the
// same kernel with one query at position o - 1.
#include "sa_device.h"
#include "sa_kernels.h"

namespace {

constexpr int kMaxD = 256;

__global__ __launch_bounds__(64) void attn_rows_f32_kernel(AttnArgs a) {
  __shared__ float qs[kMaxD];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  int64_t id = blockIdx.x;
  const int h = (int)(id % a.n_q);
  id /= a.n_q;
  const int t = (int)(id % a.T_q);
  const int b = (int)(id / a.T_q);
  const int g = h / a.q_mult;
  const int D = a.d;
  const int64_t C = a.C;

  const float* q = reinterpret_cast<const float*>(a.q) + (((int64_t)b * a.T_q + t) * a.n_q + h) * D;
  const float* kc = reinterpret_cast<const float*>(a.kc);
  const float* vc = reinterpret_cast<const float*>(a.vc);
  for (int i = lane; i < D; i += 64) qs[i] = q[i];
  __syncthreads();

  const int64_t P = a.q_offset + t;
  const int64_t lo = a.window > 0 ? max((int64_t)0, P - a.window + 1) : 0;
  const int64_t hi = P + 1;

  const float sg = a.sinks[h];
  float m_run = sg;
  float l_run = (sg == -INFINITY) ? 0.f : 1.f;
  constexpr int PER = kMaxD / 64;
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.f;

  for (int64_t k0 = lo; k0 < hi; k0 += 64) {
    const int64_t key = k0 + lane;
    float s = -INFINITY;
    if (key < hi) {
      const float* krow = kc + ((b * C + key) * a.n_kv + g) * D;
      float dot = 0.f;
      for (int i = 0; i < D; ++i) dot = fmaf(qs[i], krow[i], dot);
      s = dot * a.sm_scale;
    }
    const float m_new = fmaxf(m_run, wave_max(s));
    const float alpha = (m_run == -INFINITY) ? 0.f : expf(m_run - m_new);
    const float p = (key < hi) ? expf(s - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum(p);
    m_run = m_new;
    __syncthreads();
    ps[lane] = p;
    __syncthreads();
    const int nk = (int)min((int64_t)64, hi - k0);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int dd = lane + 64 * i;
      if (dd >= D) break;
      float v_acc = acc[i] * alpha;
      for (int kk = 0; kk < nk; ++kk) {
        const int64_t kj = k0 + kk;
        const float v = vc[((b * (C / 32) + kj / 32) * a.n_kv + g) * (int64_t)(D * 32) + dd * 32 + (kj & 31)];
        v_acc = fmaf(ps[kk], v, v_acc);
      }
      acc[i] = v_acc;
    }
  }
  float* out = reinterpret_cast<float*>(a.out) + (((int64_t)b * a.T_q + t) * a.n_q + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int dd = lane + 64 * i;
    if (dd < D) out[dd] = acc[i] / l_run;
  }
}

}  // namespace

hipError_t launch_attn_rows_f32(const AttnArgs& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.B * a.T_q * a.n_q;
  hipLaunchKernelGGL(attn_rows_f32_kernel, dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}
