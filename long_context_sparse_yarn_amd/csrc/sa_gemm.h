// The matrix-core GEMM core shared by the fused qkv projection and the MoE
// expert layers: C^T (F features x TM tokens) = W x^T over a contraction of
// K elements, both operands contiguous along K (a linear layer's [out, in]
// weight rows and the tokens' rows), for a workgroup of 8 waves.
//
//  * 64-wide slices of the F weight rows and the TM token rows go global ->
//    LDS with 16-byte global_load_lds (no staging registers): slot l of a
//    1 KB block receives one 16-byte chunk; chunk c of row r sits at slot
//    c ^ (r & 7), so the operand reads below are free of bank conflicts.
//    Where the rows come from is the caller's: it hands in, per lane, the
//    element offset of the chunk it fetches (w_slot / x_slot tell which row
//    and chunk that is), so tokens can be gathered through an index list.
//  * Two LDS stages, one barrier per stage.
//  * Wave (wf, wt) = (wave & 1, wave >> 1) owns features [F/2 wf, +F/2) and
//    tokens [TM/4 wt, +TM/4); v_mfma_f32_16x16x32_bf16 leaves lane l with
//    features 16 f + 4 (l / 16) + r (r < 4) of token 16 t + (l % 16) of its
//    part in acc[f][t][r].
#pragma once

#include "sa_device.h"

namespace sa_gemm {

constexpr int kThreads = 512;   // 8 waves
constexpr int kWaves = kThreads / 64;
constexpr int kTM = 256;        // tokens per workgroup
constexpr int kKS = 64;         // contraction elements per LDS stage

__device__ __forceinline__ void lds_direct16(const void* src, const uint16_t* lds_block) {
  __builtin_amdgcn_global_load_lds(
      src, (__attribute__((address_space(3))) void*)(const_cast<uint16_t*>(lds_block)), 16, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

template <int F, int TM = kTM>
struct Gemm {
  static constexpr int WBUF = F * kKS;            // elements per stage
  static constexpr int XBUF = TM * kKS;
  static constexpr int LDS_ELEMS = 2 * (WBUF + XBUF);
  static constexpr int WBLK = F * 8 / 64;         // 1 KB blocks per weight stage
  static constexpr int XBLK = TM * 8 / 64;
  static constexpr int WBW = WBLK / kWaves, XBW = XBLK / kWaves;   // blocks per wave
  static constexpr int FT = F / 2 / 16;           // 16-feature tiles per wave
  static constexpr int TQ = TM / 4;               // tokens per wave
  static constexpr int TT = TQ / 16;              // 16-token tiles per wave
  static_assert(WBLK % kWaves == 0 && XBLK % kWaves == 0, "blocks split evenly over the waves");

  // Row (within the F weight rows, or the 256 tokens) and 16-byte chunk
  // (0..7 of a 64-wide slice) that this lane fetches for its i-th block.
  __device__ static void w_slot(int i, int* row, int* chunk) {
    const int sl = 64 * ((int)(threadIdx.x >> 6) + kWaves * i) + (int)(threadIdx.x & 63);
    *row = sl >> 3;
    *chunk = (sl & 7) ^ (*row & 7);
  }
  __device__ static void x_slot(int i, int* row, int* chunk) { w_slot(i, row, chunk); }

  // acc += W x^T over K (a multiple of 64).  w_off / x_off: element offsets
  // (slice start excluded) of this lane's chunks from wg / xg.
  __device__ static void run(const uint16_t* wg, const uint32_t (&w_off)[WBW], const uint16_t* xg,
                             const uint32_t (&x_off)[XBW], int K, uint16_t* lds,
                             f32x4 (&acc)[FT][TT]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane & 15, g4 = lane >> 4;
    const int wf = wave & 1, wt = wave >> 1;
    auto Wb = [&](int s) { return lds + s * (WBUF + XBUF); };
    auto Xb = [&](int s) { return lds + s * (WBUF + XBUF) + WBUF; };
    auto load_stage = [&](int s, int k0) {
#pragma unroll
      for (int i = 0; i < WBW; ++i) lds_direct16(wg + w_off[i] + k0, &Wb(s)[512 * (wave + kWaves * i)]);
#pragma unroll
      for (int i = 0; i < XBW; ++i) lds_direct16(xg + x_off[i] + k0, &Xb(s)[512 * (wave + kWaves * i)]);
    };
    // rows of a lane's tiles differ by multiples of 16, so r & 7 = j & 7
    const int swz = j & 7;
    const int wrow0 = (F / 2) * wf + j, xrow0 = TQ * wt + j;
#pragma unroll
    for (int f = 0; f < FT; ++f)
#pragma unroll
      for (int t = 0; t < TT; ++t) acc[f][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nks = K / kKS;
    load_stage(0, 0);
    wait_vmem();
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
      const int s = ks & 1;
      if (ks + 1 < nks) load_stage(s ^ 1, (ks + 1) * kKS);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int cofs = 8 * ((g4 + 4 * kk) ^ swz);
        u32x4 A[FT], Bx[TT];
#pragma unroll
        for (int f = 0; f < FT; ++f) A[f] = ld16(&Wb(s)[(wrow0 + 16 * f) * kKS + cofs]);
#pragma unroll
        for (int t = 0; t < TT; ++t) Bx[t] = ld16(&Xb(s)[(xrow0 + 16 * t) * kKS + cofs]);
#pragma unroll
        for (int f = 0; f < FT; ++f)
#pragma unroll
          for (int t = 0; t < TT; ++t) acc[f][t] = mfma16x16x32(A[f], Bx[t], acc[f][t]);
      }
      wait_vmem();
      __syncthreads();
    }
  }
};

}  // namespace sa_gemm
