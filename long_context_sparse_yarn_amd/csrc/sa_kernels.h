// Internal launch interface between the C ABI (sinkattn_abi.hip) and the
// kernel translation units.  Every launcher enqueues on `s` and returns the
// HIP error of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define SA_MAX_HALF 128   // d_h <= 256

#include "sa_attn.h"

struct RopeArgs {
  const void* src;      // rows read from here ...
  void* x;              // ... and written here (may be the same buffer)
  int64_t offset;
  int BT, T, H, d;
  double conc;
  double inv_freq[SA_MAX_HALF];
};
hipError_t launch_rope(const RopeArgs& a, int elt_bytes, hipStream_t s);

struct AppendArgs {
  const void* k_src;    // [B, src_T, n_kv, d]
  const void* v_src;
  void* kc;
  void* vc;
  int B, T_new, n_kv, d;
  int64_t C, o;         // cache rows [o, o + T_new) receive source rows
  int src_T, src_t0;    //   [src_t0, src_t0 + T_new) of each sequence
  int64_t pos0;         // global position of cache row o (for the rotation)
};
hipError_t launch_append(const AppendArgs& a, int elt_bytes, hipStream_t s);

// Copy the rows of positions [p0, p0 + n) from one cache to another (K rows
// and blocked V).  Each side maps a position to a row: a ring holds p at
// row p mod C, a linear cache at row p - base.
struct CopyRowsArgs {
  const void* ks;
  const void* vs;
  void* kd;
  void* vd;
  int64_t Cs, Cd;       // capacities (rows, multiples of 32)
  int64_t base_s, base_d;
  int ring_s, ring_d;
  int64_t p0;
  int n;
  int B, n_kv, d;
};
hipError_t launch_copy_rows(const CopyRowsArgs& a, int elt_bytes, hipStream_t s);

struct AppendRopeArgs {  // rotate K rows at their cache positions, then append
  AppendArgs ap;         // k_src holds unrotated rows
  const void* q_src;     // optional [B, src_T, n_q, d]: rotated at the same
  void* q_dst;           //   positions into q_dst (may be q_src); null: none
  int n_q;
  double conc;
  double inv_freq[SA_MAX_HALF];
};
hipError_t launch_append_rope(const AppendRopeArgs& a, int elt_bytes, hipStream_t s);

// Fused qkv projection with the RoPE + append epilogue.
struct QkvArgs {
  const void* x;        // [B*T, d_model] bf16 (hidden states after the norm)
  const void* w;        // [d_qkv, d_model] bf16, d_qkv = d (n_q + 2 n_kv)
  const void* bias;     // [d_qkv] bf16
  void* q_rot;          // [B, T, n_q, d] bf16
  void* kc;             // cache K [B, C, n_kv, d]
  void* vc;             // cache V [B, C/32, n_kv, d, 32]
  double2* tab;         // workspace [T][d/2]: (c cos, c sin) at position pos0 + t
  int B, T, d_model, n_q, n_kv, d;
  int64_t C;            // cache capacity (rows)
  int64_t row0;         // cache row of token 0
  int64_t pos0;         // global position of token 0
  double conc;
  double inv_freq[SA_MAX_HALF];
};
hipError_t launch_qkv_rope_append(const QkvArgs& a, hipStream_t s);

// MoE layer: router, dispatch, experts, combine.
struct MoeArgs {
  const void* x;          // [N, d_model] bf16
  const void* w_router;   // [E, d_model] bf16
  int N, d_model, E, k;   // E <= 64, k <= 8
  void* logits;           // [N, E] bf16
  int32_t* ids;           // [N, k]
  float* weights;         // [N, k]
  int32_t* counts;        // [blocks of 256 tokens, E]
  int32_t* offsets;       // [blocks, E]
  int32_t* expert_start;  // [E + 1]
  int32_t* tile_start;    // [E + 1]: first 256-row tile of each expert
  int32_t* rows;          // [N * k]: token * k + slot, by expert then token
  float* out_slots;       // [N, k + 1, d_model]: weighted expert outputs (slot k: shared)
  void* y;                // [N, d_model] bf16
};
struct MoeGroup {         // one set of SwiGLU experts
  const void* w13;        // [E, 2 ffn, d_model]: gate rows, then up rows
  const void* w2;         // [E, d_model, ffn]
  void* h;                // [rows, ffn] bf16 scratch
  int ffn;
  int shared;             // 1: one expert over every token, weight 1, slot k
};
hipError_t launch_moe_route(const MoeArgs& a, hipStream_t s);
hipError_t launch_moe_dispatch(const MoeArgs& a, hipStream_t s);
// combine: the shared group's down pass also sums the routed slots into y
hipError_t launch_moe_experts(const MoeArgs& a, const MoeGroup& g, bool combine, hipStream_t s);
hipError_t launch_moe_combine(const MoeArgs& a, int nslots, hipStream_t s);


struct DecodeArgs {
  AttnArgs at;          // T_q == 1, q_offset == cache offset - 1
  float* ws;            // workspace (fp32)
  int n_splits;
};
int decode_splits(int B, int n_kv, int64_t span_rows);
int decode_max_splits(int B, int n_kv, int64_t capacity);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);

// A whole decode step in the attention launch: the token's Q and K rotated
// at its position, its K/V row written to the cache, and attention over the
// cache with that row in it.  DecodeArgs.at.q is unused (q_raw holds Q).
struct StepArgs {
  const void* q_raw;    // [B, n_q, d] unrotated
  void* q_rot;          // optional [B, n_q, d]: receives the rotated Q (null: not written)
  const void* k_raw;    // [B, n_kv, d] unrotated
  const void* v_raw;    // [B, n_kv, d]
  int64_t row;          // cache row that receives the token (same numbering as at.q_offset)
  int64_t pos;          // the token's global position (its rotation angle)
  double conc;
  double inv_freq[SA_MAX_HALF];
};
hipError_t launch_decode_step_bf16(const DecodeArgs& a, const StepArgs& st, hipStream_t s);
