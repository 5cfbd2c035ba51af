// Launch interface of the attention kernels (prefill, decode, fp32 rows),
// kept apart from the other launchers so that a change elsewhere does not
// touch what the attention kernels are built from.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef SA_MAX_HALF
#define SA_MAX_HALF 128   // d_h <= 256
#endif

struct AttnArgs {
  const void* q;        // [B, T_q, n_q, d]
  const void* kc;       // [B, C, n_kv, d]
  const void* vc;       // [B, C/32, n_kv, d, 32]
  const float* sinks;   // [n_q]
  void* out;            // [B, T_q, n_q, d]
  int B, T_q, n_q, n_kv, d, q_mult, window;
  int64_t C;            // capacity (rows)
  int64_t q_offset;     // cache row of query 0 (its global position minus
                        //   the cache's base; masks use row differences)
  float sm_scale;
};
struct RopeTab {         // YaRN tables for rotating Q inside the prefill kernel
  int64_t pos_base;     // global position of cache row 0 (q_offset is a row)
  double conc;
  double inv_freq[SA_MAX_HALF];
};
// rope == nullptr: q is already rotated; otherwise q holds unrotated rows and
// the kernel rotates them at their positions first (yarn_rope's arithmetic).
hipError_t launch_prefill_bf16(const AttnArgs& a, const RopeTab* rope, hipStream_t s);
hipError_t launch_attn_rows_f32(const AttnArgs& a, hipStream_t s);
