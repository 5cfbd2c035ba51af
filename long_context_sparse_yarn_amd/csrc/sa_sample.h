// Launch arguments of the sampling kernels (sample.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sinkattn.h"

constexpr int kSampleChunk = 4096;      // vocabulary entries per prep / histogram workgroup
constexpr int kSampleBuckets = 4096;    // first-level histogram: the top 12 bits of the key
constexpr int kSampleHist = kSampleBuckets + 64;   // then 64 sums of 64 buckets
constexpr int kSampleMaxV = 64 * 4096;  // the draw keeps one mass per 64 ids in LDS
constexpr int kSampleCap = 4096;        // candidates sorted in LDS

struct SampleArgs {
  const float* logits;
  int64_t logits_stride;
  const float* bias;                    // null: no bias
  int64_t bias_stride;                  // 0: one row shared by the batch
  int32_t* counts;                      // [B, V] or null
  const sa_sample_params* params;       // [B]
  const float* u;                       // [B]
  int32_t* tokens;                      // [B]
  int32_t* n_kept;                      // [B] or null
  float* processed;                     // [B, V] or null
  // workspace
  float* zp;                            // [B, zs] processed logits
  int64_t zs;                           // row stride of zp: V rounded up to 64
  float* chunk_max;                     // [B, C]
  int32_t* chunk_arg;                   // [B, C]
  uint32_t* hist_count;                 // [B, kSampleHist]
  unsigned long long* hist_mass;        // [B, kSampleHist]
  unsigned long long* cand;             // [B, kSampleCap] candidates (key << 32 | ~id)
  uint32_t* ncand;                      // [B]
  unsigned long long* chunk_mass;       // [B, C] mass of each chunk
  unsigned long long* chunk_kmass;      // [B, C] mass of each chunk above the edge bucket
  int B, V, C;
  int hist_cpw;                         // chunks per histogram workgroup
  int update_counts;
};

hipError_t launch_sample(const SampleArgs& a, hipStream_t s);
hipError_t launch_sample_count(const int32_t* ids, int B, int H, int64_t ids_stride, int32_t* counts,
                               int V, hipStream_t s);
