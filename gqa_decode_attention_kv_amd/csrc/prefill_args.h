// Interface between the C-ABI host code (api.cpp) and the chunk (prefill)
// attention kernel (prefill_attn.hip).  Passed to the kernel by value.
#pragma once

#include "launch.h"

namespace uaii {

// Chunk attention (prefill): the T chunk queries of sequence b sit at
// positions len[b] - T .. len[b] - 1, their keys already in the cache; query
// t attends the keys [lo_t, len[b] - T + t] (lo_t from the window).
struct PrefillArgs {
  int32_t H, Hkv, cap, T, window;
  const void* k;
  const void* v;
  const float* q;      // [B][T][H][D], rotated queries
  const float* sinks;  // [H] or nullptr
  float* out;          // [B][T][H][D]
  float q_mul;         // multiplies q on load: scale*log2(e), or scale with a softcap
  float softcap;
  const float* k_scale;  // int8 keys: [.][Hkv][cap] per-token scales, or nullptr
  const float* v_scale;  // int8 values: the same, or nullptr
  const int32_t* block_table;  // paged cache, or nullptr
  int32_t block_size, log2_bs, max_blocks, num_blocks;
  int32_t len[kMaxBatch];
};

// One work-group per (64 or 128 query rows, kv head, sequence).  Caches:
// bf16 K and V, vq8 (bf16 K, int8 V), q8 (int8 K and V), or f32 K and V
// (head dim 64 or 128).
hipError_t launch_prefill_attn(int D, int G, int B, int k_dtype, int v_dtype, const PrefillArgs& a,
                               hipStream_t stream);
hipError_t launch_prefill_bf16(int D, int G, int B, const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_vq8(int D, int G, int B, const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_q8(int D, int G, int B, const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(int D, int G, int B, const PrefillArgs& a, hipStream_t stream);

}  // namespace uaii
