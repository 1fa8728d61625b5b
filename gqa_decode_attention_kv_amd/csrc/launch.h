// Internal interface between the C-ABI host code (api.cpp) and the HIP
// kernels.  Everything here is passed to kernels by value: the library
// allocates nothing, and its only device-side state is the static scratch
// array of uaii_decode_step_noalloc (decode_step_noalloc.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace uaii {

constexpr int kMaxBatch = 32;
constexpr int kMaxPairs = 128;  // rotation pairs of the largest head (d = 256)

enum : int { kF32 = 0, kBF16 = 1, kI8 = 2 };
enum : int { kNeox = 0, kInterleaved = 1 };

// Per-sequence schedule of one decode step.  Sequence b has splits
// first_split[b] .. first_split[b] + n_b - 1, n_b = work_prefix[b + 1] -
// work_prefix[b] (the splits that hold visible keys, [lo[b], len[b])).
//
// Launch order of the partial kernel's work index w, longest first: the
// "body" splits (all but the last of each sequence, whole splits apart from
// a window's first one) come first, sequence by sequence, w in
// [body_prefix[b], body_prefix[b + 1]) being split first_split[b] + w -
// body_prefix[b]; then the last splits, which ragged lengths leave short,
// w = body_prefix[n_seq] + k being the last split of sequence tail_order[k]
// (sequences by the last split's visible keys, most first).  The hardware
// dispatches work-groups in order, so the short items fill in at the end.
struct SeqTable {
  int32_t n_seq;
  int32_t work_prefix[kMaxBatch + 1];
  int32_t first_split[kMaxBatch];
  int32_t lo[kMaxBatch];
  int32_t len[kMaxBatch];
  int32_t body_prefix[kMaxBatch + 1];
  int32_t tail_order[kMaxBatch];
};

struct ProduceArgs {
  int32_t B, H, Hkv, D;
  int32_t pairing;
  // Rotary frequency g_i of pair i (plain, Llama-3, linear or YaRN), the same
  // for every token of a call, so the host evaluates the scheme once.
  double freq[kMaxPairs];
  // The factor that multiplies the rotated q and k (YaRN; 1 otherwise).
  double attn_factor;
  int32_t norm_enabled, norm_offset;
  float norm_eps;
  const float* w_q;
  const float* w_k;
  const float* q_in;
  const float* k_in;
  const float* v_in;
  int32_t k_dtype, v_dtype, cap;
  void* k;
  void* v;
  float* k_scale;  // q8 keys
  float* v_scale;  // vq8 / q8 values
  float* q_out;
  // Paged cache (block_table != nullptr): slot p of (b, u) is row p % bs of
  // physical block block_table[b][p / bs], pools [num_blocks][Hkv][bs][D].
  const int32_t* block_table;
  int32_t block_size, max_blocks, num_blocks;
  // Tokens per sequence: q_in, q_out [B][T][H][D], k_in, v_in [B][T][Hkv][D];
  // token t of sequence b sits at position pos[b] + t.  T = 1 for decode.
  int32_t T;
  // Head vectors per wave of the standalone producer: the wave evaluates the
  // token's rotation angles once and applies them to hpw consecutive heads.
  int32_t hpw;
  int32_t pos[kMaxBatch];
};

struct AttnArgs {
  int32_t H, Hkv, cap, split_size, max_splits;
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  const float* q;
  float* part_o;
  float* part_lse;
  float q_mul;    // multiplies q on load: scale*log2(e), or scale with a softcap
  float softcap;  // c > 0, or 0 for none
  // Paged cache only (see ProduceArgs); log2_bs = log2(block_size).
  const int32_t* block_table;
  int32_t block_size, log2_bs, max_blocks, num_blocks;
  // 0: each wave of a work-group takes its own work item.  1: the four
  // waves of a work-group share one item, a quarter of its rows each, and
  // merge their softmax states in LDS (more waves in flight for small steps).
  int32_t coop;
  // 1: the work-groups of a step with one wave per item and items of unequal
  // size take the work table's longest-first order in serpentine rounds of
  // kCUs work-groups (see decode_partial_kernel.h); 0: in order.
  int32_t serp;
  SeqTable t;
};

// Steps with fewer (split, kv head) work items than this run cooperatively:
// four waves per item keep more loads in flight when the grid alone would
// leave most of the 1024 SIMDs idle.
#ifndef UAII_COOP_BELOW
#define UAII_COOP_BELOW 2048
#endif
constexpr int kCoopBelow = UAII_COOP_BELOW;

// Compute units of an MI355X: the hardware hands out work-groups to them in
// turn, so work-group position p of a launch lands on CU p mod kCUs.
constexpr int kCUs = 256;

// uaii_decode_step runs as one kernel up to this many (split, kv head) work
// items, and as the three kernels back to back above it.  In one kernel,
// every split's partial must be released at device scope before the last
// split combines it: on gfx950 that is an L2 write-back per work item,
// which costs more than two kernel boundaries once there are more than a
// few hundred items.
#ifndef UAII_STEP_ONE_LAUNCH_MAX
#define UAII_STEP_ONE_LAUNCH_MAX 256
#endif
constexpr int kStepOneLaunchMax = UAII_STEP_ONE_LAUNCH_MAX;

struct CombineArgs {
  int32_t H, max_splits;
  const float* part_o;
  const float* part_lse;
  const float* sinks;  // [H] attention-sink logits, or nullptr
  float* out;
  SeqTable t;
};

// The fused decode step: the producer, the partials and the combine in one
// launch (see decode_partial_kernel.h).  a.q is unused (the queries are
// computed in the kernel) and p.pos is unused (the new token of sequence b
// sits at slot a.t.len[b] - 1).
struct StepArgs {
  AttnArgs a;
  ProduceArgs p;
  const float* sinks;  // [H] attention-sink logits, or nullptr
  float* out;
  int32_t* counters;   // [B][Hkv] arrival counters: zero on entry, zero on exit
};

// Static scratch of uaii_decode_step_noalloc, one array per GPU: the
// arrival counters in [0, kNoAllocCounterBytes), then the split partials
// (part_lse, then part_o, each starting on a 256-byte boundary), at most
// kNoAllocScratchBytes in all.
constexpr int kNoAllocCounterWords = 16384;
constexpr size_t kNoAllocCounterBytes = static_cast<size_t>(kNoAllocCounterWords) * 4;
constexpr size_t kNoAllocScratchBytes = (static_cast<size_t>(16) << 20) + kNoAllocCounterBytes;

// The current GPU's scratch address (hipGetSymbolAddress, taken once per
// device); the first call on a device also enqueues a kernel on `stream`
// that zeroes the counters.
hipError_t noalloc_scratch(void** base, hipStream_t stream);

hipError_t launch_kv_produce(const ProduceArgs& a, hipStream_t stream);

// One wave per (work item, kv head): t.work_prefix[t.n_seq] * Hkv waves.
hipError_t launch_decode_partial(int D, int G, int k_dtype, int v_dtype, const AttnArgs& a,
                                 hipStream_t stream);
hipError_t launch_decode_partial_paged(int D, int G, int k_dtype, int v_dtype, const AttnArgs& a,
                                       hipStream_t stream);
hipError_t launch_decode_combine(int D, int B, const CombineArgs& a, hipStream_t stream);
// One wave per (work item, kv head), as launch_decode_partial.
hipError_t launch_decode_step(int D, int G, int k_dtype, int v_dtype, const StepArgs& s, hipStream_t stream);
hipError_t launch_decode_step_paged(int D, int G, int k_dtype, int v_dtype, const StepArgs& s,
                                    hipStream_t stream);

}  // namespace uaii
