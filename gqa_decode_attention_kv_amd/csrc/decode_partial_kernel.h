// Kernel template shared by decode_partial.hip (contiguous caches) and
// decode_partial_paged.hip (paged caches); each translation unit
// instantiates one addressing mode.
//
// Split-K flash-decoding partials for grouped-query attention, one query
// token per sequence, over B <= 32 ragged sequences.
//
// Sources: "Algenta - Model support matrix" (Kernel path capabilities:
// split-K decode partials, batched decode partial with B <= 32; Structural
// fact requirements: GQA ratio, attention scale 1/sqrt(head_dim));
// "Universal AI Inference - Hugging Face decoder completeness" (P1.4:
// sliding window and attention-logit softcap as a tanh clip); "llamay -
// Models and formats" (The KV cache, in three precisions: vq8 values, q8
// keys and values).
//
// Design (gfx950, bandwidth bound: one query row per kv head is a GEMV with
// 2-5 flop per KV byte, far below the ridge; the bf16 and f32 kernels run
// it on the vector ALUs, the int8-value kernels on the matrix cores, which
// takes the code widening and the per-element FMAs off the vector ALUs):
//   * one wave64 per (sequence, kv head, split) work item, taken from a
//     flattened per-sequence work table, so ragged batches and windows only
//     launch waves that hold visible keys; four independent waves share a
//     work-group but never synchronise (no barriers, no cross-wave merge).
//     The table launches the items longest first (every sequence's body
//     splits, then the last splits by decreasing length);
//   * steps with fewer than 2048 items run cooperatively instead: the four
//     waves of a work-group share one item, interleaving row blocks (one
//     load's rows on contiguous caches, 16 rows on paged ones) so that the
//     work-group reads the split as one sequential stream, and merge their
//     softmax states in LDS;
//   * the G query heads that share the kv head are held in registers, so
//     every K and V byte is read from HBM exactly once per group;
//   * int8 values on the vector pass use 8-byte loads (see Elem);
//   * a wave walks its split in chunks of up to 512 rows with two passes per
//     chunk: K (coalesced 16-byte loads, a row spread over d*sizeof(K)/16
//     lanes, scores reduced across those lanes with DPP) with raw scores
//     parked in LDS, then V with the softmax weights broadcast from LDS; the
//     running max and sum rescale only between chunks;
//   * scores live in the log2 domain (q pre-multiplied by scale*log2 e) so the
//     exponential is one v_exp_f32; with a softcap the tanh clip is applied
//     in the weights pass (it is monotonic, so the max commutes with it);
//   * int8 values (vq8, q8), and groups of eight heads up to d128: the key
//     pass on the matrix cores (key_mfma below), and with int8 values of
//     groups of 2, 4 or 8 heads, or bf16 values of groups of eight, up to
//     d128, the value pass too (value_mfma);
//     the key's per-token scale is applied to the raw score once per row,
//     where the chunk max is taken, and the value's is folded into the
//     softmax weight;
//   * other int8 caches: codes are widened in registers (as code + 128), the
//     128 * sum offsets removed once per row (keys) or at the end (values);
//   * at the end the wave sums its row groups across lanes and writes one
//     normalised partial and its log-sum-exp per query head.
// Loads run as a rolling pipeline (the next tiles are requested as soon as
// the current one is widened, and the first value tiles before the softmax
// weights are computed).  Every load addresses a row inside the visible
// range (rows past a chunk's end are clamped to its last row and masked
// afterwards), so memory outside the visible keys is never read and masked
// lanes never touch poisoned values.
#pragma once

#include <math.h>

#include <type_traits>

#include "combine_math.h"
#include "launch.h"
#include "producer_math.h"

namespace uaii {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;                  // independent waves per work-group
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerChunk = 512;         // rows a wave scores before it reads values
constexpr int kLoadsInFlight = 8;          // 16-byte loads per lane kept in flight (or
                                           // twice as many 8-byte loads)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int CTRL>
__device__ inline float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in {4, 8, 16, 32, 64}); every lane of
// a group receives the group's sum.
template <int N>
__device__ inline float group_sum(float x) {
  x += dpp<0xB1>(x);                        // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);                        // quad_perm [2,3,0,1]: lane ^ 2
  if constexpr (N >= 8) x += dpp<0x141>(x);   // row_half_mirror: pairs the quads of 8
  if constexpr (N >= 16) x += dpp<0x140>(x);  // row_mirror: pairs the halves of 16
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// group_sum over G independent values, stage by stage, so consecutive DPP
// operations read registers written G instructions earlier (no hazard stalls).
template <int N, int G>
__device__ inline void group_sum_n(float (&x)[G]) {
#pragma unroll
  for (int g = 0; g < G; ++g) x[g] += dpp<0xB1>(x[g]);
#pragma unroll
  for (int g = 0; g < G; ++g) x[g] += dpp<0x4E>(x[g]);
  if constexpr (N >= 8) {
#pragma unroll
    for (int g = 0; g < G; ++g) x[g] += dpp<0x141>(x[g]);
  }
  if constexpr (N >= 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) x[g] += dpp<0x140>(x[g]);
  }
  if constexpr (N >= 32) {
#pragma unroll
    for (int g = 0; g < G; ++g) x[g] += __shfl_xor(x[g], 16);
  }
  if constexpr (N >= 64) {
#pragma unroll
    for (int g = 0; g < G; ++g) x[g] += __shfl_xor(x[g], 32);
  }
}

__device__ inline float wave_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ inline float wave_sum(float x) { return group_sum<64>(x); }

// KV rows are read once per step: non-temporal loads stream them past the
// caches instead of evicting reusable lines (worth about 8% of bandwidth).
template <int NB>
using vec_t = typename std::conditional<NB == 16, u32x4, u32x2>::type;

template <int NB>
__device__ inline vec_t<NB> load_nt(const void* p) {
  return __builtin_nontemporal_load(static_cast<const vec_t<NB>*>(p));
}

// Score in the log2 domain from a raw score: with a softcap c the raw score is
// the natural-scale s and the result is c*tanh(s/c)*log2(e); without one the
// raw score already carries the log2(e) factor.  Monotonic in s.
__device__ inline float capped_log2(float s, bool capped, float c, float c_inv) {
  return capped ? c * tanhf(s * c_inv) * kLog2e : s;
}

// Widen the bytes one lane loaded (16 for f32 / bf16, 8 for int8) to E floats.
template <int DT, int E, typename V>
__device__ inline void widen(const V& w, float (&out)[E]) {
  if constexpr (DT == kF32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) out[e] = __uint_as_float(w[e]);
  } else if constexpr (DT == kBF16) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      out[2 * e] = __uint_as_float(w[e] << 16);
      out[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
  } else {
    // int8 codes are widened as code + 128 (one v_cvt_f32_ubyte per code after
    // flipping the sign bits); for values the caller removes 128 * sum(p) at
    // the end, for keys 128 * sum(q) from each raw score.
#pragma unroll
    for (int e = 0; e < E; ++e)
      out[e] = static_cast<float>(((w[e >> 2] ^ 0x80808080u) >> (8 * (e & 3))) & 0xFFu);
  }
}

// Element size and the bytes one lane loads per row segment.  Keys use
// 16-byte loads (a wider segment means fewer cross-lane reduction steps per
// byte), except int8 keys with G = 8, whose 16 query entries per head would
// not fit in registers.  int8 values use 8-byte loads, so a lane
// accumulates 8 values per head: the accumulator keeps the bf16 layout
// instead of twice as many registers.
template <int DT>
struct Elem {
  static constexpr int bytes = DT == kF32 ? 4 : (DT == kBF16 ? 2 : 1);
  static constexpr int value_load = DT == kI8 ? 8 : 16;
  template <int G>
  static constexpr int key_load() { return (DT == kI8 && G >= 8) ? 8 : 16; }
};

// ---- key pass on the matrix cores ----------------------------------------
// Over caches with int8 values (where the vector pass is bound by the
// vector ALUs; with bf16 values it is bound by HBM and the staging below
// measured slower), and for groups of eight heads (whose vector pass spends
// eight products and a cross-lane reduction per key element), keys are
// scored 16 at a time on the matrix cores.  bf16 and int8 keys take groups
// of four heads per MFMA chain, one MFMA per 32 dims (bf16) or 64 dims
// (int8).
// The A operand holds the query group, row 4 h + t being term t of head h;
// the B operand is the 16 key rows, loaded as whole rows (1 KB per wave
// load), staged in LDS and read back so that lane l holds key l % 16, the
// 16 bytes of segment 4 s + l / 16 of its row for step s (dims taken in
// that order on both sides); lane l of the 16 x 16 result holds rows
// 4 (l / 16) + i of key l % 16, the terms of one head, which the lane adds.
// Keys are never widened, and the cross-lane reduction of the vector pass
// disappears.
//   * bf16 keys: q (f32) is cut into three bf16 terms whose sum is exactly q
//     (truncation leaves the low 16, then 8 significand bits), so every
//     product is exact and the sum runs in the f32 accumulator.
//   * int8 keys: q / sigma (sigma a power of two per head, |q / sigma| < 64)
//     is written as four base-128 int8 digits and multiplied by the codes
//     in exact i32 arithmetic; the digits leave out at most 2^-22 sigma of
//     each q.
//   * f32 keys (G = 8): v_mfma_f32_16x16x4_f32 with row h of the A operand
//     head h itself (rows past G zero), one MFMA per 4 dims: lane l takes
//     dims (d / 4) (l / 16) + s at step s on both sides, so its key operand
//     for four steps is one 16-byte LDS read; the result lane holds heads
//     4 (l / 16) + i of key l % 16.  The matrix core rounds each product
//     and each four-product sum (the vector pass fuses its multiply-adds);
//     four accumulator chains, added pairwise, keep the rounding per score
//     to d / 16 + 2 steps.
template <int D, int G, int KT, int VT>
constexpr bool key_mfma() {
  return ((KT == kBF16 || KT == kI8) && ((G <= 4 && VT == kI8) || (G == 8 && VT != kF32 && D <= 128))) ||
         (KT == kF32 && VT == kF32 && G == 8 && D <= 128);
}

// The value pass on the matrix cores: int8 values with G of 2, 4 or 8, and
// bf16 values with G = 8, d <= 128.
template <int D, int G, int KT, int VT>
constexpr bool value_mfma() {
  return key_mfma<D, G, KT, VT>() && D <= 128 && ((VT == kI8 && G >= 2) || (VT == kBF16 && G == 8));
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// Term t (0, 1, 2) of x as bf16 bits: term 0 + term 1 + term 2 == x exactly.
__device__ inline uint32_t bf16_term(float x, int t) {
  const uint32_t u = __float_as_uint(x);
  const float r1 = x - __uint_as_float(u & 0xFFFF0000u);  // the low 16 significand bits, exact
  const uint32_t u1 = __float_as_uint(r1);
  const float r2 = r1 - __uint_as_float(u1 & 0xFFFF0000u);  // at most 8 significant bits, exact
  return (t == 0 ? u : (t == 1 ? u1 : __float_as_uint(r2))) >> 16;
}

// Digit t (0..3) of y, |y| < 64, in base 128 with nearest-integer digits:
// y = d0 + d1 / 128 + d2 / 128^2 + d3 / 128^3 + e with |e| <= 2^-22 and every
// |d| <= 64.  Each step is exact in f32.
__device__ inline int i8_digit(float y, int t) {
  float d[4];
  d[0] = rintf(y);
#pragma unroll
  for (int i = 1; i < 4; ++i) {
    y = (y - d[i - 1]) * 128.0f;
    d[i] = rintf(y);
  }
  return static_cast<int>(t == 0 ? d[0] : (t == 1 ? d[1] : (t == 2 ? d[2] : d[3])));
}

// Kernel arguments: the partials alone, or the fused step (partials plus
// the producer's inputs, the sinks, the output and the arrival counters).
template <bool FUSED>
using KernelArgs = typename std::conditional<FUSED, StepArgs, AttnArgs>::type;

__host__ __device__ inline const AttnArgs& attn_of(const AttnArgs& a) { return a; }
__host__ __device__ inline const AttnArgs& attn_of(const StepArgs& s) { return s.a; }
__device__ inline const StepArgs* step_of(const AttnArgs&) { return nullptr; }
__device__ inline const StepArgs* step_of(const StepArgs& s) { return &s; }

// FUSED = false: the split-K partials of uaii_decode_attn.
// FUSED = true: the whole decode step of uaii_decode_step in one launch.
//   * Each wave computes its G query heads from q_in (norm, RoPE, in double
//     precision, exactly as the producer does) instead of loading q_out;
//     the wave of the first split also writes q_out.
//   * The wave whose split holds the new token's slot (the last one) stores
//     the new key and value in the cache format and keeps the stored values
//     in registers: its K and V passes read the cache rows before the slot,
//     and the new row is merged into the softmax afterwards.  No wave reads
//     a cache row that another wave of the same launch writes.
//   * After writing its partial, a wave takes a ticket from the arrival
//     counter of its (sequence, kv head); the last of that pair's splits to
//     arrive combines the G heads (with the optional sink) and returns the
//     counter to zero, so the counters need no clearing between launches.
//
// amdgpu_waves_per_eu(2, 8): at least two waves per SIMD.  Without the hint
// the allocator spends registers freely (the vq8 kernel spilled into AGPRs at
// one wave per SIMD); with it the bf16 d128 kernel fits three waves per SIMD.
// The paged d128 partial kernels (G <= 4, bf16 or f32 keys, values not on
// the matrix cores) are held to three waves per SIMD too: with half as many
// loads in flight (below) they fit without spilling, where the per-tile
// block lookups otherwise leave room for two.
template <int D, int G, int KT, int VT, bool PAGED, bool FUSED>
constexpr int min_waves() {
  return (PAGED && !FUSED && D == 128 && G <= 4 && KT != kI8 && !value_mfma<D, G, KT, VT>()) ? 3 : 2;
}

template <int D, int G, int KT, int VT, bool PAGED, bool FUSED, bool ILV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(min_waves<D, G, KT, VT, PAGED, FUSED>(), 8))) void
decode_partial_kernel(const KernelArgs<FUSED> args) {
  const AttnArgs& a = attn_of(args);
  const StepArgs* x = step_of(args);
  // Matrix key pass (key_mfma): a K tile is 16 rows, each lane loading KNL
  // 16-byte segments of one row; otherwise a tile is one wave load.
  constexpr bool KMF = key_mfma<D, G, KT, VT>();
  constexpr int KB = Elem<KT>::bytes, VB = Elem<VT>::bytes;
  constexpr int KLB = KMF ? 16 : Elem<KT>::template key_load<G>(), VLB = Elem<VT>::value_load;
  constexpr int KLPR = KMF ? 4 : D * KB / KLB;  // lanes per K row
  constexpr int KRPL = 64 / KLPR;               // K rows per tile
  constexpr int KNL = KMF ? D * KB / 64 : 1;    // loads per lane per K tile
  constexpr int KE = KLB / KB;                  // K elements per lane and load
  constexpr int KRB = D * KB;                   // bytes per key row
  constexpr int KSPR = KRB / 16;                // 16-byte segments per key row
  constexpr int KRPI = KRB <= 1024 ? 1024 / KRB : 1;  // key rows per 1 KB wave load
  constexpr int VLPR = D * VB / VLB;
  constexpr int VRPL = 64 / VLPR;
  constexpr int VE = VLB / VB;
  // Eight 16-byte loads per lane in flight (the same bytes in 8-byte loads);
  // half as many for G = 8, whose query and accumulator registers would
  // otherwise leave room for one wave per SIMD, and for paged caches, whose
  // tiles each carry their own block's base (more waves per SIMD instead;
  // measured better also for cooperative items, which leave two waves per
  // SIMD at most: B=32 ctx 8K 82.4% against 79.8% of 8 TB/s).
  constexpr int LF = (G >= 8 || PAGED) ? kLoadsInFlight / 2 : kLoadsInFlight;
  constexpr int LFK = LF * 16 / KLB, LFV = LF * 16 / VLB;
  constexpr int LFKT = (LFK / KNL > 0) ? LFK / KNL : 1;  // K tiles in flight
  // Rows per chunk: 512, or 256 for the matrix key pass at G = 8, whose
  // [row][G] scores and key staging would otherwise leave LDS for one
  // work-group per CU.
  constexpr int CH = (KMF && G == 8) ? kRowsPerChunk / 2 : kRowsPerChunk;
  constexpr int UK = (LFKT * KRPL <= CH) ? LFKT : CH / KRPL;
  constexpr int UV = (LFV * VRPL <= CH) ? LFV : CH / VRPL;
  // Paged caches align tiles to blocks, so a chunk's rows sit up to 15 rows
  // after the start of its LDS window.
  // Matrix value pass (int8 values, G of 2, 4 or 8, d <= 128): blocks of 64
  // keys, staged like the key tiles and read back transposed.
  constexpr bool VMF = value_mfma<D, G, KT, VT>();
  constexpr bool VMB = VMF && VT == kBF16;       // bf16 values: weights as two bf16 terms
  constexpr int VBK = VMB ? 32 : 64;             // keys per value block
  constexpr int VRPI = 1024 / (D * VB);          // value rows per 1 KB wave load
  constexpr int VNL = VMF ? VBK / VRPI : 1;      // loads per lane per value block
  constexpr int NT = D / 16;                     // 16-dim output tiles
  // Paged chunks align their value blocks to 16 rows, up to 63 rows before
  // the chunk.
  constexpr int kLdsRows = CH + (PAGED ? (VMF ? 64 : 16) : 0);
  constexpr int kStageBytes = (VMF && VBK * D * VB > 16 * KRB) ? VBK * D * VB : 16 * KRB;
  constexpr int kScaleRegs = (VT == kI8) ? (kLdsRows + 63) / 64 : 1;
  constexpr int kKScaleRegs = (KT == kI8) ? (kLdsRows + 63) / 64 : 1;
  static_assert(CH % (UK * KRPL) == 0 && CH % (UV * VRPL) == 0, "tiling");
  static_assert(KLPR >= 4 && VLPR >= 4, "row must span at least a quad");

  __shared__ __attribute__((aligned(16))) float smem[kWaves * kLdsRows * G];
  // Matrix key pass: per wave, one 16-row key tile staged between the
  // coalesced loads and the operand reads.
  __shared__ __attribute__((aligned(16))) uint32_t kstage[KMF ? kWaves * kStageBytes / 4 : 4];
  // Fused step: per-wave staging of one head vector in double precision.
  __shared__ double sxd[FUSED ? kWaves * D : 1];
  static_assert(!FUSED || kLdsRows * G >= (G + 1) * D, "query and value staging must fit a wave's LDS");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // Work item (work index w, kv head); w names (sequence, split).  Alone,
  // each wave of the work-group takes its own item; cooperatively, the
  // work-group takes one item and its waves (part = wave) share the split's
  // rows as described below, merged through LDS at the end.
  const bool coop = ILV || a.coop != 0;
  // Serpentine placement (serp: one wave per item, items of unequal size).
  // Work-group position p runs on CU p mod kCUs, and the work table lists
  // the items longest first, so in plain order the CUs of the first
  // positions of every round get the largest items of each round.  Taking
  // every other round of kCUs positions in reverse pairs them with the
  // smallest instead, which evens the work per CU (HBM bandwidth is shared
  // per CU).  The map is a permutation of the positions.
  int lg = static_cast<int>(blockIdx.x);
  if (!coop && a.serp != 0) {
    const int n = static_cast<int>(gridDim.x);
    const int rnd = lg / kCUs, j = lg % kCUs;
    const int in_rnd = min(kCUs, n - rnd * kCUs);
    lg = rnd * kCUs + ((rnd & 1) ? in_rnd - 1 - j : j);
  }
  const int item = coop ? lg : lg * kWaves + wave;
  const int part = coop ? wave : 0;
  const int total = a.t.work_prefix[a.t.n_seq] * a.Hkv;
  // Idle waves leave at once.  Cooperative work-groups leave as a whole (the
  // item is per work-group), so the one barrier below is reached by all or
  // none of a work-group's waves.
  if (item >= total) return;
  // Work index w in launch order (SeqTable): body splits, then last splits.
  const int kvh = item % a.Hkv;
  const int w = item / a.Hkv;
  const int n_body = a.t.body_prefix[a.t.n_seq];
  int b = 0, sigma = 0;
  if (w < n_body) {
    for (int i = 1; i < a.t.n_seq; ++i) b += (w >= a.t.body_prefix[i]) ? 1 : 0;
    sigma = a.t.first_split[b] + (w - a.t.body_prefix[b]);
  } else {
    b = a.t.tail_order[w - n_body];
    sigma = a.t.first_split[b] + (a.t.work_prefix[b + 1] - a.t.work_prefix[b]) - 1;
  }
  // Cache rows [r0, r1) are read.  The fused step leaves out the new
  // token's slot L - 1: the split that holds it (has_new) merges it from
  // registers after its last chunk, in the wave of part 0.
  const int L = a.t.len[b];
  const bool has_new = FUSED && (sigma + 1) * a.split_size >= L;
  int r0 = max(sigma * a.split_size, a.t.lo[b]);
  int r1 = min((sigma + 1) * a.split_size, FUSED ? L - 1 : L);
  // A wave walks rows [r0, r1) in chunks; row x of a chunk that starts at
  // row c is cache row chunk_row(c) + xrow(x).  Alone, a wave reads its rows
  // in order (chunk_row(c) = c, xrow(x) = x).  Cooperative work-groups split
  // the item among their four waves:
  //   * ILV: the waves interleave blocks of BR rows (wave `part` takes
  //     blocks part, part + 4, ...), so the work-group reads the split as
  //     one sequential stream, measured faster than four separate streams.
  //     Contiguous caches use the rows of one load as a block.  The wave's
  //     own rows become local rows [0, n), local row l being cache row
  //     R0 + 4 BR (l / BR) + BR part + l % BR.  Paged caches use 16-row
  //     blocks counted from the item's first row aligned down to 16 (Rb),
  //     so that a block never straddles a cache block; wave 0 starts at
  //     local row r0 - Rb (the rows before the item are never visible);
  //   * otherwise (the fused step): each wave takes a quarter in whole
  //     16-row tiles.
  constexpr bool PILV = PAGED && ILV;
  constexpr int BR = PAGED ? 16 : (KRPL > VRPL ? KRPL : VRPL);
  static_assert(!PILV || (16 % KRPL == 0 && 16 % VRPL == 0), "paged interleaving blocks hold whole tiles");
  const int R0 = r0;
  const int Rb = PILV ? (r0 & ~15) : r0;
  if (coop) {
    if constexpr (ILV) {
      const int first = r0 - Rb;                 // rows of the first block before the item
      const int N = max(r1 - r0, 0) + first;
      const int nb = (N + BR - 1) / BR;  // blocks of the item, the last one possibly partial
      const int mine = nb > part ? (nb - 1 - part) / kWaves + 1 : 0;
      int n = mine * BR;
      if (mine > 0 && (nb - 1) % kWaves == part) n -= nb * BR - N;
      r0 = part == 0 ? first : 0;
      r1 = max(n, r0);
    } else {
      const int N = max(r1 - r0, 0);  // this wave's quarter, in whole 16-row tiles (possibly empty)
      const int piece = ((N + kWaves - 1) / kWaves + 15) & ~15;
      r0 = min(r0 + part * piece, r1);
      r1 = min(r0 + piece, r1);
    }
  }
  // Chunk starts are multiples of CH local rows, hence of BR.
  auto chunk_row = [&](int c) -> int {
    if constexpr (ILV) {
      return R0 + kWaves * c + BR * part;
    } else {
      return c;
    }
  };
  auto xrow = [&](int x) -> int {
    if constexpr (ILV) {
      return x + static_cast<int>(static_cast<uint32_t>(x) / BR) * (BR * (kWaves - 1));
    } else {
      return x;
    }
  };
  const bool new_here = has_new && part == 0;

  // Contiguous: the (b, kvh) slab starts at row slab of the cache.  Paged:
  // row r lives in physical block block_table[b][r / bs] at offset r % bs.
  const int64_t slab = PAGED ? 0 : (static_cast<int64_t>(b) * a.Hkv + kvh) * a.cap;
  const char* kbase = static_cast<const char*>(a.k) + slab * (D * KB);
  const char* vbase = static_cast<const char*>(a.v) + slab * (D * VB);
  const float* sbase = (VT == kI8) ? a.v_scale + slab : nullptr;
  const float* ksbase = (KT == kI8) ? a.k_scale + slab : nullptr;

  // Vector key pass: the query group in registers, lane holding
  // q[h][kc*KE .. kc*KE + KE) for its K segment.  Matrix key pass: lane
  // loads segment kc of key row kr of each tile, and qa is the A operand.
  const int kr = KMF ? (lane & 15) : lane / KLPR, kc = KMF ? (lane >> 4) : lane % KLPR;
  const int vr = lane / VLPR, vc = lane % VLPR;
  float* sc = smem + wave * (kLdsRows * G);  // this wave's [row][G] scores / weights
  float q[KMF ? 1 : G][KMF ? 1 : KE];
  using AOp = typename std::conditional<KT == kI8, i32x4, bf16x8>::type;
  // Matrix key pass over bf16 and int8 keys: heads are handled in groups of
  // four (HG groups; G = 8 has two), one A operand and one MFMA chain per
  // group.  f32 keys take all G heads in one A operand (qk).
  constexpr bool KF32 = KMF && KT == kF32;
  constexpr int HG = KMF ? (KF32 ? 1 : (G + 3) / 4) : 1;
  AOp qa[KF32 ? 1 : HG][KF32 ? 1 : KNL];
  float qk[KF32 ? D / 4 : 1];  // f32 keys: q[lane % 16][(D / 4) (lane / 16) + s]
  (void)qk;
  float qsig[HG];  // int8 keys: sigma of this lane's output head 4 hg + kc
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) qsig[hg] = 1.0f;
  // A operand of head group hg from the G query rows at qsrc (row h at
  // qsrc + h D, scaled by q_mul here): lane (m, kc), m = lane % 16, holds
  // term / digit m % 4 of head 4 hg + m / 4 (zero past the group, and for
  // bf16 row 4 h + 3), dims 32 s + 8 kc + j (bf16) or 64 s + 16 kc + j
  // (int8) for step s.
  auto build_qa = [&](const float* qsrc) {
    if constexpr (KF32) {
      const int m = lane & 15;
      const float* qh = qsrc + min(m, G - 1) * D + (D / 4) * kc;
#pragma unroll
      for (int j = 0; j < D / 4; j += 4) {
        const float4 v = *reinterpret_cast<const float4*>(qh + j);
        qk[j] = m < G ? v.x * a.q_mul : 0.0f;
        qk[j + 1] = m < G ? v.y * a.q_mul : 0.0f;
        qk[j + 2] = m < G ? v.z * a.q_mul : 0.0f;
        qk[j + 3] = m < G ? v.w * a.q_mul : 0.0f;
      }
      return;
    }
#pragma unroll
    for (int hg = 0; hg < (KF32 ? 0 : HG); ++hg) {
      const int m = lane & 15, t = m & 3;
      const int h = 4 * hg + (m >> 2);
      const bool live = h < G && (KT == kI8 || t < 3);
      const float* qh = qsrc + min(h, G - 1) * D;
      constexpr int SD = KT == kI8 ? 16 : 8;  // dims per lane and step
      float x[KNL][SD];
#pragma unroll
      for (int st = 0; st < KNL; ++st)
#pragma unroll
        for (int j = 0; j < SD; j += 4) {
          const float4 v = *reinterpret_cast<const float4*>(qh + 4 * SD * st + SD * kc + j);
          x[st][j] = v.x * a.q_mul;
          x[st][j + 1] = v.y * a.q_mul;
          x[st][j + 2] = v.z * a.q_mul;
          x[st][j + 3] = v.w * a.q_mul;
        }
      if constexpr (KT == kI8) {
        float mx = 0.0f;
#pragma unroll
        for (int st = 0; st < KNL; ++st)
#pragma unroll
          for (int j = 0; j < SD; ++j) mx = fmaxf(mx, fabsf(x[st][j]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));  // max |q| of head m / 4
        const int ex = mx > 0.0f ? ilogbf(mx) - 5 : 0;  // |q| / 2^ex < 64
#pragma unroll
        for (int st = 0; st < KNL; ++st) {
          uint32_t w[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            uint32_t word = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const int dg = live ? i8_digit(ldexpf(x[st][4 * j + k], -ex), t) : 0;
              word |= (static_cast<uint32_t>(dg) & 0xFFu) << (8 * k);
            }
            w[j] = word;
          }
          qa[hg][st] = i32x4{static_cast<int32_t>(w[0]), static_cast<int32_t>(w[1]),
                             static_cast<int32_t>(w[2]), static_cast<int32_t>(w[3])};
        }
        qsig[hg] = __shfl(ldexpf(1.0f, ex), 4 * min(kc, G - 1 - 4 * hg));
      } else {
#pragma unroll
        for (int st = 0; st < KNL; ++st) {
          u32x4 w;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            w[j] = live ? (bf16_term(x[st][2 * j], t) | (bf16_term(x[st][2 * j + 1], t) << 16)) : 0u;
          qa[hg][st] = __builtin_bit_cast(bf16x8, w);
        }
      }
    }
  };
  float s_new[G];  // fused step: raw scores of the new token's row
  float vnew[VE];  // fused step: its stored value, this lane's V segment
  if constexpr (FUSED) {
    const ProduceArgs& p = x->p;
    constexpr int EPL = pm::Shape<D>::EPL, NP = pm::Shape<D>::NP;
    const int pos = L - 1;
    double* sx = sxd + wave * D;
    float* qs = sc;  // G rows of D floats: the rotated queries
    pm::Angles<D> an;
    pm::rope_angles<D>(p, pos, lane, an);
    const bool write_q = sigma == a.t.first_split[b] && part == 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int64_t hrow = static_cast<int64_t>(b) * a.H + kvh * G + g;
      float xin[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) xin[e] = p.q_in[hrow * D + lane + 64 * e];
      pm::Rotated<D> r;
      pm::norm_rope<D>(p, xin, p.w_q, an, sx, lane, r);
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        if (!r.ok[j]) continue;
        const float fa = static_cast<float>(r.ya[j]), fb = static_cast<float>(r.yb[j]);
        qs[g * D + r.ia[j]] = fa;
        qs[g * D + r.ib[j]] = fb;
        if (write_q) {
          p.q_out[hrow * D + r.ia[j]] = fa;
          p.q_out[hrow * D + r.ib[j]] = fb;
        }
      }
    }
    pm::wave_sync();
    if constexpr (KMF) {
      build_qa(qs);
    } else {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < KE; ++e) q[g][e] = qs[g * D + kc * KE + e] * a.q_mul;
    }
    if (new_here) {
      const int64_t krow = static_cast<int64_t>(b) * a.Hkv + kvh;
      float kin[EPL], vin[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        kin[e] = p.k_in[krow * D + lane + 64 * e];
        vin[e] = p.v_in[krow * D + lane + 64 * e];
      }
      pm::Rotated<D> r;
      pm::norm_rope<D>(p, kin, p.w_k, an, sx, lane, r);
      const int64_t slot = pm::cache_slot<D>(p, b, kvh, pos);
      float kst[2 * NP], vst[EPL];
      pm::store_key<D>(p, r, slot, lane, kst);
      pm::store_value<D>(p, vin, slot, lane, vst);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float t = 0.0f;
#pragma unroll
        for (int j = 0; j < NP; ++j) {
          if (!r.ok[j]) continue;
          t = fmaf(qs[g * D + r.ia[j]] * a.q_mul, kst[2 * j], t);
          t = fmaf(qs[g * D + r.ib[j]] * a.q_mul, kst[2 * j + 1], t);
        }
        s_new[g] = wave_sum(t);
      }
      float* vs = sc + G * D;  // the stored value row, then this lane's segment
#pragma unroll
      for (int e = 0; e < EPL; ++e) vs[lane + 64 * e] = vst[e];
      pm::wave_sync();
#pragma unroll
      for (int e = 0; e < VE; ++e) vnew[e] = vs[vc * VE + e];
      if constexpr (VMF) {
        // The matrix value pass reads the stored value row at the merge
        // (the prologue's staging row, free from here on, holds it).
        float* vkeep = reinterpret_cast<float*>(sx);
#pragma unroll
        for (int e = 0; e < EPL; ++e) vkeep[lane + 64 * e] = vst[e];
      }
    }
    pm::wave_sync();  // the staging area is the K pass's score buffer
  } else if constexpr (KMF) {
    build_qa(a.q + (static_cast<int64_t>(b) * a.H + kvh * G) * D);
  } else {
    const float* qb = a.q + (static_cast<int64_t>(b) * a.H + kvh * G) * D + kc * KE;
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int e = 0; e < KE; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(qb + g * D + e);
        q[g][e] = v.x * a.q_mul;
        q[g][e + 1] = v.y * a.q_mul;
        q[g][e + 2] = v.z * a.q_mul;
        q[g][e + 3] = v.w * a.q_mul;
      }
    }
  }
  (void)s_new;
  (void)vnew;
  (void)q;
  (void)qsig;
  // q8 keys in the vector pass: each raw score carries 128 * sum(q_h) from
  // the code offset (the matrix pass multiplies the signed codes).
  float c128[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    float t = 0.0f;
    if constexpr (KT == kI8 && !KMF) {
#pragma unroll
      for (int e = 0; e < KE; ++e) t += q[g][e];
    }
    c128[g] = t;
  }
  if constexpr (KT == kI8 && !KMF) {
    group_sum_n<KLPR, G>(c128);
#pragma unroll
    for (int g = 0; g < G; ++g) c128[g] *= 128.0f;
  }
  const bool capped = a.softcap > 0.0f;
  const float cap_c = a.softcap, cap_inv = capped ? 1.0f / a.softcap : 0.0f;

  // Vector value pass: acc[g][e] of this lane's value segment.  Matrix
  // value pass: vacc[s][T] = head vhead(s), dim 16 T + lane % 16,
  // complete (no reduction across lanes).
  float acc[VMF ? 1 : G][VMF ? 1 : VE];
#pragma unroll
  for (int g = 0; g < (VMF ? 1 : G); ++g)
#pragma unroll
    for (int e = 0; e < (VMF ? 1 : VE); ++e) acc[g][e] = 0.0f;
  // Heads per lane: int8 values 4 hg + kc (one per head group), bf16
  // values 2 kc and 2 kc + 1 (rows 4 kc .. 4 kc + 3 of the result are their
  // two weight terms).
  constexpr int VH = VMB ? 2 : HG;
  auto vhead = [&](int s) { return VMB ? 2 * kc + s : 4 * s + kc; };
  (void)vhead;
  float vacc[VMF ? VH : 1][VMF ? NT : 1];
#pragma unroll
  for (int hg = 0; hg < (VMF ? VH : 1); ++hg)
#pragma unroll
    for (int t = 0; t < (VMF ? NT : 1); ++t) vacc[hg][t] = 0.0f;
  (void)acc;
  (void)vacc;
  float m_run[G], l_run[G];
  float psum[G];  // int8 values: sum of the scaled weights this lane wrote (removes the +128)
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.0f;
    psum[g] = 0.0f;
  }

  for (int a0 = r0; a0 < r1; a0 += CH) {
    const int nrows = min(CH, r1 - a0);  // rows [a0, a0 + nrows), wave-uniform

    // Loads address a row clamped into [a0, last]: every load is
    // unconditional and in the visible range; rows outside are masked after
    // the load.  Addresses are a wave-uniform base plus a 32-bit lane offset.
    // Tiles start at TK0 / TV0 and LDS row x holds absolute row A + x.  A
    // contiguous chunk starts its tiles at a0; a paged one aligns them (and
    // A) down so that no tile straddles a block.
    const int last = a0 + nrows - 1;
    const int A = PAGED ? (a0 & ~15) : a0;
    const int TK0 = PAGED ? (a0 & ~(KRPL - 1)) : a0;
    const int TV0 = VMF ? A : (PAGED ? (a0 & ~(VRPL - 1)) : a0);
    const int nk = (a0 + nrows - TK0 + KRPL - 1) / KRPL;  // K tiles of KRPL rows
    constexpr int VTR = VMF ? VBK : VRPL;                   // rows per V tile
    const int nv = (a0 + nrows - TV0 + VTR - 1) / VTR;      // V tiles (matrix pass: blocks)
    const char* kblk = kbase + static_cast<int64_t>(chunk_row(a0)) * (D * KB);
    const char* vblk = vbase + static_cast<int64_t>(chunk_row(a0)) * (D * VB);
    // Paged: lane j holds the physical id of logical block j0 + j (a chunk
    // spans at most 512 / 16 + 1 blocks); ids outside the pool are clamped.
    // Interleaved (PILV): rows are local, lane j holds the id of the cache
    // block of the chunk's 16-row block j0 + j, and abs_row maps a local row
    // to its cache row.
    auto abs_row = [&](int R) -> int {
      if constexpr (PILV) {
        return Rb + (R >> 4) * (16 * kWaves) + 16 * part + (R & 15);
      } else {
        return R;
      }
    };
    auto blk_lane = [&](int R) -> int { return (PILV ? (R >> 4) : (R >> a.log2_bs)); };
    int j0 = 0, idreg = 0;
    if constexpr (PAGED) {
      j0 = blk_lane(a0);
      const int nb = blk_lane(last) - j0 + 1;
      const int jb = PILV ? (abs_row(16 * (j0 + min(lane, nb - 1))) >> a.log2_bs) : j0 + min(lane, nb - 1);
      const int id = a.block_table[static_cast<int64_t>(b) * a.max_blocks + jb];
      idreg = min(max(id, 0), a.num_blocks - 1);
    }
    // Wave-uniform start of a tile whose first row is R (its rows are
    // consecutive cache rows of one block).
    auto tile_base = [&](const void* pool, int R, int row_bytes) -> const char* {
      const int pid = __builtin_amdgcn_readlane(idreg, blk_lane(R) - j0);
      return static_cast<const char*>(pool) +
             ((static_cast<int64_t>(pid) * a.Hkv + kvh) * a.block_size + (abs_row(R) & (a.block_size - 1))) *
                 row_bytes;
    };
    auto kaddr = [&](int t) -> const char* {
      if constexpr (PAGED) {
        const int R = TK0 + t * KRPL;
        const int row = min(max(R + kr, a0), last);
        return tile_base(a.k, R, D * KB) + static_cast<uint32_t>((row - R) * (D * KB) + kc * KLB);
      } else {
        return kblk + static_cast<uint32_t>(xrow(min(t * KRPL + kr, nrows - 1)) * (D * KB) + kc * KLB);
      }
    };
    auto vaddr = [&](int t) -> const char* {
      if constexpr (PAGED) {
        const int R = TV0 + t * VRPL;
        const int row = min(max(R + vr, a0), last);
        return tile_base(a.v, R, D * VB) + static_cast<uint32_t>((row - R) * (D * VB) + vc * VLB);
      } else {
        return vblk + static_cast<uint32_t>(xrow(min(t * VRPL + vr, nrows - 1)) * (D * VB) + vc * VLB);
      }
    };

    // Per-token scale of LDS row x = lane + 64 i (clamped into the chunk).
    auto load_scale = [&](const float* pool, const float* contiguous, int i) -> float {
      if constexpr (PAGED) {
        const int row = min(max(A + lane + 64 * i, a0), last);
        const int pid = __shfl(idreg, blk_lane(row) - j0);
        return pool[(static_cast<int64_t>(pid) * a.Hkv + kvh) * a.block_size + (abs_row(row) & (a.block_size - 1))];
      } else {
        return contiguous[chunk_row(a0) + xrow(min(lane + 64 * i, nrows - 1))];
      }
    };
    // int8 caches: the chunk's per-token scales are requested now; key scales
    // are used where the chunk max is taken, value scales by the weights
    // pass.  LDS row x = lane + 64 i sits in register i.
    float sreg[kScaleRegs], ksreg[kKScaleRegs];
    if constexpr (VT == kI8) {
#pragma unroll
      for (int i = 0; i < kScaleRegs; ++i) sreg[i] = load_scale(a.v_scale, sbase, i);
    }
    if constexpr (KT == kI8) {
#pragma unroll
      for (int i = 0; i < kKScaleRegs; ++i) ksreg[i] = load_scale(a.k_scale, ksbase, i);
    }

    // ---- pass 1: raw scores of the chunk's rows (rolling prefetch) ----------
    // Rows past the chunk's end hold duplicates of its last row; the weights
    // pass ignores them.  Each tile's registers are reloaded as soon as the
    // tile has been widened.  The steady-state loop has no branches (every
    // tile and every reload is in range) so the compiler can count loads in
    // flight exactly; the last one or two batches run in a guarded tail.
    if constexpr (KMF) {
      // Matrix pass.  A tile of 16 rows is read as KNL wave loads of 1 KB
      // each (KRPI whole rows, fully coalesced: measured 15% faster than
      // loads that take 64 bytes of each of the 16 rows), staged in LDS
      // slot = lane, and read back in the operand layout (lane: row kr,
      // segment 4 st + kc for step st).  Within a row the segments are
      // permuted (XOR with a function of the row) so that those reads hit
      // distinct banks.  Each load is reissued for the tile UK ahead as soon
      // as it is staged.
      using COp = typename std::conditional<KT == kI8, i32x4, f32x4>::type;
      auto kswz = [](int rr) { return (rr ^ (rr >> (KRB == 64 ? 2 : 3))) & (KSPR - 1); };
      auto kaddr_mf = [&](int t, int st) -> const char* {
        const int rr = KRPI * st + lane / KSPR;  // row of the tile this lane loads
        const int seg = (lane % KSPR) ^ kswz(rr);
        if constexpr (PAGED) {
          const int R = TK0 + t * KRPL;
          const int row = min(max(R + rr, a0), last);
          return tile_base(a.k, R, KRB) + static_cast<uint32_t>((row - R) * KRB + 16 * seg);
        } else {
          return kblk + static_cast<uint32_t>(xrow(min(t * KRPL + rr, nrows - 1)) * KRB + 16 * seg);
        }
      };
      u32x4* stg = reinterpret_cast<u32x4*>(kstage) + wave * (kStageBytes / 16);
      u32x4 kd[UK][KNL];
      auto k_tile = [&](int u, int t_next, bool reload, int r) {
#pragma unroll
        for (int st = 0; st < KNL; ++st) {
          stg[64 * st + lane] = kd[u][st];
          if (reload) kd[u][st] = load_nt<16>(kaddr_mf(t_next, st));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        COp c[HG];
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) c[hg] = COp{0, 0, 0, 0};
        if constexpr (KF32) {
          // Segment KNL kc + st of row kr: dims 4 (KNL kc + st) + e, step
          // 4 st + e.  Four accumulators (one per e) added pairwise at the
          // end: each sum then takes KNL + 2 roundings instead of 4 KNL,
          // which keeps the scores as close as the vector pass's short
          // chains and reduction tree.
          COp ce[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) ce[e] = COp{0, 0, 0, 0};
#pragma unroll
          for (int st = 0; st < KNL; ++st) {
            const int seg = KNL * kc + st;
            const u32x4 kb = stg[64 * (kr / KRPI) + (kr % KRPI) * KSPR + (seg ^ kswz(kr))];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              ce[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(qk[4 * st + e], __uint_as_float(kb[e]), ce[e], 0, 0, 0);
          }
          c[0] = (ce[0] + ce[1]) + (ce[2] + ce[3]);
        }
#pragma unroll
        for (int st = 0; st < (KF32 ? 0 : KNL); ++st) {
          const int seg = 4 * st + kc;
          const u32x4 kb = stg[64 * (kr / KRPI) + (kr % KRPI) * KSPR + (seg ^ kswz(kr))];
#pragma unroll
          for (int hg = 0; hg < HG; ++hg) {
            if constexpr (KT == kI8) {
              c[hg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa[hg][st], __builtin_bit_cast(i32x4, kb), c[hg], 0, 0,
                                                            0);
            } else {
              c[hg] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hg][st], __builtin_bit_cast(bf16x8, kb), c[hg], 0,
                                                              0, 0);
            }
          }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if constexpr (KF32) {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * kc + i < G) sc[r * G + 4 * kc + i] = c[0][i];
        }
#pragma unroll
        for (int hg = 0; hg < (KF32 ? 0 : HG); ++hg) {
          float sv;
          if constexpr (KT == kI8) {
            constexpr float k7 = 1.0f / 128.0f;
            sv = fmaf(fmaf(fmaf(static_cast<float>(c[hg][3]), k7, static_cast<float>(c[hg][2])), k7,
                           static_cast<float>(c[hg][1])),
                      k7, static_cast<float>(c[hg][0])) *
                 qsig[hg];
          } else {
            sv = (c[hg][0] + c[hg][1]) + c[hg][2];
          }
          if (4 * hg + kc < G) sc[r * G + 4 * hg + kc] = sv;
        }
      };
#pragma unroll
      for (int u = 0; u < UK; ++u)
#pragma unroll
        for (int st = 0; st < KNL; ++st) kd[u][st] = load_nt<16>(kaddr_mf(min(u, nk - 1), st));
      const int kx0 = TK0 - A + kr;  // LDS row of tile 0 for this lane's output key
      int t0 = 0;
      for (; t0 + 2 * UK <= nk; t0 += UK) {
#pragma unroll
        for (int u = 0; u < UK; ++u) k_tile(u, t0 + UK + u, true, kx0 + (t0 + u) * KRPL);
      }
      for (; t0 < nk; t0 += UK) {
#pragma unroll
        for (int u = 0; u < UK; ++u)
          if (t0 + u < nk) k_tile(u, t0 + UK + u, t0 + UK + u < nk, kx0 + (t0 + u) * KRPL);
      }
    } else {
      vec_t<KLB> kd[UK];
      auto k_scores = [&](const float (&kf)[KE], int r) {
        float s[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float p = q[g][0] * kf[0];
#pragma unroll
          for (int e = 1; e < KE; ++e) p = fmaf(q[g][e], kf[e], p);
          s[g] = p;
        }
        group_sum_n<KLPR, G>(s);
        if (kc == 0) {
#pragma unroll
          for (int g = 0; g < G; ++g) sc[r * G + g] = s[g];
        }
      };
#pragma unroll
      for (int u = 0; u < UK; ++u) kd[u] = load_nt<KLB>(kaddr(min(u, nk - 1)));
      const int kx0 = TK0 - A + kr;  // LDS row of tile 0 for this lane
      int t0 = 0;
      for (; t0 + 2 * UK <= nk; t0 += UK) {
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          float kf[KE];
          widen<KT, KE>(kd[u], kf);
          kd[u] = load_nt<KLB>(kaddr(t0 + UK + u));
          k_scores(kf, kx0 + (t0 + u) * KRPL);
        }
      }
      for (; t0 < nk; t0 += UK) {
#pragma unroll
        for (int u = 0; u < UK; ++u) {
          if (t0 + u < nk) {
            float kf[KE];
            widen<KT, KE>(kd[u], kf);
            if (t0 + UK + u < nk) kd[u] = load_nt<KLB>(kaddr(t0 + UK + u));
            k_scores(kf, kx0 + (t0 + u) * KRPL);
          }
        }
      }
    }
    // First value tiles are in flight while the weights are computed.
    // Matrix value pass: load st of block t brings rows VRPI st + lane / CB
    // of the block, 16-byte column block lane % CB (1 KB per wave load).
    constexpr int CB = D * VB / 16;
    auto vaddr_mf = [&](int t, int st) -> const char* {
      const int rr = VRPI * st + lane / CB;
      const int col = 16 * (lane % CB);
      if constexpr (PAGED) {
        // A load's VRPI rows lie in one 16-row group, hence in one block; a
        // load wholly past the chunk reads its last row.
        const int R = min(TV0 + t * VBK + VRPI * st, last);
        const int row = min(max(R + lane / CB, a0), last);
        return tile_base(a.v, R, D * VB) + static_cast<uint32_t>((row - R) * (D * VB) + col);
      } else {
        return vblk + static_cast<uint32_t>(xrow(min(t * VBK + rr, nrows - 1)) * (D * VB) + col);
      }
    };
    vec_t<VLB> vd[VMF ? 1 : UV];
    u32x4 vdm[VMF ? VNL : 1];
    if constexpr (VMF) {
#pragma unroll
      for (int st = 0; st < VNL; ++st) vdm[st] = load_nt<16>(vaddr_mf(0, st));
    } else {
#pragma unroll
      for (int u = 0; u < UV; ++u) vd[u] = load_nt<VLB>(vaddr(min(u, nv - 1)));
    }
    (void)vd;
    (void)vdm;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // ---- chunk max (raw scores of valid rows, from LDS), running max, rescale
    float mloc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) mloc[g] = -INFINITY;
    const int xlo = a0 - A, xhi = a0 - A + nrows;  // LDS rows of the chunk's keys
    if constexpr (KT == kI8) {
      // Finish the raw scores in place, (dot - 128 sum q) * key scale; each
      // lane rewrites exactly the rows it reads again in the weights pass.
#pragma unroll
      for (int i = 0; i < kKScaleRegs; ++i) {
        const int r = lane + 64 * i;
        if (64 * i >= xhi) break;  // wave-uniform
        if (r >= xlo && r < xhi) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float sv = (sc[r * G + g] - c128[g]) * ksreg[i];
            sc[r * G + g] = sv;
            mloc[g] = fmaxf(mloc[g], sv);
          }
        }
      }
    } else {
      for (int r = xlo + lane; r < xhi; r += 64) {
#pragma unroll
        for (int g = 0; g < G; ++g) mloc[g] = fmaxf(mloc[g], sc[r * G + g]);
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float m_chunk = wave_max(mloc[g]);  // finite: the chunk has >= 1 row
      const float m_new = fmaxf(m_run[g], capped_log2(m_chunk, capped, cap_c, cap_inv));
      const float alpha = (m_run[g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[g] - m_new);
      l_run[g] *= alpha;
      if constexpr (VMF) {
#pragma unroll
        for (int hg = 0; hg < VH; ++hg)
          if (vhead(hg) == g) {
#pragma unroll
            for (int t = 0; t < NT; ++t) vacc[hg][t] *= alpha;
          }
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] *= alpha;
      }
      psum[g] *= alpha;
      m_run[g] = m_new;
    }

    // Matrix value pass, int8 values: the weights pv = p * vscale of the
    // chunk are written as four base-128 int8 digits of pv / 2^vex[g],
    // 2^vex[g] a power of two with the head's largest pv of the chunk /
    // 2^vex[g] in [32, 64), packed one word per row and head (digit t in
    // byte t).  The weights that carry the output thus keep their full
    // precision whatever the spread of the value scales.  The weights pass
    // leaves pv in LDS and its largest value per head in vmx; the digits
    // replace pv after it.  bf16 values: the weights pass writes each word
    // as the weight's two bf16 terms at once (no scale).
    int vex[G];
    float vmx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      vex[g] = 0;
      vmx[g] = 0.0f;
    }
    (void)vex;
    (void)vmx;

    // ---- weights p = 2^(s - m) for every row the value tiles cover (0 past
    // the end); vq8 folds the token's scale into p ---------------------------
    const int xend = TV0 - A + nv * VTR;  // LDS rows the value tiles read
#pragma unroll
    for (int i = 0; i < (kLdsRows + 63) / 64; ++i) {
      const int r = lane + 64 * i;
      if (64 * i >= xend) break;  // wave-uniform
      if (r < xend) {
        const bool ok = r >= xlo && r < xhi;
        const float vs = (VT == kI8) ? sreg[VT == kI8 ? i : 0] : 1.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float p =
              ok ? __builtin_amdgcn_exp2f(capped_log2(sc[r * G + g], capped, cap_c, cap_inv) - m_run[g]) : 0.0f;
          l_run[g] += p;
          const float pv = p * vs;
          if constexpr (VMB) {
            // bf16 values: the weight as its bf16 high part (low half of
            // the word) and the bf16 of the remainder (high half).
            const uint32_t hi = __builtin_bit_cast(uint16_t, static_cast<__bf16>(pv));
            const float rem = pv - __uint_as_float(hi << 16);
            const uint32_t lo = __builtin_bit_cast(uint16_t, static_cast<__bf16>(rem));
            reinterpret_cast<uint32_t*>(sc)[r * G + g] = hi | (lo << 16);
          } else {
            sc[r * G + g] = pv;
          }
          if constexpr (VMF && !VMB) {
            vmx[g] = fmaxf(vmx[g], pv);
          } else if constexpr (VT == kI8) {
            psum[g] += pv;
          }
        }
      }
    }
    if constexpr (VMF && !VMB) {
      // Each lane rewrites its own rows, so no wave barrier is needed here.
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mx = wave_max(vmx[g]);
        vex[g] = mx > 0.0f ? ilogbf(mx) - 5 : 0;
      }
#pragma unroll
      for (int i = 0; i < (kLdsRows + 63) / 64; ++i) {
        const int r = lane + 64 * i;
        if (64 * i >= xend) break;  // wave-uniform
        if (r < xend) {
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float y = ldexpf(sc[r * G + g], -vex[g]);
            uint32_t word = 0;
#pragma unroll
            for (int t = 0; t < 4; ++t) word |= (static_cast<uint32_t>(i8_digit(y, t)) & 0xFFu) << (8 * t);
            reinterpret_cast<uint32_t*>(sc)[r * G + g] = word;
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    if constexpr (VMB) {
      // ---- pass 2 on the matrix cores, bf16 values (G = 8): per 32-key
      // block, O += P V with v_mfma_f32_16x16x32_bf16.  The weights' bf16
      // terms sit in LDS as [key][2 h + t] (the words written above), so the
      // transposing 16-bit LDS read gives the A operand directly (row
      // 2 h + t: term t of head h, eight keys per lane); the block's value
      // rows are staged like the int8 blocks and read the same way for the
      // B operand.  Both reads take keys 4 quad + 0..3 and 16 + 4 quad +
      // 0..3 of the block for lane group quad, so the two operands agree on
      // the order of the keys.  Result row 4 quad + i of lane (quad, n):
      // head 2 quad + i / 2, term i % 2, dim 16 T + n; the two terms are
      // added into vacc at the end of the chunk.
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      // 16-byte column blocks of a staged row are XOR-permuted so that the
      // four rows one 16-lane group reads land on distinct banks.
      auto vswz = [](int rr) { return D == 64 ? 2 * ((rr >> 1) & 1) : 2 * (rr & 3); };
      char* vst = reinterpret_cast<char*>(kstage) + wave * kStageBytes;
      const char* wts = reinterpret_cast<const char*>(sc);
      const int qd = lane >> 4, n16 = lane & 15;
      const int tr_row = 4 * qd + (n16 >> 2);  // rows of this lane's reads: tr_row, 16 + tr_row
      f32x4 cacc[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) cacc[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      for (int t = 0; t < nv; ++t) {
        const bool more = t + 1 < nv;  // wave-uniform
#pragma unroll
        for (int st = 0; st < VNL; ++st) {
          const int rr = VRPI * st + lane / CB;
          *reinterpret_cast<u32x4*>(vst + rr * (D * VB) + 16 * ((lane % CB) ^ vswz(rr))) = vdm[st];
          if (more) vdm[st] = load_nt<16>(vaddr_mf(t + 1, st));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // A: weight terms of keys tr_row, 16 + tr_row (4 G bytes per key),
        // 8 bytes at column 8 (n16 % 4) of the key's 16 terms.
        const int xb = TV0 - A + t * VBK + tr_row;
        const s16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(wts + xb * (4 * G) + 8 * (n16 & 3)));
        const s16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(wts + (xb + 16) * (4 * G) + 8 * (n16 & 3)));
        const bf16x8 av = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          // B: dims 16 tt + 4 (n16 % 4) .. of the same keys.
          const int cb = 2 * tt + ((n16 & 3) >> 1), off = 8 * (n16 & 1);
          const s16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vst + tr_row * (D * VB) + 16 * (cb ^ vswz(tr_row)) + off));
          const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_s16x4*)(vst + (tr_row + 16) * (D * VB) + 16 * (cb ^ vswz(tr_row + 16)) + off));
          const bf16x8 bv = __builtin_bit_cast(bf16x8, __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7));
          cacc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, cacc[tt], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        vacc[0][tt] += cacc[tt][0] + cacc[tt][1];
        vacc[VMB ? 1 : 0][tt] += cacc[tt][2] + cacc[tt][3];
      }
    } else if constexpr (VMF) {
      // ---- pass 2 on the matrix cores: per 64-key block, O += P V with the
      // weights' digits as the A operand (row 4 h + t: digit t of head h)
      // and the codes as the B operand.  The block is staged in LDS (rows
      // of D bytes, 16-byte column blocks permuted within a row so that the
      // transposing reads below hit distinct banks); gfx950's transposing
      // 8-bit LDS read gives lane (q, n) dim n of 8 keys at a time, and the
      // same read over the digit rows (4 G bytes per key) gives the A
      // operand.  Each load is reissued for the next block once staged.
      // The i32 products are exact; the chunk's digit rows are combined
      // into vacc at the end of the chunk.
      typedef int32_t v2i32 __attribute__((ext_vector_type(2)));
      typedef __attribute__((address_space(3))) v2i32 lds_v2i32;
      auto vswz = [](int rr) { return ((rr >> (D == 64 ? 2 : 1)) ^ ((rr >> 4) << (D == 64 ? 1 : 2))) & (CB - 1); };
      char* vst = reinterpret_cast<char*>(kstage) + wave * kStageBytes;
      const char* dig = reinterpret_cast<const char*>(sc);
      const int s16 = lane & 15, qg = lane >> 4;
      i32x4 cacc[HG][NT];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg)
#pragma unroll
        for (int t = 0; t < NT; ++t) cacc[hg][t] = i32x4{0, 0, 0, 0};
      for (int t = 0; t < nv; ++t) {
        const bool more = t + 1 < nv;  // wave-uniform
#pragma unroll
        for (int st = 0; st < VNL; ++st) {
          const int rr = VRPI * st + lane / CB;
          *reinterpret_cast<u32x4*>(vst + rr * (D * VB) + 16 * ((lane % CB) ^ vswz(rr))) = vdm[st];
          if (more) vdm[st] = load_nt<16>(vaddr_mf(t + 1, st));
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // A of head group hg: digits of keys 16 qg + (0..15) of the block,
        // row s16 (bytes 16 hg .. 16 hg + 15 of a key's 4 G digit bytes).
        const int xb = TV0 - A + t * VBK + 16 * qg + (s16 >> 1);
        i32x4 av[HG];
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const int dh = (G >= 4) ? 16 * hg + 8 * (s16 & 1) : 0;
          const v2i32 d0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(dig + xb * (4 * G) + dh));
          const v2i32 d1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32*)(dig + (xb + 8) * (4 * G) + dh));
          av[hg] = i32x4{d0.x, d0.y, d1.x, d1.y};
        }
        const int vb = 16 * qg + (s16 >> 1);  // staged row of this lane's first read
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const v2i32 b0 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_v2i32*)(vst + vb * (D * VB) + 16 * (tt ^ vswz(vb)) + 8 * (s16 & 1)));
          const v2i32 b1 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              (lds_v2i32*)(vst + (vb + 8) * (D * VB) + 16 * (tt ^ vswz(vb + 8)) + 8 * (s16 & 1)));
#pragma unroll
          for (int hg = 0; hg < HG; ++hg)
            cacc[hg][tt] =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(av[hg], i32x4{b0.x, b0.y, b1.x, b1.y}, cacc[hg][tt], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      constexpr float k7 = 1.0f / 128.0f;
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        int vexl = 0;  // the digit scale of this lane's head 4 hg + kc
#pragma unroll
        for (int g = 0; g < G; ++g) vexl = (4 * hg + kc == g) ? vex[g] : vexl;
        const float vsig = ldexpf(1.0f, vexl);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          const i32x4 c = cacc[hg][tt];
          const float x = fmaf(fmaf(fmaf(static_cast<float>(c[3]), k7, static_cast<float>(c[2])), k7,
                                    static_cast<float>(c[1])),
                               k7, static_cast<float>(c[0]));
          vacc[hg][tt] = fmaf(x, vsig, vacc[hg][tt]);
        }
      }
    } else {
      // ---- pass 2: weighted sum of values (rolling prefetch of UV tiles) ------
      auto v_accum = [&](const float (&vf)[VE], int r) {
        float p[G];
#pragma unroll
        for (int g = 0; g < G; ++g) p[g] = sc[r * G + g];
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(p[g], vf[e], acc[g][e]);
        }
      };
      const int vx0 = TV0 - A + vr;  // LDS row of tile 0 for this lane
      int t0 = 0;
      for (; t0 + 2 * UV <= nv; t0 += UV) {
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          float vf[VE];
          widen<VT, VE>(vd[u], vf);
          vd[u] = load_nt<VLB>(vaddr(t0 + UV + u));
          v_accum(vf, vx0 + (t0 + u) * VRPL);
        }
      }
      for (; t0 < nv; t0 += UV) {
#pragma unroll
        for (int u = 0; u < UV; ++u) {
          if (t0 + u < nv) {
            float vf[VE];
            widen<VT, VE>(vd[u], vf);
            if (t0 + UV + u < nv) vd[u] = load_nt<VLB>(vaddr(t0 + UV + u));
            v_accum(vf, vx0 + (t0 + u) * VRPL);
          }
        }
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // ---- fused step: merge the new token's row (scores from the prologue) ----
  if constexpr (FUSED) {
    if (new_here) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float sl = capped_log2(s_new[g], capped, cap_c, cap_inv);
        const float m_new = fmaxf(m_run[g], sl);
        const float alpha = (m_run[g] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run[g] - m_new);
        l_run[g] *= alpha;
        psum[g] *= alpha;
        m_run[g] = m_new;
        const float pn = __builtin_amdgcn_exp2f(sl - m_new);
        if (lane == 0) l_run[g] += pn;  // l is summed over the whole wave below
        if constexpr (VMF) {
          const float* vkeep = reinterpret_cast<const float*>(sxd + wave * D);
#pragma unroll
          for (int hg = 0; hg < VH; ++hg)
            if (vhead(hg) == g) {
#pragma unroll
              for (int t = 0; t < NT; ++t)
                vacc[hg][t] = fmaf(pn, vkeep[16 * t + (lane & 15)], vacc[hg][t] * alpha);
            }
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[g][e] *= alpha;
          if (vr == 0) {  // acc is summed over the row groups below
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(pn, vnew[e], acc[g][e]);
          }
        }
      }
    }
  }

  // ---- merge the wave's row groups and write the split's partial ----------
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_run[g] = wave_sum(l_run[g]);
    if constexpr (!VMF) {  // the matrix value pass leaves vacc complete
      if constexpr (VT == kI8) psum[g] = wave_sum(psum[g]);  // one lane wrote each row's weight
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        float x = acc[g][e];
#pragma unroll
        for (int m = VLPR; m < 64; m <<= 1) x += __shfl_xor(x, m);
        acc[g][e] = (VT == kI8) ? fmaf(-128.0f, psum[g], x) : x;
      }
    }
  }
  // Matrix value pass: this lane's heads 4 hg + kc (rows of heads >= G are
  // unused) and its output dims 16 t + vn.
  const int vn = lane & 15;
  (void)vn;
  // ---- cooperative item: part 0 merges the four parts' states -------------
  if (coop) {
    // This wave's area of LDS (free after the last chunk) holds its state:
    // m[G], l[G], then the unnormalised accumulator [G][D].
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        sc[g] = m_run[g];
        sc[G + g] = l_run[g];
      }
    }
    if constexpr (VMF) {
#pragma unroll
      for (int hg = 0; hg < VH; ++hg)
        if (vhead(hg) < G) {
#pragma unroll
          for (int t = 0; t < NT; ++t) sc[2 * G + vhead(hg) * D + 16 * t + vn] = vacc[hg][t];
        }
    } else if (vr == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < VE; ++e) sc[2 * G + g * D + vc * VE + e] = acc[g][e];
    }
    __syncthreads();
    if (part != 0) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float M = -INFINITY;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) M = fmaxf(M, smem[q * (kLdsRows * G) + g]);
      float l = 0.0f;
      if constexpr (VMF) {
#pragma unroll
        for (int hg = 0; hg < VH; ++hg)
          if (vhead(hg) == g) {
#pragma unroll
            for (int t = 0; t < NT; ++t) vacc[hg][t] = 0.0f;
          }
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = 0.0f;
      }
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        const float* st = smem + q * (kLdsRows * G);
        const float mq = st[g];
        // an empty part has m = -inf and contributes nothing
        const float wq = (mq == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mq - M);
        l = fmaf(wq, st[G + g], l);
        if constexpr (VMF) {
#pragma unroll
          for (int hg = 0; hg < VH; ++hg)
            if (vhead(hg) == g) {
#pragma unroll
              for (int t = 0; t < NT; ++t) vacc[hg][t] = fmaf(wq, st[2 * G + g * D + 16 * t + vn], vacc[hg][t]);
            }
        } else {
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(wq, st[2 * G + g * D + vc * VE + e], acc[g][e]);
        }
      }
      m_run[g] = M;
      l_run[g] = l;
    }
  }

  const int64_t row0 = (static_cast<int64_t>(b) * a.H + kvh * G) * a.max_splits + sigma;
  if constexpr (VMF) {
#pragma unroll
    for (int hg = 0; hg < VH; ++hg) {
      const int h = vhead(hg);
      float inv = 0.0f;
#pragma unroll
      for (int g = 0; g < G; ++g) inv = (h == g) ? 1.0f / l_run[g] : inv;
      if (h < G) {
        float* dst = a.part_o + (row0 + static_cast<int64_t>(h) * a.max_splits) * D + vn;
#pragma unroll
        for (int t = 0; t < NT; ++t) dst[16 * t] = vacc[hg][t] * inv;
      }
    }
  } else if (vr == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float inv = 1.0f / l_run[g];
      float* dst = a.part_o + (row0 + static_cast<int64_t>(g) * a.max_splits) * D + vc * VE;
#pragma unroll
      for (int e = 0; e < VE; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            make_float4(acc[g][e] * inv, acc[g][e + 1] * inv, acc[g][e + 2] * inv, acc[g][e + 3] * inv);
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
      a.part_lse[row0 + static_cast<int64_t>(g) * a.max_splits] = (m_run[g] + log2f(l_run[g])) * kLn2;
  }

  // ---- fused step: the last split of (b, kvh) to arrive combines ----------
  if constexpr (FUSED) {
    const int ns = a.t.work_prefix[b + 1] - a.t.work_prefix[b];
    int32_t* ctr = x->counters + static_cast<int64_t>(b) * a.Hkv + kvh;
    // Release this wave's partial before taking the ticket; the combining
    // wave acquires before reading the others' partials.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    int ticket = 0;
    if (lane == 0) ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ticket = __shfl(ticket, 0);
    if (ticket != ns - 1) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int s0 = a.t.first_split[b];
    const int h0 = kvh * G;
    const int64_t crow = (static_cast<int64_t>(b) * a.H + h0) * a.max_splits + s0;
    combine_group<D, G>(a.part_lse + crow, a.max_splits, a.part_o + crow * D + lane,
                        static_cast<int64_t>(a.max_splits) * D, ns, x->sinks != nullptr ? x->sinks + h0 : nullptr,
                        x->out + (static_cast<int64_t>(b) * a.H + h0) * D, lane);
    if (lane == 0) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Cooperative launches of the partials (contiguous or paged caches) use the
// interleaved instantiation (ILV); everything else the plain one.
template <int D, int G, int KT, int VT, bool PAGED, bool FUSED>
hipError_t launch_one(const KernelArgs<FUSED>& args, hipStream_t stream) {
  const AttnArgs& a = attn_of(args);
  const int items = a.t.work_prefix[a.t.n_seq] * a.Hkv;
  const dim3 grid(a.coop ? items : (items + kWaves - 1) / kWaves);
  if constexpr (!FUSED) {
    if (a.coop) {
      hipLaunchKernelGGL((decode_partial_kernel<D, G, KT, VT, PAGED, FUSED, true>), grid, dim3(kThreads), 0, stream,
                         args);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_partial_kernel<D, G, KT, VT, PAGED, FUSED, false>), grid, dim3(kThreads), 0, stream,
                     args);
  return hipGetLastError();
}

template <int D, int G, bool PAGED, bool FUSED>
hipError_t by_dtype(int kt, int vt, const KernelArgs<FUSED>& a, hipStream_t s) {
  if (kt == kF32 && vt == kF32) return launch_one<D, G, kF32, kF32, PAGED, FUSED>(a, s);
  if (kt == kF32 && vt == kBF16) return launch_one<D, G, kF32, kBF16, PAGED, FUSED>(a, s);
  if (kt == kF32 && vt == kI8) return launch_one<D, G, kF32, kI8, PAGED, FUSED>(a, s);
  if (kt == kBF16 && vt == kF32) return launch_one<D, G, kBF16, kF32, PAGED, FUSED>(a, s);
  if (kt == kBF16 && vt == kBF16) return launch_one<D, G, kBF16, kBF16, PAGED, FUSED>(a, s);
  if (kt == kBF16 && vt == kI8) return launch_one<D, G, kBF16, kI8, PAGED, FUSED>(a, s);
  if (kt == kI8 && vt == kI8) return launch_one<D, G, kI8, kI8, PAGED, FUSED>(a, s);
  return hipErrorInvalidValue;
}

template <int D, bool PAGED, bool FUSED>
hipError_t by_group(int G, int kt, int vt, const KernelArgs<FUSED>& a, hipStream_t s) {
  switch (G) {
    case 1: return by_dtype<D, 1, PAGED, FUSED>(kt, vt, a, s);
    case 2: return by_dtype<D, 2, PAGED, FUSED>(kt, vt, a, s);
    case 4: return by_dtype<D, 4, PAGED, FUSED>(kt, vt, a, s);
    case 8: return by_dtype<D, 8, PAGED, FUSED>(kt, vt, a, s);
    default: return hipErrorInvalidValue;
  }
}

template <bool PAGED, bool FUSED>
hipError_t dispatch(int D, int G, int k_dtype, int v_dtype, const KernelArgs<FUSED>& a, hipStream_t stream) {
  switch (D) {
    case 64: return by_group<64, PAGED, FUSED>(G, k_dtype, v_dtype, a, stream);
    case 128: return by_group<128, PAGED, FUSED>(G, k_dtype, v_dtype, a, stream);
    case 256: return by_group<256, PAGED, FUSED>(G, k_dtype, v_dtype, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace uaii
