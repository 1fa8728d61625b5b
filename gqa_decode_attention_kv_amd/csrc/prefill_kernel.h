// Chunk attention (prefill) for grouped-query attention on the matrix cores.
//
// Sources: "Algenta - Model support matrix" (Kernel path capabilities: a
// grouped-FA prefill for d128 and d64 and a parametric prefill for
// power-of-two head dims; Structural fact requirements: GQA ratio,
// attention scale 1/sqrt(head_dim)); "Universal AI Inference - Hugging Face
// decoder completeness" (P1.3: positions follow the absolute KV index; P1.4:
// sliding window, logit softcap as a tanh clip); "llamay - Models and
// formats" (Architectures: gpt-oss's per-head sink in the softmax
// denominator).
//
// What is computed: the T queries of a chunk of sequence b sit at positions
// L - T .. L - 1 (L = keys including the chunk, whose keys and values the
// chunk producer has already written).  Query t attends causally: the keys
// at positions lo_t .. L - T + t, where lo_t = max(0, L - T + t + 1 - W)
// under a window of W keys (W = 0: none).  Softmax over scale * <q, k>,
// softcapped if asked, optionally with a sink logit in the denominator.
//
// Design (gfx950, bf16 K and V):
//   * One work-group of four waves per (128 query rows, kv head, sequence),
//     or 64 rows at d256 and for small grids.
//     The rows are (token, head) pairs t * G + g of one kv head's group, so
//     the G heads that share a kv head share every K and V tile (grouped
//     flash attention): each tile is read from HBM once per work-group.
//   * Work-group order: all row groups of one (sequence, kv head) run on
//     one XCD (they read the same K and V prefix through its L2), longest
//     first within it (the causal tail is short).
//   * Key tiles of 32 rows of K and V are staged in LDS by the whole
//     work-group with 16-byte loads, double-buffered: one barrier per tile,
//     or per two tiles (64 rows staged at once) with two query blocks per
//     wave up to d128.
//     Padded rows, so the matrix and transposing reads below do not collide
//     on banks.  The next tile's loads go to registers while the current
//     tile's products run.
//   * Each wave owns 32 query rows (16 at d256 or in small grids) and
//     computes the transposed
//     scores S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (two 16-key blocks);
//     each K and V operand read from LDS feeds both 16-row blocks.  In the
//     transposed form the score registers of a lane already hold what the
//     PV product needs as its A operand (one query, eight keys), so the
//     probabilities never go through LDS; V, which that product needs one
//     dim across eight keys per lane, is read with gfx950's transposing LDS
//     load.
//   * Online softmax per query in f32, in the log2 domain (q pre-multiplied
//     by scale * log2 e); keys outside a query's causal window get weight 0.
//     The reference a query's weights are taken against moves only when a
//     tile exceeds it by more than 2^8, and the scores come out of the
//     matrix product already relative to it, so the common tile costs an
//     exp2 and an add per weight; the tile max, the rescale and the
//     reduction across lanes run on a rare wave-uniform path.
//   * Precision: q (f32) and the probabilities (f32) are each split into a
//     bf16 high part and a bf16 remainder, and both parts are multiplied by
//     the exact bf16 K or V: two MFMAs per product, about 16 significant bits
//     per operand and f32 accumulation (plain bf16 rounding of q and p would
//     cost about 3 significant digits of the output).
// Arithmetic intensity is about 4 * 64 flop per K/V byte in LDS and one HBM
// read of each tile per 64 rows: the kernel is bound by the matrix cores.
#pragma once

#include <math.h>

#include "prefill_args.h"

namespace uaii {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kKeys = 32;    // keys per tile
// The softmax reference of a query moves only when a tile's max exceeds it
// by more than this many powers of two (weights stay below 2^kSlack).
constexpr float kSlack = 8.0f;
constexpr float kSlackW = 256.0f;  // 2^kSlack
constexpr float kLog2eP = 1.4426950408889634f;
// Word 3 of a raw buffer descriptor on gfx9 parts: 32-bit data format,
// offsets checked against the record count (reads past it return zero).
constexpr int kBufferWord3 = 0x00020000;

// max / sum of x over lanes l and l ^ 16, then over l and l ^ 32, with
// gfx950's row swaps (v_permlane16_swap, v_permlane32_swap): swapping a
// register with itself leaves {x[l], x[l ^ 16]} (resp. l ^ 32) in the two
// results, in the same order in both lanes of a pair, so both get the same
// value.  Plain VALU instead of an LDS permute.
// The max of two scores is med3(a, b, +inf): one instruction, where fmaxf
// on the swapped registers would first quiet possible signalling NaNs (the
// scores are never NaN for finite inputs).
__device__ inline float max2(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, INFINITY); }

__device__ inline float pair_max_16_32(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max2(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float pair_sum_16_32(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float capped(float s, bool cap, float c, float c_inv) {
  return cap ? c * tanhf(s * c_inv) * kLog2eP : s;
}

// Split 8 floats into bf16 high parts (round to nearest even) and bf16
// remainders (x ~ hi + lo).  Pairs are converted with one packed convert;
// the high parts come back to f32 from the packed word by a shift and a
// mask.
__device__ inline void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const bf16x2 hp = __builtin_convertvector(f32x2{x[2 * k], x[2 * k + 1]}, bf16x2);
    h[k] = __builtin_bit_cast(uint32_t, hp);
    const float r0 = x[2 * k] - __uint_as_float(h[k] << 16);
    const float r1 = x[2 * k + 1] - __uint_as_float(h[k] & 0xFFFF0000u);
    l[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{r0, r1}, bf16x2));
  }
  hi = __builtin_bit_cast(bf16x8, u32x4{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, u32x4{l[0], l[1], l[2], l[3]});
}

// QB blocks of 16 query rows per wave.  With QB = 2 each K and V operand
// read from LDS feeds twice as many matrix products; it is used for head
// dims up to 128 (d256 registers would not hold two blocks) when the grid
// still has at least two work-groups per CU.
template <int QB>
constexpr int rows_per_group() { return 4 * 16 * QB; }

// amdgpu_waves_per_eu(2, 2): a register budget of 256 per lane, so the
// allocator keeps the output accumulator in VGPRs (without the hint it kept
// it in AGPRs and copied it to VGPRs and back on every tile).
// Staging of one operand (K or V) of a tile: EB bytes per element in the
// cache (2: bf16, 1: int8 codes, widened to bf16 in LDS, which holds them
// exactly).  NL 16-byte loads per thread cover the tile's 32 rows.
template <int D, int EB, int KT_ROWS>
struct Stage {
  static constexpr int CPR = D * EB / 16;  // 16-byte chunks per row in the cache
  static constexpr int TOTAL = KT_ROWS * CPR;
  static constexpr int NL = (TOTAL + 255) / 256;
};

// Widen 16 int8 codes to bf16 (exact: |code| <= 128 needs 8 significant
// bits), as two 16-byte LDS rows' worth of bf16 pairs.
__device__ inline void widen_i8(const u32x4& w, u32x4& lo, u32x4& hi) {
  uint32_t out[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t word = w[k >> 1] >> (16 * (k & 1));
    const float f0 = static_cast<float>(static_cast<int8_t>(word & 0xFFu));
    const float f1 = static_cast<float>(static_cast<int8_t>((word >> 8) & 0xFFu));
    out[k] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xFFFF0000u);
  }
  lo = u32x4{out[0], out[1], out[2], out[3]};
  hi = u32x4{out[4], out[5], out[6], out[7]};
}

template <int D, int G, int QB, bool PAGED, bool CAP, int KT, int VT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_attn_kernel(
    const PrefillArgs a) {
  constexpr int ROWS = rows_per_group<QB>();  // query rows per work-group
  // Rows staged per barrier: two 32-key halves with two query blocks per
  // wave up to d128 (half the barriers and staging bookkeeping per key),
  // one otherwise (d256 tiles would not fit two work-groups' LDS).
  // f32 caches (keys and values both f32) stage f32 tiles, one 32-key half
  // per barrier, and multiply on the f32 matrix cores (16x16x4): q, the
  // weights, K and V enter the products as they are.
  constexpr bool F32 = KT == kF32;
  static_assert(F32 == (VT == kF32), "f32 keys go with f32 values");
  constexpr int KST = (QB == 2 && D <= 128 && !F32) ? 2 * kKeys : kKeys;
  constexpr int KEB = F32 ? 4 : (KT == kI8 ? 1 : 2), VEB = F32 ? 4 : (VT == kI8 ? 1 : 2);
  using SK = Stage<D, KEB, KST>;
  using SV = Stage<D, VEB, KST>;
  constexpr int KSTEPS = D / 32;  // k-steps of the score product
  constexpr int NB = D / 16;      // 16-column blocks of the output
  // LDS row strides in bf16 elements.  K (16-byte pad): a 16-lane group of
  // 16-byte reads, one per row, covers the banks once.  V (32-byte pad):
  // the transposing reads take 8 bytes from each of 8 rows per 32 lanes,
  // and rows 8 banks apart cover the banks once.
  // f32 tiles (strides in floats, 16-byte pad): the score reads (four
  // floats of each of 16 rows) and the value reads (16 floats of each of 4
  // rows, 4 rows apart) both cover the banks once.
  constexpr int LS = F32 ? D + 4 : D + 8;
  constexpr int LSV = F32 ? D + 4 : D + 16;
  using LE = typename std::conditional<F32, float, uint16_t>::type;  // LDS element
  constexpr int CE = 16 / static_cast<int>(sizeof(LE));  // LDS elements per 16-byte chunk
  // Two buffers of K and V tiles (and, for int8 caches, the tiles' per-token
  // key and value scales): one is read while the next tile is staged.
  __shared__ __attribute__((aligned(16))) LE ks[2][KST * LS];
  __shared__ __attribute__((aligned(16))) LE vs[2][KST * LSV];
  __shared__ float ksc[2][KT == kI8 ? KST : 1];
  __shared__ float vsc[2][VT == kI8 ? KST : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int qi = lane & 15;   // query column of this lane (and row of the A operand)
  const int quad = lane >> 4;
  // Work-group order.  The hardware hands work-group L (x fastest) to XCD
  // L % 8.  Remapped so that all row groups of one (sequence, kv head), which
  // read the same K and V prefix, run on one XCD and share its L2, and so
  // that within it the longest row groups (the last queries of the causal
  // chunk see the most keys) start first and the short ones fill the tail.
  const int n_x = gridDim.x, n_sets = gridDim.y * gridDim.z, n_wg = n_x * n_sets;
  const int wg = blockIdx.x + n_x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int lam = (n_wg % 8 == 0) ? (wg % 8) * (n_wg / 8) + wg / 8 : wg;
  const int set = lam / n_x;
  const int b = set / gridDim.y, kvh = set % gridDim.y;
  const int gx = n_x - 1 - lam % n_x;
  const int T = a.T, L = a.len[b];
  const int P0 = L - T;  // position of the chunk's first token
  const int rows = T * G;
  const int row0 = gx * ROWS;
  const int wrow0 = row0 + wave * 16 * QB;  // first row of this wave

  // This lane's query in each block q (S^T column qi of block q).
  bool row_ok[QB];
  int my_t[QB], my_g[QB], my_p[QB], my_lo[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const int r = wrow0 + q * 16 + qi;
    row_ok[q] = r < rows;
    my_t[q] = row_ok[q] ? r / G : T - 1;
    my_g[q] = row_ok[q] ? r % G : 0;
    my_p[q] = P0 + my_t[q];
    my_lo[q] = (a.window > 0 && my_p[q] + 1 > a.window) ? my_p[q] + 1 - a.window : 0;
  }

  // Keys any row of the work-group attends: [lo_first, k_end).
  const int t_first = row0 / G;
  const int t_last = min((row0 + ROWS - 1) / G, T - 1);
  const int p_first = P0 + t_first;
  const int lo_first = (a.window > 0 && p_first + 1 > a.window) ? p_first + 1 - a.window : 0;
  const int k_end = P0 + t_last + 1;
  const int k_begin = lo_first & ~(kKeys - 1);
  // Tiles every row of the work-group sees whole need no mask.
  const int p_last = P0 + t_last;
  const int lo_last = (a.window > 0 && p_last + 1 > a.window) ? p_last + 1 - a.window : 0;
  const bool rows_full = row0 + ROWS <= rows;

  // Queries: B operand of S^T = K Q^T, lane holds q[qi][ks*32 + 8*quad + j]
  // of each block (f32: qf holds q[qi][4 s + quad] for step s).
  bf16x8 qh[QB][F32 ? 1 : KSTEPS], ql[QB][F32 ? 1 : KSTEPS];
  float qf[QB][F32 ? D / 4 : 1];
  (void)qh;
  (void)ql;
  (void)qf;
  if constexpr (F32) {
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const float* qp = a.q + ((static_cast<int64_t>(b) * T + my_t[q]) * a.H + kvh * G + my_g[q]) * D + quad;
#pragma unroll
      for (int st = 0; st < D / 4; ++st) qf[q][st] = qp[4 * st] * a.q_mul;
    }
  }
#pragma unroll
  for (int q = 0; q < (F32 ? 0 : QB); ++q) {
    const float* qp =
        a.q + ((static_cast<int64_t>(b) * T + my_t[q]) * a.H + kvh * G + my_g[q]) * D + 8 * quad;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) {
      const float4 x0 = *reinterpret_cast<const float4*>(qp + s * 32);
      const float4 x1 = *reinterpret_cast<const float4*>(qp + s * 32 + 4);
      const float x[8] = {x0.x * a.q_mul, x0.y * a.q_mul, x0.z * a.q_mul, x0.w * a.q_mul,
                          x1.x * a.q_mul, x1.y * a.q_mul, x1.z * a.q_mul, x1.w * a.q_mul};
      split8(x, qh[q][s], ql[q][s]);
    }
  }
  constexpr bool cap = CAP;  // softcap (the tanh clip) compiled in or out
  const float cap_c = a.softcap, cap_inv = cap ? 1.0f / a.softcap : 0.0f;

  f32x4 o[QB][NB];
#pragma unroll
  for (int q = 0; q < QB; ++q)
#pragma unroll
    for (int n = 0; n < NB; ++n) o[q][n] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // Softmax state of this lane's query in each block: the reference m (-inf
  // until the query's first visible key; rows past the end, which see no
  // key, start at 0 so that they never hold the wave on the exact path), and
  // this lane's share of the weight sum relative to m (the lanes of a query
  // hold different keys; their shares are added at the end).
  // The reference r itself (m, or 0 while m is -inf) is kept negated in all
  // four slots, the initial accumulator of the score product.
  float m[QB], l[QB];
  f32x4 nref[QB];
  uint64_t unref[QB];  // lanes whose query has no reference yet (wave-uniform)
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    m[q] = row_ok[q] ? -INFINITY : 0.0f;
    l[q] = 0.0f;
    nref[q] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    unref[q] = __builtin_amdgcn_ballot_w64(row_ok[q]);
  }

  const int64_t slab = PAGED ? 0 : (static_cast<int64_t>(b) * a.Hkv + kvh) * a.cap;
  // Element offset of key row r of this (b, kv head).
  auto row_off = [&](int r) -> int64_t {
    if constexpr (PAGED) {
      int pid = a.block_table[static_cast<int64_t>(b) * a.max_blocks + (r >> a.log2_bs)];
      pid = min(max(pid, 0), a.num_blocks - 1);
      return ((static_cast<int64_t>(pid) * a.Hkv + kvh) * a.block_size + (r & (a.block_size - 1))) * D;
    } else {
      return (slab + r) * D;
    }
  };
  // This thread's share of a tile: 16-byte chunks of K and of V (and, for
  // int8 caches, one scale: threads 0..31 a key's, 32..63 a value's).  Rows
  // outside [lo_first, k_end) are replaced by the nearest row inside (every
  // row read holds a visible key of some query of the work-group); their
  // weights are zero.  A tile of a contiguous cache that lies inside that
  // range (all but the first and last) is addressed as one uniform base plus
  // a fixed per-thread offset.
  u32x4 kreg[SK::NL], vreg[SV::NL];
  float sreg = 0.0f;
  const char* kslab = static_cast<const char*>(a.k) + slab * D * KEB;
  const char* vslab = static_cast<const char*>(a.v) + slab * D * VEB;
  auto clamp_row = [&](int r) { return min(max(r, lo_first), k_end - 1); };
  // Byte offset of a thread's first 16-byte chunk within a K (V) tile; its
  // load i is 4096 i bytes further (256 threads of 16 bytes, and a row
  // spans a power of two of chunks up to 256).
  static_assert(256 % SK::CPR == 0 && 256 % SV::CPR == 0, "tile chunks");
  const int koff0 = tid / SK::CPR * (D * KEB) + tid % SK::CPR * 16;
  const int voff0 = tid / SV::CPR * (D * VEB) + tid % SV::CPR * 16;
  (void)koff0;
  (void)voff0;
  auto load_tile = [&](int k0) {
    if (!PAGED && k0 >= lo_first && k0 + KST <= k_end) {
      // Buffer loads over the tile's bytes (a descriptor built from the
      // uniform tile base in scalar registers): load i of a thread reads
      // chunk tid + 256 i, 4096 i bytes after its first, so the per-load
      // offsets are scalar and no vector address is formed per tile.
      const char* kt = kslab + static_cast<int64_t>(k0) * (D * KEB);
      const char* vt = vslab + static_cast<int64_t>(k0) * (D * VEB);
      const __amdgpu_buffer_rsrc_t krs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kt), 0, KST * D * KEB, kBufferWord3);
      const __amdgpu_buffer_rsrc_t vrs =
          __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vt), 0, KST * D * VEB, kBufferWord3);
#pragma unroll
      for (int i = 0; i < SK::NL; ++i) {
        const int c = tid + 256 * i;
        if (SK::NL * 256 == SK::TOTAL || c < SK::TOTAL)
          kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, koff0, 4096 * i, 0));
      }
#pragma unroll
      for (int i = 0; i < SV::NL; ++i) {
        const int c = tid + 256 * i;
        if (SV::NL * 256 == SV::TOTAL || c < SV::TOTAL)
          vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff0, 4096 * i, 0));
      }
      if constexpr (KT == kI8 || VT == kI8) {
        const bool is_k = tid < KST;
        const float* pool = is_k ? a.k_scale : a.v_scale;
        if (tid < 2 * KST && pool != nullptr) sreg = pool[slab + k0 + (tid & (KST - 1))];
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < SK::NL; ++i) {
      const int c = tid + 256 * i;
      if (SK::NL * 256 == SK::TOTAL || c < SK::TOTAL) {
        const int r = c / SK::CPR, cc = c % SK::CPR;
        const int64_t off = row_off(clamp_row(k0 + r)) * KEB + cc * 16;
        kreg[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.k) + off);
      }
    }
#pragma unroll
    for (int i = 0; i < SV::NL; ++i) {
      const int c = tid + 256 * i;
      if (SV::NL * 256 == SV::TOTAL || c < SV::TOTAL) {
        const int r = c / SV::CPR, cc = c % SV::CPR;
        const int64_t off = row_off(clamp_row(k0 + r)) * VEB + cc * 16;
        vreg[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v) + off);
      }
    }
    if constexpr (KT == kI8 || VT == kI8) {
      const bool is_k = tid < KST;
      const float* pool = is_k ? a.k_scale : a.v_scale;
      if (tid < 2 * KST && pool != nullptr) sreg = pool[row_off(clamp_row(k0 + (tid & (KST - 1)))) / D];
    }
  };
  // Write the staged registers to LDS buffer `buf` (int8 codes widened to
  // bf16).
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < SK::NL; ++i) {
      const int c = tid + 256 * i;
      if (SK::NL * 256 == SK::TOTAL || c < SK::TOTAL) {
        const int r = c / SK::CPR, cc = c % SK::CPR;
        if constexpr (KT == kI8) {
          u32x4 lo, hi;
          widen_i8(kreg[i], lo, hi);
          *reinterpret_cast<u32x4*>(&ks[buf][r * LS + cc * 16]) = lo;
          *reinterpret_cast<u32x4*>(&ks[buf][r * LS + cc * 16 + 8]) = hi;
        } else {
          *reinterpret_cast<u32x4*>(&ks[buf][r * LS + cc * CE]) = kreg[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < SV::NL; ++i) {
      const int c = tid + 256 * i;
      if (SV::NL * 256 == SV::TOTAL || c < SV::TOTAL) {
        const int r = c / SV::CPR, cc = c % SV::CPR;
        if constexpr (VT == kI8) {
          u32x4 lo, hi;
          widen_i8(vreg[i], lo, hi);
          *reinterpret_cast<u32x4*>(&vs[buf][r * LSV + cc * 16]) = lo;
          *reinterpret_cast<u32x4*>(&vs[buf][r * LSV + cc * 16 + 8]) = hi;
        } else {
          *reinterpret_cast<u32x4*>(&vs[buf][r * LSV + cc * CE]) = vreg[i];
        }
      }
    }
    if constexpr (KT == kI8) {
      if (tid < KST) ksc[buf][tid] = sreg;
    }
    if constexpr (VT == kI8) {
      if (tid >= KST && tid < 2 * KST) vsc[buf][tid - KST] = sreg;
    }
  };

  // Tiles j = 0 .. n_tiles - 1 (keys k_begin + 32 j) alternate between the
  // two LDS buffers.  Iteration j computes tile j from buffer j % 2, then
  // stages tile j + 1 (loaded during iteration j - 1) into the other buffer,
  // whose previous tile every wave finished reading before the last
  // barrier, and starts the loads of tile j + 2: one barrier per tile.
  const int n_tiles = (k_end - k_begin + KST - 1) / KST;
  load_tile(k_begin);
  store_tile(0);
  if (n_tiles > 1) load_tile(k_begin + KST);
  __syncthreads();
  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
#pragma unroll
    for (int h = 0; h < KST / kKeys; ++h) {
    const int k0 = k_begin + j * KST + h * kKeys;  // this half's first key
    if (h > 0 && k0 >= k_end) break;               // wave-uniform: past the last key
    const LE* kb = ks[buf] + h * kKeys * LS;
    const LE* vb_ = vs[buf] + h * kKeys * LSV;
    const float* kscb = ksc[buf] + (KT == kI8 ? h * kKeys : 0);
    const float* vscb = vsc[buf] + (VT == kI8 ? h * kKeys : 0);

    // S^T for keys k0 + mb*16 + (0..15) against the wave's query blocks:
    // lane holds keys k0 + mb*16 + 4*quad + j of query qi of block q.  The
    // scores come out relative to the query's reference r = m (0 while m is
    // -inf): where nothing is applied to the raw product, the accumulator
    // starts at -r.
    constexpr bool fold = !cap && KT != kI8;
    float r[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) r[q] = -nref[q][0];
    f32x4 s[QB][2];
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) s[q][mb] = fold ? nref[q] : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (F32) {
      // A = K (lane: key mb*16 + qi, dim 4 st + quad), B = Q^T.
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
        for (int st = 0; st < D / 4; ++st) {
          const float ka = kb[(mb * 16 + qi) * LS + 4 * st + quad];
#pragma unroll
          for (int q = 0; q < QB; ++q) s[q][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(ka, qf[q][st], s[q][mb], 0, 0, 0);
        }
      }
    } else {
      // Both 16-key blocks per step, high terms then low terms: the 2 QB
      // accumulators take turns, so consecutive products into one
      // accumulator are 2 QB issues apart.
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        bf16x8 ka[2];
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
          ka[mb] = *reinterpret_cast<const bf16x8*>(&kb[(mb * 16 + qi) * LS + st * 32 + 8 * quad]);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int q = 0; q < QB; ++q)
            s[q][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[mb], qh[q][st], s[q][mb], 0, 0, 0);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int q = 0; q < QB; ++q)
            s[q][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[mb], ql[q][st], s[q][mb], 0, 0, 0);
      }
    }

    // t = score - r: int8 keys scale the raw product (q . code) by the key's
    // scale; the softcap clips the score.  Masked keys (outside a row's
    // causal window) get -inf unless every row of the work-group sees the
    // whole tile (the common case).
    const bool full = rows_full && k0 >= lo_last && k0 + kKeys - 1 <= p_first;
    float t[QB][8];
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float x = s[q][e >> 2][e & 3];
        if constexpr (KT == kI8) {
          const float kscale = kscb[(e >> 2) * 16 + 4 * quad + (e & 3)];
          x = cap ? capped(x * kscale, cap, cap_c, cap_inv) - r[q] : fmaf(x, kscale, -r[q]);
        } else if constexpr (cap) {
          x = capped(x, cap, cap_c, cap_inv) - r[q];
        }
        t[q][e] = x;
      }
    if (!full) {
#pragma unroll
      for (int q = 0; q < QB; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = k0 + (e >> 2) * 16 + 4 * quad + (e & 3);
          const bool vis = row_ok[q] && key >= my_lo[q] && key <= my_p[q];
          t[q][e] = vis ? t[q][e] : -INFINITY;
        }
    }

    // Online softmax with a lazy reference.  Fast path: the weights are
    // 2^t, each lane adds its own; valid while every weight stays at most
    // 2^kSlack, which the lane's sum bounds.  When some lane's sum exceeds
    // it, or a query of the wave has no reference yet, the wave takes the
    // exact path: the tile max over the query's lanes, and a new reference
    // when it exceeds the old one by more than kSlack, with the rescale of
    // the accumulator and the sums; the weights are recomputed in place.
    bf16x8 ph[QB], pl[QB];
    float pf[QB][F32 ? 8 : 1];  // f32: the weights themselves, the A operand
    (void)pf;
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      float p[8];
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(t[q][e]);
        ps += p[e];
      }
      if ((unref[q] | __builtin_amdgcn_ballot_w64(ps > kSlackW)) != 0) {
        float lm = t[q][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) lm = max2(lm, t[q][e]);
        const float ms = r[q] + pair_max_16_32(lm);  // tile max (-inf: no visible key)
        const bool bump = ms > m[q] + kSlack;        // m = -inf: any visible key bumps
        const float m_new = bump ? ms : m[q];
        const float r_new = (m_new == -INFINITY) ? 0.0f : m_new;
        const float d = r_new - r[q];
        const float alpha = __builtin_amdgcn_exp2f(m[q] - r_new);  // m = -inf gives 0
        ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(t[q][e] - d);
          ps += p[e];
        }
        l[q] *= alpha;
        m[q] = m_new;
        nref[q] = f32x4{-r_new, -r_new, -r_new, -r_new};
        unref[q] = __builtin_amdgcn_ballot_w64(m_new == -INFINITY);
        // Rescale the accumulator: its rows are queries 4*quad + jj, whose
        // alpha lives in lane 4*quad + jj.  Skipped when no query's
        // reference moved (every alpha is 1, or 0 for a query with no key
        // yet, whose row is still 0).
        if (__builtin_amdgcn_ballot_w64(bump) != 0) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const float aj = __shfl(alpha, 4 * quad + jj);
#pragma unroll
            for (int n = 0; n < NB; ++n) o[q][n][jj] *= aj;
          }
        }
      }
      l[q] += ps;
      // int8 values: the weight of key j carries its value scale (the
      // codes are the V operand), the sum l does not.
      if constexpr (VT == kI8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] *= vscb[(e < 4) ? 4 * quad + e : 16 + 4 * quad + (e - 4)];
      }
      if constexpr (F32) {
#pragma unroll
        for (int e = 0; e < 8; ++e) pf[q][e] = p[e];
      } else {
        split8(p, ph[q], pl[q]);
      }
    }

    // O += P V.  A operand: lane holds P[qi][k = 8*quad + e], where k < 4 of
    // the lane's group maps to key 4*quad + e and k >= 4 to key 16 + 4*quad +
    // (e - 4) (the same keys the lane's S^T registers hold).  The B operand
    // needs V at those keys in dim n*16 + qi: two transposing LDS reads
    // (ds_read_b64_tr_b16).  Within each 16-lane group, the reading lane s
    // points at 4 dims (n*16 + 4*(s%4) ..) of key base + s/4, and lane i
    // receives dim n*16 + i of keys base .. base + 3.
    if constexpr (F32) {
      // f32: step e multiplies key (e / 4) * 16 + 4*quad + e % 4 (k = quad),
      // the key of the lane's weight pf[q][e]; B = V at that key, dim
      // n*16 + qi.
#pragma unroll
      for (int n = 0; n < NB; ++n) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float vv = vb_[((e >> 2) * 16 + 4 * quad + (e & 3)) * LSV + n * 16 + qi];
#pragma unroll
          for (int q = 0; q < QB; ++q) o[q][n] = __builtin_amdgcn_mfma_f32_16x16x4f32(pf[q][e], vv, o[q][n], 0, 0, 0);
        }
      }
    } else {
      const int tr_row = 4 * quad + (qi >> 2), tr_col = 4 * (qi & 3);
      // Two 16-column blocks at a time, high terms then low terms: 2 QB
      // accumulators take turns.
#pragma unroll
      for (int n0 = 0; n0 < NB; n0 += 2) {
        bf16x8 vb[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int n = n0 + i;
          const s16x4 v0 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb_[tr_row * LSV + n * 16 + tr_col]));
          const s16x4 v1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb_[(16 + tr_row) * LSV + n * 16 + tr_col]));
          vb[i] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < QB; ++q)
            o[q][n0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[q], vb[i], o[q][n0 + i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < QB; ++q)
            o[q][n0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[q], vb[i], o[q][n0 + i], 0, 0, 0);
      }
    }

    }  // halves

    if (j + 1 < n_tiles) {
      store_tile(buf ^ 1);
      if (j + 2 < n_tiles) load_tile(k_begin + (j + 2) * KST);
    }
    __syncthreads();  // tile j + 1 is staged; every wave is done with tile j
  }

  // Normalise (with the sink, if any) and write.  Accumulator rows are
  // queries 4*quad + j of each block; their m and l live in lane 4*quad + j.
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const float lq = pair_sum_16_32(l[q]);  // the query's four lanes
    float sink2 = -INFINITY;
    if (a.sinks != nullptr && row_ok[q]) sink2 = a.sinks[kvh * G + my_g[q]] * kLog2eP;
    const float m_fin = fmaxf(m[q], sink2);
    const float keep = __builtin_amdgcn_exp2f(m[q] - m_fin);
    const float den = lq * keep + __builtin_amdgcn_exp2f(sink2 - m_fin);
    const float f = keep / den;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float fj = __shfl(f, 4 * quad + j);
      const int r = wrow0 + q * 16 + 4 * quad + j;
      if (r < rows) {
        const int t = r / G, g = r % G;
        float* dst = a.out + ((static_cast<int64_t>(b) * T + t) * a.H + kvh * G + g) * D + qi;
#pragma unroll
        for (int n = 0; n < NB; ++n) dst[n * 16] = o[q][n][j] * fj;
      }
    }
  }
}

template <int D, int G, int QB, bool PAGED, int KT, int VT>
void launch_q(int B, const PrefillArgs& a, hipStream_t stream) {
  constexpr int ROWS = rows_per_group<QB>();
  const dim3 grid((a.T * G + ROWS - 1) / ROWS, a.Hkv, B);
  if (a.softcap > 0.0f)
    hipLaunchKernelGGL((prefill_attn_kernel<D, G, QB, PAGED, true, KT, VT>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_attn_kernel<D, G, QB, PAGED, false, KT, VT>), grid, dim3(256), 0, stream, a);
}

template <int D, int G, bool PAGED, int KT, int VT>
void launch_p(int B, const PrefillArgs& a, hipStream_t stream) {
  constexpr int kCUs = 256;
  const int64_t groups2 = static_cast<int64_t>((a.T * G + rows_per_group<2>() - 1) / rows_per_group<2>()) *
                          a.Hkv * B;
  if constexpr (D <= 128) {
    if (groups2 >= 2 * kCUs) return launch_q<D, G, 2, PAGED, KT, VT>(B, a, stream);
  }
  launch_q<D, G, 1, PAGED, KT, VT>(B, a, stream);
}

template <int D, int G, int KT, int VT>
hipError_t launch_dg(int B, const PrefillArgs& a, hipStream_t stream) {
  if (a.block_table != nullptr)
    launch_p<D, G, true, KT, VT>(B, a, stream);
  else
    launch_p<D, G, false, KT, VT>(B, a, stream);
  return hipGetLastError();
}

template <int D, int KT, int VT>
hipError_t launch_d(int G, int B, const PrefillArgs& a, hipStream_t stream) {
  switch (G) {
    case 1: return launch_dg<D, 1, KT, VT>(B, a, stream);
    case 2: return launch_dg<D, 2, KT, VT>(B, a, stream);
    case 4: return launch_dg<D, 4, KT, VT>(B, a, stream);
    case 8: return launch_dg<D, 8, KT, VT>(B, a, stream);
    default: return hipErrorInvalidValue;
  }
}

// The launch for one (K, V) cache type over head dim and GQA ratio.
template <int KT, int VT>
hipError_t launch_prefill_typed(int D, int G, int B, const PrefillArgs& a, hipStream_t stream) {
  switch (D) {
    case 64: return launch_d<64, KT, VT>(G, B, a, stream);
    case 128: return launch_d<128, KT, VT>(G, B, a, stream);
    case 256: return launch_d<256, KT, VT>(G, B, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace uaii
