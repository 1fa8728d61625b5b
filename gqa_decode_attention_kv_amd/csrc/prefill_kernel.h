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
//   * Key tiles of 32 rows of K and V are staged in LDS by the whole
//     work-group with 16-byte loads (padded rows, so the matrix reads below
//     do not collide on banks).  The next tile's loads go to registers while
//     the current tile's products run (16 registers at d128; with two query
//     blocks per wave the kernel runs two waves per SIMD either way).
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
//   * Precision: q (f32) and the probabilities (f32) are each split into a
//     bf16 high part and a bf16 remainder, and both parts are multiplied by
//     the exact bf16 K or V: two MFMAs per product, about 16 significant bits
//     per operand and f32 accumulation (plain bf16 rounding of q and p would
//     cost about 3 significant digits of the output).
// Arithmetic intensity is about 4 * 64 flop per K/V byte in LDS and one HBM
// read of each tile per 64 rows: the kernel is bound by the matrix cores.
#pragma once

#include <math.h>

#include <type_traits>

#include "prefill_args.h"

namespace uaii {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kKeys = 32;    // keys per tile
// The softmax reference of a query moves only when a tile's max exceeds it
// by more than this many powers of two (weights stay below 2^kSlack).
constexpr float kSlack = 8.0f;
constexpr float kLog2eP = 1.4426950408889634f;

// max / sum of x over lanes l and l ^ 16, then over l and l ^ 32, with
// gfx950's row swaps (v_permlane16_swap, v_permlane32_swap): swapping a
// register with itself leaves {x[l], x[l ^ 16]} (resp. l ^ 32) in the two
// results, in the same order in both lanes of a pair, so both get the same
// value.  Plain VALU instead of an LDS permute.
__device__ inline float pair_max_16_32(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// Split 8 floats into bf16 high parts and bf16 remainders (x ~ hi + lo).
__device__ inline void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const __bf16 h = static_cast<__bf16>(x[j]);
    hi[j] = h;
    lo[j] = static_cast<__bf16>(x[j] - static_cast<float>(h));
  }
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
template <int D, int EB>
struct Stage {
  static constexpr int CPR = D * EB / 16;  // 16-byte chunks per row in the cache
  static constexpr int TOTAL = kKeys * CPR;
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
  constexpr int KEB = KT == kI8 ? 1 : 2, VEB = VT == kI8 ? 1 : 2;
  using SK = Stage<D, KEB>;
  using SV = Stage<D, VEB>;
  constexpr int KSTEPS = D / 32;  // k-steps of the score product
  constexpr int NB = D / 16;      // 16-column blocks of the output
  constexpr int LS = D + 8;       // K and V tiles: LDS row stride in bf16 elements (16-byte pad)
  // Two-deep rings of K and V tiles (and, for int8 caches, the tiles'
  // per-token key and value scales).  K runs one tile ahead of V.
  __shared__ __attribute__((aligned(16))) uint16_t ks[2][kKeys * LS];
  __shared__ __attribute__((aligned(16))) uint16_t vs[2][kKeys * LS];
  __shared__ float ksc[2][KT == kI8 ? kKeys : 1];
  __shared__ float vsc[2][VT == kI8 ? kKeys : 1];

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
  // of each block.
  bf16x8 qh[QB][KSTEPS], ql[QB][KSTEPS];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
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
  float m[QB], l[QB];  // running max and sum of this lane's queries
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    m[q] = -INFINITY;
    l[q] = 0.0f;
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
  // This thread's share of a tile: 16-byte chunks of K or of V (and, for
  // int8 caches, one scale: threads 0..31 a key's, 32..63 a value's).  Rows
  // outside [lo_first, k_end) are replaced by the nearest row inside (every
  // row read holds a visible key of some query of the work-group); their
  // weights are zero.
  auto clamp_row = [&](int r) { return min(max(r, lo_first), k_end - 1); };
  auto load_k = [&](int k0, u32x4 (&kr)[SK::NL], float& sr) {
#pragma unroll
    for (int i = 0; i < SK::NL; ++i) {
      const int c = tid + 256 * i;
      if (SK::NL * 256 == SK::TOTAL || c < SK::TOTAL) {
        const int r = c / SK::CPR, cc = c % SK::CPR;
        const int64_t off = row_off(clamp_row(k0 + r)) * KEB + cc * 16;
        kr[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.k) + off);
      }
    }
    if constexpr (KT == kI8) {
      if (tid < kKeys && a.k_scale != nullptr) sr = a.k_scale[row_off(clamp_row(k0 + tid)) / D];
    }
  };
  auto load_v = [&](int k0, u32x4 (&vr)[SV::NL], float& sr) {
#pragma unroll
    for (int i = 0; i < SV::NL; ++i) {
      const int c = tid + 256 * i;
      if (SV::NL * 256 == SV::TOTAL || c < SV::TOTAL) {
        const int r = c / SV::CPR, cc = c % SV::CPR;
        const int64_t off = row_off(clamp_row(k0 + r)) * VEB + cc * 16;
        vr[i] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(a.v) + off);
      }
    }
    if constexpr (VT == kI8) {
      if (tid >= kKeys && tid < 2 * kKeys && a.v_scale != nullptr)
        sr = a.v_scale[row_off(clamp_row(k0 + tid - kKeys)) / D];
    }
  };
  // Write staged registers to LDS buffer `buf` (int8 codes widened to bf16).
  auto store_rows = [&](auto& sh, const u32x4* rg, auto stage, auto eb) {
    using S = decltype(stage);
    constexpr bool i8 = decltype(eb)::value == 1;
#pragma unroll
    for (int i = 0; i < S::NL; ++i) {
      const int c = tid + 256 * i;
      if (S::NL * 256 == S::TOTAL || c < S::TOTAL) {
        const int r = c / S::CPR, cc = c % S::CPR;
        if constexpr (i8) {
          u32x4 lo, hi;
          widen_i8(rg[i], lo, hi);
          *reinterpret_cast<u32x4*>(&sh[r * LS + cc * 16]) = lo;
          *reinterpret_cast<u32x4*>(&sh[r * LS + cc * 16 + 8]) = hi;
        } else {
          *reinterpret_cast<u32x4*>(&sh[r * LS + cc * 8]) = rg[i];
        }
      }
    }
  };
  auto store_k = [&](const u32x4 (&kr)[SK::NL], float sr, int buf) {
    store_rows(ks[buf], kr, SK{}, std::integral_constant<int, KEB>{});
    if constexpr (KT == kI8) {
      if (tid < kKeys) ksc[buf][tid] = sr;
    }
  };
  auto store_v = [&](const u32x4 (&vr)[SV::NL], float sr, int buf) {
    store_rows(vs[buf], vr, SV{}, std::integral_constant<int, VEB>{});
    if constexpr (VT == kI8) {
      if (tid >= kKeys && tid < 2 * kKeys) vsc[buf][tid - kKeys] = sr;
    }
  };

  // S^T for the 32 keys of the K tile in buffer `buf` against the wave's
  // query blocks: lane holds keys mb*16 + 4*quad + j of query qi of block q.
  // int8 keys: each raw score is q . code; the key's scale makes it q . k.
  auto scores = [&](int buf, f32x4 (&s)[QB][2]) {
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) s[q][mb] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
      for (int st = 0; st < KSTEPS; ++st) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&ks[buf][(mb * 16 + qi) * LS + st * 32 + 8 * quad]);
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          s[q][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qh[q][st], s[q][mb], 0, 0, 0);
          s[q][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, ql[q][st], s[q][mb], 0, 0, 0);
        }
      }
    }
    if constexpr (KT == kI8) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float kscale = ksc[buf][mb * 16 + 4 * quad + j];
#pragma unroll
          for (int q = 0; q < QB; ++q) s[q][mb][j] *= kscale;
        }
    }
  };

  // Software pipeline over tiles j = 0 .. n_tiles - 1 (keys k_begin + 32 j):
  // iteration j computes the softmax and PV product of tile j and, from the
  // other K buffer, the scores of tile j + 1, which are independent of the
  // softmax, so the matrix products overlap its vector work.  LDS holds K(j),
  // V(j) in buffer j % 2 and K(j + 1), V(j + 1) in the other one; iteration j
  // stages K(j + 2) into buffer j % 2 (K(j) was read in iteration j - 1) and
  // V(j + 1) into buffer (j + 1) % 2 (V(j - 1)'s), so one barrier per tile
  // suffices.  Past the last tile the clamped rows are loaded and their
  // scores computed but never used.
  const int n_tiles = (k_end - k_begin + kKeys - 1) / kKeys;
  u32x4 kreg[SK::NL], vreg[SV::NL];
  float sreg = 0.0f;
  {
    u32x4 k0r[SK::NL], v0r[SV::NL], k1r[SK::NL];
    float s0 = 0.0f, s1 = 0.0f;
    load_k(k_begin, k0r, s0);
    load_v(k_begin, v0r, s0);
    load_k(k_begin + kKeys, k1r, s1);
    load_k(k_begin + 2 * kKeys, kreg, sreg);
    load_v(k_begin + kKeys, vreg, sreg);
    store_k(k0r, s0, 0);
    store_v(v0r, s0, 0);
    store_k(k1r, s1, 1);
  }
  __syncthreads();
  f32x4 s[QB][2];
  scores(0, s);
  __syncthreads();  // every wave has read K(0) before iteration 0 replaces it

  for (int j = 0; j < n_tiles; ++j) {
    const int k0 = k_begin + j * kKeys;
    store_k(kreg, sreg, j & 1);
    store_v(vreg, sreg, (j + 1) & 1);
    load_k(k0 + 3 * kKeys, kreg, sreg);
    load_v(k0 + 2 * kKeys, vreg, sreg);

    // Tile j: capped scores, and the mask unless every row of the
    // work-group sees the whole tile (the common case).
    float sv[QB][8];
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[q][e] = capped(s[q][e >> 2][e & 3], cap, cap_c, cap_inv);
    const bool full = rows_full && k0 >= lo_last && k0 + kKeys - 1 <= p_first;
    if (!full) {
#pragma unroll
      for (int q = 0; q < QB; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int key = k0 + (e >> 2) * 16 + 4 * quad + (e & 3);
          const bool vis = row_ok[q] && key >= my_lo[q] && key <= my_p[q];
          sv[q][e] = vis ? sv[q][e] : -INFINITY;
        }
    }

    f32x4 sn[QB][2];
    scores((j + 1) & 1, sn);

    // Online softmax of tile j; the weights as the PV product's A operand.
    bf16x8 ph[QB], pl[QB];
    float alpha[QB];
    bool bump[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      float mt = sv[q][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mt = fmaxf(mt, sv[q][e]);
      mt = pair_max_16_32(mt);
      // m is a reference, not always the running max: it moves only when a
      // tile's max exceeds it by more than kSlack (log2 units), so the
      // weights stay below 2^kSlack and most tiles need no rescale.  The
      // final normalisation divides by l, which carries the same reference.
      bump[q] = mt > m[q] + kSlack;  // m = -inf: any visible key bumps
      const float m_new = bump[q] ? mt : m[q];
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;  // no key yet: keep weights 0
      alpha[q] = __builtin_amdgcn_exp2f(m[q] - m_use);           // m = -inf gives 0
      float p[8];
      float ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(sv[q][e] - m_use);
        ps += p[e];
      }
      ps = pair_sum_16_32(ps);
      l[q] = l[q] * alpha[q] + ps;
      m[q] = m_new;
      // int8 values: the weight of key j carries its value scale (the
      // codes are the V operand), the sum l does not.
      if constexpr (VT == kI8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] *= vsc[j & 1][(e < 4) ? 4 * quad + e : 16 + 4 * quad + (e - 4)];
      }
      split8(p, ph[q], pl[q]);
    }
    // Rescale the accumulator: its rows are queries 4*quad + j, whose alpha
    // lives in lane 4*quad + j.  Skipped when no query's reference moved
    // (every alpha is 1, or 0 for a query with no key yet, whose row is
    // still 0).
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      if (__builtin_amdgcn_ballot_w64(bump[q]) != 0) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float aj = __shfl(alpha[q], 4 * quad + jj);
#pragma unroll
          for (int n = 0; n < NB; ++n) o[q][n][jj] *= aj;
        }
      }
    }

    // O += P V.  A operand: lane holds P[qi][k = 8*quad + e], where k < 4 of
    // the lane's group maps to key 4*quad + e and k >= 4 to key 16 + 4*quad +
    // (e - 4) (the same keys the lane's S^T registers hold).  The B operand
    // needs V at those keys in dim n*16 + qi: two transposing LDS reads
    // (ds_read_b64_tr_b16).  Within each 16-lane group, the reading lane s
    // points at 4 dims (n*16 + 4*(s%4) ..) of key base + s/4, and lane i
    // receives dim n*16 + i of keys base .. base + 3.
    const uint16_t* vb_ = vs[j & 1];
    const int tr_row = 4 * quad + (qi >> 2), tr_col = 4 * (qi & 3);
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      const s16x4 v0 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb_[tr_row * LS + n * 16 + tr_col]));
      const s16x4 v1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(&vb_[(16 + tr_row) * LS + n * 16 + tr_col]));
      const s16x8 vv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
      const bf16x8 vb = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        o[q][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph[q], vb, o[q][n], 0, 0, 0);
        o[q][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl[q], vb, o[q][n], 0, 0, 0);
      }
    }
    __syncthreads();  // tile j's buffers are read; the stores above are visible
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) s[q][mb] = sn[q][mb];
  }

  // Normalise (with the sink, if any) and write.  Accumulator rows are
  // queries 4*quad + j of each block; their m and l live in lane 4*quad + j.
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    float sink2 = -INFINITY;
    if (a.sinks != nullptr && row_ok[q]) sink2 = a.sinks[kvh * G + my_g[q]] * kLog2eP;
    const float m_fin = fmaxf(m[q], sink2);
    const float keep = __builtin_amdgcn_exp2f(m[q] - m_fin);
    const float den = l[q] * keep + __builtin_amdgcn_exp2f(sink2 - m_fin);
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
