// Per-vector math of the KV producer, shared by the standalone producer
// (kv_produce.hip) and the fused single-launch step (decode_partial_kernel.h):
// QK-RMSNorm, RoPE at an absolute position, and the storage formats of the
// cache (f32, bf16 round-to-nearest-even, int8 with one f32 scale per row).
//
// Sources: "Universal AI Inference - Hugging Face decoder completeness"
// (P0.2 RoPE scaling, P1.1 RMSNorm gain (1+w), P1.2 QK-norm before RoPE,
// P1.3 absolute positions); "llamay - Models and formats" (Architectures:
// interleaved vs NeoX rotary, gpt-oss YaRN; The KV cache, in three
// precisions: vq8 and q8); "Algenta - Model support matrix" (Decoder
// families: linear scaling); "FreeToken PR #722" (Changes: Llama-3 scaling
// constants).
//
// One 64-lane wave handles one head vector: lane l holds elements l + 64 e
// and rotates pairs i = l + 64 j.  The norm and the rotation run in double
// precision and round once to the stored format.  Every function body turns
// off floating-point contraction, so the result does not depend on where it
// is inlined.
#pragma once

#include <math.h>

#include "launch.h"

namespace uaii {
namespace pm {

__device__ inline double wave_sum_d(double x) {
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ inline float wave_max_f(float x) {
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// LDS hand-off between the lanes of one wave.
__device__ inline void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Round a double to the nearest bf16 (ties to even) straight from its bits:
// in the normal range, round the 52-bit fraction to 7 bits on the integer
// magnitude (a carry into the exponent is the correct result), then rebias
// the exponent from 1023 to 127; below 2^-126 round on the fixed subnormal
// grid 2^-133.  Overflow gives infinity.  Inputs here are finite.
__device__ inline uint16_t bf16_from_double(double x) {
#pragma clang fp contract(off)
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(x));
  const uint32_t sign = static_cast<uint32_t>(u >> 48) & 0x8000u;
  const uint64_t mag = u & 0x7FFFFFFFFFFFFFFFull;
  const int exp = static_cast<int>(mag >> 52) - 1023;
  if (exp >= -126) {
    const uint64_t rounded = (mag + 0x00000FFFFFFFFFFFull + ((mag >> 45) & 1ull)) >> 45;
    uint64_t bits = rounded - (static_cast<uint64_t>(1023 - 127) << 7);
    if (bits >= 0x7F80ull) bits = 0x7F80ull;
    return static_cast<uint16_t>(sign | static_cast<uint32_t>(bits));
  }
  const double r = rint(fabs(x) * 0x1p133);  // 0..128, exact scaling
  return static_cast<uint16_t>(sign | static_cast<uint32_t>(r));
}

__device__ inline float bf16_to_float(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

template <int D>
struct Shape {
  static constexpr int EPL = D / 64;             // elements per lane
  static constexpr int NP = (D / 2 + 63) / 64;   // rotation pairs per lane
};

// cos and sin of pos * g_i for this lane's pairs i = lane + 64 j (g_i from
// the host's frequency table).
template <int D>
struct Angles {
  double cs[Shape<D>::NP], sn[Shape<D>::NP];
};

template <int D>
__device__ inline void rope_angles(const ProduceArgs& a, int pos, int lane, Angles<D>& an) {
#pragma clang fp contract(off)
#pragma unroll
  for (int j = 0; j < Shape<D>::NP; ++j) {
    const int i = lane + 64 * j;
    an.cs[j] = 1.0;
    an.sn[j] = 0.0;
    if (i < D / 2) sincos(static_cast<double>(pos) * a.freq[i], &an.sn[j], &an.cs[j]);
  }
}

// One head vector after the norm and the rotation: pair j of this lane holds
// elements (ia[j], ib[j]) with values (ya[j], yb[j]); ok[j] is false for
// lanes past the last pair (d = 64).
template <int D>
struct Rotated {
  int ia[Shape<D>::NP], ib[Shape<D>::NP];
  double ya[Shape<D>::NP], yb[Shape<D>::NP];
  bool ok[Shape<D>::NP];
};

// Norm (if enabled, with weight w) and RoPE of the head vector x (lane holds
// x[e] = element lane + 64 e), then YaRN's attention factor.  sx is this
// wave's LDS staging array of D doubles; it is free again on return.
template <int D>
__device__ inline void norm_rope(const ProduceArgs& a, const float (&x)[Shape<D>::EPL], const float* w,
                                 const Angles<D>& an, double* sx, int lane, Rotated<D>& r) {
#pragma clang fp contract(off)
  constexpr int EPL = Shape<D>::EPL;
  double xv[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) xv[e] = static_cast<double>(x[e]);
  if (a.norm_enabled) {
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) ss += xv[e] * xv[e];
    ss = wave_sum_d(ss);
    const double rr = 1.0 / sqrt(ss / static_cast<double>(D) + static_cast<double>(a.norm_eps));
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      xv[e] = xv[e] * rr * (static_cast<double>(w[lane + 64 * e]) + static_cast<double>(a.norm_offset));
  }
#pragma unroll
  for (int e = 0; e < EPL; ++e) sx[lane + 64 * e] = xv[e];
  wave_sync();
#pragma unroll
  for (int j = 0; j < Shape<D>::NP; ++j) {
    const int i = lane + 64 * j;
    r.ok[j] = i < D / 2;
    const int ii = r.ok[j] ? i : 0;
    const int ia = (a.pairing == kNeox) ? ii : 2 * ii;
    const int ib = (a.pairing == kNeox) ? ii + D / 2 : 2 * ii + 1;
    const double c = an.cs[j], sv = an.sn[j];
    const double xa = sx[ia], xb = sx[ib];
    double ya = xa * c - xb * sv;
    double yb = xa * sv + xb * c;
    if (a.attn_factor != 1.0) {  // YaRN scales the rotated q and k
      ya *= a.attn_factor;
      yb *= a.attn_factor;
    }
    r.ia[j] = ia;
    r.ib[j] = ib;
    r.ya[j] = ya;
    r.yb[j] = yb;
  }
  wave_sync();  // sx may be overwritten by the caller from here on
}

// Symmetric int8 quantiser of one row held across the wave, E values per
// lane at element indices idx[e] (valid[e] false for padding): scale =
// max|x| / 127 in f32, code = clamp(round_half_away(x / scale), -127, 127);
// an all-zero row gives scale 0 and codes 0.  Writes the codes to dst and
// the scale through scale_out (lane 0); returns the scale and leaves the
// codes (as floats) in code.  Used for vq8 values and q8 keys.
template <int E>
__device__ inline float quantize_row(const float (&x)[E], const int (&idx)[E], const bool (&valid)[E],
                                     int8_t* dst, float* scale_out, int lane, float (&code)[E]) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (valid[e]) amax = fmaxf(amax, fabsf(x[e]));
  amax = wave_max_f(amax);
  const float scale = amax == 0.0f ? 0.0f : __fdiv_rn(amax, 127.0f);
#pragma unroll
  for (int e = 0; e < E; ++e) {
    float r = 0.0f;
    if (valid[e] && amax != 0.0f) {
      r = roundf(__fdiv_rn(x[e], scale));
      r = fminf(fmaxf(r, -127.0f), 127.0f);
    }
    code[e] = r;
    if (valid[e]) dst[idx[e]] = static_cast<int8_t>(static_cast<int>(r));
  }
  if (lane == 0) *scale_out = scale;
  return scale;
}

// Element offset of slot pos of (b, u): contiguous [B][Hkv][cap][D], or
// paged [num_blocks][Hkv][bs][D] through the block table (ids outside the
// pool are clamped, so a bad table cannot write outside it).
template <int D>
__device__ inline int64_t cache_slot(const ProduceArgs& a, int b, int u, int pos) {
  if (a.block_table != nullptr) {
    int pid = a.block_table[static_cast<int64_t>(b) * a.max_blocks + pos / a.block_size];
    pid = min(max(pid, 0), a.num_blocks - 1);
    return ((static_cast<int64_t>(pid) * a.Hkv + u) * a.block_size + pos % a.block_size) * D;
  }
  return ((static_cast<int64_t>(b) * a.Hkv + u) * a.cap + pos) * D;
}

// Store the rotated key r in the cache's key format at element offset slot.
// kst receives the stored values widened to f32 (pair j: kst[2j] at ia[j],
// kst[2j + 1] at ib[j]); q8 keys are the rotated key rounded to f32, then
// quantised (code * scale).
template <int D>
__device__ inline void store_key(const ProduceArgs& a, const Rotated<D>& r, int64_t slot, int lane,
                                 float (&kst)[2 * Shape<D>::NP]) {
#pragma clang fp contract(off)
  constexpr int NP = Shape<D>::NP;
  if (a.k_dtype == kI8) {
    float kq[2 * NP], code[2 * NP];
    int idx[2 * NP];
    bool ok[2 * NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      kq[2 * j] = r.ok[j] ? static_cast<float>(r.ya[j]) : 0.0f;
      kq[2 * j + 1] = r.ok[j] ? static_cast<float>(r.yb[j]) : 0.0f;
      idx[2 * j] = r.ia[j];
      idx[2 * j + 1] = r.ib[j];
      ok[2 * j] = ok[2 * j + 1] = r.ok[j];
    }
    const float s = quantize_row<2 * NP>(kq, idx, ok, static_cast<int8_t*>(a.k) + slot, a.k_scale + slot / D,
                                         lane, code);
#pragma unroll
    for (int e = 0; e < 2 * NP; ++e) kst[e] = code[e] * s;
    return;
  }
#pragma unroll
  for (int j = 0; j < NP; ++j) {
    kst[2 * j] = kst[2 * j + 1] = 0.0f;
    if (!r.ok[j]) continue;
    if (a.k_dtype == kF32) {
      float* k = static_cast<float*>(a.k) + slot;
      kst[2 * j] = static_cast<float>(r.ya[j]);
      kst[2 * j + 1] = static_cast<float>(r.yb[j]);
      k[r.ia[j]] = kst[2 * j];
      k[r.ib[j]] = kst[2 * j + 1];
    } else {
      uint16_t* k = static_cast<uint16_t*>(a.k) + slot;
      const uint16_t ba = bf16_from_double(r.ya[j]), bb = bf16_from_double(r.yb[j]);
      k[r.ia[j]] = ba;
      k[r.ib[j]] = bb;
      kst[2 * j] = bf16_to_float(ba);
      kst[2 * j + 1] = bf16_to_float(bb);
    }
  }
}

// Store the value row v (lane holds elements lane + 64 e) at element offset
// slot: f32 as given, bf16 rounded to nearest even, or int8 quantised.  vst
// receives the stored values widened to f32 (int8: code * scale).
template <int D>
__device__ inline void store_value(const ProduceArgs& a, const float (&v)[Shape<D>::EPL], int64_t slot, int lane,
                                   float (&vst)[Shape<D>::EPL]) {
#pragma clang fp contract(off)
  constexpr int EPL = Shape<D>::EPL;
  if (a.v_dtype == kF32) {
    float* dst = static_cast<float*>(a.v) + slot;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      dst[lane + 64 * e] = v[e];
      vst[e] = v[e];
    }
  } else if (a.v_dtype == kBF16) {
    uint16_t* dst = static_cast<uint16_t*>(a.v) + slot;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const uint16_t bits = bf16_from_double(static_cast<double>(v[e]));
      dst[lane + 64 * e] = bits;
      vst[e] = bf16_to_float(bits);
    }
  } else {
    int idx[EPL];
    bool ok[EPL];
    float code[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      idx[e] = lane + 64 * e;
      ok[e] = true;
    }
    const float s = quantize_row<EPL>(v, idx, ok, static_cast<int8_t*>(a.v) + slot, a.v_scale + slot / D, lane, code);
#pragma unroll
    for (int e = 0; e < EPL; ++e) vst[e] = code[e] * s;
  }
}

}  // namespace pm
}  // namespace uaii
