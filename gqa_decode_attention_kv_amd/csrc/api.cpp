// C-ABI entry points of the GQA decode-step library: argument validation
// (fail closed, typed messages), the per-sequence work table, and the
// kernel launches on the caller's stream.  See include/uaii_decode.h for
// the contract of each call.
//
// Refusals are typed and specific, after "Algenta - Model support matrix"
// (Conformance CLI: the refusal identifies the offending fact with its value
// and the accepted range) and "Universal AI Inference - Hugging Face decoder
// completeness" (section 6 on error messages, which state the failure and
// the remedy; support contract: unsupported inputs fail closed as
// InvalidArgument or NotImplemented).
#include "uaii_decode.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "launch.h"
#include "prefill_args.h"

namespace {

thread_local std::string g_error;

uaii_status fail(uaii_status st, const char* fn, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = std::string(fn) + ": " + buf;
  return st;
}

#define REQUIRE(cond, st, ...)                    \
  do {                                            \
    if (!(cond)) return fail((st), fn, __VA_ARGS__); \
  } while (0)

constexpr uaii_status kInvalid = UAII_ERR_INVALID_ARGUMENT;
constexpr uaii_status kNotImpl = UAII_ERR_NOT_IMPLEMENTED;
constexpr int32_t kMaxCapacity = 1 << 30;

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) & (n - 1)) == 0; }

uaii_status check_device_ptr(const char* fn, const char* name, const void* p, uintptr_t align) {
  REQUIRE(p != nullptr, kInvalid, "%s is NULL; pass a device buffer", name);
  REQUIRE(aligned(p, align), kInvalid, "%s=%p is not %u-byte aligned; allocate it with the device allocator",
          name, p, static_cast<unsigned>(align));
  return UAII_OK;
}

#define CHECK_PTR(name, p, align)                                        \
  do {                                                                   \
    uaii_status st_ = check_device_ptr(fn, (name), (p), (align));        \
    if (st_ != UAII_OK) return st_;                                      \
  } while (0)

uaii_status check_shape(const char* fn, const uaii_attn_shape* s) {
  REQUIRE(s != nullptr, kInvalid, "shape is NULL; pass a uaii_attn_shape");
  REQUIRE(s->batch >= 1, kInvalid, "batch=%d is invalid (must be >= 1)", s->batch);
  REQUIRE(s->batch <= uaii::kMaxBatch, kNotImpl,
          "batch=%d is not supported (supported: 1..%d); split the batch into calls of at most %d sequences",
          s->batch, uaii::kMaxBatch, uaii::kMaxBatch);
  REQUIRE(s->n_heads >= 1, kInvalid, "n_heads=%d is invalid (must be >= 1)", s->n_heads);
  REQUIRE(s->n_kv_heads >= 1, kInvalid, "n_kv_heads=%d is invalid (must be >= 1)", s->n_kv_heads);
  REQUIRE(s->n_heads <= 65535, kNotImpl, "n_heads=%d is not supported (supported: 1..65535)",
          s->n_heads);
  REQUIRE(s->n_heads % s->n_kv_heads == 0, kInvalid,
          "n_heads=%d is not an exact multiple of n_kv_heads=%d (the GQA ratio must be integral)",
          s->n_heads, s->n_kv_heads);
  REQUIRE(s->head_dim >= 1, kInvalid, "head_dim=%d is invalid (must be >= 1)", s->head_dim);
  REQUIRE(s->head_dim == 64 || s->head_dim == 128 || s->head_dim == 256, kNotImpl,
          "head_dim=%d is not supported (supported: {64, 128, 256})", s->head_dim);
  const int g = s->n_heads / s->n_kv_heads;
  REQUIRE(g == 1 || g == 2 || g == 4 || g == 8, kNotImpl,
          "GQA ratio n_heads/n_kv_heads=%d is not supported (supported: {1, 2, 4, 8})", g);
  return UAII_OK;
}

uaii_status check_cache(const char* fn, const uaii_kv_cache* c) {
  REQUIRE(c != nullptr, kInvalid, "cache is NULL; pass a uaii_kv_cache");
  REQUIRE(c->k_dtype == UAII_F32 || c->k_dtype == UAII_BF16 || c->k_dtype == UAII_I8, kInvalid,
          "k_dtype=%d is not a dtype code (f32=0, bf16=1, int8=2)", c->k_dtype);
  REQUIRE(c->v_dtype == UAII_F32 || c->v_dtype == UAII_BF16 || c->v_dtype == UAII_I8, kInvalid,
          "v_dtype=%d is not a dtype code (f32=0, bf16=1, int8=2)", c->v_dtype);
  REQUIRE(c->k_dtype != UAII_I8 || c->v_dtype == UAII_I8, kNotImpl,
          "k_dtype=int8 with v_dtype=%d is not supported (supported: int8 keys only in the q8 cache, "
          "with int8 values); use f32 or bf16 keys, or v_dtype int8",
          c->v_dtype);
  REQUIRE(c->capacity >= 1, kInvalid, "capacity=%d is invalid (must be >= 1)", c->capacity);
  REQUIRE(c->capacity <= kMaxCapacity, kNotImpl, "capacity=%d is not supported (supported: 1..%d)",
          c->capacity, kMaxCapacity);
  if (c->block_table != nullptr) {
    const int32_t bs = c->block_size;
    REQUIRE(bs >= 16 && bs <= 1024 && (bs & (bs - 1)) == 0, kNotImpl,
            "block_size=%d is not supported (supported: a power of two in [16, 1024])", bs);
    REQUIRE(c->max_blocks >= 1, kInvalid, "max_blocks=%d is invalid (must be >= 1)", c->max_blocks);
    REQUIRE(c->num_blocks >= 1, kInvalid, "num_blocks=%d is invalid (must be >= 1)", c->num_blocks);
    REQUIRE(static_cast<int64_t>(c->max_blocks) * bs == c->capacity, kInvalid,
            "capacity=%d must equal max_blocks*block_size=%lld for a paged cache", c->capacity,
            static_cast<long long>(c->max_blocks) * bs);
    CHECK_PTR("cache.block_table", c->block_table, 4);
  }
  CHECK_PTR("cache.k", c->k, 16);
  CHECK_PTR("cache.v", c->v, 16);
  if (c->v_dtype == UAII_I8) {
    REQUIRE(c->v_scale != nullptr, kInvalid,
            "cache.v_scale is NULL but v_dtype is int8 (vq8 needs one f32 scale per token per kv head)");
    CHECK_PTR("cache.v_scale", c->v_scale, 4);
  }
  if (c->k_dtype == UAII_I8) {
    REQUIRE(c->k_scale != nullptr, kInvalid,
            "cache.k_scale is NULL but k_dtype is int8 (q8 needs one f32 key scale per token per kv head)");
    CHECK_PTR("cache.k_scale", c->k_scale, 4);
  }
  return UAII_OK;
}

bool finite_pos(double x) { return std::isfinite(x) && x > 0.0; }

// Visible keys [lo, L) and the splits [first, last] that intersect them,
// and the launch order of the splits (SeqTable: body splits first, then
// the last splits by decreasing visible keys).  Returns true when the
// splits do not all hold the same number of visible keys.
bool build_table(int B, const int32_t* lens, int32_t window, int32_t split, uaii::SeqTable* t) {
  std::memset(t, 0, sizeof *t);
  int32_t prefix = 0, body = 0;
  int32_t tail_rows[uaii::kMaxBatch];
  int32_t rmin = split, rmax = 0;
  auto rows = [&](int32_t r) {
    rmin = std::min(rmin, r);
    rmax = std::max(rmax, r);
  };
  for (int b = 0; b < B; ++b) {
    const int32_t L = lens[b];
    const int32_t lo = (window > 0 && L > window) ? L - window : 0;
    const int32_t first = lo / split, last = (L - 1) / split;
    t->len[b] = L;
    t->lo[b] = lo;
    t->first_split[b] = first;
    t->work_prefix[b] = prefix;
    prefix += last - first + 1;
    t->body_prefix[b] = body;
    body += last - first;
    tail_rows[b] = L - std::max(last * split, lo);
    t->tail_order[b] = b;
    rows(tail_rows[b]);
    if (last > first) rows((first + 1) * split - lo);
    if (last > first + 1) rows(split);
  }
  t->work_prefix[B] = prefix;
  t->body_prefix[B] = body;
  t->n_seq = B;
  std::stable_sort(t->tail_order, t->tail_order + B,
                   [&](int32_t x, int32_t y) { return tail_rows[x] > tail_rows[y]; });
  return rmin != rmax;
}

uaii_status device_status(const char* fn, hipError_t e) {
  if (e == hipSuccess) return UAII_OK;
  return fail(UAII_ERR_DEVICE, fn, "HIP error %d (%s) while enqueuing the kernel", static_cast<int>(e),
              hipGetErrorString(e));
}

uaii_status check_lens(const char* fn, const uaii_attn_shape* s, const int32_t* seq_lens, int32_t cap,
                       int32_t split_size, int32_t max_splits, int32_t window) {
  REQUIRE(seq_lens != nullptr, kInvalid, "seq_lens is NULL; pass a host array of batch=%d lengths",
          s->batch);
  REQUIRE(window >= 0, kInvalid, "window=%d is invalid (0 = no window, W > 0 keeps the last W keys)",
          window);
  REQUIRE(split_size >= 1, kInvalid, "split_size=%d is invalid (must be >= 1)", split_size);
  int32_t max_len = 0;
  for (int b = 0; b < s->batch; ++b) {
    REQUIRE(seq_lens[b] >= 1 && seq_lens[b] <= cap, kInvalid,
            "seq_lens[%d]=%d is outside [1, %d] (keys including the new token, at most the capacity)", b,
            seq_lens[b], cap);
    if (seq_lens[b] > max_len) max_len = seq_lens[b];
  }
  const int64_t need = (static_cast<int64_t>(max_len) + split_size - 1) / split_size;
  REQUIRE(max_splits >= need, kInvalid,
          "max_splits=%d is too small: seq_lens up to %d with split_size=%d need %lld splits", max_splits,
          max_len, split_size, static_cast<long long>(need));
  int64_t work = 0;
  for (int b = 0; b < s->batch; ++b) {
    const int64_t L = seq_lens[b];
    const int64_t lo = (window > 0 && L > window) ? L - window : 0;
    work += (L - 1) / split_size - lo / split_size + 1;
  }
  work *= s->n_kv_heads;
  REQUIRE(work <= (int64_t{1} << 30), kNotImpl,
          "%lld (split, kv head) work items are not supported (supported: up to 2^30); use a larger "
          "split_size",
          static_cast<long long>(work));
  return UAII_OK;
}

// Rotary frequency g_i of every pair i < d/2 over the full head, with the
// scheme's scaling ("Universal AI Inference - Hugging Face decoder
// completeness", P0.2: plain theta, Llama-3 scaling matching Hugging Face,
// YaRN; "FreeToken PR #722", Changes: Llama-3 band constants; "Algenta -
// Model support matrix", Decoder families: linear scaling).  f_i =
// theta^(-2i/d).  Llama-3: with wavelength 2 pi / f, keep f below
// original/high, divide by factor above original/low, blend linearly in
// original/wavelength between.  Linear: f / factor.  YaRN: blend f / factor
// and f with a weight linear in the pair index between the indices that
// turn beta_fast and beta_slow times over the original context (rounded
// outwards when truncate is set).  Evaluated once per call in double.
void rope_freqs(const uaii_rope* r, int d, double* g) {
  const double pi = 3.14159265358979323846;
  double c_lo = 0.0, c_hi = 1.0;
  if (r->scaling == UAII_ROPE_YARN) {
    const double orig = static_cast<double>(r->original_max_position);
    c_lo = d * std::log(orig / (2.0 * pi * r->high_freq_factor)) / (2.0 * std::log(r->theta));
    c_hi = d * std::log(orig / (2.0 * pi * r->low_freq_factor)) / (2.0 * std::log(r->theta));
    if (r->truncate) {
      c_lo = std::floor(c_lo);
      c_hi = std::ceil(c_hi);
    }
    c_lo = std::max(c_lo, 0.0);
    c_hi = std::min(c_hi, d - 1.0);
    if (c_hi == c_lo) c_hi += 0.001;
  }
  for (int i = 0; i < d / 2; ++i) {
    const double f = std::pow(r->theta, -2.0 * static_cast<double>(i) / static_cast<double>(d));
    double gi = f;
    if (r->scaling == UAII_ROPE_LINEAR) {
      gi = f / r->factor;
    } else if (r->scaling == UAII_ROPE_YARN) {
      const double t = std::min(std::max((static_cast<double>(i) - c_lo) / (c_hi - c_lo), 0.0), 1.0);
      gi = t * f / r->factor + (1.0 - t) * f;
    } else if (r->scaling == UAII_ROPE_LLAMA3) {
      const double orig = static_cast<double>(r->original_max_position);
      const double wavelen = 2.0 * pi / f;
      if (wavelen < orig / r->high_freq_factor) {
        gi = f;
      } else if (wavelen > orig / r->low_freq_factor) {
        gi = f / r->factor;
      } else {
        const double mu = (orig / wavelen - r->low_freq_factor) / (r->high_freq_factor - r->low_freq_factor);
        gi = (1.0 - mu) * f / r->factor + mu * f;
      }
    }
    g[i] = gi;
  }
}

// Checks the producer's arguments (rope, norm, inputs, q_out) and fills
// everything in ProduceArgs except the positions.  Shape and cache are
// checked by the caller.
uaii_status produce_args(const char* fn, const uaii_attn_shape* shape, const uaii_rope* rope,
                         const uaii_qk_norm* qk_norm, const float* q_in, const float* k_in,
                         const float* v_in, const uaii_kv_cache* cache, float* q_out,
                         uaii::ProduceArgs* out) {
  REQUIRE(rope != nullptr, kInvalid, "rope is NULL; pass a uaii_rope");
  REQUIRE(rope->pairing == UAII_ROPE_NEOX || rope->pairing == UAII_ROPE_INTERLEAVED, kInvalid,
          "rope.pairing=%d is not a pairing code (neox=0, interleaved=1)", rope->pairing);
  REQUIRE(rope->scaling >= UAII_ROPE_PLAIN && rope->scaling <= UAII_ROPE_YARN, kNotImpl,
          "unsupported rope_scaling.type=%d (supported: plain=0, llama3=1, linear=2, yarn=3)",
          rope->scaling);
  REQUIRE(finite_pos(rope->theta), kInvalid, "rope.theta=%g is invalid (must be finite and > 0)",
          rope->theta);
  if (rope->scaling == UAII_ROPE_LINEAR)
    REQUIRE(finite_pos(rope->factor), kInvalid,
            "rope.factor=%g is invalid for linear scaling (must be finite and > 0)", rope->factor);
  if (rope->scaling == UAII_ROPE_YARN) {
    REQUIRE(std::isfinite(rope->factor) && rope->factor >= 1.0, kInvalid,
            "rope.factor=%g is invalid for yarn scaling (must be finite and >= 1)", rope->factor);
    REQUIRE(finite_pos(rope->low_freq_factor), kInvalid,
            "rope.low_freq_factor (yarn beta_slow)=%g is invalid (must be finite and > 0)",
            rope->low_freq_factor);
    REQUIRE(std::isfinite(rope->high_freq_factor) && rope->high_freq_factor > rope->low_freq_factor,
            kInvalid, "rope.high_freq_factor (yarn beta_fast)=%g must be finite and > beta_slow=%g",
            rope->high_freq_factor, rope->low_freq_factor);
    REQUIRE(rope->original_max_position > 0, kInvalid,
            "rope.original_max_position=%d is invalid (must be > 0)", rope->original_max_position);
    REQUIRE(std::isfinite(rope->attention_factor) && rope->attention_factor >= 0.0, kInvalid,
            "rope.attention_factor=%g is invalid (must be finite and > 0, or 0 for the default)",
            rope->attention_factor);
  }
  if (rope->scaling == UAII_ROPE_LLAMA3) {
    REQUIRE(std::isfinite(rope->factor) && rope->factor >= 1.0, kInvalid,
            "rope.factor=%g is invalid for llama3 scaling (must be finite and >= 1)", rope->factor);
    REQUIRE(finite_pos(rope->low_freq_factor), kInvalid,
            "rope.low_freq_factor=%g is invalid (must be finite and > 0)", rope->low_freq_factor);
    REQUIRE(std::isfinite(rope->high_freq_factor) && rope->high_freq_factor > rope->low_freq_factor,
            kInvalid, "rope.high_freq_factor=%g must be finite and > low_freq_factor=%g",
            rope->high_freq_factor, rope->low_freq_factor);
    REQUIRE(rope->original_max_position > 0, kInvalid,
            "rope.original_max_position=%d is invalid (must be > 0)", rope->original_max_position);
  }
  const bool norm = qk_norm != nullptr && qk_norm->enabled != 0;
  if (norm) {
    REQUIRE(std::isfinite(qk_norm->eps) && qk_norm->eps > 0.0f, kInvalid,
            "qk_norm.eps=%g is invalid (must be finite and > 0)", static_cast<double>(qk_norm->eps));
    REQUIRE(qk_norm->offset == 0 || qk_norm->offset == 1, kInvalid,
            "qk_norm.offset=%d is invalid (0: gain w, 1: gain 1 + w)", qk_norm->offset);
    CHECK_PTR("qk_norm.q_weight", qk_norm->q_weight, 4);
    CHECK_PTR("qk_norm.k_weight", qk_norm->k_weight, 4);
  }
  CHECK_PTR("q_in", q_in, 16);
  CHECK_PTR("k_in", k_in, 16);
  CHECK_PTR("v_in", v_in, 16);
  CHECK_PTR("q_out", q_out, 16);

  uaii::ProduceArgs a{};
  a.B = shape->batch;
  a.H = shape->n_heads;
  a.Hkv = shape->n_kv_heads;
  a.D = shape->head_dim;
  a.pairing = rope->pairing;
  rope_freqs(rope, shape->head_dim, a.freq);
  a.attn_factor = 1.0;
  if (rope->scaling == UAII_ROPE_YARN)
    a.attn_factor = rope->attention_factor > 0.0
                        ? rope->attention_factor
                        : (rope->factor <= 1.0 ? 1.0 : 0.1 * std::log(rope->factor) + 1.0);
  a.norm_enabled = norm ? 1 : 0;
  a.norm_offset = norm ? qk_norm->offset : 0;
  a.norm_eps = norm ? qk_norm->eps : 0.0f;
  a.w_q = norm ? qk_norm->q_weight : nullptr;
  a.w_k = norm ? qk_norm->k_weight : nullptr;
  a.q_in = q_in;
  a.k_in = k_in;
  a.v_in = v_in;
  a.k_dtype = cache->k_dtype;
  a.v_dtype = cache->v_dtype;
  a.cap = cache->capacity;
  a.k = cache->k;
  a.v = cache->v;
  a.k_scale = cache->k_dtype == UAII_I8 ? cache->k_scale : nullptr;
  a.v_scale = cache->v_dtype == UAII_I8 ? cache->v_scale : nullptr;
  a.q_out = q_out;
  a.block_table = cache->block_table;
  a.block_size = cache->block_table ? cache->block_size : 0;
  a.max_blocks = cache->block_table ? cache->max_blocks : 0;
  a.num_blocks = cache->block_table ? cache->num_blocks : 0;
  a.T = 1;
  a.hpw = 1;
  *out = a;
  return UAII_OK;
}

// Checks the attention arguments (lengths, window, softcap, scale,
// partials) and fills AttnArgs with the work table.  Shape and cache are
// checked by the caller; q is checked here only when check_q is set (the
// fused step computes the queries itself).
uaii_status attn_args(const char* fn, const uaii_attn_shape* shape, const uaii_kv_cache* cache,
                      const float* q, bool check_q, const int32_t* seq_lens, float scale, int32_t window,
                      float softcap, int32_t split_size, int32_t max_splits, float* part_o, float* part_lse,
                      uaii::AttnArgs* out, bool check_parts = true) {
  uaii_status st = check_lens(fn, shape, seq_lens, cache->capacity, split_size, max_splits, window);
  if (st != UAII_OK) return st;
  REQUIRE(std::isfinite(softcap) && softcap >= 0.0f, kInvalid,
          "softcap=%g is invalid (0 = none, c > 0 applies c*tanh(s/c))", static_cast<double>(softcap));
  REQUIRE(std::isfinite(scale), kInvalid, "scale=%g is invalid (must be finite)", static_cast<double>(scale));
  const double want = 1.0 / std::sqrt(static_cast<double>(shape->head_dim));
  REQUIRE(std::fabs(static_cast<double>(scale) - want) <= 1e-6 * want, kNotImpl,
          "scale=%.9g is not supported (supported: 1/sqrt(head_dim)=%.9g; a differing "
          "query_pre_attn_scalar is refused)",
          static_cast<double>(scale), want);
  if (check_q) CHECK_PTR("q", q, 16);
  if (check_parts) {
    CHECK_PTR("part_o", part_o, 16);
    CHECK_PTR("part_lse", part_lse, 4);
  }

  uaii::AttnArgs a{};
  a.H = shape->n_heads;
  a.Hkv = shape->n_kv_heads;
  a.cap = cache->capacity;
  a.split_size = split_size;
  a.max_splits = max_splits;
  a.k = cache->k;
  a.v = cache->v;
  a.k_scale = cache->k_dtype == UAII_I8 ? cache->k_scale : nullptr;
  a.v_scale = cache->v_dtype == UAII_I8 ? cache->v_scale : nullptr;
  a.q = q;
  a.part_o = part_o;
  a.part_lse = part_lse;
  const float log2e = 1.4426950408889634f;
  const float s = static_cast<float>(want);
  a.q_mul = softcap > 0.0f ? s : s * log2e;
  a.softcap = softcap;
  const bool uneven = build_table(shape->batch, seq_lens, window, split_size, &a.t);
  a.coop = a.t.work_prefix[shape->batch] * shape->n_kv_heads < uaii::kCoopBelow ? 1 : 0;
  a.serp = (!a.coop && uneven) ? 1 : 0;
  if (cache->block_table != nullptr) {
    a.block_table = cache->block_table;
    a.block_size = cache->block_size;
    a.log2_bs = 0;
    while ((1 << a.log2_bs) < cache->block_size) ++a.log2_bs;
    a.max_blocks = cache->max_blocks;
    a.num_blocks = cache->num_blocks;
  }
  *out = a;
  return UAII_OK;
}

// The one-call step (validation, then one kernel or three) shared by
// uaii_decode_step and uaii_decode_step_noalloc; fn names the entry point
// in messages.  With scratch set, part_o, part_lse and counters are ignored
// and taken from the GPU's static scratch once every argument has passed.
uaii_status decode_step_impl(const char* fn, const uaii_attn_shape* shape, const uaii_rope* rope,
                             const uaii_qk_norm* qk_norm, const float* q_in, const float* k_in,
                             const float* v_in, const int32_t* seq_lens, const uaii_kv_cache* cache,
                             float scale, int32_t window, float softcap, int32_t split_size,
                             int32_t max_splits, const float* sinks, float* q_out, float* part_o,
                             float* part_lse, int32_t* counters, float* out, void* stream,
                             bool scratch);

}  // namespace

extern "C" {

const char* uaii_last_error(void) { return g_error.c_str(); }

uaii_status uaii_kv_produce(const uaii_attn_shape* shape, const uaii_rope* rope,
                            const uaii_qk_norm* qk_norm, const float* q_in, const float* k_in,
                            const float* v_in, const int32_t* positions, const uaii_kv_cache* cache,
                            float* q_out, void* stream) {
  const char* fn = "uaii_kv_produce";
  g_error.clear();
  uaii_status st = check_shape(fn, shape);
  if (st != UAII_OK) return st;
  st = check_cache(fn, cache);
  if (st != UAII_OK) return st;
  uaii::ProduceArgs a{};
  st = produce_args(fn, shape, rope, qk_norm, q_in, k_in, v_in, cache, q_out, &a);
  if (st != UAII_OK) return st;
  REQUIRE(positions != nullptr, kInvalid, "positions is NULL; pass a host array of batch=%d positions",
          shape->batch);
  for (int b = 0; b < shape->batch; ++b)
    REQUIRE(positions[b] >= 0 && positions[b] < cache->capacity, kInvalid,
            "positions[%d]=%d is outside [0, capacity=%d)", b, positions[b], cache->capacity);
  for (int b = 0; b < shape->batch; ++b) a.pos[b] = positions[b];
  return device_status(fn, uaii::launch_kv_produce(a, static_cast<hipStream_t>(stream)));
}

uaii_status uaii_decode_attn(const uaii_attn_shape* shape, const uaii_kv_cache* cache, const float* q,
                             const int32_t* seq_lens, float scale, int32_t window, float softcap,
                             int32_t split_size, int32_t max_splits, float* part_o, float* part_lse,
                             void* stream) {
  const char* fn = "uaii_decode_attn";
  g_error.clear();
  uaii_status st = check_shape(fn, shape);
  if (st != UAII_OK) return st;
  st = check_cache(fn, cache);
  if (st != UAII_OK) return st;
  uaii::AttnArgs a{};
  st = attn_args(fn, shape, cache, q, true, seq_lens, scale, window, softcap, split_size, max_splits, part_o,
                 part_lse, &a);
  if (st != UAII_OK) return st;
  const int G = shape->n_heads / shape->n_kv_heads;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (cache->block_table != nullptr)
    return device_status(
        fn, uaii::launch_decode_partial_paged(shape->head_dim, G, cache->k_dtype, cache->v_dtype, a, s));
  return device_status(fn,
                       uaii::launch_decode_partial(shape->head_dim, G, cache->k_dtype, cache->v_dtype, a, s));
}

uaii_status uaii_kv_produce_chunk(const uaii_attn_shape* shape, const uaii_rope* rope,
                                  const uaii_qk_norm* qk_norm, const float* q_in, const float* k_in,
                                  const float* v_in, const int32_t* start_positions, int32_t n_tokens,
                                  const uaii_kv_cache* cache, float* q_out, void* stream) {
  const char* fn = "uaii_kv_produce_chunk";
  g_error.clear();
  uaii_status st = check_shape(fn, shape);
  if (st != UAII_OK) return st;
  st = check_cache(fn, cache);
  if (st != UAII_OK) return st;
  uaii::ProduceArgs a{};
  st = produce_args(fn, shape, rope, qk_norm, q_in, k_in, v_in, cache, q_out, &a);
  if (st != UAII_OK) return st;
  REQUIRE(n_tokens >= 1, kInvalid, "n_tokens=%d is invalid (must be >= 1)", n_tokens);
  REQUIRE(n_tokens <= 65535, kNotImpl, "n_tokens=%d is not supported (supported: 1..65535 per call)",
          n_tokens);
  REQUIRE(start_positions != nullptr, kInvalid,
          "start_positions is NULL; pass a host array of batch=%d positions", shape->batch);
  for (int b = 0; b < shape->batch; ++b)
    REQUIRE(start_positions[b] >= 0 &&
                static_cast<int64_t>(start_positions[b]) + n_tokens <= cache->capacity,
            kInvalid, "start_positions[%d]=%d with n_tokens=%d is outside [0, capacity=%d]", b,
            start_positions[b], n_tokens, cache->capacity);
  a.T = n_tokens;
  // Several tokens: each wave rotates up to 8 head vectors of a token with
  // one evaluation of that token's angles.
  a.hpw = n_tokens > 1 ? std::min(8, shape->n_heads + shape->n_kv_heads) : 1;
  for (int b = 0; b < shape->batch; ++b) a.pos[b] = start_positions[b];
  return device_status(fn, uaii::launch_kv_produce(a, static_cast<hipStream_t>(stream)));
}

uaii_status uaii_prefill_attn(const uaii_attn_shape* shape, const uaii_kv_cache* cache, const float* q,
                              const int32_t* seq_lens, int32_t n_tokens, float scale, int32_t window,
                              float softcap, const float* sinks, float* out, void* stream) {
  const char* fn = "uaii_prefill_attn";
  g_error.clear();
  uaii_status st = check_shape(fn, shape);
  if (st != UAII_OK) return st;
  st = check_cache(fn, cache);
  if (st != UAII_OK) return st;
  REQUIRE((cache->k_dtype == UAII_BF16 && cache->v_dtype == UAII_BF16) ||
              (cache->k_dtype == UAII_BF16 && cache->v_dtype == UAII_I8) ||
              (cache->k_dtype == UAII_I8 && cache->v_dtype == UAII_I8) ||
              (cache->k_dtype == UAII_F32 && cache->v_dtype == UAII_F32),
          kNotImpl,
          "prefill over k_dtype=%d, v_dtype=%d is not supported (supported: bf16 keys with bf16 or int8 "
          "values, int8 keys and values, or f32 keys and values: (1,1), (1,2), (2,2), (0,0))",
          cache->k_dtype, cache->v_dtype);
  REQUIRE(cache->k_dtype != UAII_F32 || shape->head_dim <= 128, kNotImpl,
          "prefill over f32 caches with head_dim=%d is not supported (supported: 64 and 128; the f32 "
          "tiles of head_dim 256 would not fit two work-groups' LDS)",
          shape->head_dim);
  REQUIRE(n_tokens >= 1, kInvalid, "n_tokens=%d is invalid (must be >= 1)", n_tokens);
  REQUIRE(n_tokens <= (1 << 20), kNotImpl, "n_tokens=%d is not supported (supported: 1..%d per call)",
          n_tokens, 1 << 20);
  REQUIRE(seq_lens != nullptr, kInvalid, "seq_lens is NULL; pass a host array of batch=%d lengths",
          shape->batch);
  REQUIRE(window >= 0, kInvalid, "window=%d is invalid (0 = no window, W > 0 keeps the last W keys)",
          window);
  for (int b = 0; b < shape->batch; ++b)
    REQUIRE(seq_lens[b] >= n_tokens && seq_lens[b] <= cache->capacity, kInvalid,
            "seq_lens[%d]=%d is outside [n_tokens=%d, capacity=%d] (keys including the chunk)", b,
            seq_lens[b], n_tokens, cache->capacity);
  REQUIRE(std::isfinite(softcap) && softcap >= 0.0f, kInvalid,
          "softcap=%g is invalid (0 = none, c > 0 applies c*tanh(s/c))", static_cast<double>(softcap));
  REQUIRE(std::isfinite(scale), kInvalid, "scale=%g is invalid (must be finite)", static_cast<double>(scale));
  const double want = 1.0 / std::sqrt(static_cast<double>(shape->head_dim));
  REQUIRE(std::fabs(static_cast<double>(scale) - want) <= 1e-6 * want, kNotImpl,
          "scale=%.9g is not supported (supported: 1/sqrt(head_dim)=%.9g; a differing "
          "query_pre_attn_scalar is refused)",
          static_cast<double>(scale), want);
  CHECK_PTR("q", q, 16);
  CHECK_PTR("out", out, 16);
  if (sinks != nullptr) CHECK_PTR("sinks", sinks, 4);

  uaii::PrefillArgs a{};
  a.H = shape->n_heads;
  a.Hkv = shape->n_kv_heads;
  a.cap = cache->capacity;
  a.T = n_tokens;
  a.window = window;
  a.k = cache->k;
  a.v = cache->v;
  a.q = q;
  a.sinks = sinks;
  a.out = out;
  a.k_scale = cache->k_dtype == UAII_I8 ? cache->k_scale : nullptr;
  a.v_scale = cache->v_dtype == UAII_I8 ? cache->v_scale : nullptr;
  const float s = static_cast<float>(want);
  a.q_mul = softcap > 0.0f ? s : s * 1.4426950408889634f;
  a.softcap = softcap;
  if (cache->block_table != nullptr) {
    a.block_table = cache->block_table;
    a.block_size = cache->block_size;
    a.log2_bs = 0;
    while ((1 << a.log2_bs) < cache->block_size) ++a.log2_bs;
    a.max_blocks = cache->max_blocks;
    a.num_blocks = cache->num_blocks;
  }
  for (int b = 0; b < shape->batch; ++b) a.len[b] = seq_lens[b];
  const int G = shape->n_heads / shape->n_kv_heads;
  return device_status(fn, uaii::launch_prefill_attn(shape->head_dim, G, shape->batch, cache->k_dtype,
                                                     cache->v_dtype, a, static_cast<hipStream_t>(stream)));
}

uaii_status uaii_decode_step(const uaii_attn_shape* shape, const uaii_rope* rope, const uaii_qk_norm* qk_norm,
                             const float* q_in, const float* k_in, const float* v_in, const int32_t* seq_lens,
                             const uaii_kv_cache* cache, float scale, int32_t window, float softcap,
                             int32_t split_size, int32_t max_splits, const float* sinks, float* q_out,
                             float* part_o, float* part_lse, int32_t* counters, float* out, void* stream) {
  g_error.clear();
  return decode_step_impl("uaii_decode_step", shape, rope, qk_norm, q_in, k_in, v_in, seq_lens, cache, scale,
                          window, softcap, split_size, max_splits, sinks, q_out, part_o, part_lse, counters, out,
                          stream, false);
}

uaii_status uaii_decode_step_noalloc(const uaii_attn_shape* shape, const uaii_rope* rope,
                                     const uaii_qk_norm* qk_norm, const float* q_in, const float* k_in,
                                     const float* v_in, const int32_t* seq_lens, const uaii_kv_cache* cache,
                                     float scale, int32_t window, float softcap, int32_t split_size,
                                     const float* sinks, float* q_out, float* out, void* stream) {
  const char* fn = "uaii_decode_step_noalloc";
  g_error.clear();
  uaii_status st = check_shape(fn, shape);
  if (st != UAII_OK) return st;
  st = check_cache(fn, cache);
  if (st != UAII_OK) return st;
  REQUIRE(seq_lens != nullptr, kInvalid, "seq_lens is NULL; pass a host array of batch=%d lengths", shape->batch);
  REQUIRE(split_size >= 1, kInvalid, "split_size=%d is invalid (must be >= 1)", split_size);
  int32_t max_len = 1;
  for (int b = 0; b < shape->batch; ++b) {
    REQUIRE(seq_lens[b] >= 1 && seq_lens[b] <= cache->capacity, kInvalid,
            "seq_lens[%d]=%d is outside [1, capacity=%d]", b, seq_lens[b], cache->capacity);
    max_len = std::max(max_len, seq_lens[b]);
  }
  const int64_t max_splits = (static_cast<int64_t>(max_len) + split_size - 1) / split_size;
  const int64_t rows = static_cast<int64_t>(shape->batch) * shape->n_heads * max_splits;
  const int64_t lse_bytes = (rows * 4 + 255) / 256 * 256;
  const int64_t o_bytes = rows * shape->head_dim * 4;
  const int64_t room = static_cast<int64_t>(uaii::kNoAllocScratchBytes - uaii::kNoAllocCounterBytes);
  REQUIRE(static_cast<int64_t>(shape->batch) * shape->n_kv_heads <= uaii::kNoAllocCounterWords, kNotImpl,
          "batch*n_kv_heads=%lld is not supported (supported: up to %d arrival counters in the static "
          "scratch); use uaii_decode_step with a caller-owned counter buffer",
          static_cast<long long>(shape->batch) * shape->n_kv_heads, uaii::kNoAllocCounterWords);
  REQUIRE(lse_bytes + o_bytes <= room, kNotImpl,
          "the split partials need %lld bytes (batch*n_heads*ceil(max seq_len/split_size)*(head_dim+1)*4, "
          "split_size=%d) and the static scratch holds %lld; raise split_size, or use uaii_decode_step "
          "with caller-owned partial buffers",
          static_cast<long long>(lse_bytes + o_bytes), split_size, static_cast<long long>(room));
  return decode_step_impl(fn, shape, rope, qk_norm, q_in, k_in, v_in, seq_lens, cache, scale, window, softcap,
                          split_size, static_cast<int32_t>(max_splits), sinks, q_out, nullptr, nullptr, nullptr,
                          out, stream, true);
}

}  // extern "C"

namespace {

uaii_status decode_step_impl(const char* fn, const uaii_attn_shape* shape, const uaii_rope* rope,
                             const uaii_qk_norm* qk_norm, const float* q_in, const float* k_in,
                             const float* v_in, const int32_t* seq_lens, const uaii_kv_cache* cache,
                             float scale, int32_t window, float softcap, int32_t split_size,
                             int32_t max_splits, const float* sinks, float* q_out, float* part_o,
                             float* part_lse, int32_t* counters, float* out, void* stream,
                             bool scratch) {
  uaii_status st = check_shape(fn, shape);
  if (st != UAII_OK) return st;
  st = check_cache(fn, cache);
  if (st != UAII_OK) return st;
  uaii::StepArgs x{};
  st = produce_args(fn, shape, rope, qk_norm, q_in, k_in, v_in, cache, q_out, &x.p);
  if (st != UAII_OK) return st;
  st = attn_args(fn, shape, cache, q_out, false, seq_lens, scale, window, softcap, split_size, max_splits, part_o,
                 part_lse, &x.a, !scratch);
  if (st != UAII_OK) return st;
  if (sinks != nullptr) CHECK_PTR("sinks", sinks, 4);
  if (!scratch) CHECK_PTR("counters", counters, 4);
  CHECK_PTR("out", out, 16);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (scratch) {
    // Every argument is valid: only now is the device touched, to find this
    // GPU's static scratch (counters, then part_lse, then part_o).
    void* base = nullptr;
    st = device_status(fn, uaii::noalloc_scratch(&base, s));
    if (st != UAII_OK) return st;
    const int64_t rows = static_cast<int64_t>(shape->batch) * shape->n_heads * max_splits;
    unsigned char* p = static_cast<unsigned char*>(base);
    counters = reinterpret_cast<int32_t*>(p);
    part_lse = reinterpret_cast<float*>(p + uaii::kNoAllocCounterBytes);
    part_o = reinterpret_cast<float*>(p + uaii::kNoAllocCounterBytes + (rows * 4 + 255) / 256 * 256);
    x.a.part_o = part_o;
    x.a.part_lse = part_lse;
  }
  x.sinks = sinks;
  x.out = out;
  x.counters = counters;
  const int G = shape->n_heads / shape->n_kv_heads;
  const int items = x.a.t.work_prefix[shape->batch] * shape->n_kv_heads;
  if (items <= uaii::kStepOneLaunchMax) {
    if (cache->block_table != nullptr)
      return device_status(
          fn, uaii::launch_decode_step_paged(shape->head_dim, G, cache->k_dtype, cache->v_dtype, x, s));
    return device_status(fn,
                         uaii::launch_decode_step(shape->head_dim, G, cache->k_dtype, cache->v_dtype, x, s));
  }
  // A large step: the producer, the partials and the combine back to back
  // on the stream (the kernel boundaries order them; the counters are not
  // touched and stay zero).
  for (int b = 0; b < shape->batch; ++b) x.p.pos[b] = seq_lens[b] - 1;
  st = device_status(fn, uaii::launch_kv_produce(x.p, s));
  if (st != UAII_OK) return st;
  st = device_status(fn, cache->block_table != nullptr
                             ? uaii::launch_decode_partial_paged(shape->head_dim, G, cache->k_dtype,
                                                                 cache->v_dtype, x.a, s)
                             : uaii::launch_decode_partial(shape->head_dim, G, cache->k_dtype, cache->v_dtype,
                                                           x.a, s));
  if (st != UAII_OK) return st;
  uaii::CombineArgs c{};
  c.H = shape->n_heads;
  c.max_splits = max_splits;
  c.part_o = part_o;
  c.part_lse = part_lse;
  c.sinks = sinks;
  c.out = out;
  c.t = x.a.t;
  return device_status(fn, uaii::launch_decode_combine(shape->head_dim, shape->batch, c, s));
}

uaii_status combine(const char* fn, const uaii_attn_shape* shape, const int32_t* seq_lens, int32_t window,
                    int32_t split_size, int32_t max_splits, const float* part_o, const float* part_lse,
                    const float* sinks, float* out, void* stream) {
  g_error.clear();
  uaii_status st = check_shape(fn, shape);
  if (st != UAII_OK) return st;
  st = check_lens(fn, shape, seq_lens, kMaxCapacity, split_size, max_splits, window);
  if (st != UAII_OK) return st;
  CHECK_PTR("part_o", part_o, 16);
  CHECK_PTR("part_lse", part_lse, 4);
  CHECK_PTR("out", out, 16);

  uaii::CombineArgs a{};
  a.H = shape->n_heads;
  a.max_splits = max_splits;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.sinks = sinks;
  a.out = out;
  build_table(shape->batch, seq_lens, window, split_size, &a.t);
  return device_status(fn, uaii::launch_decode_combine(shape->head_dim, shape->batch, a,
                                                       static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

uaii_status uaii_decode_combine(const uaii_attn_shape* shape, const int32_t* seq_lens, int32_t window,
                                int32_t split_size, int32_t max_splits, const float* part_o,
                                const float* part_lse, float* out, void* stream) {
  return combine("uaii_decode_combine", shape, seq_lens, window, split_size, max_splits, part_o, part_lse,
                 nullptr, out, stream);
}

uaii_status uaii_decode_combine_sink(const uaii_attn_shape* shape, const int32_t* seq_lens,
                                     int32_t window, int32_t split_size, int32_t max_splits,
                                     const float* part_o, const float* part_lse, const float* sinks,
                                     float* out, void* stream) {
  const char* fn = "uaii_decode_combine_sink";
  g_error.clear();
  CHECK_PTR("sinks", sinks, 4);
  return combine(fn, shape, seq_lens, window, split_size, max_splits, part_o, part_lse, sinks, out,
                 stream);
}

}  // extern "C"
