/*
 * uaii_decode.h -- C ABI of the MI355X (gfx950) GQA decode-step library.
 *
 * One decode step of a grouped-query attention layer, in three calls:
 *
 *   uaii_kv_produce      optional per-head QK-RMSNorm, RoPE, append of the new
 *                        token's K and V to an f32 / bf16 / vq8 cache
 *   uaii_decode_attn     split-K flash-decoding partials over B <= 32 ragged
 *                        sequences, with an optional sliding window and
 *                        attention-logit softcap
 *   uaii_decode_combine  log-sum-exp combine of the partials
 *   uaii_decode_combine_sink  the same combine with a per-head attention
 *                        sink in the softmax denominator
 *   uaii_decode_step     all of the above in a single launch
 *
 * and, for a chunk of new tokens per sequence (prefill):
 *
 *   uaii_kv_produce_chunk  the producer for T tokens per sequence
 *   uaii_prefill_attn      causal attention of the chunk's queries
 *
 * Sources (page title, then section):
 *   [UAII]      "Universal AI Inference - Hugging Face decoder completeness"
 *   [ALGENTA]   "Algenta - Model support matrix"
 *   [FREETOKEN] "FreeToken PR #722 - serve Llama and Mistral llama-arch GGUF
 *               checkpoints"
 *   [LLAMAY]    "llamay - Models and formats"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Ownership.  The caller owns every buffer.  The library never allocates or
 *   frees memory, keeps no state between calls (except the thread-local error
 *   text), never synchronises, and enqueues all work on the caller's stream.
 * Pointers.  "device" pointers address GPU memory of the current device and
 *   must be 16-byte aligned; "host" arrays are read during the call only.
 * Layouts (row-major, innermost last):
 *   q_in, q_out, q           [batch][n_heads][head_dim]            f32
 *   k_in, v_in               [batch][n_kv_heads][head_dim]         f32
 *   cache K, V               [batch][n_kv_heads][capacity][head_dim] (contiguous;
 *                            the paged layout is described at uaii_kv_cache)
 *                            K: f32, bf16 or int8 (q8); V: f32, bf16 or
 *                            int8 (vq8, q8)
 *   k_scale (q8), v_scale (vq8, q8)  [batch][n_kv_heads][capacity]  f32
 *   part_o                   [batch][n_heads][max_splits][head_dim] f32
 *   part_lse                 [batch][n_heads][max_splits]          f32
 *   out                      [batch][n_heads][head_dim]            f32
 *   bf16 is stored as its 16-bit pattern (upper half of an f32); it is
 *   widened to f32 when read, never reinterpreted ([UAII] P0.1 BF16 ingest).
 * Query-to-kv-head map.  n_heads is an exact multiple of n_kv_heads and query
 *   head h reads kv head h / (n_heads / n_kv_heads): consecutive groups
 *   ([ALGENTA] Structural fact requirements: integral GQA ratio).
 * Lengths.  seq_lens[b] counts the keys sequence b attends, the new token
 *   included; the new token sits at slot seq_lens[b] - 1, which is also its
 *   absolute RoPE position ([UAII] P1.3: positions follow the absolute KV
 *   index, same as RoPE).
 * Window.  window = W > 0 keeps the last W keys, the new one included:
 *   keys [max(0, L - W), L).  W = 0 means no window ([UAII] P1.4).
 * Errors.  Every argument is checked before any work is enqueued; on error
 *   nothing is written and the call returns a status, with a message that
 *   names the fact, its value and the supported range
 *   ([ALGENTA] Conformance CLI: typed refusals; [UAII] section 6: every
 *   message says what failed and what to do).  Sizes of caller buffers
 *   cannot be checked through plain pointers and are the caller's contract.
 *   UAII_ERR_INVALID_ARGUMENT  malformed input (null pointer, bad range)
 *   UAII_ERR_NOT_IMPLEMENTED   a valid fact outside the supported ranges
 *   UAII_ERR_DEVICE            a HIP error when enqueuing (message from HIP)
 * Supported ranges.  head_dim in {64, 128, 256}; batch in 1..32 ([ALGENTA]
 *   Kernel path capabilities: batched decode partial, B <= 32);
 *   n_heads / n_kv_heads in {1, 2, 4, 8}; K dtype f32 or bf16; V dtype f32,
 *   bf16 or int8 with an f32 scale per token per kv head (vq8: values
 *   quantised, keys exact; [LLAMAY] The KV cache, in three precisions);
 *   int8 keys only together with int8 values (q8: both quantised, each
 *   with its own scale per token per kv head; same section).
 * Threads.  Re-entrant; calls on different streams may overlap.  Calls that
 *   write the same cache slot or partial rows concurrently race.
 */
#ifndef UAII_DECODE_H
#define UAII_DECODE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum uaii_status {
    UAII_OK = 0,
    UAII_ERR_INVALID_ARGUMENT = 1,
    UAII_ERR_NOT_IMPLEMENTED = 2,
    UAII_ERR_DEVICE = 3
} uaii_status;

/* Cache element types (int32 codes in the structs below). */
enum { UAII_F32 = 0, UAII_BF16 = 1, UAII_I8 = 2 };

/* RoPE pairing: NeoX rotates (i, i + d/2), interleaved rotates (2i, 2i + 1)
 * ([UAII] P0.2; [LLAMAY] Architectures; [FREETOKEN] Changes). */
enum { UAII_ROPE_NEOX = 0, UAII_ROPE_INTERLEAVED = 1 };

/* RoPE frequency scheme: plain theta^(-2i/d), Llama-3 frequency scaling
 * ([UAII] P0.2: match Hugging Face's Llama-3 rotary embedding;
 * [ALGENTA] Structural fact requirements: plain or llama3), linear scaling
 * ([ALGENTA] Decoder families: gemma3 linear global scaling) or YaRN
 * ([UAII] P0.2 names it; [LLAMAY] Architectures: gpt-oss). */
enum { UAII_ROPE_PLAIN = 0, UAII_ROPE_LLAMA3 = 1, UAII_ROPE_LINEAR = 2, UAII_ROPE_YARN = 3 };

typedef struct uaii_attn_shape {
    int32_t batch;      /* B, 1..32 */
    int32_t n_heads;    /* H, query heads */
    int32_t n_kv_heads; /* Hkv, H % Hkv == 0 */
    int32_t head_dim;   /* d in {64, 128, 256} */
} uaii_attn_shape;

/* Rotary embedding of one layer.  A Gemma-style local/global layer pair is
 * two calls, each with its own theta ([ALGENTA] Decoder families: dual
 * theta; [LLAMAY] Architectures: a second rotary base on local layers).
 * Frequencies cover the full head ([ALGENTA]: partial rotary is refused).
 * Llama-3 scaling, with wavelength lambda_i = 2 pi / f_i and
 * f_i = theta^(-2i/d):
 *   lambda < original/high  -> f;    lambda > original/low -> f / factor;
 *   otherwise mu = (original/lambda - low)/(high - low) and
 *   (1 - mu) f / factor + mu f   ([FREETOKEN] Changes: low 1, high 4,
 *   original 8192 for every Llama 3.1-3.3 release).
 * Linear scaling: f / factor for every pair (positions divided by factor).
 * YaRN, as Hugging Face computes it: low_freq_factor is beta_slow and
 *   high_freq_factor is beta_fast, the numbers of turns over the original
 *   context that bound the blend.  With c(n) = d ln(original / (2 pi n)) /
 *   (2 ln theta), the pair index that turns n times, the blend runs from
 *   c_lo = c(beta_fast) to c_hi = c(beta_slow) (rounded outwards to whole
 *   indices if truncate != 0, clamped to [0, d - 1]):
 *   t_i = clamp((i - c_lo)/(c_hi - c_lo), 0, 1), g_i = t_i f / factor +
 *   (1 - t_i) f.  The rotated q and k are multiplied by attention_factor
 *   (0 selects 1 + 0.1 ln(factor) for factor > 1, else 1). */
typedef struct uaii_rope {
    int32_t pairing;               /* UAII_ROPE_NEOX | UAII_ROPE_INTERLEAVED */
    int32_t scaling;               /* UAII_ROPE_PLAIN | _LLAMA3 | _LINEAR | _YARN */
    double theta;                  /* > 0 */
    double factor;                 /* llama3, yarn: >= 1; linear: > 0 */
    double low_freq_factor;        /* llama3: > 0; yarn: beta_slow > 0 */
    double high_freq_factor;       /* llama3: > low_freq_factor; yarn: beta_fast > beta_slow */
    int32_t original_max_position; /* llama3, yarn: > 0 */
    int32_t truncate;              /* yarn: round the blend edges to whole pair indices */
    double attention_factor;       /* yarn: > 0, or 0 for the default */
} uaii_rope;

/* Per-head QK-RMSNorm, applied to every q and k head before RoPE
 * ([UAII] P1.2), y = x (mean x^2 + eps)^-1/2 (w + offset), with offset 0
 * (gain w) or 1 (gain 1 + w, Gemma; [UAII] P1.1).  One weight vector of
 * head_dim entries for q and one for k, shared by all heads.  Passing NULL
 * for the whole struct, or enabled = 0, disables the norm. */
typedef struct uaii_qk_norm {
    int32_t enabled;
    float eps;               /* > 0 */
    int32_t offset;          /* 0 or 1 */
    const float *q_weight;   /* device [head_dim] */
    const float *k_weight;   /* device [head_dim] */
} uaii_qk_norm;

/* KV cache of one layer, in one of two layouts.
 *
 * Contiguous (block_table == NULL): one slab per (sequence, kv head),
 *   k, v     device [B][Hkv][capacity][d]
 *   v_scale  device [B][Hkv][capacity]          (int8 values only)
 *   k_scale  device [B][Hkv][capacity]          (int8 keys only)
 *
 * Paged (block_table != NULL): pools of fixed-size blocks shared by all
 * sequences, and a table that maps each sequence's logical blocks to
 * physical ones.  Slot p of (sequence b, kv head u) is row p % block_size of
 * physical block block_table[b][p / block_size]:
 *   k, v         device [num_blocks][Hkv][block_size][d]
 *   v_scale, k_scale  device [num_blocks][Hkv][block_size]  (int8 only)
 *   block_table  device [B][max_blocks] int32
 *   capacity     must equal max_blocks * block_size (logical slots per
 *                sequence)
 * The table must hold an id in [0, num_blocks) for every logical block that
 * covers a visible key or the new token's slot; the kernels clamp ids
 * outside the pool (so a bad table cannot reach memory outside it) but the
 * result is then undefined.  Blocks may be shared between sequences for
 * reading; the producer writes only the new token's slot, so two sequences
 * must not share the block that receives it.
 * (Paged KV pages: "llamay - Models and formats", What is refused: a KV
 * page, the paged allocator, copy-on-write fork.) */
typedef struct uaii_kv_cache {
    int32_t k_dtype;   /* UAII_F32 | UAII_BF16 | UAII_I8 (q8, with v_dtype int8) */
    int32_t v_dtype;   /* UAII_F32 | UAII_BF16 | UAII_I8 (vq8, q8) */
    int32_t capacity;  /* slots per (sequence, kv head), >= 1 */
    void *k;           /* device, see the layouts above */
    void *v;           /* device */
    float *v_scale;    /* device, vq8 only (else ignored) */
    const int32_t *block_table; /* device [B][max_blocks], or NULL (contiguous) */
    int32_t block_size; /* paged: rows per block, a power of two in [16, 1024] */
    int32_t max_blocks; /* paged: table entries per sequence, >= 1 */
    int32_t num_blocks; /* paged: blocks in each pool, >= 1 */
    float *k_scale;    /* device, q8 only (else ignored); same layout as v_scale */
} uaii_kv_cache;

/* Text of the last error on the calling thread ("" if none); valid until the
 * next call on the same thread. */
const char *uaii_last_error(void);

/* KV producer.  For every sequence b at position p = positions[b]:
 *   q' = RoPE(norm_q(q_in[b][h]), p)   -> q_out[b][h]           (f32)
 *   k' = RoPE(norm_k(k_in[b][u]), p)   -> K[b][u][p]  (f32, or bf16 rounded
 *        to nearest even; q8: k' rounded to f32, then quantised like v
 *        below, scale -> k_scale[b][u][p])
 *   v  = v_in[b][u]                    -> V[b][u][p]  (f32; bf16 rounded to
 *        nearest even; vq8: scale = max|v| / 127 in f32, code =
 *        clamp(round_half_away(v / scale), -127, 127), all-zero v gives
 *        scale 0 and codes 0; scale -> v_scale[b][u][p])
 * RoPE is the pairing and frequency scheme of rope; for YaRN, q' and k' are
 * also multiplied by its attention factor.  The norm and the rotation are
 * evaluated in double precision and rounded once to the stored format.
 * Only slot p of each (b, u) is written.
 *   shape      host, required
 *   rope       host, required
 *   qk_norm    host, may be NULL (no norm)
 *   q_in, k_in, v_in, q_out   device
 *   positions  host [batch], each in [0, capacity)
 *   cache      host struct describing device buffers
 *   stream     hipStream_t (NULL = the null stream) */
uaii_status uaii_kv_produce(const uaii_attn_shape *shape, const uaii_rope *rope,
                            const uaii_qk_norm *qk_norm, const float *q_in,
                            const float *k_in, const float *v_in,
                            const int32_t *positions, const uaii_kv_cache *cache,
                            float *q_out, void *stream);

/* Split-K flash-decoding partials ([ALGENTA] Kernel path capabilities:
 * split-K decode partial, batched decode partial; Conformance CLI:
 * decode_attn=splitk_flash_decoding).  For every sequence b, query head h
 * and split sigma that intersects the visible keys [lo_b, L_b), where split
 * sigma covers keys [sigma * split_size, (sigma + 1) * split_size):
 *   s_j   = scale * <q[b][h], K[b][h / G][j]>,  then c * tanh(s_j / c) if
 *           softcap c > 0 ([UAII] P1.4 logit softcap; [ALGENTA] attention
 *           scale 1/sqrt(head_dim))
 *   part_o[b][h][sigma]   = sum_j e^(s_j - m) v_j / sum_j e^(s_j - m)
 *   part_lse[b][h][sigma] = m + ln sum_j e^(s_j - m)
 * over the split's visible keys, with m their largest score; K and v_j are
 * the cached entries widened to f32 (int8: code * scale).  Accumulation is
 * f32.
 * Entries of splits outside the visible range are not written.
 *   scale       must equal 1/sqrt(head_dim) (any other value is refused)
 *   seq_lens    host [batch], each in [1, capacity]
 *   window      >= 0 (0 = none);  softcap >= 0 and finite (0 = none)
 *   split_size  >= 1;  max_splits >= ceil(max_b seq_lens[b] / split_size)
 *   q           device, normally q_out of uaii_kv_produce
 *   part_o, part_lse  device, sized with max_splits */
uaii_status uaii_decode_attn(const uaii_attn_shape *shape, const uaii_kv_cache *cache,
                             const float *q, const int32_t *seq_lens, float scale,
                             int32_t window, float softcap, int32_t split_size,
                             int32_t max_splits, float *part_o, float *part_lse,
                             void *stream);

/* Log-sum-exp combine of the partials written by uaii_decode_attn with the
 * same seq_lens, window, split_size and max_splits: over the splits that
 * intersect the visible keys, M = max lse, and
 *   out[b][h] = sum_sigma e^(lse_sigma - M) part_o_sigma / sum_sigma e^(lse_sigma - M).
 * Only the valid splits are read. */
uaii_status uaii_decode_combine(const uaii_attn_shape *shape, const int32_t *seq_lens,
                                int32_t window, int32_t split_size, int32_t max_splits,
                                const float *part_o, const float *part_lse, float *out,
                                void *stream);

/* The combine with an attention sink: one learned logit per query head that
 * joins the softmax denominator but carries no value ([LLAMAY]
 * Architectures: gpt-oss puts a per-head sink in the denominator).  The sink
 * belongs to no split, so the partials are those of uaii_decode_attn
 * unchanged and
 *   out[b][h] = sum_sigma e^(lse_sigma - M) part_o_sigma /
 *               (sum_sigma e^(lse_sigma - M) + e^(sinks[h] - M)),
 * with M the largest of the split lse values and sinks[h] (the sink is in
 * the units of the scaled, softcapped scores).
 *   sinks  device [n_heads] f32, finite (not checked: device memory) */
uaii_status uaii_decode_combine_sink(const uaii_attn_shape *shape, const int32_t *seq_lens,
                                     int32_t window, int32_t split_size, int32_t max_splits,
                                     const float *part_o, const float *part_lse,
                                     const float *sinks, float *out, void *stream);

/* The whole decode step in one launch: uaii_kv_produce at positions
 * seq_lens[b] - 1, then uaii_decode_attn, then uaii_decode_combine (or
 * uaii_decode_combine_sink when sinks != NULL), with the same results.
 * ([ALGENTA] Kernel path capabilities lists a KV-producer-fused decode
 * partial; here the combine is folded in as well.)  Each wave computes the
 * rotated queries of its kv head's group itself; the wave whose split holds
 * the new token's slot stores the new K and V and merges that row from
 * registers; the last split of each (sequence, kv head) to finish combines
 * that group's heads.  That costs a device-scope release per split, so only
 * small steps run this way: up to 256 (split, kv head) work items, i.e.
 * sum_b (splits of b) * n_kv_heads <= 256.  Larger steps run the producer,
 * partial and combine kernels back to back on the stream, as the three
 * calls would.
 *   q_in, k_in, v_in, rope, qk_norm   as uaii_kv_produce; the position of
 *               sequence b is seq_lens[b] - 1
 *   seq_lens, scale, window, softcap, split_size, max_splits   as
 *               uaii_decode_attn
 *   sinks       device [n_heads] f32, or NULL (no sink)
 *   q_out       device, receives the rotated queries, as uaii_kv_produce
 *   part_o, part_lse   device, sized as for uaii_decode_attn; they hold the
 *               split partials afterwards
 *   counters    device [batch][n_kv_heads] int32 arrival counters: all zero
 *               before the first call (e.g. from a zero fill), and left at
 *               zero by every call that completes, so one buffer serves any
 *               number of consecutive calls.  Calls that share counters,
 *               partials or cache slots must not run concurrently.
 *   out         device [batch][n_heads][head_dim] f32 */
uaii_status uaii_decode_step(const uaii_attn_shape *shape, const uaii_rope *rope,
                             const uaii_qk_norm *qk_norm, const float *q_in,
                             const float *k_in, const float *v_in,
                             const int32_t *seq_lens, const uaii_kv_cache *cache,
                             float scale, int32_t window, float softcap,
                             int32_t split_size, int32_t max_splits,
                             const float *sinks, float *q_out, float *part_o,
                             float *part_lse, int32_t *counters, float *out,
                             void *stream);

/* uaii_decode_step for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The caller passes the inputs and outputs only; the split
 * partials and arrival counters live in a static scratch array that the
 * library holds on each GPU it runs on until the process ends
 * (16 MiB + 64 KiB per GPU).  The call allocates nothing and frees nothing.
 *   arguments   as uaii_decode_step, without max_splits (taken as
 *               ceil(max seq_len / split_size)) and without part_o,
 *               part_lse and counters
 * Limits, refused with UAII_ERR_NOT_IMPLEMENTED before anything is
 * launched: batch*n_heads*ceil(max seq_len/split_size)*(head_dim+1)*4 bytes
 * of partials at most 16 MiB (256-byte alignment of the lse block
 * included), and batch*n_kv_heads <= 16384.
 * Every call on a GPU shares that GPU's scratch, which keeps the last call's
 * partials: calls that overlap on one GPU (on different streams, or from
 * different threads without ordering) race and must not be issued.  The
 * counters are zeroed by a kernel enqueued on the stream of the first call
 * on each GPU, and every completed call leaves them at zero. */
uaii_status uaii_decode_step_noalloc(const uaii_attn_shape *shape, const uaii_rope *rope,
                                     const uaii_qk_norm *qk_norm, const float *q_in,
                                     const float *k_in, const float *v_in,
                                     const int32_t *seq_lens, const uaii_kv_cache *cache,
                                     float scale, int32_t window, float softcap,
                                     int32_t split_size, const float *sinks, float *q_out,
                                     float *out, void *stream);

/* --------------------------------------------------------------------------
 * Chunks of new tokens (prefill)
 * ------------------------------------------------------------------------ */

/* The KV producer for a chunk of n_tokens = T new tokens per sequence:
 * token t of sequence b is at position start_positions[b] + t, and each
 * token is produced exactly as uaii_kv_produce produces one (norm, RoPE at
 * its own position, append at its own slot).  With T = 1 it is
 * uaii_kv_produce.
 *   q_in, q_out        device [batch][T][n_heads][head_dim] f32
 *   k_in, v_in         device [batch][T][n_kv_heads][head_dim] f32
 *   start_positions    host [batch]; start + T <= capacity
 *   n_tokens           1..65535
 * Slots start .. start + T - 1 of each (b, kv head) are written. */
uaii_status uaii_kv_produce_chunk(const uaii_attn_shape *shape, const uaii_rope *rope,
                                  const uaii_qk_norm *qk_norm, const float *q_in,
                                  const float *k_in, const float *v_in,
                                  const int32_t *start_positions, int32_t n_tokens,
                                  const uaii_kv_cache *cache, float *q_out, void *stream);

/* Causal attention of a chunk ([ALGENTA] Kernel path capabilities:
 * grouped-FA prefill and parametric prefill).  The chunk's T queries of
 * sequence b sit at positions L - T .. L - 1 with L = seq_lens[b]; their keys
 * and values are already in the cache (uaii_kv_produce_chunk).  Query t
 * attends the keys at positions lo .. L - T + t, lo = max(0, L - T + t + 1 -
 * window) with a window (0: lo = 0):
 *   s_j = scale * <q[b][t][h], K[b][h / G][j]>, then c * tanh(s_j / c) if
 *         softcap c > 0
 *   out[b][t][h] = sum_j e^(s_j - m) v_j / (sum_j e^(s_j - m) [+ e^(sink_h - m)])
 * with m the largest of the s_j (and sink_h).  This is uaii_decode_attn +
 * uaii_decode_combine(_sink) of each query over its own prefix, in one
 * launch on the matrix cores.
 *   cache     contiguous or paged, with (k_dtype, v_dtype) one of
 *             (BF16, BF16), (BF16, I8) (vq8), (I8, I8) (q8) or (F32, F32)
 *             (head_dim 64 or 128); other pairs, and f32 at head_dim 256,
 *             are refused with UAII_ERR_NOT_IMPLEMENTED
 *   q         device [batch][T][n_heads][head_dim] f32 (q_out of the chunk
 *             producer)
 *   seq_lens  host [batch], each in [T, capacity]
 *   n_tokens  1..2^20
 *   sinks     device [n_heads] f32, or NULL (no sink)
 *   out       device [batch][T][n_heads][head_dim] f32
 * Accumulation is f32.  bf16 and int8 caches: q and the softmax weights
 * enter the matrix products as a bf16 pair (high part and remainder), K and
 * V as stored.  f32 caches: every operand enters as f32 (f32 matrix
 * products). */
uaii_status uaii_prefill_attn(const uaii_attn_shape *shape, const uaii_kv_cache *cache,
                              const float *q, const int32_t *seq_lens, int32_t n_tokens,
                              float scale, int32_t window, float softcap,
                              const float *sinks, float *out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* UAII_DECODE_H */
