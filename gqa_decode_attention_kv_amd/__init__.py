"""GQA decode step on MI355X (gfx950): KV producer (QK-RMSNorm, RoPE, append
to an f32 / bf16 / vq8 cache) and split-K flash-decoding attention with a
log-sum-exp combine, behind the C ABI of ``include/uaii_decode.h``.

The compute lives in ``libuaii_decode.so`` (hand-written HIP); this package
only marshals arguments (``binding``) and draws seeded inputs (``workloads``).
"""
