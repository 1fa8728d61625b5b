"""ctypes binding of ``libuaii_decode.so`` (declared in include/uaii_decode.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI.  The raw functions take integer device pointers
and host integer arrays; ``UaiiError`` carries the library's status and
message.  The library must have been built (``__graft_entry__.build()``);
there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(HERE, "libuaii_decode.so")

OK, ERR_INVALID_ARGUMENT, ERR_NOT_IMPLEMENTED, ERR_DEVICE = 0, 1, 2, 3
F32, BF16, I8 = 0, 1, 2
ROPE_NEOX, ROPE_INTERLEAVED = 0, 1
ROPE_PLAIN, ROPE_LLAMA3, ROPE_LINEAR, ROPE_YARN = 0, 1, 2, 3

EXPORTS = ("uaii_last_error", "uaii_kv_produce", "uaii_decode_attn", "uaii_decode_combine",
           "uaii_decode_combine_sink", "uaii_decode_step", "uaii_decode_step_noalloc",
           "uaii_kv_produce_chunk", "uaii_prefill_attn")


class UaiiError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status
        self.message = message


class Shape(C.Structure):
    _fields_ = [("batch", C.c_int32), ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32)]


class Rope(C.Structure):
    _fields_ = [("pairing", C.c_int32), ("scaling", C.c_int32), ("theta", C.c_double),
                ("factor", C.c_double), ("low_freq_factor", C.c_double),
                ("high_freq_factor", C.c_double), ("original_max_position", C.c_int32),
                ("truncate", C.c_int32), ("attention_factor", C.c_double)]


class QKNorm(C.Structure):
    _fields_ = [("enabled", C.c_int32), ("eps", C.c_float), ("offset", C.c_int32),
                ("q_weight", C.c_void_p), ("k_weight", C.c_void_p)]


class KVCache(C.Structure):
    _fields_ = [("k_dtype", C.c_int32), ("v_dtype", C.c_int32), ("capacity", C.c_int32),
                ("k", C.c_void_p), ("v", C.c_void_p), ("v_scale", C.c_void_p),
                ("block_table", C.c_void_p), ("block_size", C.c_int32),
                ("max_blocks", C.c_int32), ("num_blocks", C.c_int32), ("k_scale", C.c_void_p)]


_lib = None


def load() -> C.CDLL:
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is missing: build it first with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        lib = C.CDLL(LIBRARY)
        vp, ip = C.c_void_p, C.POINTER(C.c_int32)
        lib.uaii_last_error.restype = C.c_char_p
        lib.uaii_last_error.argtypes = []
        lib.uaii_kv_produce.restype = C.c_int
        lib.uaii_kv_produce.argtypes = [C.POINTER(Shape), C.POINTER(Rope), C.POINTER(QKNorm),
                                        vp, vp, vp, ip, C.POINTER(KVCache), vp, vp]
        lib.uaii_decode_attn.restype = C.c_int
        lib.uaii_decode_attn.argtypes = [C.POINTER(Shape), C.POINTER(KVCache), vp, ip, C.c_float,
                                         C.c_int32, C.c_float, C.c_int32, C.c_int32, vp, vp, vp]
        lib.uaii_decode_combine.restype = C.c_int
        lib.uaii_decode_combine.argtypes = [C.POINTER(Shape), ip, C.c_int32, C.c_int32, C.c_int32,
                                            vp, vp, vp, vp]
        lib.uaii_decode_combine_sink.restype = C.c_int
        lib.uaii_decode_combine_sink.argtypes = [C.POINTER(Shape), ip, C.c_int32, C.c_int32,
                                                 C.c_int32, vp, vp, vp, vp, vp]
        lib.uaii_decode_step.restype = C.c_int
        lib.uaii_decode_step.argtypes = [C.POINTER(Shape), C.POINTER(Rope), C.POINTER(QKNorm),
                                         vp, vp, vp, ip, C.POINTER(KVCache), C.c_float, C.c_int32,
                                         C.c_float, C.c_int32, C.c_int32, vp, vp, vp, vp, vp, vp,
                                         vp]
        lib.uaii_decode_step_noalloc.restype = C.c_int
        lib.uaii_decode_step_noalloc.argtypes = [C.POINTER(Shape), C.POINTER(Rope),
                                                 C.POINTER(QKNorm), vp, vp, vp, ip,
                                                 C.POINTER(KVCache), C.c_float, C.c_int32,
                                                 C.c_float, C.c_int32, vp, vp, vp, vp]
        lib.uaii_kv_produce_chunk.restype = C.c_int
        lib.uaii_kv_produce_chunk.argtypes = [C.POINTER(Shape), C.POINTER(Rope), C.POINTER(QKNorm),
                                              vp, vp, vp, ip, C.c_int32, C.POINTER(KVCache), vp,
                                              vp]
        lib.uaii_prefill_attn.restype = C.c_int
        lib.uaii_prefill_attn.argtypes = [C.POINTER(Shape), C.POINTER(KVCache), vp, ip, C.c_int32,
                                          C.c_float, C.c_int32, C.c_float, vp, vp, vp]
        _lib = lib
    return _lib


def last_error() -> str:
    return load().uaii_last_error().decode()


def _check(status: int):
    if status != OK:
        raise UaiiError(status, last_error())


def _host_i32(a, n: int | None = None):
    if a is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    if n is not None and arr.size < n:
        raise ValueError(f"host array has {arr.size} entries, need {n}")
    return arr, arr.ctypes.data_as(C.POINTER(C.c_int32))


def kv_produce(shape: Shape, rope: Rope, qk_norm: QKNorm | None, q_in: int, k_in: int, v_in: int,
               positions, cache: KVCache, q_out: int, stream: int = 0) -> None:
    arr, p = _host_i32(positions, shape.batch)
    _check(load().uaii_kv_produce(C.byref(shape), C.byref(rope),
                                  C.byref(qk_norm) if qk_norm is not None else None,
                                  q_in, k_in, v_in, p, C.byref(cache), q_out, stream))


def decode_attn(shape: Shape, cache: KVCache, q: int, seq_lens, scale: float, window: int,
                softcap: float, split_size: int, max_splits: int, part_o: int, part_lse: int,
                stream: int = 0) -> None:
    arr, p = _host_i32(seq_lens, shape.batch)
    _check(load().uaii_decode_attn(C.byref(shape), C.byref(cache), q, p, scale, window, softcap,
                                   split_size, max_splits, part_o, part_lse, stream))


def decode_combine(shape: Shape, seq_lens, window: int, split_size: int, max_splits: int,
                   part_o: int, part_lse: int, out: int, stream: int = 0) -> None:
    arr, p = _host_i32(seq_lens, shape.batch)
    _check(load().uaii_decode_combine(C.byref(shape), p, window, split_size, max_splits, part_o,
                                      part_lse, out, stream))


def decode_combine_sink(shape: Shape, seq_lens, window: int, split_size: int, max_splits: int,
                        part_o: int, part_lse: int, sinks: int, out: int, stream: int = 0) -> None:
    arr, p = _host_i32(seq_lens, shape.batch)
    _check(load().uaii_decode_combine_sink(C.byref(shape), p, window, split_size, max_splits,
                                           part_o, part_lse, sinks, out, stream))


def decode_step(shape: Shape, rope: Rope, qk_norm: QKNorm | None, q_in: int, k_in: int, v_in: int,
                seq_lens, cache: KVCache, scale: float, window: int, softcap: float,
                split_size: int, max_splits: int, sinks: int | None, q_out: int, part_o: int,
                part_lse: int, counters: int, out: int, stream: int = 0) -> None:
    arr, p = _host_i32(seq_lens, shape.batch)
    _check(load().uaii_decode_step(C.byref(shape), C.byref(rope),
                                   C.byref(qk_norm) if qk_norm is not None else None,
                                   q_in, k_in, v_in, p, C.byref(cache), scale, window, softcap,
                                   split_size, max_splits, sinks, q_out, part_o, part_lse,
                                   counters, out, stream))


def decode_step_noalloc(shape: Shape, rope: Rope, qk_norm: QKNorm | None, q_in: int, k_in: int,
                        v_in: int, seq_lens, cache: KVCache, scale: float, window: int,
                        softcap: float, split_size: int, sinks: int | None, q_out: int, out: int,
                        stream: int = 0) -> None:
    arr, p = _host_i32(seq_lens, shape.batch)
    _check(load().uaii_decode_step_noalloc(C.byref(shape), C.byref(rope),
                                           C.byref(qk_norm) if qk_norm is not None else None,
                                           q_in, k_in, v_in, p, C.byref(cache), scale, window,
                                           softcap, split_size, sinks, q_out, out, stream))


def kv_produce_chunk(shape: Shape, rope: Rope, qk_norm: QKNorm | None, q_in: int, k_in: int,
                     v_in: int, start_positions, n_tokens: int, cache: KVCache, q_out: int,
                     stream: int = 0) -> None:
    arr, p = _host_i32(start_positions, shape.batch)
    _check(load().uaii_kv_produce_chunk(C.byref(shape), C.byref(rope),
                                        C.byref(qk_norm) if qk_norm is not None else None,
                                        q_in, k_in, v_in, p, n_tokens, C.byref(cache), q_out,
                                        stream))


def prefill_attn(shape: Shape, cache: KVCache, q: int, seq_lens, n_tokens: int, scale: float,
                 window: int, softcap: float, sinks: int | None, out: int,
                 stream: int = 0) -> None:
    arr, p = _host_i32(seq_lens, shape.batch)
    _check(load().uaii_prefill_attn(C.byref(shape), C.byref(cache), q, p, n_tokens, scale, window,
                                    softcap, sinks, out, stream))
