"""ctypes binding of the CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the product path never imports it.

All arrays are numpy arrays in the layouts of the C functions:
``q [B][H][d]``, caches ``[B][Hkv][cap][d]``, ``v_scale [B][Hkv][cap]``.
bf16 caches are ``uint16`` bit patterns, vq8 value caches ``int8`` codes.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

F32, BF16, I8 = 0, 1, 2
NEOX, INTERLEAVED = 0, 1
PLAIN, LLAMA3, LINEAR, YARN = 0, 1, 2, 3

_dp = C.POINTER(C.c_double)
_fp = C.POINTER(C.c_float)
_ip = C.POINTER(C.c_int32)
_vp = C.c_void_p


def _ptr(a, ctype=None):
    if a is None:
        return None
    if ctype is None:
        return a.ctypes.data_as(_vp)
    return a.ctypes.data_as(C.POINTER(ctype))


def _need(a, dtype, name):
    if a.dtype != dtype or not a.flags["C_CONTIGUOUS"]:
        raise TypeError(f"{name}: expected C-contiguous {np.dtype(dtype).name}, "
                        f"got {a.dtype} contiguous={a.flags['C_CONTIGUOUS']}")
    return a


_STORAGE = {F32: np.float32, BF16: np.uint16, I8: np.int8}


class Oracle:
    """One loaded copy of the oracle library (a path lets tests load variants)."""

    def __init__(self, path: str | None = None):
        if path is None:
            path = _build.LIBRARY
            if not os.path.exists(path):
                _build.build()
        self.path = path
        lib = C.CDLL(path)
        lib.oracle_bf16_to_double.restype = C.c_double
        lib.oracle_bf16_to_double.argtypes = [C.c_uint16]
        lib.oracle_bf16_from_double.restype = C.c_uint16
        lib.oracle_bf16_from_double.argtypes = [C.c_double]
        lib.oracle_quantize_v.restype = None
        lib.oracle_quantize_v.argtypes = [_fp, C.c_int, C.POINTER(C.c_int8), _fp]
        lib.oracle_rms_norm.restype = None
        lib.oracle_rms_norm.argtypes = [_dp, C.c_int, _fp, C.c_int, C.c_double, _dp]
        lib.oracle_rope_freqs.restype = None
        lib.oracle_rope_freqs.argtypes = [C.c_int, C.c_int] + [C.c_double] * 5 + [C.c_int, _dp]
        lib.oracle_yarn_attn_factor.restype = C.c_double
        lib.oracle_yarn_attn_factor.argtypes = [C.c_double]
        lib.oracle_rope_apply.restype = None
        lib.oracle_rope_apply.argtypes = [_dp, C.c_int, C.c_int, _dp, C.c_int64]
        lib.oracle_kv_produce.restype = C.c_int
        lib.oracle_kv_produce.argtypes = (
            [C.c_int] * 4 + [C.c_int, C.c_int] + [C.c_double] * 5 + [C.c_int, C.c_double]
            + [C.c_int, C.c_double, C.c_int, _fp, _fp, _fp, _fp, _fp, _ip,
               C.c_int, C.c_int, C.c_int, _vp, _vp, _fp, _fp, _dp])
        lib.oracle_scores.restype = None
        lib.oracle_scores.argtypes = ([C.c_int] * 5 + [_vp, _fp, _dp, C.c_int, C.c_int, C.c_int64,
                                                       C.c_int64, C.c_double, _dp])
        lib.oracle_decode_pairs.restype = C.c_int
        lib.oracle_decode_pairs.argtypes = ([C.c_int] * 7 + [_vp, _vp, _fp, _fp, _dp, _ip, C.c_int32,
                                                            C.c_double, _dp, _ip, C.c_int, _dp])
        lib.oracle_split_partial.restype = C.c_int64
        lib.oracle_split_partial.argtypes = ([C.c_int] * 6 + [_vp, _vp, _fp, _fp, _dp, C.c_int,
                                                              C.c_int]
                                             + [C.c_int64, C.c_int64, C.c_double, C.c_int64,
                                                C.c_int64, _dp, _dp])
        lib.oracle_combine.restype = C.c_int
        lib.oracle_combine.argtypes = [C.c_int, C.c_int, _dp, _dp, C.c_int, C.c_double, _dp]
        self.lib = lib

    # -- codecs -----------------------------------------------------------
    def bf16_to_double(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_double(int(bits))

    def bf16_from_double(self, x: float) -> int:
        return int(self.lib.oracle_bf16_from_double(float(x)))

    def bf16_encode(self, x) -> np.ndarray:
        """Round every element of x (any float array) to bf16 bits."""
        x = np.asarray(x, dtype=np.float64)
        f = self.lib.oracle_bf16_from_double
        return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)

    def bf16_decode(self, bits) -> np.ndarray:
        bits = np.asarray(bits, dtype=np.uint16)
        f = self.lib.oracle_bf16_to_double
        return np.array([f(int(v)) for v in bits.ravel()], dtype=np.float64).reshape(bits.shape)

    def quantize_v(self, v):
        v = np.ascontiguousarray(v, dtype=np.float32)
        codes = np.zeros(v.shape[-1], dtype=np.int8)
        scale = np.zeros(1, dtype=np.float32)
        self.lib.oracle_quantize_v(_ptr(v, C.c_float), v.shape[-1], _ptr(codes, C.c_int8),
                                   _ptr(scale, C.c_float))
        return codes, np.float32(scale[0])

    # -- producer pieces ----------------------------------------------------
    def rms_norm(self, x, w, offset: int, eps: float):
        x = np.ascontiguousarray(x, dtype=np.float64)
        w = np.ascontiguousarray(w, dtype=np.float32)
        y = np.zeros_like(x)
        self.lib.oracle_rms_norm(_ptr(x, C.c_double), x.size, _ptr(w, C.c_float), int(offset),
                                 float(eps), _ptr(y, C.c_double))
        return y

    def rope_freqs(self, d: int, scaling: int = PLAIN, theta: float = 10000.0,
                   factor: float = 1.0, low: float = 1.0, high: float = 4.0,
                   orig: float = 8192.0, truncate: bool = True):
        g = np.zeros(d // 2, dtype=np.float64)
        self.lib.oracle_rope_freqs(d, scaling, theta, factor, low, high, orig, int(truncate),
                                   _ptr(g, C.c_double))
        return g

    def yarn_attn_factor(self, factor: float) -> float:
        return float(self.lib.oracle_yarn_attn_factor(float(factor)))

    def rope_apply(self, x, pairing: int, g, pos: int):
        y = np.array(x, dtype=np.float64, copy=True)
        g = np.ascontiguousarray(g, dtype=np.float64)
        self.lib.oracle_rope_apply(_ptr(y, C.c_double), y.size, pairing, _ptr(g, C.c_double),
                                   int(pos))
        return y

    def kv_produce(self, *, rope: dict, norm: dict | None, q_in, k_in, v_in, positions,
                   k_dtype: int, v_dtype: int, cache_k, cache_v, v_scale=None, k_scale=None):
        """Run the producer; writes slot positions[b] of the caches in place and
        returns q' as double [B][H][d]."""
        B, H, d = q_in.shape
        Hkv = k_in.shape[1]
        _need(q_in, np.float32, "q_in"), _need(k_in, np.float32, "k_in")
        _need(v_in, np.float32, "v_in")
        positions = np.ascontiguousarray(positions, dtype=np.int32)
        _need(cache_k, _STORAGE[k_dtype], "cache_k")
        _need(cache_v, _STORAGE[v_dtype], "cache_v")
        cap = cache_k.shape[2]
        q_out = np.zeros((B, H, d), dtype=np.float64)
        if norm and norm.get("enabled"):
            w_q = np.ascontiguousarray(norm["w_q"], dtype=np.float32)
            w_k = np.ascontiguousarray(norm["w_k"], dtype=np.float32)
            ne, eps, off = 1, float(norm["eps"]), int(norm["offset"])
        else:
            w_q = w_k = None
            ne, eps, off = 0, 1e-6, 0
        rc = self.lib.oracle_kv_produce(
            B, H, Hkv, d, int(rope["pairing"]), int(rope["scaling"]), float(rope["theta"]),
            float(rope.get("factor", 1.0)), float(rope.get("low", 1.0)),
            float(rope.get("high", 4.0)), float(rope.get("orig", 8192.0)),
            int(rope.get("truncate", True)),
            float(rope.get("attn_factor") or self.yarn_attn_factor(rope.get("factor", 1.0))),
            ne, eps, off, _ptr(w_q, C.c_float), _ptr(w_k, C.c_float),
            _ptr(q_in, C.c_float), _ptr(k_in, C.c_float), _ptr(v_in, C.c_float),
            _ptr(positions, C.c_int32), k_dtype, v_dtype, cap, _ptr(cache_k), _ptr(cache_v),
            _ptr(k_scale, C.c_float), _ptr(v_scale, C.c_float), _ptr(q_out, C.c_double))
        if rc != 0:
            raise ValueError("oracle_kv_produce rejected its arguments")
        return q_out

    # -- attention -----------------------------------------------------------
    def _cache_args(self, cache_k, cache_v, v_scale, k_dtype, v_dtype, k_scale=None):
        _need(cache_k, _STORAGE[k_dtype], "cache_k")
        _need(cache_v, _STORAGE[v_dtype], "cache_v")
        if v_dtype == I8:
            _need(v_scale, np.float32, "v_scale")
        if k_dtype == I8:
            _need(k_scale, np.float32, "k_scale")
        return cache_k.shape[2]

    def scores(self, *, q, cache_k, k_dtype, n_heads, b, h, L, window=0, softcap=0.0,
               k_scale=None):
        Hkv, cap, d = cache_k.shape[1], cache_k.shape[2], cache_k.shape[3]
        _need(cache_k, _STORAGE[k_dtype], "cache_k")
        if k_dtype == I8:
            _need(k_scale, np.float32, "k_scale")
        qv = np.ascontiguousarray(q, dtype=np.float64)
        s = np.zeros(int(L), dtype=np.float64)
        self.lib.oracle_scores(n_heads, Hkv, d, k_dtype, cap, _ptr(cache_k),
                               _ptr(k_scale, C.c_float), _ptr(qv, C.c_double),
                               int(b), int(h), int(L), int(window), float(softcap),
                               _ptr(s, C.c_double))
        return s

    def decode(self, *, q, cache_k, cache_v, v_scale=None, k_dtype, v_dtype, seq_lens,
               window=0, softcap=0.0, pairs=None, sinks=None, k_scale=None):
        """Single-pass attention; q is [B][H][d] (any float dtype, widened to
        double); sinks is an optional per-head attention-sink logit [H].
        Returns [B][H][d] double, or [len(pairs)][d] for a list of (b, h)
        pairs."""
        B, H, d = q.shape
        Hkv = cache_k.shape[1]
        cap = self._cache_args(cache_k, cache_v, v_scale, k_dtype, v_dtype, k_scale)
        qd = np.ascontiguousarray(q, dtype=np.float64)
        lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        if pairs is None:
            pr = np.array([(b, h) for b in range(B) for h in range(H)], dtype=np.int32)
        else:
            pr = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        out = np.zeros((len(pr), d), dtype=np.float64)
        sk = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float64)
        if sk is not None and sk.shape != (H,):
            raise ValueError(f"sinks must have shape ({H},)")
        rc = self.lib.oracle_decode_pairs(B, H, Hkv, d, k_dtype, v_dtype, cap, _ptr(cache_k),
                                          _ptr(cache_v), _ptr(k_scale, C.c_float),
                                          _ptr(v_scale, C.c_float),
                                          _ptr(qd, C.c_double), _ptr(lens, C.c_int32),
                                          int(window), float(softcap), _ptr(sk, C.c_double),
                                          _ptr(pr, C.c_int32), len(pr), _ptr(out, C.c_double))
        if rc != 0:
            raise ValueError("oracle_decode_pairs rejected its arguments")
        return out.reshape(B, H, d) if pairs is None else out

    def split_partial(self, *, q_bh, cache_k, cache_v, v_scale=None, k_dtype, v_dtype,
                      n_heads, b, h, L, window, softcap, split_size, sigma, k_scale=None):
        """(o[d], lse, n_keys) of split sigma for one (b, h); q_bh is [d]."""
        Hkv, d = cache_k.shape[1], cache_k.shape[3]
        cap = self._cache_args(cache_k, cache_v, v_scale, k_dtype, v_dtype, k_scale)
        qv = np.ascontiguousarray(q_bh, dtype=np.float64)
        o = np.zeros(d, dtype=np.float64)
        lse = np.zeros(1, dtype=np.float64)
        n = self.lib.oracle_split_partial(n_heads, Hkv, d, k_dtype, v_dtype, cap, _ptr(cache_k),
                                          _ptr(cache_v), _ptr(k_scale, C.c_float),
                                          _ptr(v_scale, C.c_float),
                                          _ptr(qv, C.c_double), int(b), int(h), int(L),
                                          int(window), float(softcap), int(split_size),
                                          int(sigma), _ptr(o, C.c_double),
                                          _ptr(lse, C.c_double))
        return o, float(lse[0]), int(n)

    def combine(self, o, lse, sink=None):
        o = np.ascontiguousarray(o, dtype=np.float64)
        lse = np.ascontiguousarray(lse, dtype=np.float64)
        out = np.zeros(o.shape[1], dtype=np.float64)
        used = self.lib.oracle_combine(o.shape[0], o.shape[1], _ptr(o, C.c_double),
                                       _ptr(lse, C.c_double), 0 if sink is None else 1,
                                       0.0 if sink is None else float(sink),
                                       _ptr(out, C.c_double))
        return out, int(used)


    # -- chunks of new tokens (prefill) ---------------------------------------
    def kv_produce_chunk(self, *, rope: dict, norm: dict | None, q_in, k_in, v_in,
                         start_positions, k_dtype: int, v_dtype: int, cache_k, cache_v,
                         v_scale=None, k_scale=None):
        """The producer for T new tokens per sequence ("Universal AI Inference"
        P1.3: every token is rotated at its own absolute position and stored at
        that slot): token t of sequence b is produced exactly as a single-token
        producer produces it at position start_positions[b] + t.  q_in is
        [B][T][H][d], k_in and v_in [B][T][Hkv][d]; returns q' [B][T][H][d]
        (double) and writes the T slots of every (b, kv head) in place."""
        B, T, H, d = q_in.shape
        start = np.asarray(start_positions, dtype=np.int64)
        q_out = np.zeros((B, T, H, d), dtype=np.float64)
        for t in range(T):
            q_out[:, t] = self.kv_produce(
                rope=rope, norm=norm, q_in=np.ascontiguousarray(q_in[:, t]),
                k_in=np.ascontiguousarray(k_in[:, t]), v_in=np.ascontiguousarray(v_in[:, t]),
                positions=(start + t).astype(np.int32), k_dtype=k_dtype, v_dtype=v_dtype,
                cache_k=cache_k, cache_v=cache_v, v_scale=v_scale, k_scale=k_scale)
        return q_out

    def prefill(self, *, q, cache_k, cache_v, v_scale=None, k_dtype, v_dtype, seq_lens,
                window=0, softcap=0.0, sinks=None, k_scale=None, triples=None):
        """Causal attention of a chunk: the T queries of sequence b sit at
        positions L_b - T .. L_b - 1 and query t sees the keys up to its own
        position, within its own window ("Universal AI Inference" P1.3 and
        P1.4).  That is decode attention of query t over the first
        L_b - T + t + 1 keys, which is what this computes.  q is
        [B][T][H][d]; returns [B][T][H][d] double, or [n][d] for a list of
        (b, t, h) triples."""
        B, T, H, d = q.shape
        lens = np.asarray(seq_lens, dtype=np.int64)

        def prefix(t):  # keys that query t may see: positions 0 .. L - T + t
            return (lens - T + t + 1).astype(np.int32)

        if triples is None:
            out = np.zeros((B, T, H, d), dtype=np.float64)
            for t in range(T):
                out[:, t] = self.decode(q=np.ascontiguousarray(q[:, t]), cache_k=cache_k,
                                        cache_v=cache_v, v_scale=v_scale, k_scale=k_scale,
                                        k_dtype=k_dtype, v_dtype=v_dtype,
                                        seq_lens=prefix(t), window=window, softcap=softcap,
                                        sinks=sinks)
            return out
        tr = np.asarray(triples, dtype=np.int64).reshape(-1, 3)
        out = np.zeros((len(tr), d), dtype=np.float64)
        for t in np.unique(tr[:, 1]):
            sel = np.nonzero(tr[:, 1] == t)[0]
            pairs = tr[sel][:, [0, 2]]
            out[sel] = self.decode(q=np.ascontiguousarray(q[:, t]), cache_k=cache_k,
                                   cache_v=cache_v, v_scale=v_scale, k_scale=k_scale,
                                   k_dtype=k_dtype, v_dtype=v_dtype,
                                   seq_lens=prefix(t), window=window, softcap=softcap,
                                   sinks=sinks, pairs=pairs)
        return out


_default: Oracle | None = None


def load() -> Oracle:
    """The oracle built from ``oracle.c`` (built on first use if missing)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
