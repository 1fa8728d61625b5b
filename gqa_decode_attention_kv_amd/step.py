"""One decode step on the GPU for a seeded workload.

torch provides device memory and the stream only; the three calls go
through the C ABI (``binding``) into the HIP kernels.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import binding as B
from .workloads import BF16, F32, I8, Inputs, PagedInputs, Workload

_TORCH = {F32: torch.float32, BF16: torch.int16, I8: torch.int8}


def _dev(a: np.ndarray, device) -> torch.Tensor:
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


class DeviceStep:
    """Device buffers of one layer's decode step and the calls that run it."""

    def __init__(self, inputs: Inputs, device: str = "cuda", split_size: int | None = None,
                 paged: PagedInputs | None = None):
        if not torch.cuda.is_available():
            raise RuntimeError("DeviceStep needs a GPU (torch.cuda.is_available() is False)")
        w: Workload = inputs.workload
        self.w, self.inputs, self.device = w, inputs, device
        self.split_size = int(split_size or w.split_size)
        lens = inputs.seq_lens
        self.seq_lens = np.ascontiguousarray(lens, dtype=np.int32)
        self.positions = np.ascontiguousarray(inputs.positions, dtype=np.int32)
        self.max_splits = int(-(-int(lens.max()) // self.split_size))
        Bn, H, Hkv, d = w.batch, w.n_heads, w.n_kv_heads, w.head_dim

        self.q_in = _dev(inputs.q_in, device)
        self.k_in = _dev(inputs.k_in, device)
        self.v_in = _dev(inputs.v_in, device)
        self.paged = paged
        src_k = paged.pool_k if paged else inputs.cache_k
        src_v = paged.pool_v if paged else inputs.cache_v
        src_s = paged.pool_scale if paged else inputs.v_scale
        src_ks = paged.pool_k_scale if paged else inputs.k_scale
        self.cache_k = _dev(src_k, device)
        self.cache_v = _dev(src_v, device)
        self.v_scale = _dev(src_s, device) if src_s is not None else None
        self.k_scale = _dev(src_ks, device) if src_ks is not None else None
        self.sinks = _dev(inputs.sinks, device) if inputs.sinks is not None else None
        self.block_table = _dev(paged.block_table, device) if paged else None
        self.w_q = _dev(inputs.w_q, device) if inputs.w_q is not None else None
        self.w_k = _dev(inputs.w_k, device) if inputs.w_k is not None else None
        self.q_out = torch.empty((Bn, H, d), dtype=torch.float32, device=device)
        self.part_o = torch.empty((Bn, H, self.max_splits, d), dtype=torch.float32, device=device)
        self.part_lse = torch.empty((Bn, H, self.max_splits), dtype=torch.float32, device=device)
        self.out = torch.empty((Bn, H, d), dtype=torch.float32, device=device)
        # Arrival counters of the single-launch step: zero once, and every
        # completed step leaves them at zero.
        self.counters = torch.zeros((Bn, Hkv), dtype=torch.int32, device=device)

        self.shape = B.Shape(Bn, H, Hkv, d)
        r = w.rope
        self.rope = B.Rope(r.pairing, r.scaling, r.theta, r.factor, r.low, r.high, r.orig,
                           int(r.truncate), r.attn_factor)
        n = w.qk_norm
        self.qk_norm = (B.QKNorm(1, n.eps, n.offset, self.w_q.data_ptr(), self.w_k.data_ptr())
                        if n.enabled else None)
        vs_ptr = self.v_scale.data_ptr() if self.v_scale is not None else None
        ks_ptr = self.k_scale.data_ptr() if self.k_scale is not None else None
        if paged:
            self.cache = B.KVCache(w.k_dtype, w.v_dtype, paged.capacity, self.cache_k.data_ptr(),
                                   self.cache_v.data_ptr(), vs_ptr, self.block_table.data_ptr(),
                                   paged.block_size, paged.max_blocks, paged.num_blocks, ks_ptr)
        else:
            self.cache = B.KVCache(w.k_dtype, w.v_dtype, w.capacity, self.cache_k.data_ptr(),
                                   self.cache_v.data_ptr(), vs_ptr, None, 0, 0, 0, ks_ptr)
        self.scale = 1.0 / math.sqrt(d)

    @staticmethod
    def stream() -> int:
        return torch.cuda.current_stream().cuda_stream

    def produce(self):
        B.kv_produce(self.shape, self.rope, self.qk_norm, self.q_in.data_ptr(),
                     self.k_in.data_ptr(), self.v_in.data_ptr(), self.positions, self.cache,
                     self.q_out.data_ptr(), self.stream())

    def attn(self):
        B.decode_attn(self.shape, self.cache, self.q_out.data_ptr(), self.seq_lens, self.scale,
                      self.w.window, self.w.softcap, self.split_size, self.max_splits,
                      self.part_o.data_ptr(), self.part_lse.data_ptr(), self.stream())

    def combine(self):
        if self.sinks is not None:
            B.decode_combine_sink(self.shape, self.seq_lens, self.w.window, self.split_size,
                                  self.max_splits, self.part_o.data_ptr(),
                                  self.part_lse.data_ptr(), self.sinks.data_ptr(),
                                  self.out.data_ptr(), self.stream())
        else:
            B.decode_combine(self.shape, self.seq_lens, self.w.window, self.split_size,
                             self.max_splits, self.part_o.data_ptr(), self.part_lse.data_ptr(),
                             self.out.data_ptr(), self.stream())

    def step(self):
        self.produce()
        self.attn()
        self.combine()

    def fused_step(self):
        """The same step as one launch (uaii_decode_step)."""
        B.decode_step(self.shape, self.rope, self.qk_norm, self.q_in.data_ptr(),
                      self.k_in.data_ptr(), self.v_in.data_ptr(), self.seq_lens, self.cache,
                      self.scale, self.w.window, self.w.softcap, self.split_size, self.max_splits,
                      self.sinks.data_ptr() if self.sinks is not None else None,
                      self.q_out.data_ptr(), self.part_o.data_ptr(), self.part_lse.data_ptr(),
                      self.counters.data_ptr(), self.out.data_ptr(), self.stream())

    # -- host copies for checking ------------------------------------------------
    def host(self, t: torch.Tensor, dtype=None) -> np.ndarray:
        a = t.cpu().numpy()
        if dtype is not None:
            a = a.view(dtype)
        return a

    def slot_index(self):
        """(first index, row index) of each sequence's new-token slot: (b, p)
        for a contiguous cache, (physical block, p % block_size) for a paged one."""
        p = self.positions.astype(np.int64)
        if self.paged:
            bs = self.paged.block_size
            blk = self.paged.block_table[np.arange(self.w.batch), p // bs].astype(np.int64)
            return blk, p % bs
        return np.arange(self.w.batch), p

    def cache_rows(self) -> dict:
        """The produced slot of every (b, kv head): K, V and (vq8) scale rows."""
        first, row = self.slot_index()
        bi = torch.as_tensor(first, device=self.device)
        idx = torch.as_tensor(row, device=self.device)
        k = self.cache_k[bi, :, idx].cpu().numpy()
        v = self.cache_v[bi, :, idx].cpu().numpy()
        if self.w.k_dtype == BF16:
            k = k.view(np.uint16)
        if self.w.v_dtype == BF16:
            v = v.view(np.uint16)
        s = self.v_scale[bi, :, idx].cpu().numpy() if self.v_scale is not None else None
        ks = self.k_scale[bi, :, idx].cpu().numpy() if self.k_scale is not None else None
        return dict(k=k, v=v, scale=s, k_scale=ks)


class DevicePrefill:
    """Device buffers of one layer's chunk step (T new tokens per sequence)
    and the two calls that run it: the chunk producer, then the chunk's
    causal attention."""

    def __init__(self, inputs, device: str = "cuda", paged: PagedInputs | None = None):
        if not torch.cuda.is_available():
            raise RuntimeError("DevicePrefill needs a GPU (torch.cuda.is_available() is False)")
        w: Workload = inputs.workload
        self.w, self.inputs, self.device, self.paged = w, inputs, device, paged
        self.T = int(w.chunk)
        self.seq_lens = np.ascontiguousarray(inputs.seq_lens, dtype=np.int32)
        self.start = np.ascontiguousarray(inputs.start, dtype=np.int32)
        Bn, H, Hkv, d = w.batch, w.n_heads, w.n_kv_heads, w.head_dim
        self.q_in = _dev(inputs.q_in, device)
        self.k_in = _dev(inputs.k_in, device)
        self.v_in = _dev(inputs.v_in, device)
        self.cache_k = _dev(paged.pool_k if paged else inputs.cache_k, device)
        self.cache_v = _dev(paged.pool_v if paged else inputs.cache_v, device)
        src_s = paged.pool_scale if paged else inputs.v_scale
        src_ks = paged.pool_k_scale if paged else inputs.k_scale
        self.v_scale = _dev(src_s, device) if src_s is not None else None
        self.k_scale = _dev(src_ks, device) if src_ks is not None else None
        self.block_table = _dev(paged.block_table, device) if paged else None
        self.sinks = _dev(inputs.sinks, device) if inputs.sinks is not None else None
        self.w_q = _dev(inputs.w_q, device) if inputs.w_q is not None else None
        self.w_k = _dev(inputs.w_k, device) if inputs.w_k is not None else None
        self.q_out = torch.empty((Bn, self.T, H, d), dtype=torch.float32, device=device)
        self.out = torch.empty((Bn, self.T, H, d), dtype=torch.float32, device=device)
        self.shape = B.Shape(Bn, H, Hkv, d)
        r = w.rope
        self.rope = B.Rope(r.pairing, r.scaling, r.theta, r.factor, r.low, r.high, r.orig,
                           int(r.truncate), r.attn_factor)
        n = w.qk_norm
        self.qk_norm = (B.QKNorm(1, n.eps, n.offset, self.w_q.data_ptr(), self.w_k.data_ptr())
                        if n.enabled else None)
        vs_ptr = self.v_scale.data_ptr() if self.v_scale is not None else None
        ks_ptr = self.k_scale.data_ptr() if self.k_scale is not None else None
        if paged:
            self.cache = B.KVCache(w.k_dtype, w.v_dtype, paged.capacity, self.cache_k.data_ptr(),
                                   self.cache_v.data_ptr(), vs_ptr, self.block_table.data_ptr(),
                                   paged.block_size, paged.max_blocks, paged.num_blocks, ks_ptr)
        else:
            self.cache = B.KVCache(w.k_dtype, w.v_dtype, w.capacity, self.cache_k.data_ptr(),
                                   self.cache_v.data_ptr(), vs_ptr, None, 0, 0, 0, ks_ptr)
        self.scale = 1.0 / math.sqrt(d)

    @staticmethod
    def stream() -> int:
        return torch.cuda.current_stream().cuda_stream

    def produce(self):
        B.kv_produce_chunk(self.shape, self.rope, self.qk_norm, self.q_in.data_ptr(),
                           self.k_in.data_ptr(), self.v_in.data_ptr(), self.start, self.T,
                           self.cache, self.q_out.data_ptr(), self.stream())

    def attn(self):
        B.prefill_attn(self.shape, self.cache, self.q_out.data_ptr(), self.seq_lens, self.T,
                       self.scale, self.w.window, self.w.softcap,
                       self.sinks.data_ptr() if self.sinks is not None else None,
                       self.out.data_ptr(), self.stream())

    def step(self):
        self.produce()
        self.attn()
