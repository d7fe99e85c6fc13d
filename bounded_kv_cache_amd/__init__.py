"""Prefix Sliding attention for MI355X (gfx950): thin Python binding over the C ABI.

The functions here only check tensor metadata and pass pointers, sizes and
the current HIP stream to ``libprefix_sliding.so``; every step of the
computation runs in the library's HIP kernels.  torch supplies device memory
and streams.  Cache layout, semantics and error behaviour are documented in
include/prefix_sliding.h.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
from typing import Optional

import torch

from . import _lib
from ._lib import PS_BF16, PS_F32, PS_PE_CONTINUE, PS_PE_RESET, PS_PE_RESET_RECOMPUTE, PSError

__all__ = ["AttnSpec", "CacheSpec", "PSError", "ps_kv_append", "ps_decode_attn", "ps_prefill_attn",
           "ps_chunk_prefill_attn", "ps_chunk_prefill_workspace_size", "ps_prefill_attn_backward",
           "ps_prefill_backward_workspace_size", "ps_prefill_backward_ds_workspace_size", "ps_heavy_decode_step", "ps_heavy_workspace_size", "HeavyState",
           "ps_prefill_plan", "ps_decode_workspace_size", "ps_decode_num_splits", "ps_prefill_workspace_size",
           "ps_prefill_tile_shape", "ps_read_probe", "ps_decode_step", "ps_decode_step_noalloc", "ps_abi_version", "cache_shapes", "PS_BF16", "PS_F32", "PS_PE_CONTINUE",
           "PS_PE_RESET", "PS_PE_RESET_RECOMPUTE"]

_TORCH_DTYPE = {PS_BF16: torch.bfloat16, PS_F32: torch.float32}


@dataclasses.dataclass(frozen=True)
class AttnSpec:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: int = PS_BF16
    rope_theta: float = 10000.0
    softmax_scale: Optional[float] = None  # default 1/sqrt(head_dim)
    pe_mode: int = PS_PE_CONTINUE          # PS_PE_RESET / PS_PE_RESET_RECOMPUTE: decode only

    def c(self) -> _lib.AttnDesc:
        scale = self.softmax_scale if self.softmax_scale is not None else 1.0 / math.sqrt(self.head_dim)
        return _lib.AttnDesc(self.num_q_heads, self.num_kv_heads, self.head_dim, self.dtype, float(self.rope_theta),
                             float(scale), int(self.pe_mode))

    @property
    def torch_dtype(self) -> torch.dtype:
        return _TORCH_DTYPE[self.dtype]


@dataclasses.dataclass(frozen=True)
class CacheSpec:
    window: int
    slot_capacity: int          # multiple of 64, >= prefix_len + window of every sequence
    page_size: int = 0          # 0 contiguous, 64 paged
    num_pages: int = 0          # paged: pool size

    def c(self) -> _lib.CacheDesc:
        mp = self.slot_capacity // 64 if self.page_size == 64 else 0
        return _lib.CacheDesc(self.window, self.page_size, self.slot_capacity, mp, self.num_pages)


def cache_shapes(attn: AttnSpec, cache: CacheSpec, num_seqs: int):
    """Tensor shapes of one layer's K and V caches (see the layout in the header)."""
    d, h = attn.head_dim, attn.num_kv_heads
    if cache.page_size == 64:
        return (cache.num_pages, h, 64, d), (cache.num_pages, h, 8, d, 8)
    return (num_seqs, h, cache.slot_capacity, d), (num_seqs, h, cache.slot_capacity // 8, d, 8)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, numel: Optional[int] = None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def ps_abi_version() -> int:
    return _lib.load().ps_abi_version()


def ps_decode_num_splits(attn: AttnSpec, cache: CacheSpec, num_seqs: int) -> int:
    a, c = attn.c(), cache.c()
    return _lib.load().ps_decode_num_splits(ctypes.byref(a), ctypes.byref(c), num_seqs)


def ps_decode_workspace_size(attn: AttnSpec, cache: CacheSpec, num_seqs: int, num_splits: int = 0) -> int:
    a, c = attn.c(), cache.c()
    return _lib.load().ps_decode_workspace_size(ctypes.byref(a), ctypes.byref(c), num_seqs, num_splits)


def ps_prefill_workspace_size(attn: AttnSpec, batch: int, num_queries: int, num_keys: int) -> int:
    a = attn.c()
    return _lib.load().ps_prefill_workspace_size(ctypes.byref(a), batch, num_queries, num_keys)


def ps_read_probe(src: torch.Tensor, checksum: torch.Tensor, *, stream=None) -> torch.Tensor:
    """Read every byte of `src` once on the GPU; `checksum` (one int32 on the
    device) receives the XOR of its 32-bit words.  A bandwidth-measurement helper."""
    if not src.is_cuda or not checksum.is_cuda or checksum.dtype != torch.int32 or checksum.numel() < 1:
        raise ValueError("src and a one-element int32 checksum must be device tensors")
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    _lib.check(_lib.load().ps_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(checksum),
                                         _stream(stream)))
    return checksum


def ps_prefill_tile_shape(attn: AttnSpec):
    a = attn.c()
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _lib.check(_lib.load().ps_prefill_tile_shape(ctypes.byref(a), ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def ps_kv_append(attn: AttnSpec, cache: CacheSpec, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 prefix_len: torch.Tensor, start_pos: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, *,
                 block_table: Optional[torch.Tensor] = None, seq_tokens: Optional[torch.Tensor] = None,
                 slot_pos: Optional[torch.Tensor] = None, stream=None) -> None:
    """Append k_new/v_new [num_seqs, T, Hkv, D] at positions start_pos[s] + t."""
    dt = attn.torch_dtype
    num_seqs, tokens = k_new.shape[0], k_new.shape[1]
    _need(k_new, "k_new", dt, num_seqs * tokens * attn.num_kv_heads * attn.head_dim)
    _need(v_new, "v_new", dt, k_new.numel())
    ks, vs = cache_shapes(attn, cache, num_seqs)
    _need(k_cache, "k_cache", dt, math.prod(ks))
    _need(v_cache, "v_cache", dt, math.prod(vs))
    _need(prefix_len, "prefix_len", torch.int32, num_seqs)
    _need(start_pos, "start_pos", torch.int64, num_seqs)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32, num_seqs * (cache.slot_capacity // 64))
    if seq_tokens is not None:
        _need(seq_tokens, "seq_tokens", torch.int32, num_seqs)
    if slot_pos is not None:
        _need(slot_pos, "slot_pos", torch.int32, num_seqs * cache.slot_capacity)
    a, c = attn.c(), cache.c()
    _lib.check(_lib.load().ps_kv_append(ctypes.byref(a), ctypes.byref(c), _ptr(k_cache), _ptr(v_cache),
                                        _ptr(block_table), _ptr(prefix_len), _ptr(start_pos), _ptr(seq_tokens),
                                        tokens, _ptr(k_new), _ptr(v_new), num_seqs, _ptr(slot_pos),
                                        _stream(stream)))


def ps_decode_attn(attn: AttnSpec, cache: CacheSpec, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   prefix_len: torch.Tensor, pos: torch.Tensor, q: torch.Tensor, out: torch.Tensor, *,
                   block_table: Optional[torch.Tensor] = None, num_splits: int = 0,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Decode attention of q [num_seqs, Hq, D] at positions pos; writes out [num_seqs, Hq, D]."""
    dt = attn.torch_dtype
    num_seqs = q.shape[0]
    _need(q, "q", dt, num_seqs * attn.num_q_heads * attn.head_dim)
    _need(out, "out", dt, q.numel())
    ks, vs = cache_shapes(attn, cache, num_seqs)
    _need(k_cache, "k_cache", dt, math.prod(ks))
    _need(v_cache, "v_cache", dt, math.prod(vs))
    _need(prefix_len, "prefix_len", torch.int32, num_seqs)
    _need(pos, "pos", torch.int64, num_seqs)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32, num_seqs * (cache.slot_capacity // 64))
    need = ps_decode_workspace_size(attn, cache, num_seqs, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a, c = attn.c(), cache.c()
    _lib.check(_lib.load().ps_decode_attn(ctypes.byref(a), ctypes.byref(c), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(block_table), _ptr(prefix_len), _ptr(pos), _ptr(q), _ptr(out),
                                          num_seqs, num_splits, _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def ps_decode_step_noalloc(attn: AttnSpec, cache: CacheSpec, k_cache: torch.Tensor, v_cache: torch.Tensor,
                           prefix_len: torch.Tensor, pos: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                           v_new: torch.Tensor, out: torch.Tensor, *, block_table: Optional[torch.Tensor] = None,
                           num_splits: int = 0, stream=None) -> torch.Tensor:
    """ps_decode_step without a workspace: the split partials use the library's
    static device scratch, so the call allocates nothing (see the header)."""
    dt = attn.torch_dtype
    num_seqs = q.shape[0]
    _need(q, "q", dt, num_seqs * attn.num_q_heads * attn.head_dim)
    _need(out, "out", dt, q.numel())
    _need(k_new, "k_new", dt, num_seqs * attn.num_kv_heads * attn.head_dim)
    _need(v_new, "v_new", dt, k_new.numel())
    ks, vs = cache_shapes(attn, cache, num_seqs)
    _need(k_cache, "k_cache", dt, math.prod(ks))
    _need(v_cache, "v_cache", dt, math.prod(vs))
    _need(prefix_len, "prefix_len", torch.int32, num_seqs)
    _need(pos, "pos", torch.int64, num_seqs)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32, num_seqs * (cache.slot_capacity // 64))
    a, c = attn.c(), cache.c()
    _lib.check(_lib.load().ps_decode_step_noalloc(ctypes.byref(a), ctypes.byref(c), _ptr(k_cache), _ptr(v_cache),
                                                  _ptr(block_table), _ptr(prefix_len), _ptr(pos), _ptr(q),
                                                  _ptr(k_new), _ptr(v_new), _ptr(out), num_seqs, num_splits,
                                                  _stream(stream)))
    return out


def ps_decode_step(attn: AttnSpec, cache: CacheSpec, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   prefix_len: torch.Tensor, pos: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                   v_new: torch.Tensor, out: torch.Tensor, *, block_table: Optional[torch.Tensor] = None,
                   num_splits: int = 0, workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Append the token at pos (k_new, v_new [num_seqs, 1, Hkv, D]) and attend with q at pos (see the header)."""
    dt = attn.torch_dtype
    num_seqs = q.shape[0]
    _need(q, "q", dt, num_seqs * attn.num_q_heads * attn.head_dim)
    _need(out, "out", dt, q.numel())
    _need(k_new, "k_new", dt, num_seqs * attn.num_kv_heads * attn.head_dim)
    _need(v_new, "v_new", dt, k_new.numel())
    ks, vs = cache_shapes(attn, cache, num_seqs)
    _need(k_cache, "k_cache", dt, math.prod(ks))
    _need(v_cache, "v_cache", dt, math.prod(vs))
    _need(prefix_len, "prefix_len", torch.int32, num_seqs)
    _need(pos, "pos", torch.int64, num_seqs)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32, num_seqs * (cache.slot_capacity // 64))
    need = ps_decode_workspace_size(attn, cache, num_seqs, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    a, c = attn.c(), cache.c()
    _lib.check(_lib.load().ps_decode_step(ctypes.byref(a), ctypes.byref(c), _ptr(k_cache), _ptr(v_cache),
                                          _ptr(block_table), _ptr(prefix_len), _ptr(pos), _ptr(q), _ptr(k_new),
                                          _ptr(v_new), _ptr(out), num_seqs, num_splits, _ptr(workspace), ws_bytes,
                                          _stream(stream)))
    return out


def ps_prefill_attn(attn: AttnSpec, window: int, prefix_len: int, kv_start: int, q: torch.Tensor,
                    k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, *, lse: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Masked attention of q [B, T, Hq, D] over k, v [B, Nk, Hkv, D]; writes out [B, T, Hq, D]."""
    dt = attn.torch_dtype
    batch, num_q = q.shape[0], q.shape[1]
    num_k = k.shape[1]
    _need(q, "q", dt, batch * num_q * attn.num_q_heads * attn.head_dim)
    _need(k, "k", dt, batch * num_k * attn.num_kv_heads * attn.head_dim)
    _need(v, "v", dt, k.numel())
    _need(out, "out", dt, q.numel())
    if lse is not None:
        _need(lse, "lse", torch.float32, batch * attn.num_q_heads * num_q)
    need = ps_prefill_workspace_size(attn, batch, num_q, num_k)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    a = attn.c()
    _lib.check(_lib.load().ps_prefill_attn(ctypes.byref(a), window, prefix_len, kv_start, _ptr(q), _ptr(k), _ptr(v),
                                           batch, num_q, num_k, _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                           _stream(stream)))
    return out


def ps_heavy_workspace_size(attn: AttnSpec, cache: CacheSpec, num_seqs: int, num_splits: int = 0) -> int:
    a, c = attn.c(), cache.c()
    return _lib.load().ps_heavy_workspace_size(ctypes.byref(a), ctypes.byref(c), num_seqs, num_splits)


@dataclasses.dataclass
class HeavyState:
    """Caller-owned state of prefix + heavy hitters + window decoding (zeros = new sequences)."""
    score: torch.Tensor        # [num_seqs, Hkv, slot_capacity] float32
    heavy_count: torch.Tensor  # [num_seqs, Hkv] int32
    heavy_pos: torch.Tensor    # [num_seqs, Hkv, heavy_slots] int64

    @staticmethod
    def new(attn: AttnSpec, cache: CacheSpec, num_seqs: int, heavy_slots: int, device="cuda") -> "HeavyState":
        h = attn.num_kv_heads
        return HeavyState(torch.zeros((num_seqs, h, cache.slot_capacity), dtype=torch.float32, device=device),
                          torch.zeros((num_seqs, h), dtype=torch.int32, device=device),
                          torch.full((num_seqs, h, max(heavy_slots, 1)), -1, dtype=torch.int64, device=device))


def ps_heavy_decode_step(attn: AttnSpec, cache: CacheSpec, heavy_slots: int, k_cache: torch.Tensor,
                         v_cache: torch.Tensor, prefix_len: torch.Tensor, pos: torch.Tensor, q: torch.Tensor,
                         k_new: torch.Tensor, v_new: torch.Tensor, out: torch.Tensor, state: HeavyState, *,
                         block_table: Optional[torch.Tensor] = None, num_splits: int = 0,
                         workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decode step at positions pos with prefix + heavy hitters + window (see the header)."""
    dt = attn.torch_dtype
    num_seqs = q.shape[0]
    _need(q, "q", dt, num_seqs * attn.num_q_heads * attn.head_dim)
    _need(out, "out", dt, q.numel())
    _need(k_new, "k_new", dt, num_seqs * attn.num_kv_heads * attn.head_dim)
    _need(v_new, "v_new", dt, k_new.numel())
    ks, vs = cache_shapes(attn, cache, num_seqs)
    _need(k_cache, "k_cache", dt, math.prod(ks))
    _need(v_cache, "v_cache", dt, math.prod(vs))
    _need(prefix_len, "prefix_len", torch.int32, num_seqs)
    _need(pos, "pos", torch.int64, num_seqs)
    _need(state.score, "score", torch.float32, num_seqs * attn.num_kv_heads * cache.slot_capacity)
    _need(state.heavy_count, "heavy_count", torch.int32, num_seqs * attn.num_kv_heads)
    _need(state.heavy_pos, "heavy_pos", torch.int64)
    if state.heavy_pos.numel() < num_seqs * attn.num_kv_heads * heavy_slots:
        raise ValueError("heavy_pos too small")
    if block_table is not None:
        _need(block_table, "block_table", torch.int32, num_seqs * (cache.slot_capacity // 64))
    need = ps_heavy_workspace_size(attn, cache, num_seqs, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    a, c = attn.c(), cache.c()
    _lib.check(_lib.load().ps_heavy_decode_step(ctypes.byref(a), ctypes.byref(c), heavy_slots, _ptr(k_cache),
                                                _ptr(v_cache), _ptr(block_table), _ptr(prefix_len), _ptr(pos),
                                                _ptr(q), _ptr(k_new), _ptr(v_new), _ptr(out), num_seqs,
                                                _ptr(state.score), _ptr(state.heavy_count), _ptr(state.heavy_pos),
                                                num_splits, _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def ps_prefill_backward_workspace_size(attn: AttnSpec, batch: int, num_queries: int, num_keys: int) -> int:
    a = attn.c()
    return _lib.load().ps_prefill_backward_workspace_size(ctypes.byref(a), batch, num_queries, num_keys)


def ps_prefill_backward_ds_workspace_size(attn: AttnSpec, window: int, prefix_len: int, kv_start: int, batch: int,
                                          num_queries: int, num_keys: int) -> int:
    a = attn.c()
    return _lib.load().ps_prefill_backward_ds_workspace_size(ctypes.byref(a), window, prefix_len, kv_start, batch,
                                                             num_queries, num_keys)


def ps_prefill_attn_backward(attn: AttnSpec, window: int, prefix_len: int, kv_start: int, q: torch.Tensor,
                             k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, d_out: torch.Tensor,
                             lse: torch.Tensor, dq: torch.Tensor, dk: torch.Tensor, dv: torch.Tensor, *,
                             workspace: Optional[torch.Tensor] = None, keep_ds: Optional[bool] = None,
                             stream=None):
    """Gradients of ps_prefill_attn: writes dq [B, T, Hq, D], dk and dv [B, Nk, Hkv, D].

    Without a workspace one is allocated: with the extra dS room (the dq pass then
    reads the dk/dv pass's dS tiles) when keep_ds is True, or when keep_ds is None and
    that room is at most a quarter of the free device memory."""
    dt = attn.torch_dtype
    batch, num_q = q.shape[0], q.shape[1]
    num_k = k.shape[1]
    _need(q, "q", dt, batch * num_q * attn.num_q_heads * attn.head_dim)
    _need(k, "k", dt, batch * num_k * attn.num_kv_heads * attn.head_dim)
    _need(v, "v", dt, k.numel())
    _need(out, "out", dt, q.numel())
    _need(d_out, "d_out", dt, q.numel())
    _need(lse, "lse", torch.float32, batch * attn.num_q_heads * num_q)
    _need(dq, "dq", dt, q.numel())
    _need(dk, "dk", dt, k.numel())
    _need(dv, "dv", dt, k.numel())
    need = ps_prefill_backward_workspace_size(attn, batch, num_q, num_k)
    if workspace is None:
        extra = ps_prefill_backward_ds_workspace_size(attn, window, prefix_len, kv_start, batch, num_q, num_k)
        if keep_ds is None:
            keep_ds = extra <= torch.cuda.mem_get_info(q.device)[0] // 4
        workspace = torch.empty(max(need + (extra if keep_ds else 0), 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    a = attn.c()
    _lib.check(_lib.load().ps_prefill_attn_backward(ctypes.byref(a), window, prefix_len, kv_start, _ptr(q), _ptr(k),
                                                    _ptr(v), _ptr(out), _ptr(d_out), _ptr(lse), batch, num_q, num_k,
                                                    _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                                                    _stream(stream)))
    return dq, dk, dv


def ps_chunk_prefill_workspace_size(attn: AttnSpec, cache: CacheSpec, num_seqs: int, chunk_len: int) -> int:
    a, c = attn.c(), cache.c()
    return _lib.load().ps_chunk_prefill_workspace_size(ctypes.byref(a), ctypes.byref(c), num_seqs, chunk_len)


def ps_chunk_prefill_attn(attn: AttnSpec, cache: CacheSpec, k_cache: torch.Tensor, v_cache: torch.Tensor,
                          prefix_len: torch.Tensor, start_pos: torch.Tensor, q: torch.Tensor, k_new: torch.Tensor,
                          v_new: torch.Tensor, out: torch.Tensor, *, block_table: Optional[torch.Tensor] = None,
                          lse: Optional[torch.Tensor] = None, slot_pos: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Chunk q/k_new/v_new [num_seqs, T, H, D] at positions start_pos[s] + t: attention over each ring plus
    the chunk (writes out [num_seqs, T, Hq, D]), then the chunk is appended to the rings."""
    dt = attn.torch_dtype
    num_seqs, chunk = q.shape[0], q.shape[1]
    _need(q, "q", dt, num_seqs * chunk * attn.num_q_heads * attn.head_dim)
    _need(k_new, "k_new", dt, num_seqs * chunk * attn.num_kv_heads * attn.head_dim)
    _need(v_new, "v_new", dt, k_new.numel())
    _need(out, "out", dt, q.numel())
    ks, vs = cache_shapes(attn, cache, num_seqs)
    _need(k_cache, "k_cache", dt, math.prod(ks))
    _need(v_cache, "v_cache", dt, math.prod(vs))
    _need(prefix_len, "prefix_len", torch.int32, num_seqs)
    _need(start_pos, "start_pos", torch.int64, num_seqs)
    if block_table is not None:
        _need(block_table, "block_table", torch.int32, num_seqs * (cache.slot_capacity // 64))
    if lse is not None:
        _need(lse, "lse", torch.float32, num_seqs * attn.num_q_heads * chunk)
    if slot_pos is not None:
        _need(slot_pos, "slot_pos", torch.int32, num_seqs * cache.slot_capacity)
    need = ps_chunk_prefill_workspace_size(attn, cache, num_seqs, chunk)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    a, c = attn.c(), cache.c()
    _lib.check(_lib.load().ps_chunk_prefill_attn(ctypes.byref(a), ctypes.byref(c), _ptr(k_cache), _ptr(v_cache),
                                                 _ptr(block_table), _ptr(prefix_len), _ptr(start_pos), chunk,
                                                 _ptr(q), _ptr(k_new), _ptr(v_new), num_seqs, _ptr(out), _ptr(lse),
                                                 _ptr(slot_pos), _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def ps_prefill_plan(attn: AttnSpec, window: int, prefix_len: int, kv_start: int, num_queries: int, num_keys: int,
                    tiles: torch.Tensor, num_tiles: torch.Tensor, stream=None) -> None:
    """Write the executed tile list ((q_tile, k_tile, kind) int32 triples) into tiles [max_tiles, 3]."""
    _need(num_tiles, "num_tiles", torch.int32, 1)
    _need(tiles, "tiles", torch.int32)
    if tiles.dim() != 2 or tiles.shape[1] != 3:
        raise ValueError("tiles must be [max_tiles, 3]")
    a = attn.c()
    _lib.check(_lib.load().ps_prefill_plan(ctypes.byref(a), window, prefix_len, kv_start, num_queries, num_keys,
                                           _ptr(tiles), tiles.shape[0], _ptr(num_tiles), _stream(stream)))
