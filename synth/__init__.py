"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to a storage dtype.  It
holds none of the attention arithmetic: no visibility rule, no slot map, no
rotary embedding, no softmax.  Both the CPU oracle and the HIP path consume
what it returns, so a value that reaches the GPU and the float64 copy that
reaches the oracle are the same numbers bit for bit.

Every stream is keyed by ``numpy.random.SeedSequence([seed, *key])`` with a
PCG64 bit generator, so a tensor for one (sequence, layer, position-block) can
be regenerated on its own without drawing the tensors before it.

Workload shapes mirror the pages' settings: a Qwen3-1.7B attention geometry
(28 layers, 2 KV heads, head dim 128), a 100-token prefix with a 4096-token
window, positions of 32K and 128K, and a 7B-shaped truncated-backprop chunk
(28 query heads, 4 KV heads, an 8192-token chunk behind a 100-token prefix).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# tensor ids used in the seed key (stable: changing one changes every input)
T_Q, T_K, T_V, T_MISC = 1, 2, 3, 9

# positions are generated in blocks of this many tokens so that a long history
# can be regenerated block by block
POS_BLOCK = 4096


def rng(seed: int, *key: int) -> np.random.Generator:
    """A PCG64 generator for one named stream."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *[int(k) for k in key]])))


def normal(shape, seed: int, *key: int, std: float = 1.0) -> np.ndarray:
    """i.i.d. N(0, std^2) draws in float64."""
    return rng(seed, *key).standard_normal(size=shape) * float(std)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round a float64 array to ``dtype`` ('bf16' or 'f32') with round-to-nearest-even
    and return the rounded values as float64 (exactly representable)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        f = x.astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        # round to nearest even on the upper 16 bits (inputs here are finite)
        bias = ((u >> 16) & 1) + 0x7FFF
        r = ((u + bias) >> 16) << 16
        return r.astype(np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def history(seed: int, cfg_id: int, tensor: int, seq: int, layer: int, lo: int, hi: int,
            heads: int, dim: int, std: float, dtype: str) -> np.ndarray:
    """Raw per-position vectors for positions [lo, hi) of one (sequence, layer):
    shape [hi-lo, heads, dim], already rounded to ``dtype``.  Position blocks of
    POS_BLOCK tokens have their own streams, so any range is cheap to rebuild."""
    out = np.empty((max(hi - lo, 0), heads, dim), dtype=np.float64)
    if hi <= lo:
        return out
    b0, b1 = lo // POS_BLOCK, (hi - 1) // POS_BLOCK
    for b in range(b0, b1 + 1):
        blk = normal((POS_BLOCK, heads, dim), seed, cfg_id, tensor, seq, layer, b, std=std)
        s = max(lo, b * POS_BLOCK)
        e = min(hi, (b + 1) * POS_BLOCK)
        out[s - lo:e - lo] = blk[s - b * POS_BLOCK:e - b * POS_BLOCK]
    return round_to(out, dtype)


def query(seed: int, cfg_id: int, seq: int, layer: int, step: int, heads: int, dim: int,
          std: float, dtype: str) -> np.ndarray:
    """Raw query vectors [heads, dim] of one decode step."""
    return round_to(normal((heads, dim), seed, cfg_id, T_Q, seq, layer, step, std=std), dtype)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """Shape of a decode workload (one layer's cache per layer)."""
    name: str
    cfg_id: int
    num_seqs: int
    layers: int
    hq: int
    hkv: int
    dim: int
    dtype: str
    prefix: int          # L_prefix (uniform; ragged configs draw per sequence)
    window: int          # W
    position: int        # first measured query position P
    steps: int
    q_std: float
    kv_std: float
    rope_theta: float = 10000.0
    ragged: bool = False
    page_size: int = 0   # 0: contiguous ring per sequence; 64: paged

    @property
    def group(self) -> int:
        return self.hq // self.hkv


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    """Shape of a masked prefill / training-forward workload."""
    name: str
    cfg_id: int
    batch: int
    hq: int
    hkv: int
    dim: int
    dtype: str
    prefix: int
    window: int
    kv_start: int        # absolute position of the first chunk token
    chunk: int           # tokens in the chunk (keys after the prefix)
    queries: int         # T: queries are the last T keys
    q_std: float = 1.0
    kv_std: float = 1.0
    rope_theta: float = 10000.0

    @property
    def nk(self) -> int:
        return self.prefix + self.chunk


# Tiny single-layer check: fp32, Hq=4, Hkv=1, D=64, L=16, W=64, 80-slot ring,
# 1024 decode steps from an empty cache plus one masked prefill over 1024 tokens.
C1_DECODE = DecodeConfig("c1-tiny-decode", 1, num_seqs=1, layers=1, hq=4, hkv=1, dim=64, dtype="f32",
                         prefix=16, window=64, position=0, steps=1024, q_std=1.0, kv_std=1.0)
C1_PREFILL = PrefillConfig("c1-tiny-prefill", 1, batch=1, hq=4, hkv=1, dim=64, dtype="f32", prefix=16,
                           window=64, kv_start=16, chunk=1024 - 16, queries=1024)
# Qwen3-1.7B-shaped decode at 32K: 64 sequences, L=100, W=4096, 256 steps.
C2_DECODE = DecodeConfig("c2-decode-32k", 2, num_seqs=64, layers=28, hq=16, hkv=2, dim=128, dtype="bf16",
                         prefix=100, window=4096, position=32768, steps=256,
                         q_std=1.0, kv_std=0.5)
# Long-position decode: 256 sequences at 131072, W in {4096, 8192}.
C3_DECODE_W4096 = DecodeConfig("c3-decode-128k-w4096", 3, num_seqs=256, layers=28, hq=16, hkv=2, dim=128,
                               dtype="bf16", prefix=100, window=4096, position=131072, steps=256,
                               q_std=1.0, kv_std=0.5)
C3_DECODE_W8192 = dataclasses.replace(C3_DECODE_W4096, name="c3-decode-128k-w8192", window=8192)
# Full-attention comparator at the same position: the window covers the whole history.
C3_DECODE_FULL = dataclasses.replace(C3_DECODE_W4096, name="c3-decode-128k-full", prefix=0,
                                     window=1 << 30)
# Truncated-backprop forward, 7B-shaped: 8 x 8192-token chunk at 98304 behind a 100-token prefix.
C4_PREFILL = PrefillConfig("c4-prefill-7b", 4, batch=8, hq=28, hkv=4, dim=128, dtype="bf16", prefix=100,
                           window=2048, kv_start=98304, chunk=8192, queries=8192)
# Full-causal comparator: every position 0..106495 is a key.
C4_PREFILL_FULL = PrefillConfig("c4-prefill-7b-full-causal", 4, batch=8, hq=28, hkv=4, dim=128,
                                dtype="bf16", prefix=0, window=1 << 30, kv_start=0,
                                chunk=98304 + 8192, queries=8192)
# Ragged paged decode: 1024 sequences, p ~ U{1024..262144}, L ~ U{50..2000}, W=4096, 64-slot pages.
C5_DECODE = DecodeConfig("c5-ragged-paged", 5, num_seqs=1024, layers=28, hq=16, hkv=2, dim=128,
                         dtype="bf16", prefix=0, window=4096, position=0, steps=128,
                         q_std=1.0, kv_std=0.5, ragged=True, page_size=64)


@dataclasses.dataclass(frozen=True)
class ChunkConfig:
    """A chunk of new tokens continuing cached traces (ring + chunk attention)."""
    name: str
    cfg_id: int
    num_seqs: int
    hq: int
    hkv: int
    dim: int
    dtype: str
    prefix: int
    window: int
    position: int        # P: first chunk position (the ring holds positions < P)
    chunk: int           # T: chunk tokens
    q_std: float = 1.0
    kv_std: float = 0.5
    rope_theta: float = 10000.0
    page_size: int = 0


# Long external content (a tool output) poured into 64 live Qwen3-1.7B-shaped
# traces at 32768: L=100, W=4096, 2048-token chunk.
C6_CHUNK = ChunkConfig("c6-chunk-32k", 6, num_seqs=64, hq=16, hkv=2, dim=128, dtype="bf16", prefix=100,
                       window=4096, position=32768, chunk=2048)


def ragged_draws(seed: int, num_seqs: int, p_lo: int = 1024, p_hi: int = 262144,
                 l_lo: int = 50, l_hi: int = 2000):
    """Per-sequence query positions and prefix lengths, integer-uniform and inclusive."""
    g = rng(seed, 5, T_MISC, 0)
    pos = g.integers(p_lo, p_hi + 1, size=num_seqs, dtype=np.int64)
    pre = g.integers(l_lo, l_hi + 1, size=num_seqs, dtype=np.int64).astype(np.int32)
    return pos, pre


def page_permutation(seed: int, num_pages: int) -> np.ndarray:
    """A seeded random physical order of cache pages."""
    return rng(seed, 5, T_MISC, 1).permutation(num_pages).astype(np.int32)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def pages_for(slots: int, page: int) -> int:
    return ceil_div(slots, page)


__all__ = [name for name in dir() if not name.startswith("_") and name not in ("dataclasses", "math", "np")]
