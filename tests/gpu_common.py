"""Helpers shared by the GPU parity tests: cache construction, ring filling
through the library's own append call, and the error metric.

Error metric: row-normwise relative error, max over rows of
max|got - want| / max|want| (element-wise relative error is meaningless for
outputs near zero)."""
from __future__ import annotations

import math

import numpy as np
import torch

import synth

BF16_TOL = 1e-2
F32_TOL = 1e-5


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def normwise_err(got: np.ndarray, want: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64).reshape(-1, want.shape[-1])
    want = np.asarray(want, dtype=np.float64).reshape(-1, want.shape[-1])
    num = np.abs(got - want).max(axis=1)
    den = np.abs(want).max(axis=1)
    return float((num / den).max())


def to_dev(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """Upload values already rounded to ``dtype`` (exact conversion)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype).cuda()


def new_cache(ps, attn, cache, num_seqs: int, fill=float("nan")):
    """K and V cache tensors of one layer, pre-filled with NaN so that reading a
    slot that was never written would poison the result."""
    ks, vs = ps.cache_shapes(attn, cache, num_seqs)
    k = torch.full(ks, fill, dtype=attn.torch_dtype, device="cuda")
    v = torch.full(vs, fill, dtype=attn.torch_dtype, device="cuda")
    return k, v


def paged_table(num_seqs: int, pages_per_seq: int, seed: int, spare: int = 3):
    """Block table [num_seqs, pages_per_seq] over a pool with a seeded random
    physical page order (plus a few unused pages)."""
    num_pages = num_seqs * pages_per_seq + spare
    perm = synth.page_permutation(seed, num_pages)
    table = perm[: num_seqs * pages_per_seq].reshape(num_seqs, pages_per_seq)
    return torch.from_numpy(np.ascontiguousarray(table)).cuda(), num_pages


def fill_ring(ps, attn, cache, k_cache, v_cache, prefix_len, p_before, k_hist, v_hist, block_table=None,
              slot_pos=None):
    """Make each sequence's ring hold positions A(p_before[s]) (as if positions
    0..p_before[s] had been appended one by one), with two bulk appends: the
    prefix tokens, then the window tokens.  k_hist[s] / v_hist[s] are raw
    [>= p_before+1, Hkv, D] arrays (float64 values exactly representable in
    the kernel dtype).  p_before[s] may be -1 (empty ring)."""
    n = len(prefix_len)
    hkv, d = attn.num_kv_heads, attn.head_dim
    dt = attn.torch_dtype
    pre_cnt = [max(0, min(int(prefix_len[s]), int(p_before[s]) + 1)) for s in range(n)]
    win_start = [max(int(prefix_len[s]), int(p_before[s]) - cache.window + 1) for s in range(n)]
    win_cnt = [max(0, int(p_before[s]) - win_start[s] + 1) for s in range(n)]
    pl = torch.tensor(np.asarray(prefix_len, dtype=np.int32), device="cuda")
    for starts, counts in ((np.zeros(n, dtype=np.int64), pre_cnt), (np.asarray(win_start, dtype=np.int64), win_cnt)):
        t = max(max(counts), 1)
        kn = np.zeros((n, t, hkv, d))
        vn = np.zeros((n, t, hkv, d))
        for s in range(n):
            c = counts[s]
            if c:
                kn[s, :c] = k_hist[s][starts[s]:starts[s] + c]
                vn[s, :c] = v_hist[s][starts[s]:starts[s] + c]
        ps.ps_kv_append(attn, cache, k_cache, v_cache, pl, torch.tensor(starts, device="cuda"),
                        to_dev(kn, dt), to_dev(vn, dt), block_table=block_table,
                        seq_tokens=torch.tensor(np.asarray(counts, dtype=np.int32), device="cuda"),
                        slot_pos=slot_pos)


def fill_rings_sampled(ps, attn, cache, k_cache, v_cache, prefix_len, p_before, sampled, block_table=None, seed=0):
    """Like fill_ring for a large batch: every sequence's ring receives
    A(p_before[s]); sequences in ``sampled`` (dict s -> (k_hist, v_hist) raw
    arrays) get those exact values, all others seeded device-side random
    values (never compared).  Uses two bulk appends with per-sequence counts."""
    n = len(prefix_len)
    hkv, d, dt = attn.num_kv_heads, attn.head_dim, attn.torch_dtype
    pre_cnt = np.array([max(0, min(int(prefix_len[s]), int(p_before[s]) + 1)) for s in range(n)], dtype=np.int32)
    win_start = np.array([max(int(prefix_len[s]), int(p_before[s]) - cache.window + 1) for s in range(n)],
                         dtype=np.int64)
    win_cnt = np.array([max(0, int(p_before[s]) - int(win_start[s]) + 1) for s in range(n)], dtype=np.int32)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    pl = torch.tensor(np.asarray(prefix_len, dtype=np.int32), device="cuda")
    for starts, counts in ((np.zeros(n, dtype=np.int64), pre_cnt), (win_start, win_cnt)):
        t = int(max(int(counts.max()), 1))
        kn = (torch.randn((n, t, hkv, d), generator=gen, device="cuda") * 0.5).to(dt)
        vn = (torch.randn((n, t, hkv, d), generator=gen, device="cuda") * 0.5).to(dt)
        for s, (kh, vh) in sampled.items():
            c = int(counts[s])
            if c:
                kn[s, :c] = to_dev(kh[starts[s]:starts[s] + c], dt)
                vn[s, :c] = to_dev(vh[starts[s]:starts[s] + c], dt)
        ps.ps_kv_append(attn, cache, k_cache, v_cache, pl, torch.tensor(starts, device="cuda"), kn, vn,
                        block_table=block_table, seq_tokens=torch.tensor(counts, device="cuda"))
        del kn, vn
