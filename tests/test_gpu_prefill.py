"""GPU parity of the prefill tile plan (bit-exact) and of masked prefill attention
(fp32 debug path 1e-5, bf16 MFMA path 1e-2) against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import BF16_TOL, F32_TOL, normwise_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    require_gpu()
    import bounded_kv_cache_amd as ps
    return ps


def _plan(ps, attn, W, L, start, T, nk):
    max_tiles = 1 << 18
    tiles = torch.full((max_tiles, 3), -7, dtype=torch.int32, device="cuda")
    n = torch.zeros(1, dtype=torch.int32, device="cuda")
    ps.ps_prefill_plan(attn, W, L, start, T, nk, tiles, n)
    cnt = int(n.item())
    assert cnt <= max_tiles
    return [tuple(int(x) for x in r) for r in tiles[:cnt].cpu().numpy()]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_plan_bit_exact(ps, dtype):
    attn = ps.AttnSpec(28, 4, 128, ps.PS_BF16 if dtype == "bf16" else ps.PS_F32)
    bm, bn = ps.ps_prefill_tile_shape(attn)
    geoms = [(2048, 100, 98304, 8192, 8292),          # truncated-backprop chunk behind a 100-token prefix
             (64, 16, 16, 1024, 1024),                 # queries from position 0 (prefix queries)
             (1 << 30, 0, 0, 8192, 106496),            # full causal comparator
             (1, 0, 0, 300, 300), (3, 5, 5, 200, 205), (500, 130, 9000, 777, 1000)]
    rs = np.random.default_rng(1)
    for _ in range(20):
        L = int(rs.integers(0, 300))
        chunk = int(rs.integers(1, 3000))
        if rs.random() < 0.5:
            geoms.append((int(rs.integers(1, 4000)), L, L, int(rs.integers(1, L + chunk + 1)), L + chunk))
        else:
            geoms.append((int(rs.integers(1, 4000)), L, L + int(rs.integers(0, 10 ** 6)),
                          int(rs.integers(1, chunk + 1)), L + chunk))
    for W, L, start, T, nk in geoms:
        assert _plan(ps, attn, W, L, start, T, nk) == oracle.tile_plan(T, nk, L, W, start, bm, bn), \
            (W, L, start, T, nk)


def _prefill_case(ps, dtype, batch, hq, hkv, d, L, W, start, chunk, T, seed, rows=None, tol=None, theta=10000.0,
                  transform=None):
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16 if dtype == "bf16" else ps.PS_F32, theta, 1 / math.sqrt(d))
    nk = L + chunk
    qs, ks, vs = [], [], []
    for b in range(batch):
        qs.append(synth.history(seed, 40, synth.T_Q, b, 0, 0, T, hq, d, 1.0, dtype))
        ks.append(synth.history(seed, 40, synth.T_K, b, 0, 0, nk, hkv, d, 1.0, dtype))
        vs.append(synth.history(seed, 40, synth.T_V, b, 0, 0, nk, hkv, d, 1.0, dtype))
    q, k, v = np.stack(qs), np.stack(ks), np.stack(vs)
    if transform is not None:
        q, k, v = transform(q, k, v)
    out = torch.empty((batch, T, hq, d), dtype=dt, device="cuda")
    lse = torch.empty((batch, hq, T), dtype=torch.float32, device="cuda")
    ps.ps_prefill_attn(attn, W, L, start, to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), out, lse=lse)
    got = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy()
    tol = tol if tol is not None else (BF16_TOL if dtype == "bf16" else F32_TOL)
    for b in range(batch):
        want, want_lse = oracle.prefill_attention(q[b], k[b], v[b], L, W, start, 1 / math.sqrt(d), theta,
                                                  rows=rows)
        sel = got[b] if rows is None else got[b][rows]
        err = normwise_err(sel, want)
        assert err <= tol, (b, err)
        gl = got_lse[b].T if rows is None else got_lse[b].T[rows]
        np.testing.assert_allclose(gl, want_lse, rtol=0, atol=(2e-2 if dtype == "bf16" else 1e-4))


def test_tiny_fp32_prefill_matches_oracle_and_decode(ps):
    c = synth.C1_PREFILL
    _prefill_case(ps, "f32", 1, c.hq, c.hkv, c.dim, c.prefix, c.window, c.kv_start, c.chunk, c.queries, seed=0)


@pytest.mark.parametrize("args", [
    # batch, hq, hkv, d, L, W, kv_start, chunk, T
    (2, 8, 2, 128, 10, 100, 500, 300, 300),     # ragged q and k tails, chunk behind a gap
    (1, 4, 4, 128, 16, 64, 16, 1008, 1024),     # queries start at position 0 (prefix queries)
    (1, 7, 1, 128, 0, 1 << 30, 0, 700, 700),    # full causal
    (1, 4, 2, 64, 37, 129, 37, 400, 437),       # head_dim 64
    (1, 2, 1, 128, 100, 1, 5000, 256, 256),     # window of 1: prefix + self
])
def test_bf16_prefill_small(ps, args):
    _prefill_case(ps, "bf16", *args, seed=1)


@pytest.mark.parametrize("args", [
    (1, 4, 1, 128, 10, 100, 500, 300, 300),
    (1, 2, 2, 64, 5, 50, 5, 200, 205),
])
def test_fp32_prefill_small(ps, args):
    _prefill_case(ps, "f32", *args, seed=2)


def _score_swings(L):
    """Reference moves of the softmax (power-of-two scalings, exact in bf16;
    no rotation, so the alignments hold at every position).  Every pinned key
    is 8 k0.  Even query rows are -k0: their pinned scores are about -90
    natural units (-130 in log2), so the kernel's reference must move down
    before anything is accumulated, and the window keys' ordinary scores then
    move it up by ~130 log2 units, rescaling the pinned contributions already
    accumulated.  Odd rows are -k0 / 16: pinned scores about -6 against
    window scores near 0 (a mix with no reference move).  The scores that
    carry weight stay O(1), within the dtype's ordinary accuracy."""
    def tf(q, k, v):
        q, k = q.copy(), k.copy()
        k0 = k[:, :1, :1, :].copy()
        k[:, :L] = 8.0 * k0
        q[:, 0::2] = -k0
        q[:, 1::2] = -k0 / 16.0
        return q, k, v
    return tf


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_large_score_swings(ps, dtype):
    L, W, start, chunk, T = 40, 300, 1000, 700, 700
    _prefill_case(ps, dtype, 1, 4, 2, 128, L, W, start, chunk, T, seed=5, theta=0.0, transform=_score_swings(L))
