"""ps_decode_step (append the token at pos, then attend at pos) against the
float64 oracle over the full history, step after step, and against the two
separate calls on a twin cache: the same ring contents bit for bit, outputs
within tolerance; and a ring snapshot restored after S steps replays them
bit-identically.
bf16 with Continue PE is one launch (the decode kernel appends); fp32 and
Reset PE take the two-call path."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import (BF16_TOL, F32_TOL, fill_ring, new_cache, normwise_err, paged_table,
                              require_gpu, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    require_gpu()
    import bounded_kv_cache_amd as ps
    return ps


CASES = [  # (prefix, window, start positions, steps)
    (5, 40, [0, 3, 44, 45, 200, 1000], 60),      # warm-up, window edge, wrap; prefix ends inside a chunk
    (0, 33, [0, 32, 34, 500], 50),               # no prefix
    (100, 4096, [4190, 9000], 12),               # the headline shape: splits cover several chunks
]


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_step_trace(ps, dtype, case, paged, splits):
    L, W, starts, steps = CASES[case]
    if dtype == "f32" and case == 2:
        pytest.skip("the fp32 path of the headline shape adds nothing over the small cases")
    hq, hkv, d = 16, 2, 128
    n = len(starts)
    cap = -(-(L + W) // 64) * 64
    splits = min(splits, cap // 32)
    pt, tdt = (ps.PS_BF16, torch.bfloat16) if dtype == "bf16" else (ps.PS_F32, torch.float32)
    attn = ps.AttnSpec(hq, hkv, d, pt, 10000.0, 1 / math.sqrt(d))
    bt, num_pages = (None, 0)
    if paged:
        bt, num_pages = paged_table(n, cap // 64, seed=case + 20)
    cache = ps.CacheSpec(window=W, slot_capacity=cap, page_size=64 if paged else 0, num_pages=num_pages)
    last = [p + steps for p in starts]
    hist = [(synth.history(4, 200 + case, synth.T_K, s, 0, 0, last[s], hkv, d, 0.5, dtype),
             synth.history(4, 200 + case, synth.T_V, s, 0, 0, last[s], hkv, d, 0.5, dtype)) for s in range(n)]
    qs = [synth.history(4, 200 + case, synth.T_Q, s, 0, 0, last[s], hq, d, 1.0, dtype) for s in range(n)]
    caches = [new_cache(ps, attn, cache, n) for _ in range(2)]   # fused step / two calls
    for kc, vc in caches:
        fill_ring(ps, attn, cache, kc, vc, [L] * n, [p - 1 for p in starts], [h[0] for h in hist],
                  [h[1] for h in hist], block_table=bt)
    pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
    out = [torch.empty((n, hq, d), dtype=tdt, device="cuda") for _ in range(2)]
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    worst = 0.0
    for i in range(steps):
        p = [starts[s] + i for s in range(n)]
        pos = torch.tensor(p, dtype=torch.int64, device="cuda")
        kn = to_dev(np.stack([hist[s][0][p[s]] for s in range(n)])[:, None], tdt)
        vn = to_dev(np.stack([hist[s][1][p[s]] for s in range(n)])[:, None], tdt)
        q = to_dev(np.stack([qs[s][p[s]] for s in range(n)]), tdt)
        ps.ps_decode_step(attn, cache, caches[0][0], caches[0][1], pl, pos, q, kn, vn, out[0], block_table=bt,
                          num_splits=splits)
        ps.ps_kv_append(attn, cache, caches[1][0], caches[1][1], pl, pos, kn, vn, block_table=bt)
        ps.ps_decode_attn(attn, cache, caches[1][0], caches[1][1], pl, pos, q, out[1], block_table=bt,
                          num_splits=splits)
        got = out[0].float().cpu().numpy()
        two = out[1].float().cpu().numpy()
        for s in range(n):
            want = oracle.decode_attention(qs[s][p[s]], hist[s][0], hist[s][1], p[s], L, W, 1 / math.sqrt(d),
                                           10000.0)
            worst = max(worst, normwise_err(got[s], want))
            assert normwise_err(got[s], two[s]) <= tol, (i, s)
    assert worst <= tol, worst
    # the same ring contents as the two calls, bit for bit (the fused append
    # rotates keys with the append kernel's expression)
    (k0, v0), (k1, v1) = caches
    bits = torch.int16 if dtype == "bf16" else torch.int32
    np.testing.assert_array_equal(v0.view(bits).cpu().numpy(), v1.view(bits).cpu().numpy())
    np.testing.assert_array_equal(k0.view(bits).cpu().numpy(), k1.view(bits).cpu().numpy())


def test_decode_step_head_dim_64(ps):
    """head_dim 64 (two QK k-steps, 32 rotation pairs per token) through the
    one-launch step, 80 steps from warm-up past the window, vs the oracle."""
    hq, hkv, d, L, W, steps = 8, 1, 64, 9, 70, 80
    starts = [0, 50, 300]
    n = len(starts)
    cap = -(-(L + W) // 64) * 64
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    cache = ps.CacheSpec(window=W, slot_capacity=cap)
    last = [p + steps for p in starts]
    hist = [(synth.history(8, 300, synth.T_K, s, 0, 0, last[s], hkv, d, 0.5, "bf16"),
             synth.history(8, 300, synth.T_V, s, 0, 0, last[s], hkv, d, 0.5, "bf16")) for s in range(n)]
    qs = [synth.history(8, 300, synth.T_Q, s, 0, 0, last[s], hq, d, 1.0, "bf16") for s in range(n)]
    kc, vc = new_cache(ps, attn, cache, n)
    fill_ring(ps, attn, cache, kc, vc, [L] * n, [p - 1 for p in starts], [h[0] for h in hist], [h[1] for h in hist])
    pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
    out = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
    worst = 0.0
    for i in range(steps):
        p = [starts[s] + i for s in range(n)]
        ps.ps_decode_step(attn, cache, kc, vc, pl, torch.tensor(p, dtype=torch.int64, device="cuda"),
                          to_dev(np.stack([qs[s][p[s]] for s in range(n)]), torch.bfloat16),
                          to_dev(np.stack([hist[s][0][p[s]] for s in range(n)])[:, None], torch.bfloat16),
                          to_dev(np.stack([hist[s][1][p[s]] for s in range(n)])[:, None], torch.bfloat16), out,
                          num_splits=2)
        got = out.float().cpu().numpy()
        for s in range(n):
            want = oracle.decode_attention(qs[s][p[s]], hist[s][0], hist[s][1], p[s], L, W, 1 / math.sqrt(d),
                                           10000.0)
            worst = max(worst, normwise_err(got[s], want))
    assert worst <= BF16_TOL, worst


def test_decode_step_reset_pe_and_invalid_sequences(ps):
    """Reset PE takes the two-call path and matches it bit for bit; a sequence
    with a negative prefix gets NaN rows and its ring is left untouched, the
    others are unaffected."""
    hq, hkv, d, L, W = 16, 2, 128, 7, 50
    cap = 64
    n = 3
    cache = ps.CacheSpec(window=W, slot_capacity=cap)
    g = torch.Generator(device="cuda").manual_seed(5)
    for pe in (ps.PS_PE_RESET, ps.PS_PE_CONTINUE):
        attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d), pe_mode=pe)
        kc, vc = new_cache(ps, attn, cache, n, fill=0.0)
        hk = (torch.randn((n, 90, hkv, d), generator=g, device="cuda") * 0.5).bfloat16()
        hv = (torch.randn((n, 90, hkv, d), generator=g, device="cuda") * 0.5).bfloat16()
        pl = torch.tensor([L, -1, L], dtype=torch.int32, device="cuda")
        ps.ps_kv_append(attn, cache, kc, vc, torch.tensor([L, L, L], dtype=torch.int32, device="cuda"),
                        torch.zeros(n, dtype=torch.int64, device="cuda"), hk, hv)
        kc2, vc2 = kc.clone(), vc.clone()
        pos = torch.full((n,), 90, dtype=torch.int64, device="cuda")
        q = torch.randn((n, hq, d), generator=g, device="cuda").bfloat16()
        kn = (torch.randn((n, 1, hkv, d), generator=g, device="cuda") * 0.5).bfloat16()
        vn = (torch.randn((n, 1, hkv, d), generator=g, device="cuda") * 0.5).bfloat16()
        o1 = torch.empty_like(q)
        o2 = torch.empty_like(q)
        ps.ps_decode_step(attn, cache, kc, vc, pl, pos, q, kn, vn, o1)
        ps.ps_kv_append(attn, cache, kc2, vc2, pl, pos, kn, vn)
        ps.ps_decode_attn(attn, cache, kc2, vc2, pl, pos, q, o2)
        a_, b_ = o1.float().cpu().numpy(), o2.float().cpu().numpy()
        assert np.isnan(a_[1]).all() and np.isnan(b_[1]).all()
        if pe == ps.PS_PE_RESET:
            assert torch.equal(o1[[0, 2]].view(torch.int16), o2[[0, 2]].view(torch.int16))
        else:
            assert normwise_err(a_[[0, 2]], b_[[0, 2]]) <= BF16_TOL
        assert torch.equal(vc.view(torch.int16), vc2.view(torch.int16))
        assert torch.equal(kc[1].view(torch.int16), kc2[1].view(torch.int16))   # the invalid sequence: untouched


@pytest.mark.parametrize("splits", [1, 3])
def test_ring_snapshot_restore_replays_bit_identically(ps, splits):
    """Checkpoint / resume of the bounded cache: snapshot every ring (plain
    device copies of the K and V caches), run S decode steps, restore the
    snapshot, run the same S steps again: every output and the final rings are
    bit-identical to the first run (the kernels are deterministic and the ring
    is the whole state a sequence carries); the first run also matches the
    oracle.  Positions cross the window edge, the prefix ends inside a chunk."""
    hq, hkv, d, L, W, steps = 16, 2, 128, 37, 300, 24
    starts = [330, 1000, 5]
    n = len(starts)
    cap = -(-(L + W) // 64) * 64
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    cache = ps.CacheSpec(window=W, slot_capacity=cap)
    last = [p + steps for p in starts]
    hist = [(synth.history(9, 400, synth.T_K, s, 0, 0, last[s], hkv, d, 0.5, "bf16"),
             synth.history(9, 400, synth.T_V, s, 0, 0, last[s], hkv, d, 0.5, "bf16")) for s in range(n)]
    qs = [synth.history(9, 400, synth.T_Q, s, 0, 0, last[s], hq, d, 1.0, "bf16") for s in range(n)]
    kc, vc = new_cache(ps, attn, cache, n)
    fill_ring(ps, attn, cache, kc, vc, [L] * n, [p - 1 for p in starts], [h[0] for h in hist], [h[1] for h in hist])
    snap = (kc.clone(), vc.clone())
    pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
    inputs = []
    for i in range(steps):
        p = [starts[s] + i for s in range(n)]
        inputs.append((torch.tensor(p, dtype=torch.int64, device="cuda"),
                       to_dev(np.stack([qs[s][p[s]] for s in range(n)]), torch.bfloat16),
                       to_dev(np.stack([hist[s][0][p[s]] for s in range(n)])[:, None], torch.bfloat16),
                       to_dev(np.stack([hist[s][1][p[s]] for s in range(n)])[:, None], torch.bfloat16)))

    def run():
        outs = []
        for pos, q, kn, vn in inputs:
            out = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
            ps.ps_decode_step(attn, cache, kc, vc, pl, pos, q, kn, vn, out, num_splits=splits)
            outs.append(out)
        torch.cuda.synchronize()
        return [o.view(torch.int16).cpu().numpy() for o in outs], kc.view(torch.int16).cpu().numpy(), \
            vc.view(torch.int16).cpu().numpy()

    first, k1, v1 = run()
    for i, o in enumerate(first):
        got = torch.from_numpy(o).view(torch.bfloat16).float().numpy()
        for s in range(n):
            p = starts[s] + i
            want = oracle.decode_attention(qs[s][p], hist[s][0], hist[s][1], p, L, W, 1 / math.sqrt(d), 10000.0)
            assert normwise_err(got[s], want) <= BF16_TOL, (i, s)
    kc.copy_(snap[0])
    vc.copy_(snap[1])
    second, k2, v2 = run()
    for a_, b_ in zip(first, second):
        np.testing.assert_array_equal(a_, b_)
    np.testing.assert_array_equal(k1, k2)
    np.testing.assert_array_equal(v1, v2)
