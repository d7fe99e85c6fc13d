"""GPU parity of the chunk prefill that reads the ring (ps_chunk_prefill_attn)
against the float64 oracle, through the C ABI.

Each case fills the rings with the history before the chunk (as if appended
token by token), runs the chunk call, and checks: the chunk output and LSE
against oracle.chunk_prefill_attention over the full un-evicted history; the
ring's slot map afterwards bit-exactly against oracle.simulate_ring; and a
decode step right after the chunk against oracle.decode_attention (the chunk
was handed into the ring correctly)."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import (BF16_TOL, F32_TOL, fill_ring, new_cache, normwise_err, paged_table, require_gpu,
                              to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    require_gpu()
    import bounded_kv_cache_amd as ps
    return ps


def _run_case(ps, dtype, hq, hkv, d, W, prefixes, starts, T, cap, paged=False, seed=0, check_decode=True):
    dt_name = "bf16" if dtype == "bf16" else "f32"
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16 if dtype == "bf16" else ps.PS_F32, 10000.0, 1 / math.sqrt(d))
    n = len(starts)
    bt, num_pages = (None, 0)
    if paged:
        bt, num_pages = paged_table(n, cap // 64, seed)
    cache = ps.CacheSpec(window=W, slot_capacity=cap, page_size=64 if paged else 0, num_pages=num_pages)
    kc, vc = new_cache(ps, attn, cache, n)
    slot_pos = torch.full((n, cap), -1, dtype=torch.int32, device="cuda")
    hist = [(synth.history(seed, 7, synth.T_K, s, 0, 0, starts[s] + T + 1, hkv, d, 0.5, dt_name),
             synth.history(seed, 7, synth.T_V, s, 0, 0, starts[s] + T + 1, hkv, d, 0.5, dt_name)) for s in range(n)]
    qs = [synth.history(seed, 7, synth.T_Q, s, 0, starts[s], starts[s] + T + 1, hq, d, 1.0, dt_name)
          for s in range(n)]
    fill_ring(ps, attn, cache, kc, vc, prefixes, [p - 1 for p in starts], [h[0] for h in hist],
              [h[1] for h in hist], block_table=bt, slot_pos=slot_pos)
    pl = torch.tensor(np.asarray(prefixes, dtype=np.int32), device="cuda")
    sp = torch.tensor(np.asarray(starts, dtype=np.int64), device="cuda")
    q = to_dev(np.stack([x[:T] for x in qs]), tdt)
    kn = to_dev(np.stack([h[0][starts[s]:starts[s] + T] for s, h in enumerate(hist)]), tdt)
    vn = to_dev(np.stack([h[1][starts[s]:starts[s] + T] for s, h in enumerate(hist)]), tdt)
    out = torch.empty((n, T, hq, d), dtype=tdt, device="cuda")
    lse = torch.empty((n, hq, T), dtype=torch.float32, device="cuda")
    ps.ps_chunk_prefill_attn(attn, cache, kc, vc, pl, sp, q, kn, vn, out, block_table=bt, lse=lse,
                             slot_pos=slot_pos)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    got_lse = lse.cpu().numpy()
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    worst = 0.0
    for s in range(n):
        want, want_lse = oracle.chunk_prefill_attention(qs[s][:T], hist[s][0], hist[s][1], starts[s], prefixes[s],
                                                        W, 1 / math.sqrt(d), 10000.0)
        e = normwise_err(got[s], want)
        worst = max(worst, e)
        assert e <= tol, (s, starts[s], prefixes[s], e)
        np.testing.assert_allclose(got_lse[s].T, want_lse, rtol=0, atol=(2e-2 if dtype == "bf16" else 1e-4))
    # ring after the chunk: exactly the slot map of appending 0 .. P+T-1
    sp_host = slot_pos.cpu().numpy()
    for s in range(n):
        want_slots = oracle.simulate_ring(range(starts[s] + T), prefixes[s], W, cap)
        np.testing.assert_array_equal(sp_host[s], want_slots)
    if check_decode:
        # one decode step at P + T continues from the ring the chunk left behind
        p_next = torch.tensor([st + T for st in starts], dtype=torch.int64, device="cuda")
        kn1 = to_dev(np.stack([h[0][starts[s] + T:starts[s] + T + 1] for s, h in enumerate(hist)]), tdt)
        vn1 = to_dev(np.stack([h[1][starts[s] + T:starts[s] + T + 1] for s, h in enumerate(hist)]), tdt)
        ps.ps_kv_append(attn, cache, kc, vc, pl, p_next, kn1, vn1, block_table=bt)
        qd = to_dev(np.stack([x[T] for x in qs]), tdt)
        od = torch.empty((n, hq, d), dtype=tdt, device="cuda")
        ps.ps_decode_attn(attn, cache, kc, vc, pl, p_next, qd, od, block_table=bt)
        torch.cuda.synchronize()
        gd = od.float().cpu().numpy()
        for s in range(n):
            want = oracle.decode_attention(qs[s][T], hist[s][0], hist[s][1], starts[s] + T, prefixes[s], W,
                                           1 / math.sqrt(d), 10000.0)
            assert normwise_err(gd[s], want) <= tol
    return worst


# ragged starts: empty ring, inside the prefix, warm-up, crossing L+W, sliding far beyond
CASES = [
    # hq, hkv, d, W, prefixes, starts, T, cap, paged
    (16, 2, 128, 256, [100, 100, 100, 100, 100], [0, 50, 300, 356, 1500], 200, 384, False),
    (16, 2, 128, 256, [7, 130, 0, 64, 250], [900, 20, 700, 64, 3000], 200, 512, True),
    (4, 1, 64, 64, [16, 16, 3], [500, 37, 80], 300, 128, False),     # chunk longer than the window
    (28, 4, 128, 2048, [100, 100], [20000, 5000], 129, 2176, False),
    (8, 8, 64, 96, [0, 1, 200], [260, 1, 150], 65, 320, True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_chunk_bf16_matches_oracle(ps, case):
    hq, hkv, d, W, pre, st, T, cap, paged = CASES[case]
    print(f"chunk bf16 case {case}: Hq={hq} Hkv={hkv} D={d} W={W} L={pre} P={st} T={T} cap={cap} paged={paged}",
          flush=True)
    _run_case(ps, "bf16", hq, hkv, d, W, pre, st, T, cap, paged=paged, seed=case)


@pytest.mark.parametrize("case", [0, 2, 4])
def test_chunk_fp32_matches_oracle(ps, case):
    hq, hkv, d, W, pre, st, T, cap, paged = CASES[case]
    print(f"chunk fp32 case {case}", flush=True)
    _run_case(ps, "f32", hq, hkv, d, W, pre, st, T, cap, paged=paged, seed=10 + case)


def test_chunk_equals_token_by_token_decode_tiny_fp32(ps):
    # C1 shapes: a 1024-token trace fed as 8 chunks of 128 gives, row for row,
    # the outputs of 1024 single-token decode steps (oracle decode at each p)
    c = synth.C1_DECODE
    attn = ps.AttnSpec(c.hq, c.hkv, c.dim, ps.PS_F32, c.rope_theta, 1 / math.sqrt(c.dim))
    cache = ps.CacheSpec(window=c.window, slot_capacity=128)
    kc, vc = new_cache(ps, attn, cache, 1)
    k = synth.history(0, c.cfg_id, synth.T_K, 0, 0, 0, c.steps, c.hkv, c.dim, c.kv_std, "f32")
    v = synth.history(0, c.cfg_id, synth.T_V, 0, 0, 0, c.steps, c.hkv, c.dim, c.kv_std, "f32")
    q = synth.history(0, c.cfg_id, synth.T_Q, 0, 0, 0, c.steps, c.hq, c.dim, c.q_std, "f32")
    pl = torch.tensor([c.prefix], dtype=torch.int32, device="cuda")
    T = 128
    worst = 0.0
    for i in range(c.steps // T):
        sp = torch.tensor([i * T], dtype=torch.int64, device="cuda")
        out = torch.empty((1, T, c.hq, c.dim), dtype=torch.float32, device="cuda")
        ps.ps_chunk_prefill_attn(attn, cache, kc, vc, pl, sp, to_dev(q[None, i * T:(i + 1) * T], torch.float32),
                                 to_dev(k[None, i * T:(i + 1) * T], torch.float32),
                                 to_dev(v[None, i * T:(i + 1) * T], torch.float32), out)
        got = out.cpu().numpy()[0]
        for t in range(0, T, 7):
            p = i * T + t
            want = oracle.decode_attention(q[p], k, v, p, c.prefix, c.window, 1 / math.sqrt(c.dim), c.rope_theta)
            worst = max(worst, normwise_err(got[t], want))
    assert worst <= F32_TOL, worst


def test_chunk_unservable_sequences_give_nan_rows(ps):
    attn = ps.AttnSpec(8, 2, 128, ps.PS_BF16)
    cache = ps.CacheSpec(window=64, slot_capacity=128)
    n, T = 4, 70
    kc, vc = new_cache(ps, attn, cache, n, fill=0.0)
    # seq 0 fine; seq 1 negative L; seq 2 negative P; seq 3 ring reach min(P, L+W) = 100+64 > 128
    pl = torch.tensor([10, -1, 10, 100], dtype=torch.int32, device="cuda")
    sp = torch.tensor([40, 5, -3, 500], dtype=torch.int64, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(3)
    q = torch.randn((n, T, 8, 128), generator=g, device="cuda").bfloat16()
    kn = torch.randn((n, T, 2, 128), generator=g, device="cuda").bfloat16()
    vn = torch.randn((n, T, 2, 128), generator=g, device="cuda").bfloat16()
    out = torch.zeros((n, T, 8, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((n, 8, T), dtype=torch.float32, device="cuda")
    ps.ps_chunk_prefill_attn(attn, cache, kc, vc, pl, sp, q, kn, vn, out, lse=lse)
    torch.cuda.synchronize()
    o = out.float()
    assert torch.isfinite(o[0]).all() and torch.isfinite(lse[0]).all()
    for s in (1, 2, 3):
        assert torch.isnan(o[s]).all(), s
        assert torch.isnan(lse[s]).all(), s
