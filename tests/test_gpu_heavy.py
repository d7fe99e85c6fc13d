"""GPU parity of prefix + heavy hitters + window decoding (ps_heavy_decode_step)
against the float64 oracle (oracle.h2o_decode_trace / h2o_admit), through the
C ABI.

fp32 debug path: the GPU and the oracle run the whole trace independently;
every step's output (1e-5), the final heavy sets (exact) and the members'
scores (1e-5 relative) must agree.  bf16: admission is an argmin over
accumulated scores, a decision taken from floating point, so the test follows
the GPU's own state: at every step it checks that the admission the GPU made
is exactly what the rule gives on the GPU's scores, that the output matches
the oracle's attention over the GPU's visible set, and that the scores grew by
the oracle's attention mass (oracle.slot_attention_mass) within the bf16
row-normwise bound."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import BF16_TOL, F32_TOL, fill_ring, new_cache, normwise_err, paged_table, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    require_gpu()
    import bounded_kv_cache_amd as ps
    return ps


def _data(seed, n_seq, steps, hq, hkv, d, dtype):
    q = [synth.history(seed, 9, synth.T_Q, s, 0, 0, steps, hq, d, 1.0, dtype) for s in range(n_seq)]
    k = [synth.history(seed, 9, synth.T_K, s, 0, 0, steps, hkv, d, 1.0, dtype) for s in range(n_seq)]
    v = [synth.history(seed, 9, synth.T_V, s, 0, 0, steps, hkv, d, 1.0, dtype) for s in range(n_seq)]
    return q, k, v


def _ring_slot(j, L, W):
    return j if j < L else L + (j - L) % W


@pytest.mark.parametrize("splits", [1, 2])
def test_heavy_fp32_trace_matches_oracle(ps, splits):
    hq, hkv, d, W, H, steps = 4, 2, 64, 48, 24, 360
    prefixes = [16, 5, 0]
    n = len(prefixes)
    cap = -(-(max(prefixes) + W + H) // 64) * 64
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_F32, 10000.0, 1 / math.sqrt(d))
    cache = ps.CacheSpec(window=W, slot_capacity=cap)
    q, k, v = _data(1, n, steps, hq, hkv, d, "f32")
    want = [oracle.h2o_decode_trace(q[s], k[s], v[s], prefixes[s], W, H, 1 / math.sqrt(d), 10000.0)
            for s in range(n)]
    kc, vc = new_cache(ps, attn, cache, n)
    state = ps.HeavyState.new(attn, cache, n, H)
    pl = torch.tensor(prefixes, dtype=torch.int32, device="cuda")
    qd = to_dev(np.stack(q), torch.float32)
    kd = to_dev(np.stack(k), torch.float32)
    vd = to_dev(np.stack(v), torch.float32)
    out = torch.empty((n, hq, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(ps.ps_heavy_workspace_size(attn, cache, n, splits), dtype=torch.uint8, device="cuda")
    worst = 0.0
    for p in range(steps):
        pos = torch.full((n,), p, dtype=torch.int64, device="cuda")
        ps.ps_heavy_decode_step(attn, cache, H, kc, vc, pl, pos, qd[:, p].contiguous(),
                                kd[:, p:p + 1].contiguous(), vd[:, p:p + 1].contiguous(), out, state,
                                num_splits=splits, workspace=ws)
        got = out.cpu().numpy()
        for s in range(n):
            worst = max(worst, normwise_err(got[s], want[s][0][p]))
    assert worst <= F32_TOL, worst
    cnt = state.heavy_count.cpu().numpy()
    hpos = state.heavy_pos.cpu().numpy()
    sc = state.score.cpu().numpy()
    for s in range(n):
        for kv in range(hkv):
            L = prefixes[s]
            members = hpos[s, kv, :cnt[s, kv]]
            ref = want[s][1][kv]
            assert sorted(members.tolist()) == sorted(ref[ref >= 0].tolist()), (s, kv)
            for i, j in enumerate(members):
                np.testing.assert_allclose(sc[s, kv, L + W + i], want[s][2][kv][int(j)], rtol=1e-5)


@pytest.mark.parametrize("geom", ["narrow", "wide"])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("paged", [False, True])
def test_heavy_bf16_follows_the_rule_step_by_step(ps, paged, splits, geom):
    """splits 1: statistics kept in LDS and the scores accumulated by the decode
    kernel (narrow: 4 waves, two workgroups per CU; wide, 5312 slots: 8 waves,
    one workgroup per CU); 3: statistics through HBM and the accumulate kernel.
    The wide trace starts at 5210 from rings filled by a bulk append (empty
    heavy sets), so tokens leave the window at once."""
    hq, hkv, d = 16, 2, 128
    W, H, start, steps = (96, 40, 0, 330) if geom == "narrow" else (5200, 64, 5210, 24)
    prefixes = [20, 0, 37]
    n = len(prefixes)
    cap = -(-(max(prefixes) + W + H) // 64) * 64
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    bt, num_pages = (None, 0)
    if paged:
        bt, num_pages = paged_table(n, cap // 64, seed=4)
    cache = ps.CacheSpec(window=W, slot_capacity=cap, page_size=64 if paged else 0, num_pages=num_pages)
    q, k, v = _data(2, n, start + steps, hq, hkv, d, "bf16")
    kc, vc = new_cache(ps, attn, cache, n)
    if start:
        fill_ring(ps, attn, cache, kc, vc, prefixes, [start - 1] * n, k, v, block_table=bt)
    state = ps.HeavyState.new(attn, cache, n, H)
    pl = torch.tensor(prefixes, dtype=torch.int32, device="cuda")
    qd, kd, vd = (to_dev(np.stack(x), torch.bfloat16) for x in (q, k, v))
    out = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
    g = hq // hkv
    scale = 1 / math.sqrt(d)
    admitted = replaced = dropped = 0
    for p in range(start, start + steps):
        pre_sc = state.score.cpu().numpy()
        pre_cnt = state.heavy_count.cpu().numpy()
        pre_pos = state.heavy_pos.cpu().numpy()
        pos = torch.full((n,), p, dtype=torch.int64, device="cuda")
        ps.ps_heavy_decode_step(attn, cache, H, kc, vc, pl, pos, qd[:, p].contiguous(), kd[:, p:p + 1].contiguous(),
                                vd[:, p:p + 1].contiguous(), out, state, block_table=bt, num_splits=splits)
        got = out.float().cpu().numpy()
        sc = state.score.cpu().numpy()
        cnt = state.heavy_count.cpu().numpy()
        hpos = state.heavy_pos.cpu().numpy()
        for s in range(n):
            L = prefixes[s]
            for kv in range(hkv):
                e = p - W
                members_pre = [int(x) for x in pre_pos[s, kv, :pre_cnt[s, kv]]] + [-1] * (H - pre_cnt[s, kv])
                scores_pre = [float(pre_sc[s, kv, L + W + i]) for i in range(H)]
                if e >= L:
                    slot, _ = oracle.h2o_admit(members_pre, scores_pre, e, float(pre_sc[s, kv, _ring_slot(e, L, W)]),
                                               H)
                    if slot >= 0:
                        assert hpos[s, kv, slot] == e, (p, s, kv, slot)
                        if members_pre[slot] >= 0:
                            replaced += 1
                        else:
                            admitted += 1
                    else:
                        dropped += 1
                    members = [x for x in members_pre if x >= 0]
                    if slot >= 0:
                        members = [x for i, x in enumerate(members_pre[:max(pre_cnt[s, kv], slot + 1)])
                                   if i != slot and x >= 0] + [e]
                    assert sorted(members) == sorted(int(x) for x in hpos[s, kv, :cnt[s, kv]])
                # the output: the oracle's attention over the GPU's visible set
                heavy = [int(x) for x in hpos[s, kv, :cnt[s, kv]]]
                win = list(range(max(L, p - W + 1), p + 1))
                vis = np.array(list(range(min(L, p + 1))) + heavy + win, dtype=np.int64)
                kr = oracle.rope(k[s][vis][:, kv:kv + 1], vis[:, None], 10000.0)
                want = oracle.decode_from_slots(q[s][p][kv * g:(kv + 1) * g], p, kr, v[s][vis][:, kv:kv + 1], scale,
                                                10000.0)
                assert normwise_err(got[s, kv * g:(kv + 1) * g], want) <= BF16_TOL, (p, s, kv)
                # scores grew by the attention each visible token received
                mass = oracle.slot_attention_mass(q[s][p][kv * g:(kv + 1) * g], p, kr, scale, 10000.0)[:, 0]
                grew, want_mass = [], []
                for j, m in zip(vis, mass):
                    if j < L:
                        continue
                    if j > p - W:
                        slot_j = _ring_slot(int(j), L, W)
                        before = 0.0 if j == p else pre_sc[s, kv, slot_j]
                    else:
                        i = heavy.index(int(j))
                        slot_j = L + W + i
                        before = pre_sc[s, kv, L + W + i] if int(j) in members_pre and \
                            members_pre.index(int(j)) == i else pre_sc[s, kv, _ring_slot(int(j), L, W)]
                    grew.append(float(sc[s, kv, slot_j]) - float(before))
                    want_mass.append(m)
                if want_mass:   # the row-normwise bf16 bound over the visible non-prefix slots
                    assert normwise_err(np.array(grew), np.array(want_mass)) <= BF16_TOL, (p, s, kv)
    if geom == "narrow":
        assert admitted > 0 and replaced > 0 and dropped > 0, (admitted, replaced, dropped)
    else:   # 24 steps into 64 free heavy slots: every token leaving past the prefix is admitted
        want = sum(hkv for L in prefixes for p in range(start, start + steps) if p - W >= L)
        assert admitted == want and replaced == 0 and dropped == 0, (admitted, want)
