"""GPU parity of append + decode against the float64 oracle (through the C ABI).

Slots are compared bit-exactly; floating point with the row-normwise relative
error of gpu_common (fp32 debug path 1e-5, bf16 1e-2)."""
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


def _hist(seed, cfg_id, seq, n, hkv, d, std, dtype):
    k = synth.history(seed, cfg_id, synth.T_K, seq, 0, 0, n, hkv, d, std, dtype)
    v = synth.history(seed, cfg_id, synth.T_V, seq, 0, 0, n, hkv, d, std, dtype)
    return k, v


# ------------------------------------------------------------------ tiny fp32 config, step by step
@pytest.mark.parametrize("splits", [1, 3])
def test_tiny_fp32_autoregressive_decode(ps, splits):
    c = synth.C1_DECODE
    attn = ps.AttnSpec(c.hq, c.hkv, c.dim, ps.PS_F32, c.rope_theta, 1 / math.sqrt(c.dim))
    cache = ps.CacheSpec(window=c.window, slot_capacity=128)
    steps = c.steps
    k, v = _hist(0, c.cfg_id, 0, steps, c.hkv, c.dim, c.kv_std, "f32")
    q = synth.history(0, c.cfg_id, synth.T_Q, 0, 0, 0, steps, c.hq, c.dim, c.q_std, "f32")
    kc, vc = new_cache(ps, attn, cache, 1)
    slot_pos = torch.full((1, cache.slot_capacity), -1, dtype=torch.int32, device="cuda")
    kd, vd, qd = to_dev(k, torch.float32), to_dev(v, torch.float32), to_dev(q, torch.float32)
    pl = torch.tensor([c.prefix], dtype=torch.int32, device="cuda")
    pos_all = torch.arange(steps, dtype=torch.int64, device="cuda")
    out = torch.empty((steps, c.hq, c.dim), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(ps.ps_decode_workspace_size(attn, cache, 1, splits), 1), dtype=torch.uint8, device="cuda")
    ring_checks = {}
    for p in range(steps):
        ps.ps_kv_append(attn, cache, kc, vc, pl, pos_all[p:p + 1], kd[p:p + 1].reshape(1, 1, c.hkv, c.dim),
                        vd[p:p + 1].reshape(1, 1, c.hkv, c.dim), slot_pos=slot_pos)
        ps.ps_decode_attn(attn, cache, kc, vc, pl, pos_all[p:p + 1], qd[p:p + 1], out[p:p + 1], num_splits=splits,
                          workspace=ws)
        if p in (10, 79, 80, 500, steps - 1):
            ring_checks[p] = slot_pos.clone()
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for p in range(steps):
        want = oracle.decode_attention(q[p], k, v, p, c.prefix, c.window, 1 / math.sqrt(c.dim), c.rope_theta)
        worst = max(worst, normwise_err(got[p], want))
    assert worst <= F32_TOL, worst
    for p, sp in ring_checks.items():
        want = oracle.simulate_ring(range(p + 1), c.prefix, c.window, cache.slot_capacity)
        np.testing.assert_array_equal(sp.cpu().numpy()[0], want)


def test_tiny_fp32_ring_contents(ps):
    """K in the ring is the oracle's rotation at the absolute position; V is the raw value."""
    c = synth.C1_DECODE
    attn = ps.AttnSpec(c.hq, c.hkv, c.dim, ps.PS_F32, c.rope_theta, 0.125)
    cache = ps.CacheSpec(window=c.window, slot_capacity=128)
    p = 300
    k, v = _hist(1, c.cfg_id, 0, p + 1, c.hkv, c.dim, 1.0, "f32")
    kc, vc = new_cache(ps, attn, cache, 1)
    fill_ring(ps, attn, cache, kc, vc, [c.prefix], [p], [k], [v])
    torch.cuda.synchronize()
    ring = oracle.simulate_ring(range(p + 1), c.prefix, c.window, cache.slot_capacity)
    kg = kc.cpu().numpy()[0, 0]                               # [slots, D]
    vg = vc.cpu().numpy()[0, 0].transpose(0, 2, 1).reshape(-1, c.dim)  # blocks [slot/8][D][8] -> [slot][D]
    for slot, pos in enumerate(ring):
        if pos < 0:
            assert np.isnan(kg[slot]).all()
            continue
        want_k = oracle.rope(k[pos, 0], pos, c.rope_theta)
        np.testing.assert_allclose(kg[slot], want_k, rtol=0, atol=2e-6)
        np.testing.assert_array_equal(vg[slot], v[pos, 0])


# ------------------------------------------------------------------ bf16, GQA 8, head_dim 128
CASES = [  # (prefix, window, query positions of the sequences)
    (5, 40, [0, 3, 44, 45, 46, 200, 1000]),
    (0, 33, [0, 32, 33, 34, 500]),
    (64, 64, [63, 127, 128, 129, 4000]),
    (100, 4096, [4195, 4196, 9000]),
]


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_bf16_decode_small(ps, case, paged):
    L, W, positions = CASES[case]
    hq, hkv, d = 16, 2, 128
    n = len(positions)
    cap = -(-(L + W) // 64) * 64
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    bt = None
    num_pages = 0
    if paged:
        bt, num_pages = paged_table(n, cap // 64, seed=case)
    cache = ps.CacheSpec(window=W, slot_capacity=cap, page_size=64 if paged else 0, num_pages=num_pages)
    kc, vc = new_cache(ps, attn, cache, n)
    hist = [_hist(2, 90 + case, s, positions[s] + 1, hkv, d, 0.5, "bf16") for s in range(n)]
    fill_ring(ps, attn, cache, kc, vc, [L] * n, [p - 1 for p in positions], [h[0] for h in hist],
              [h[1] for h in hist], block_table=bt)
    # decode step: append the query token, then attend
    kn = np.stack([h[0][p] for h, p in zip(hist, positions)])[:, None]
    vn = np.stack([h[1][p] for h, p in zip(hist, positions)])[:, None]
    pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
    pos = torch.tensor(positions, dtype=torch.int64, device="cuda")
    ps.ps_kv_append(attn, cache, kc, vc, pl, pos, to_dev(kn, torch.bfloat16), to_dev(vn, torch.bfloat16),
                    block_table=bt)
    q = np.stack([synth.query(2, 90 + case, s, 0, 0, hq, d, 1.0, "bf16") for s in range(n)])
    qd = to_dev(q, torch.bfloat16)
    max_splits = cap // 32
    for splits in sorted({sp for sp in (1, 2, 3, 7, 0) if sp <= max_splits}):
        out = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
        ps.ps_decode_attn(attn, cache, kc, vc, pl, pos, qd, out, block_table=bt, num_splits=splits)
        got = out.float().cpu().numpy()
        for s in range(n):
            want = oracle.decode_attention(q[s], hist[s][0], hist[s][1], positions[s], L, W, 1 / math.sqrt(d),
                                           10000.0)
            err = normwise_err(got[s], want)
            assert err <= BF16_TOL, (splits, s, positions[s], err)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_large_score_swings(ps, dtype):
    """Softmax maxima that move by over a hundred log2 units (power-of-two
    scalings, exact in bf16; no rotation, so alignments hold at every
    position): the pinned keys are 8 k0, even sequences query with -k0
    (pinned scores about -90 natural units, then ordinary window scores) and
    odd ones with -k0 / 16 (about -6 against window scores near 0); W = 1 in
    the second geometry (prefix + self)."""
    hq, hkv, d = 16, 2, 128
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16 if dtype == "bf16" else ps.PS_F32, 0.0, 1 / math.sqrt(d))
    for L, W, positions in ((40, 300, [45, 339, 340, 2000, 5000, 77]), (40, 1, [39, 40, 41, 900])):
        n = len(positions)
        cap = -(-(L + W) // 64) * 64
        cache = ps.CacheSpec(window=W, slot_capacity=cap)
        kc, vc = new_cache(ps, attn, cache, n)
        hist = []
        for s_ in range(n):
            k, v = _hist(6, 120 + W, s_, positions[s_] + 1, hkv, d, 1.0, dtype)
            k0 = k[:1, :1, :].copy()
            k[:L] = 8.0 * k0
            hist.append((k, v, k0))
        fill_ring(ps, attn, cache, kc, vc, [L] * n, [p - 1 for p in positions], [h[0] for h in hist],
                  [h[1] for h in hist])
        kn = np.stack([h[0][p] for h, p in zip(hist, positions)])[:, None]
        vn = np.stack([h[1][p] for h, p in zip(hist, positions)])[:, None]
        pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
        pos = torch.tensor(positions, dtype=torch.int64, device="cuda")
        ps.ps_kv_append(attn, cache, kc, vc, pl, pos, to_dev(kn, dt), to_dev(vn, dt))
        q = np.stack([-hist[s_][2][0] * (1.0 if s_ % 2 == 0 else 1.0 / 16.0) for s_ in range(n)])
        q = np.broadcast_to(q, (n, hq, d)).copy()
        qd = to_dev(q, dt)
        for splits in sorted({sp for sp in (1, 2, 3, 0) if sp <= cap // 32}):
            out = torch.empty((n, hq, d), dtype=dt, device="cuda")
            ps.ps_decode_attn(attn, cache, kc, vc, pl, pos, qd, out, num_splits=splits)
            got = out.float().cpu().numpy()
            for s_ in range(n):
                want = oracle.decode_attention(q[s_], hist[s_][0], hist[s_][1], positions[s_], L, W,
                                               1 / math.sqrt(d), 0.0)
                err = normwise_err(got[s_], want)
                assert err <= (BF16_TOL if dtype == "bf16" else F32_TOL), (W, splits, s_, positions[s_], err)


def test_bf16_decode_deterministic(ps):
    L, W, hq, hkv, d, n = 7, 300, 16, 2, 128, 5
    positions = [0, 100, 306, 307, 5000]
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    cache = ps.CacheSpec(window=W, slot_capacity=320)
    kc, vc = new_cache(ps, attn, cache, n)
    hist = [_hist(3, 77, s, positions[s] + 1, hkv, d, 0.5, "bf16") for s in range(n)]
    fill_ring(ps, attn, cache, kc, vc, [L] * n, positions, [h[0] for h in hist], [h[1] for h in hist])
    pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
    pos = torch.tensor(positions, dtype=torch.int64, device="cuda")
    qd = torch.randn((n, hq, d), generator=torch.Generator(device="cuda").manual_seed(0), device="cuda").bfloat16()
    outs = []
    for _ in range(3):
        out = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
        ps.ps_decode_attn(attn, cache, kc, vc, pl, pos, qd, out, num_splits=4)
        outs.append(out.view(torch.int16).cpu())
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


def test_bulk_append_skips_tokens_evicted_within_the_call(ps):
    """Appending a whole history in one call leaves exactly A(p) in the ring."""
    L, W, d = 3, 10, 64
    attn = ps.AttnSpec(4, 1, d, ps.PS_F32, 10000.0, 0.125)
    cache = ps.CacheSpec(window=W, slot_capacity=64)
    for p in (0, 5, 12, 13, 40):
        k, v = _hist(4, 55, p, p + 1, 1, d, 1.0, "f32")
        kc, vc = new_cache(ps, attn, cache, 1)
        sp = torch.full((1, 64), -1, dtype=torch.int32, device="cuda")
        ps.ps_kv_append(attn, cache, kc, vc, torch.tensor([L], dtype=torch.int32, device="cuda"),
                        torch.tensor([0], device="cuda"), to_dev(k[None], torch.float32),
                        to_dev(v[None], torch.float32), slot_pos=sp)
        got = sp.cpu().numpy()[0]
        want = np.full(64, -1)
        for j in oracle.visible_positions(p, L, W):
            want[oracle.slot_of(int(j), L, W)] = j
        np.testing.assert_array_equal(got, want)


def test_invalid_sequence_gives_nan_rows_and_leaves_others(ps):
    hq, hkv, d, W = 16, 2, 128, 64
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    cache = ps.CacheSpec(window=W, slot_capacity=128)
    n = 3
    positions = [70, 130, 70]
    prefix = [10, 100, 10]   # sequence 1 at 130 needs min(131, 164) = 131 > 128 slots
    kc, vc = new_cache(ps, attn, cache, n)
    hist = [_hist(5, 66, s, positions[s] + 1, hkv, d, 0.5, "bf16") for s in range(n)]
    fill_ring(ps, attn, cache, kc, vc, prefix, positions, [h[0] for h in hist], [h[1] for h in hist])
    pl = torch.tensor(prefix, dtype=torch.int32, device="cuda")
    pos = torch.tensor(positions, dtype=torch.int64, device="cuda")
    pos[2] = -5  # sequence 2: negative position
    q = np.stack([synth.query(5, 66, s, 0, 0, hq, d, 1.0, "bf16") for s in range(n)])
    for splits in (1, 2):
        out = torch.zeros((n, hq, d), dtype=torch.bfloat16, device="cuda")
        ps.ps_decode_attn(attn, cache, kc, vc, pl, pos, to_dev(q, torch.bfloat16), out, num_splits=splits)
        got = out.float().cpu().numpy()
        assert np.isnan(got[1]).all() and np.isnan(got[2]).all()
        want = oracle.decode_attention(q[0], hist[0][0], hist[0][1], 70, 10, W, 1 / math.sqrt(d), 10000.0)
        assert normwise_err(got[0], want) <= BF16_TOL


def test_full_attention_comparator_is_the_same_kernel(ps):
    """W >= n: ring slot == position, every key visible (full causal attention)."""
    hq, hkv, d = 16, 2, 128
    p = 2999
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    cache = ps.CacheSpec(window=1 << 30, slot_capacity=3008)
    kc, vc = new_cache(ps, attn, cache, 1)
    k, v = _hist(6, 67, 0, p + 1, hkv, d, 0.5, "bf16")
    fill_ring(ps, attn, cache, kc, vc, [0], [p], [k], [v])
    q = synth.query(6, 67, 0, 0, 0, hq, d, 1.0, "bf16")[None]
    out = torch.empty((1, hq, d), dtype=torch.bfloat16, device="cuda")
    ps.ps_decode_attn(attn, cache, kc, vc, torch.zeros(1, dtype=torch.int32, device="cuda"),
                      torch.tensor([p], device="cuda"), to_dev(q, torch.bfloat16), out, num_splits=8)
    want = oracle.decode_attention(q[0], k, v, p, 0, 1 << 30, 1 / math.sqrt(d), 10000.0)
    assert normwise_err(out.float().cpu().numpy()[0], want) <= BF16_TOL


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("paged", [False, True])
def test_append_calls_of_mixed_lengths_keep_the_ring_exact(ps, dtype, paged):
    """Appends of 1..70 tokens per call (short calls take the per-token path,
    long ones the 8-slot block path, which rewrites partly covered blocks):
    after every call the ring holds exactly A(p) -- K rotated at its position,
    V bit-exact, the slot map bit-exact -- including prefix/window blocks that
    straddle (L = 13) and the ring wrapping inside a call (W = 45)."""
    L, W, hkv, d, theta = 13, 45, 2, 64, 10000.0
    cap = 64
    pt = ps.PS_F32 if dtype == "f32" else ps.PS_BF16
    attn = ps.AttnSpec(2 * hkv, hkv, d, pt, theta, 0.125)
    bt = None
    if paged:
        bt, num_pages = paged_table(1, cap // 64, seed=9)
        cache = ps.CacheSpec(window=W, slot_capacity=cap, page_size=64, num_pages=num_pages)
    else:
        cache = ps.CacheSpec(window=W, slot_capacity=cap)
    total = 400
    k, v = _hist(5, 31, 0, total, hkv, d, 1.0, dtype)
    kc, vc = new_cache(ps, attn, cache, 1)
    slot_pos = torch.full((1, cap), -1, dtype=torch.int32, device="cuda")
    pl = torch.tensor([L], dtype=torch.int32, device="cuda")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    rng = np.random.default_rng(3)
    p = 0
    calls = 0
    while p < total:
        n = int(min(total - p, rng.choice([1, 3, 8, 15, 16, 17, 33, 45, 46, 70])))
        ps.ps_kv_append(attn, cache, kc, vc, pl, torch.tensor([p], dtype=torch.int64, device="cuda"),
                        to_dev(k[p:p + n][None], tdt), to_dev(v[p:p + n][None], tdt), block_table=bt,
                        slot_pos=slot_pos)
        p += n
        calls += 1
        ring = oracle.simulate_ring(range(p), L, W, cap)
        np.testing.assert_array_equal(slot_pos.cpu().numpy()[0], ring)
        kf, vf = kc.float().cpu().numpy(), vc.float().cpu().numpy()
        if paged:
            page = int(bt.cpu().numpy()[0, 0])
            kg, vg = kf[page, 0], vf[page, 0]
        else:
            kg, vg = kf[0, 0], vf[0, 0]
        vg = vg.transpose(0, 2, 1).reshape(-1, d)
        for slot, pos in enumerate(ring):
            if pos < 0:
                continue
            want_k = oracle.rope(k[pos, 0], pos, theta)
            tol = 2e-6 if dtype == "f32" else 2 ** -7 * np.abs(want_k).max()
            np.testing.assert_allclose(kg[slot], want_k, rtol=0, atol=tol, err_msg=f"call {calls} slot {slot}")
            np.testing.assert_array_equal(vg[slot], v[pos, 0], err_msg=f"call {calls} slot {slot}")
    assert calls > 10
