"""Pins for the float64 oracle: each test checks it against something other than
itself -- numbers the pages print, closed forms, torch's CPU attention with a
mask built independently, the textbook definitions of a rotation, and hand-worked
tile plans.  The cases are picked so that a plausible slip in the oracle (an
off-by-one window edge, a non-causal prefix, a swapped GQA map, a sign flip in
the rotation, a transposed operand) fails at least one of them."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- visible set
@pytest.mark.parametrize("L,W", [(0, 1), (0, 5), (1, 1), (3, 2), (16, 64), (100, 7), (7, 100)])
def test_visible_count_closed_form(L, W):
    # warm-up: all n = p+1 tokens; afterwards exactly L + W (blog mask section: L_total = L_prefix + W)
    for p in list(range(0, 3 * (L + W) + 5)) + [10 * (L + W) + 3]:
        assert oracle.visible_count(p, L, W) == min(p + 1, L + W), (p, L, W)


def test_pages_max_resident_tokens():
    g = _golden("pages_numbers.json")["max_resident_tokens"]
    for p in (4195, 4196, 10_000, 100_000, 262_143):
        assert oracle.visible_count(p, g["prefix_len"], g["window"]) == g["value"]
    # and the cap is reached exactly when the sequence has L + W tokens
    assert oracle.visible_count(g["value"] - 2, g["prefix_len"], g["window"]) == g["value"] - 1


def test_visible_set_closed_form_membership():
    # prefix [0, min(L, p+1)) union window (max(p-W, L-1), p]
    for L, W, p in itertools.product((0, 1, 4, 9), (1, 2, 3, 8), range(0, 40)):
        want = set(range(min(L, p + 1))) | set(range(max(p - W, L - 1) + 1, p + 1))
        assert set(oracle.visible_positions(p, L, W).tolist()) == want


# ---------------------------------------------------------------- ring / slots
@pytest.mark.parametrize("L,W", [(0, 1), (0, 4), (3, 1), (16, 64), (5, 7)])
def test_slot_map_bijection_and_eviction(L, W):
    cap = L + W
    for p in range(0, 4 * cap + 3):
        ring = oracle.simulate_ring(range(p + 1), L, W, cap)
        held = set(int(x) for x in ring if x >= 0)
        assert held == set(oracle.visible_positions(p, L, W).tolist())
        if p >= cap - 1:
            slots = sorted(oracle.slot_of(j, L, W) for j in oracle.visible_positions(p, L, W))
            assert slots == list(range(cap))
        if p - W >= L:
            assert oracle.slot_of(p, L, W) == oracle.slot_of(p - W, L, W)


def test_ring_permutation_invariance():
    rs = np.random.default_rng(3)
    L, W, p, hq, hkv, d = 5, 11, 57, 4, 2, 8
    k = rs.standard_normal((p + 1, hkv, d))
    v = rs.standard_normal((p + 1, hkv, d))
    q = rs.standard_normal((hq, d))
    full = oracle.decode_attention(q, k, v, p, L, W, 0.3, 10000.0)
    ring = oracle.simulate_ring(range(p + 1), L, W, L + W)
    pos = ring[ring >= 0]
    k_rot = oracle.rope(k[pos], pos[:, None], 10000.0)
    for _ in range(5):
        perm = rs.permutation(pos.size)
        got = oracle.decode_from_slots(q, p, k_rot[perm], v[pos][perm], 0.3, 10000.0)
        np.testing.assert_allclose(got, full, rtol=0, atol=1e-13)


# ---------------------------------------------------------------- reductions to torch's attention
def _sdpa(q, k, v, mask, scale):
    """torch CPU attention in float64; q [T,Hq,D], k/v [N,Hkv,D] with KV heads
    expanded by repeat_interleave (consecutive query heads share a KV head)."""
    hq, hkv = q.shape[1], k.shape[1]
    kk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    vv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
    qq = torch.from_numpy(q).permute(1, 0, 2)
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=torch.from_numpy(mask),
                                                         scale=scale)
    return o.permute(1, 0, 2).numpy()


def _band_mask(n, L, W):
    """Causal band with W keys (self included) plus pinned columns [0, L), built
    from torch's triangular helpers."""
    ones = torch.ones(n, n, dtype=torch.bool)
    band = ones.tril() & ~ones.tril(-W)
    pinned = torch.zeros(n, n, dtype=torch.bool)
    pinned[:, :L] = True
    return (band | (pinned & ones.tril())).numpy()


@pytest.mark.parametrize("L,W,kind", [(0, 1 << 20, "full"), (5, 1 << 20, "full"), (40, 3, "full-prefix"),
                                      (0, 6, "swa"), (0, 1, "swa"), (3, 6, "ps")])
def test_prefill_reduces_to_reference_attention(L, W, kind):
    rs = np.random.default_rng(7)
    n, hq, hkv, d = 37, 6, 2, 16
    q = rs.standard_normal((n, hq, d))
    k = rs.standard_normal((n, hkv, d))
    v = rs.standard_normal((n, hkv, d))
    scale = 1 / math.sqrt(d)
    got, _ = oracle.prefill_attention(q, k, v, min(L, n), W, min(L, n), scale, 0.0)
    if kind.startswith("full"):
        mask = np.tril(np.ones((n, n), dtype=bool))       # L >= n or W >= n: plain causal attention
    else:
        mask = _band_mask(n, L, W)
    want = _sdpa(q, k, v, mask, scale)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,W", [(0, 1 << 20), (0, 9), (4, 9), (64, 2)])
def test_decode_reduces_to_reference_attention(L, W):
    rs = np.random.default_rng(11)
    hq, hkv, d = 8, 2, 16
    k = rs.standard_normal((60, hkv, d))
    v = rs.standard_normal((60, hkv, d))
    for p in (0, 1, 8, 13, 59):
        q = rs.standard_normal((hq, d))
        got = oracle.decode_attention(q, k, v, p, L, W, 0.25, 0.0)
        mask = _band_mask(p + 1, min(L, p + 1), W)[-1:]
        want = _sdpa(q[None], k[:p + 1], v[:p + 1], mask, 0.25)[0]
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_decode_with_rope_matches_reference_on_complex_rotation():
    # rotate with the complex-number form of RoPE (x_lo + i x_hi) * exp(i pos f), then plain attention
    rs = np.random.default_rng(5)
    L, W, p, hq, hkv, d, theta = 3, 10, 40, 4, 1, 8, 10000.0
    k = rs.standard_normal((p + 1, hkv, d))
    v = rs.standard_normal((p + 1, hkv, d))
    q = rs.standard_normal((hq, d))
    f = theta ** (-np.arange(d // 2) * 2.0 / d)

    def crot(x, pos):
        z = (x[..., : d // 2] + 1j * x[..., d // 2:]) * np.exp(1j * np.multiply.outer(pos, f))
        return np.concatenate([z.real, z.imag], axis=-1)

    pos = np.arange(p + 1)
    kr = crot(k, pos[:, None])
    qr = crot(q, np.full(hq, p))
    mask = _band_mask(p + 1, L, W)[-1:]
    want = _sdpa(qr[None], kr, v, mask, 0.2)[0]
    got = oracle.decode_attention(q, k, v, p, L, W, 0.2, theta)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("L,W", [(0, 5), (4, 6), (10, 3), (2, 100)])
def test_zero_query_gives_mean_of_visible_values(L, W):
    # q = 0 -> uniform weights over A(p).  With v_j = (1, j, j^2) the output is
    # (1, mean j, mean j^2) over A(p), written here with arithmetic-series sums.
    d = 4

    def s1(a, b):  # sum of j for a <= j < b
        return (b - a) * (a + b - 1) / 2 if b > a else 0.0

    def s2(a, b):  # sum of j^2 for a <= j < b
        f = lambda n: (n - 1) * n * (2 * n - 1) / 6  # sum_{j<n} j^2
        return f(b) - f(a) if b > a else 0.0

    for p in range(0, 60):
        j = np.arange(p + 1, dtype=np.float64)
        v = np.zeros((p + 1, 1, d))
        v[:, 0, 0], v[:, 0, 1], v[:, 0, 2] = 1.0, j, j * j
        k = np.random.default_rng(p).standard_normal((p + 1, 1, d))
        got = oracle.decode_attention(np.zeros((2, d)), k, v, p, L, W, 1.0, 10000.0)
        a = min(L, p + 1)                     # prefix part [0, a)
        b = max(p - W + 1, a)                 # window part [b, p+1), disjoint from the prefix
        n = a + (p + 1 - b)
        assert n == min(p + 1, L + W)
        want = [1.0, (s1(0, a) + s1(b, p + 1)) / n, (s2(0, a) + s2(b, p + 1)) / n, 0.0]
        np.testing.assert_allclose(got[0], want, rtol=1e-13)
        np.testing.assert_allclose(got[1], want, rtol=1e-13)


def test_single_visible_key_returns_its_value():
    rs = np.random.default_rng(1)
    k = rs.standard_normal((1, 2, 8))
    v = rs.standard_normal((1, 2, 8))
    out = oracle.decode_attention(rs.standard_normal((4, 8)), k, v, 0, 0, 1, 1.0, 10000.0)
    np.testing.assert_allclose(out, np.repeat(v[0], 2, axis=0), rtol=0, atol=0)
    # W = 1 with no prefix: every query sees only itself
    k = rs.standard_normal((9, 2, 8))
    v = rs.standard_normal((9, 2, 8))
    out = oracle.decode_attention(rs.standard_normal((4, 8)), k, v, 8, 0, 1, 1.0, 10000.0)
    np.testing.assert_allclose(out, np.repeat(v[8], 2, axis=0), rtol=0, atol=1e-15)


def test_gqa_head_map_is_consecutive():
    # Hq=4, Hkv=2: heads 0,1 -> KV head 0; heads 2,3 -> KV head 1.  With a single
    # visible key the output is that KV head's value.
    rs = np.random.default_rng(2)
    k = rs.standard_normal((1, 2, 8))
    v = rs.standard_normal((1, 2, 8))
    out = oracle.decode_attention(rs.standard_normal((4, 8)), k, v, 0, 0, 1, 1.0, 0.0)
    for h in range(4):
        np.testing.assert_array_equal(out[h], v[0, h // 2])


# ---------------------------------------------------------------- RoPE
def test_rope_two_dims_is_plane_rotation():
    x = np.array([[0.3, -1.7]])
    for pos in (0, 1, 5, 1000, 131072):
        c, s = math.cos(pos), math.sin(pos)           # D=2: the only frequency is theta^0 = 1
        want = np.array([[c * 0.3 - s * -1.7, s * 0.3 + c * -1.7]])
        np.testing.assert_allclose(oracle.rope(x, pos, 10000.0), want, rtol=0, atol=1e-15)


def test_rope_frequencies_and_pairing():
    # unit vector e_i (i < D/2) at position pos rotates into (cos, sin) on dims (i, i + D/2)
    d, theta = 8, 10000.0
    for i in range(d // 2):
        e = np.zeros(d)
        e[i] = 1.0
        pos = 37
        ang = pos * theta ** (-2 * i / d)
        want = np.zeros(d)
        want[i], want[i + d // 2] = math.cos(ang), math.sin(ang)
        np.testing.assert_allclose(oracle.rope(e, pos, theta), want, atol=1e-15)


def test_rope_relative_position_and_norm():
    rs = np.random.default_rng(4)
    q, k = rs.standard_normal(64), rs.standard_normal(64)
    base = oracle.rope(q, 100, 10000.0) @ oracle.rope(k, 70, 10000.0)
    for shift in (1, 17, 4096, 131000):
        got = oracle.rope(q, 100 + shift, 10000.0) @ oracle.rope(k, 70 + shift, 10000.0)
        assert abs(got - base) < 1e-9
    np.testing.assert_allclose(np.linalg.norm(oracle.rope(q, 262143, 10000.0)), np.linalg.norm(q), rtol=1e-14)
    np.testing.assert_array_equal(oracle.rope(q, 0, 10000.0), q)


# ---------------------------------------------------------------- decode == prefill row
def test_decode_matches_prefill_rows_tiny_config():
    c = synth.C1_PREFILL
    n = 200
    k = synth.history(0, 1, synth.T_K, 0, 0, 0, n, c.hkv, c.dim, 1.0, "f32")
    v = synth.history(0, 1, synth.T_V, 0, 0, 0, n, c.hkv, c.dim, 1.0, "f32")
    q = synth.history(0, 1, synth.T_Q, 0, 0, 0, n, c.hq, c.dim, 1.0, "f32")
    pre, _ = oracle.prefill_attention(q, k, v, c.prefix, c.window, c.prefix, 0.125, 10000.0)
    for p in (0, 15, 16, 79, 80, 81, 199):
        dec = oracle.decode_attention(q[p], k, v, p, c.prefix, c.window, 0.125, 10000.0)
        np.testing.assert_allclose(dec, pre[p], rtol=0, atol=1e-12)


def test_prefill_lse_matches_direct_sum():
    rs = np.random.default_rng(9)
    q = rs.standard_normal((12, 2, 8))
    k = rs.standard_normal((15, 1, 8))
    v = rs.standard_normal((15, 1, 8))
    _, lse = oracle.prefill_attention(q, k, v, 3, 4, 3, 0.5, 0.0)
    posk = np.arange(15)
    for t in range(12):
        pq = 3 + t
        vis = [j for j in range(15) if j <= pq and (j < 3 or j > pq - 4)]
        for h in range(2):
            want = math.log(sum(math.exp(0.5 * float(q[t, h] @ k[j, 0])) for j in vis))
            assert abs(lse[t, h] - want) < 1e-12


# ---------------------------------------------------------------- chunk continuing a trace
@pytest.mark.parametrize("L,W,start,T", [(0, 1 << 20, 20, 17), (3, 6, 0, 37), (3, 6, 25, 12), (4, 9, 2, 30),
                                         (40, 3, 10, 20), (0, 1, 30, 7)])
def test_chunk_reduces_to_reference_attention(L, W, start, T):
    # no rotation: the chunk rows are the last T rows of plain band attention
    rs = np.random.default_rng(5)
    n, hq, hkv, d = start + T, 6, 2, 16
    q = rs.standard_normal((T, hq, d))
    k = rs.standard_normal((n, hkv, d))
    v = rs.standard_normal((n, hkv, d))
    got, _ = oracle.chunk_prefill_attention(q, k, v, start, L, W, 0.25, 0.0)
    mask = _band_mask(n, min(L, n), W)[start:]
    want_q = np.zeros((n, hq, d))
    want_q[start:] = q
    want = _sdpa(want_q, k, v, _band_mask(n, min(L, n), W), 0.25)[start:]
    assert mask.shape == (T, n)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_chunk_rows_match_decode_with_rotation():
    rs = np.random.default_rng(6)
    L, W, start, T = 5, 11, 23, 19
    k = rs.standard_normal((start + T, 2, 8))
    v = rs.standard_normal((start + T, 2, 8))
    q = rs.standard_normal((T, 4, 8))
    got, _ = oracle.chunk_prefill_attention(q, k, v, start, L, W, 0.4, 10000.0)
    for t in range(T):
        dec = oracle.decode_attention(q[t], k, v, start + t, L, W, 0.4, 10000.0)
        np.testing.assert_allclose(got[t], dec, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,W,start", [(3, 5, 40), (10, 4, 3), (0, 7, 15), (6, 100, 50)])
def test_chunk_zero_query_gives_mean_of_visible_values(L, W, start):
    # q = 0 -> uniform weights over A(p) for every chunk query p = start + t;
    # v_j = (1, j, j^2) makes the output the count-normalised first and second
    # moments of the visible positions, summed here in closed form
    T, d = 25, 4
    n = start + T
    j = np.arange(n, dtype=np.float64)
    v = np.zeros((n, 1, d))
    v[:, 0, 0], v[:, 0, 1], v[:, 0, 2] = 1.0, j, j * j
    k = np.random.default_rng(start).standard_normal((n, 1, d))
    got, lse = oracle.chunk_prefill_attention(np.zeros((T, 2, d)), k, v, start, L, W, 1.0, 10000.0)
    s1 = lambda a, b: (b - a) * (a + b - 1) / 2 if b > a else 0.0
    f2 = lambda m: (m - 1) * m * (2 * m - 1) / 6
    s2 = lambda a, b: f2(b) - f2(a) if b > a else 0.0
    for t in range(T):
        p = start + t
        a = min(L, p + 1)
        b = max(p - W + 1, a)
        cnt = a + (p + 1 - b)
        want = [1.0, (s1(0, a) + s1(b, p + 1)) / cnt, (s2(0, a) + s2(b, p + 1)) / cnt, 0.0]
        np.testing.assert_allclose(got[t, 0], want, rtol=1e-13)
        np.testing.assert_allclose(got[t, 1], want, rtol=1e-13)
        assert abs(lse[t, 0] - math.log(cnt)) < 1e-12   # all scores 0: lse = log(count)


# ---------------------------------------------------------------- backward of the masked prefill
def _bwd_case(seed, t_q=9, nk=14, hq=4, hkv=2, d=8):
    rs = np.random.default_rng(seed)
    return (rs.standard_normal((t_q, hq, d)), rs.standard_normal((nk, hkv, d)), rs.standard_normal((nk, hkv, d)),
            rs.standard_normal((t_q, hq, d)))


@pytest.mark.parametrize("L,W,kv_start,theta", [(3, 4, 3, 10000.0), (2, 3, 7, 10000.0), (0, 1 << 20, 0, 500.0),
                                                (5, 2, 5, 0.0)])
def test_backward_matches_central_differences(L, W, kv_start, theta):
    q, k, v, do = _bwd_case(1)
    sc = 0.37
    dq, dk, dv = oracle.prefill_attention_backward(q, k, v, do, L, W, kv_start, sc, theta)

    def loss(q_, k_, v_):
        o, _ = oracle.prefill_attention(q_, k_, v_, L, W, kv_start, sc, theta)
        return float((o * do).sum())

    eps = 1e-6
    for arr, grad, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            args_p = [q.copy(), k.copy(), v.copy()]
            args_m = [q.copy(), k.copy(), v.copy()]
            args_p[which][idx] += eps
            args_m[which][idx] -= eps
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8)


def _torch_rope(x, pos, theta):
    # rotation written as complex multiplication of the pairs (x_i, x_{i+D/2})
    d = x.shape[-1]
    h = d // 2
    if not theta:
        return x
    f = theta ** (-2.0 * torch.arange(h, dtype=torch.float64) / d)
    rot = torch.polar(torch.ones(pos.shape[0], h, dtype=torch.float64), pos[:, None].double() * f)[:, None, :]
    z = torch.complex(x[..., :h], x[..., h:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


@pytest.mark.parametrize("L,W", [(4, 5), (0, 6), (30, 3)])
def test_backward_matches_torch_autograd(L, W):
    q, k, v, do = _bwd_case(2, t_q=21, nk=21, hq=6, hkv=3, d=16)
    sc, theta = 0.25, 10000.0
    dq, dk, dv = oracle.prefill_attention_backward(q, k, v, do, L, W, L, sc, theta)
    n = 21
    pos = torch.arange(n)
    tq = torch.from_numpy(q).requires_grad_()
    tk = torch.from_numpy(k).requires_grad_()
    tv = torch.from_numpy(v).requires_grad_()
    qr = _torch_rope(tq, pos, theta)
    kr = _torch_rope(tk, pos, theta)
    mask = torch.from_numpy(_band_mask(n, min(L, n), W))
    g = 2
    kk = kr.permute(1, 0, 2).repeat_interleave(g, dim=0)
    vv = tv.permute(1, 0, 2).repeat_interleave(g, dim=0)
    s = sc * qr.permute(1, 0, 2) @ kk.transpose(1, 2)
    o = torch.softmax(s.masked_fill(~mask, float("-inf")), dim=-1) @ vv
    (o.permute(1, 0, 2) * torch.from_numpy(do)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), rtol=0, atol=1e-12)


def test_backward_invariants_and_loss_mask_structure():
    q, k, v, do = _bwd_case(3, t_q=30, nk=40, hq=4, hkv=2, d=8)
    L, W, ks = 3, 5, 13
    # without rotation: scores are unchanged by adding one vector to every key, so dk sums to 0;
    # every probability row sums to 1, so dv sums to the upstream gradient of the group's heads
    dq, dk, dv = oracle.prefill_attention_backward(q, k, v, do, L, W, ks, 0.5, 0.0)
    np.testing.assert_allclose(dk.sum(axis=0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(axis=0), do.reshape(30, 2, 2, 8).sum(axis=(0, 2)), atol=1e-12)
    # loss mask on the last r rows (the trainer's last-W rule): keys no such row can see get exactly 0
    r = 6
    dom = do.copy()
    dom[:-r] = 0.0
    dq, dk, dv = oracle.prefill_attention_backward(q, k, v, dom, L, W, ks, 0.5, 10000.0)
    posk = oracle.key_positions(40, L, ks)
    posq = posk[-30:][-r:]
    seen = oracle.visible(posq[:, None], posk[None, :], L, W).any(axis=0)
    assert (~seen).sum() > 0 and seen.sum() > 0
    assert np.all(dk[~seen] == 0.0) and np.all(dv[~seen] == 0.0)
    assert np.all(np.abs(dv[seen]).sum(axis=(1, 2)) > 0)
    assert np.all(dq[:-r] == 0.0)


def test_backward_sampled_rows_agree_with_full_evaluation():
    q, k, v, do = _bwd_case(4, t_q=70, nk=90, hq=6, hkv=2, d=8)
    L, W, ks = 7, 11, 33
    dq, dk, dv = oracle.prefill_attention_backward(q, k, v, do, L, W, ks, 0.3, 10000.0)
    qr, kr = [0, 5, 31, 69], [0, 6, 7, 40, 89]
    for kv in range(2):
        sq, sk, sv = oracle.prefill_attention_backward_sampled(q, k, v, do, L, W, ks, 0.3, 10000.0, kv, qr, kr,
                                                               block=16)
        np.testing.assert_allclose(sq, dq[qr][:, 3 * kv:3 * kv + 3], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sk, dk[kr, kv], rtol=0, atol=1e-12)
        np.testing.assert_allclose(sv, dv[kr, kv], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- Reset PE
def test_reset_pe_numbering_hand_worked():
    # L = 3, W = 4, p = 20: visible {0, 1, 2, 17, 18, 19, 20} -> 0..6, query at 6
    vis, new = oracle.reset_pe_positions(20, 3, 4)
    assert vis.tolist() == [0, 1, 2, 17, 18, 19, 20] and new.tolist() == [0, 1, 2, 3, 4, 5, 6]
    # warm-up: nothing is renumbered
    vis, new = oracle.reset_pe_positions(5, 3, 4)
    assert vis.tolist() == new.tolist() == [0, 1, 2, 3, 4, 5]
    vis, new = oracle.reset_pe_positions(2, 10, 4)      # query inside the prefix
    assert vis.tolist() == new.tolist() == [0, 1, 2]


def test_reset_pe_against_explicit_rotation():
    rs = np.random.default_rng(12)
    k = rs.standard_normal((21, 2, 8))
    v = rs.standard_normal((21, 2, 8))
    q = rs.standard_normal((4, 8))
    got = oracle.decode_attention_reset_pe(q, k, v, 20, 3, 4, 0.5, 100.0)
    keys = [0, 1, 2, 17, 18, 19, 20]
    # rotate each pair (i, i + D/2) by position * 100^(-2i/D) with complex numbers
    def rot(x, pos):
        f = 100.0 ** (-2.0 * np.arange(4) / 8)
        z = (x[..., :4] + 1j * x[..., 4:]) * np.exp(1j * pos * f)
        return np.concatenate([z.real, z.imag], axis=-1)
    want = np.empty((4, 8))
    for h in range(4):
        qh = rot(q[h], 6)
        s = np.array([0.5 * rot(k[j, h // 2], n) @ qh for n, j in enumerate(keys)])
        w = np.exp(s - s.max())
        want[h] = (w / w.sum()) @ v[keys, h // 2]
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("L,W,p", [(0, 8, 40), (0, 1, 9), (5, 6, 9), (5, 6, 10), (30, 6, 20), (4, 100, 50),
                                   (3, 4, 20), (10, 8, 100)])
def test_reset_pe_reduces_to_continue_pe(L, W, p):
    # no prefix (only relative offsets inside the window matter), warm-up, or no
    # rotation: Reset PE and Continue PE give the same attention
    rs = np.random.default_rng(p)
    k = rs.standard_normal((p + 1, 2, 16))
    v = rs.standard_normal((p + 1, 2, 16))
    q = rs.standard_normal((4, 16))
    cont = oracle.decode_attention(q, k, v, p, L, W, 0.3, 10000.0)
    reset = oracle.decode_attention_reset_pe(q, k, v, p, L, W, 0.3, 10000.0)
    if L == 0 or p - W + 1 <= L:
        np.testing.assert_allclose(reset, cont, rtol=0, atol=1e-12)
    else:
        assert np.abs(reset - cont).max() > 1e-6      # the prefix-window distance really changed
    np.testing.assert_allclose(oracle.decode_attention_reset_pe(q, k, v, p, L, W, 0.3, 0.0),
                               oracle.decode_attention(q, k, v, p, L, W, 0.3, 0.0), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- prefix + heavy hitters + window
def test_h2o_admission_hand_worked():
    assert oracle.h2o_admit([-1, -1], [0.0, 0.0], 7, 0.1, 2) == (0, -1)          # free slot, filled in order
    assert oracle.h2o_admit([5, -1], [3.0, 0.0], 7, 0.1, 2) == (1, -1)
    assert oracle.h2o_admit([5, 6], [3.0, 1.0], 9, 2.0, 2) == (1, 6)             # beats the weakest member
    assert oracle.h2o_admit([5, 6], [3.0, 1.0], 9, 1.0, 2) == (-1, 9)            # a tie keeps the member
    assert oracle.h2o_admit([8, 6], [1.0, 1.0], 9, 1.5, 2) == (1, 6)             # equal members: oldest goes
    assert oracle.h2o_admit([5], [1.0], 9, 0.5, 1) == (-1, 9)


def test_h2o_zero_query_trace_hand_worked():
    # q = 0 makes every visible token draw the same mass; with W = 1 and one heavy
    # slot the first token enters the heavy set at step 1 and never leaves (each
    # later candidate has drawn half a step's mass against its growing total), so
    # the query at p averages v over {0, p}; features (1, j, j^2) expose the set
    n, g = 12, 2
    j = np.arange(n, dtype=np.float64)
    v = np.zeros((n, 1, 4))
    v[:, 0, 0], v[:, 0, 1], v[:, 0, 2] = 1.0, j, j * j
    k = np.random.default_rng(0).standard_normal((n, 1, 4))
    out, heavy, scores = oracle.h2o_decode_trace(np.zeros((n, g, 4)), k, v, 0, 1, 1, 1.0, 10000.0)
    assert heavy.tolist() == [[0]]
    np.testing.assert_allclose(out[0, :, :3], [[1.0, 0.0, 0.0]] * g, atol=1e-15)
    for p in range(1, n):
        np.testing.assert_allclose(out[p, 0, :3], [1.0, p / 2, p * p / 2], rtol=1e-13)
    # token 0: G at step 0, then G/2 at each of steps 1..n-1
    assert abs(scores[0][0] - (g + g * (n - 1) / 2)) < 1e-12
    assert set(scores[0]) == {0, n - 1}


@pytest.mark.parametrize("L,W", [(3, 5), (0, 4), (6, 1)])
def test_h2o_reduces_to_prefix_sliding_and_full_attention(L, W):
    rs = np.random.default_rng(L + W)
    n = 40
    q = rs.standard_normal((n, 4, 8))
    k = rs.standard_normal((n, 2, 8))
    v = rs.standard_normal((n, 2, 8))
    none, _, _ = oracle.h2o_decode_trace(q, k, v, L, W, 0, 0.4, 10000.0)          # no heavy slots: Prefix Sliding
    allk, heavy, _ = oracle.h2o_decode_trace(q, k, v, L, W, n, 0.4, 10000.0)      # room for every token: full
    for p in range(n):
        np.testing.assert_allclose(none[p], oracle.decode_attention(q[p], k, v, p, L, W, 0.4, 10000.0),
                                   rtol=0, atol=1e-12)
        np.testing.assert_allclose(allk[p], oracle.decode_attention(q[p], k, v, p, 0, 1 << 30, 0.4, 10000.0),
                                   rtol=0, atol=1e-12)
    assert sorted(heavy[0][heavy[0] >= 0].tolist()) == list(range(L, n - W))


def test_h2o_trace_invariants():
    # every step's attention sums to one per head, so the scores of the tokens
    # still cached never exceed G * steps; heavy members always outscore the
    # candidates they beat, and the heavy set is disjoint from prefix and window
    rs = np.random.default_rng(3)
    n, L, W, H = 80, 4, 6, 5
    q = rs.standard_normal((n, 6, 8)) * 2
    k = rs.standard_normal((n, 2, 8))
    v = rs.standard_normal((n, 2, 8))
    _, heavy, scores = oracle.h2o_decode_trace(q, k, v, L, W, H, 0.5, 10000.0)
    for kv in range(2):
        members = heavy[kv][heavy[kv] >= 0]
        assert members.size == H
        assert np.all(members >= L) and np.all(members <= n - 1 - W)
        assert sum(scores[kv].values()) <= 3 * n + 1e-9
        assert set(scores[kv]) == set(members.tolist()) | set(range(n - W, n))


def test_slot_attention_mass_closed_forms():
    # q = 0: every cached key draws the same weight from every head, so each slot
    # of a KV head gets G / n; two keys whose scores differ by a known amount
    # split a head's unit mass as a logistic function of that difference
    rs = np.random.default_rng(11)
    n, hq, hkv, d = 9, 6, 2, 8
    k = rs.standard_normal((n, hkv, d))
    mass = oracle.slot_attention_mass(np.zeros((hq, d)), 17, k, 0.7, 10000.0)
    np.testing.assert_allclose(mass, np.full((n, hkv), (hq // hkv) / n), rtol=0, atol=1e-15)
    # theta = 0 (no rotation): key 0 scores scale * <q, k0> = 0.5 * 2 = 1 with every
    # query head, key 1 scores 0
    q = np.zeros((4, 2))
    q[:, 0] = 2.0
    kk = np.zeros((2, 1, 2))
    kk[0, 0, 0] = 1.0
    got = oracle.slot_attention_mass(q, 5, kk, 0.5, 0.0)
    e = math.e
    np.testing.assert_allclose(got[:, 0], [4 * e / (e + 1), 4 / (e + 1)], rtol=1e-15)


def test_slot_attention_mass_against_outputs_and_trace_increments():
    rs = np.random.default_rng(12)
    hq, hkv, d, L, W, p = 8, 2, 16, 3, 50, 23
    g = hq // hkv
    q = rs.standard_normal((p + 2, hq, d))
    k = rs.standard_normal((p + 2, hkv, d))
    v = rs.standard_normal((p + 2, hkv, d))
    pos = np.arange(p + 1)
    k_rot = oracle.rope(k[:p + 1], pos[:, None], 10000.0)
    mass = oracle.slot_attention_mass(q[p], p, k_rot, 0.3, 10000.0)
    # each KV head's column sums to its G heads' unit masses
    np.testing.assert_allclose(mass.sum(axis=0), [g, g], rtol=1e-14)
    # the group's outputs summed over heads are the mass-weighted sum of values
    # (ties the weights to the pinned decode oracle: same rotation, scale, map)
    out = oracle.decode_from_slots(q[p], p, k_rot, v[:p + 1], 0.3, 10000.0)
    for kv in range(hkv):
        np.testing.assert_allclose(out[kv * g:(kv + 1) * g].sum(axis=0), mass[:, kv] @ v[:p + 1, kv],
                                   rtol=0, atol=1e-12)
    # the heavy-hitter trace adds exactly this mass at step p to every cached
    # non-prefix token (W > p: nothing has left the window yet)
    _, _, before = oracle.h2o_decode_trace(q[:p], k[:p], v[:p], L, W, 4, 0.3, 10000.0)
    _, _, after = oracle.h2o_decode_trace(q[:p + 1], k[:p + 1], v[:p + 1], L, W, 4, 0.3, 10000.0)
    for kv in range(hkv):
        for j in range(L, p + 1):
            grew = after[kv][j] - before[kv].get(j, 0.0)
            assert abs(grew - mass[j, kv]) < 1e-12, (kv, j)


# ---------------------------------------------------------------- tile plan
def test_tile_plan_hand_worked_cases():
    for case in _golden("tile_plan_small.json")["cases"]:
        plan = oracle.tile_plan(case["T"], case["Nk"], case["L"], case["W"], case["kv_start"], case["BM"],
                                case["BN"])
        want = [(qt, kt, oracle.KIND_FULL if kind == "F" else oracle.KIND_PARTIAL)
                for qt, kt, kind, _ in case["tiles"]]
        assert plan == want, case["name"]
        assert oracle.visible_pairs(case["T"], case["Nk"], case["L"], case["W"], case["kv_start"]) \
            == case["total_pairs"]


def test_tile_plan_invariants_truncated_backprop_shape():
    # chunk of 4W tokens behind a 100-token prefix, as in the truncated-backprop example
    g = _golden("pages_numbers.json")["truncated_backprop_example"]
    W, T, L, start = g["window"], g["trainer_tokens"], 100, 98304
    nk = L + T
    total = oracle.visible_pairs(T, nk, L, W, start)
    # closed form: every query sees the whole prefix plus min(t+1, W) chunk keys
    assert total == L * T + sum(min(t + 1, W) for t in range(T)) == 15_500_288
    plan = oracle.tile_plan(T, nk, L, W, start, 128, 64)
    full = [p for p in plan if p[2] == oracle.KIND_FULL]
    # full tiles carry BM*BN pairs each, partial tiles the remainder, and no pair is lost
    posk = oracle.key_positions(nk, L, start)
    posq = posk[nk - T:]
    covered = 0
    for qt, kt, kind in plan:
        cnt = int(oracle.visible(posq[qt * 128:(qt + 1) * 128, None], posk[None, kt * 64:(kt + 1) * 64],
                                 L, W).sum())
        assert cnt > 0 and (kind == oracle.KIND_PARTIAL or cnt == 128 * 64)
        covered += cnt
    assert covered == total and len(full) > 0


def test_key_positions_layout():
    np.testing.assert_array_equal(oracle.key_positions(6, 2, 100), [0, 1, 100, 101, 102, 103])
    np.testing.assert_array_equal(oracle.key_positions(4, 0, 7), [7, 8, 9, 10])


# ---------------------------------------------------------------- byte accounting from the pages
def test_kv_bytes_per_token_formula():
    for key in ("kv_bytes_per_token_qwen3_1p7b", "kv_bytes_per_token_7b"):
        g = _golden("pages_numbers.json")[key]
        b = 2 * g["layers"] * g["kv_heads"] * g["head_dim"] * g["bytes_per_elem"]
        assert round(b / 1000) == g["approx_kb"] or round(b / 1024) == g["approx_kb"]


# ---------------------------------------------------------------- synthetic input rounding
def test_bf16_rounding_matches_torch():
    x = synth.normal((4096,), 0, 99, std=3.0)
    want = torch.from_numpy(x).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(synth.round_to(x, "bf16"), want)
