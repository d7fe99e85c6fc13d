"""Float64 CPU oracle for Prefix Sliding attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the library path may import or call this
module: only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` use it.  It shares no code with the HIP kernels.

What it computes, and where each rule comes from (page titles as printed on
the pages; no page is quoted):

* Visibility.  Blog "Prefix Sliding 完全拆解" (pinghaoyang.com.cn), section
  "核心机制：注意力掩码上的两个区间", definition of the allowed set A(i): a query
  sees the prefix and the last W tokens up to itself; every other score is set
  to -inf before the softmax.  The same rule is restated in the Polish notes
  "Prefix Sliding. Myślenie może być długie, pamięć nie", section "Intuicja".
  Readings (the pages are 1-indexed and loose at the edges):
    - positions are 0-indexed absolute positions p, j of one sequence;
    - the prefix is [0, L); the window is (p - W, p], i.e. W tokens counting
      the query itself -- this is what makes "100-token prefix + 4096 window
      holds at most 4196 tokens" (agihunt.info summary; ainews.surl.tw
      article) come out exactly;
    - attention is always causal (j <= p), also inside the prefix: during
      warm-up the method behaves exactly like the unmodified model (same blog
      section, warm-up paragraph);
    - prefix and window are a set union: no key is counted twice.
* Eviction and Continue PE.  Same blog, the mask section (hidden tokens'
  K/V are not kept) and section "位置编码：Reset PE 还是 Continue PE？": every
  token keeps its absolute position; cached keys are rotated once and reused.
  Because a hidden key only ever contributes a -inf score, the method's result
  is exactly plain masked softmax attention over the *full, un-evicted*
  history, which is what this oracle evaluates.
* Rotary embedding.  The pages name RoPE without fixing a variant.  Reading:
  rotate-half pairing (i, i + D/2) with inverse frequencies theta^(-2i/D),
  theta = 10000, evaluated exactly in float64 at the absolute position.
* GQA.  Query head h uses KV head floor(h / (Hq/Hkv)) (the blog's memory
  formula counts KV heads separately from query heads).
* Prefill key set (truncated backprop, blog section
  "超长 rollouts 的反向传播：截断回传"): keys are the prefix followed by a chunk
  of consecutive positions starting at ``kv_start``; queries are the last T
  keys; nothing before the chunk other than the prefix exists.
* Chunk continuing a trace (``chunk_prefill_attention``): queries at
  start..start+T-1 over the whole history; the ring supplies what the earlier
  trace left visible, so the result is again plain masked attention.
* Reset PE (``decode_attention_reset_pe``; blog section "位置编码：Reset PE 还是
  Continue PE？", the alternative the paper ablated): same visible set, visible
  window tokens renumbered to follow the prefix, rotation at the new numbers.
* Prefix + heavy hitters + window (``h2o_admit``, ``h2o_decode_trace``,
  ``slot_attention_mass``): the combination the blog proposes when comparing
  with H2O; the admission rule and the per-KV-head score (attention received,
  summed over the group's query heads, accumulated while cached) are
  readings, stated in the docstrings.
* Backward of the masked prefill (``prefill_attention_backward``): the chain
  rule of masked softmax attention, written out; gradients are taken with
  respect to the raw (un-rotated) inputs.
* Tile plan (blog section "Kernel 实现：两层级过滤"): tiles with no visible pair
  are skipped, tiles whose every pair is visible need no element mask, the
  rest are partial.  The oracle decides this by enumerating every element.
* Ring slot of position n (the pages only say hidden tokens are not kept):
  n for n < L, else L + ((n - L) mod W).

Parity status: every function here is pinned by tests/test_oracle_pins.py
against closed forms, reductions to torch's CPU attention with independently
built masks, the pages' printed numbers (tests/golden/) and brute force.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

KIND_FULL = 1
KIND_PARTIAL = 2


# --------------------------------------------------------------------------
# visibility (blog "Prefix Sliding 完全拆解", mask section: the set A(i))
# --------------------------------------------------------------------------
def visible(pq, pk, prefix_len: int, window: int):
    """Element-wise: may a query at absolute position ``pq`` see the key at ``pk``?

    Causal, plus (key in the pinned prefix [0, L) or key in the window (pq-W, pq]).
    Works on scalars and broadcasting numpy arrays."""
    pq = np.asarray(pq, dtype=np.int64)
    pk = np.asarray(pk, dtype=np.int64)
    return (pk <= pq) & ((pk < prefix_len) | (pk > pq - window))


def visible_positions(p: int, prefix_len: int, window: int) -> np.ndarray:
    """All history positions a decode query at ``p`` sees, found by testing
    every j in [0, p]."""
    j = np.arange(p + 1, dtype=np.int64)
    return j[visible(p, j, prefix_len, window)]


def visible_count(p: int, prefix_len: int, window: int) -> int:
    """Number of keys a decode query at ``p`` sees (enumeration, not a formula)."""
    return int(visible_positions(p, prefix_len, window).size)


# --------------------------------------------------------------------------
# ring slots (bounded cache of L + W entries per sequence)
# --------------------------------------------------------------------------
def slot_of(n: int, prefix_len: int, window: int) -> int:
    """Ring slot that holds position ``n``: prefix positions sit in their own
    slot, window positions cycle through the W slots after the prefix."""
    if n < prefix_len:
        return int(n)
    return int(prefix_len + (n - prefix_len) % window)


def simulate_ring(positions: Sequence[int], prefix_len: int, window: int, capacity: int) -> np.ndarray:
    """Append ``positions`` in order into an empty ring; return, for every slot,
    the position it holds last (-1 when never written)."""
    ring = np.full(capacity, -1, dtype=np.int64)
    for n in positions:
        ring[slot_of(int(n), prefix_len, window)] = int(n)
    return ring


# --------------------------------------------------------------------------
# rotary embedding at the absolute position (Continue PE)
# --------------------------------------------------------------------------
def rope(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE in float64.  ``x`` is [..., D]; ``pos`` broadcasts
    against x.shape[:-1].  theta == 0 means "already rotated": identity."""
    x = np.asarray(x, dtype=np.float64)
    if not theta:
        return x.copy()
    d = x.shape[-1]
    half = d // 2
    inv_freq = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------
def _masked_softmax_rows(scores: np.ndarray, mask: np.ndarray):
    s = np.where(mask, scores, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=-1, keepdims=True)
    return e / z, (m + np.log(z))[..., 0]


def decode_attention(q: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray, p: int,
                     prefix_len: int, window: int, scale: float, theta: float) -> np.ndarray:
    """One decode query at absolute position ``p`` over the full history.

    q: raw query [Hq, D]; k_hist, v_hist: raw keys/values [>= p+1, Hkv, D] for
    positions 0..p (hidden positions included; the mask removes them).
    Returns [Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k_hist.shape[1]
    g = hq // hkv
    n = p + 1
    pos = np.arange(n, dtype=np.int64)
    qr = rope(q, p, theta)
    kr = rope(np.asarray(k_hist[:n], dtype=np.float64), pos[:, None], theta)
    v = np.asarray(v_hist[:n], dtype=np.float64)
    mask = visible(p, pos, prefix_len, window)
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        kv = h // g
        s = scale * (kr[:, kv, :] @ qr[h])
        w, _ = _masked_softmax_rows(s[None, :], mask[None, :])
        out[h] = w[0] @ v[:, kv, :]
    return out


def reset_pe_positions(p: int, prefix_len: int, window: int) -> Tuple[np.ndarray, np.ndarray]:
    """Reset PE numbering for a query at ``p`` (blog section "位置编码：Reset PE 还是
    Continue PE？"): the visible window tokens are renumbered so that they
    directly follow the prefix, oldest first (0-indexed: the prefix keeps
    0..L-1, the oldest visible window token becomes L).  Returns (visible
    absolute positions, their new positions); the query's new position is the
    last entry."""
    vis = visible_positions(p, prefix_len, window)
    pre = vis[vis < prefix_len]
    win = vis[vis >= prefix_len]
    return vis, np.concatenate([pre, prefix_len + np.arange(win.size, dtype=np.int64)])


def decode_attention_reset_pe(q: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray, p: int,
                              prefix_len: int, window: int, scale: float, theta: float) -> np.ndarray:
    """Decode at ``p`` with Reset PE: the same visible set as Continue PE, but
    every visible key and the query are rotated at their renumbered positions
    (``reset_pe_positions``) instead of their absolute ones.  Raw inputs as in
    ``decode_attention``; returns [Hq, D] float64."""
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k_hist.shape[1]
    g = hq // hkv
    vis, newpos = reset_pe_positions(p, prefix_len, window)
    assert vis[-1] == p
    qr = rope(q, newpos[-1], theta)
    kr = rope(np.asarray(k_hist[vis], dtype=np.float64), newpos[:, None], theta)
    v = np.asarray(v_hist[vis], dtype=np.float64)
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        kv = h // g
        s = scale * (kr[:, kv, :] @ qr[h])
        e = np.exp(s - s.max())
        out[h] = (e @ v[:, kv, :]) / e.sum()
    return out


def h2o_admit(heavy_pos: Sequence[int], heavy_score: Sequence[float], cand_pos: int, cand_score: float,
              capacity: int):
    """Heavy-hitter admission for a token leaving the window (the prefix +
    heavy-hitter + window combination the blog proposes in its comparison with
    H2O: keep, besides prefix and window, the middle tokens that have drawn the
    most attention so far).  Reading: the heavy set fills its ``capacity``
    slots in order; once full, the candidate replaces the member with the
    smallest accumulated score (ties: the oldest position) if its own score is
    strictly larger, else the candidate is dropped.  Returns (slot index the
    candidate is written to, or -1; evicted position, or -1)."""
    n = sum(1 for x in heavy_pos if x >= 0)
    if n < capacity:
        return n, -1
    m = min(range(capacity), key=lambda i: (heavy_score[i], heavy_pos[i]))
    if cand_score > heavy_score[m]:
        return m, int(heavy_pos[m])
    return -1, int(cand_pos)


def h2o_decode_trace(q: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray, prefix_len: int, window: int,
                     heavy: int, scale: float, theta: float):
    """Decode positions 0..N-1 of one sequence with prefix + heavy hitters +
    window, per KV head (the cache is per KV head).  Step p: the token p - W
    leaves the window and competes for the heavy set (``h2o_admit``) with its
    accumulated score; the query at p attends, under plain masked softmax, to
    the prefix, the heavy set and the window (p - W, p]; then every visible
    non-prefix token adds the attention it received, summed over the query
    heads of its KV head.  q: raw [N, Hq, D]; k_hist, v_hist: raw [N, Hkv, D].
    Returns (out [N, Hq, D], heavy positions [Hkv, heavy] (-1 empty),
    scores: list per KV head of dict position -> accumulated score)."""
    q = np.asarray(q, dtype=np.float64)
    n_steps, hq, d = q.shape
    hkv = k_hist.shape[1]
    g = hq // hkv
    pos_all = np.arange(n_steps, dtype=np.int64)
    kr = rope(np.asarray(k_hist, dtype=np.float64), pos_all[:, None], theta)
    v = np.asarray(v_hist, dtype=np.float64)
    out = np.empty((n_steps, hq, d), dtype=np.float64)
    heavy_pos = np.full((hkv, heavy), -1, dtype=np.int64)
    heavy_sc = np.zeros((hkv, heavy), dtype=np.float64)
    scores = [dict() for _ in range(hkv)]
    for p in range(n_steps):
        e = p - window
        for kv in range(hkv):
            if e >= prefix_len and heavy > 0:
                slot, dropped = h2o_admit(heavy_pos[kv], heavy_sc[kv], e, scores[kv][e], heavy)
                if slot >= 0:
                    heavy_pos[kv, slot] = e
                    heavy_sc[kv, slot] = scores[kv][e]
                if dropped >= 0:
                    scores[kv].pop(dropped)
            elif e >= prefix_len:
                scores[kv].pop(e)
            if p >= prefix_len:
                scores[kv][p] = 0.0
        qr = rope(q[p], p, theta)
        for kv in range(hkv):
            hp = heavy_pos[kv][heavy_pos[kv] >= 0]
            win = np.arange(max(prefix_len, p - window + 1), p + 1, dtype=np.int64)
            vis = np.concatenate([np.arange(min(prefix_len, p + 1), dtype=np.int64), hp, win])
            assert np.unique(vis).size == vis.size
            mass = np.zeros(vis.size)
            for h in range(kv * g, (kv + 1) * g):
                sc = scale * (kr[vis, kv, :] @ qr[h])
                w = np.exp(sc - sc.max())
                w /= w.sum()
                out[p, h] = w @ v[vis, kv, :]
                mass += w
            for j, m in zip(vis, mass):
                if j >= prefix_len:
                    scores[kv][int(j)] += m
            for i in range(heavy):
                if heavy_pos[kv, i] >= 0:
                    heavy_sc[kv, i] = scores[kv][int(heavy_pos[kv, i])]
    return out, heavy_pos, scores


def decode_from_slots(q: np.ndarray, p: int, k_rot: np.ndarray, v: np.ndarray, scale: float,
                      theta: float) -> np.ndarray:
    """Attention of a query at ``p`` over an explicit set of cached keys that are
    already rotated at their own positions (the ring's contents, in any
    order).  No mask: the cache holds exactly the visible keys."""
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k_rot.shape[1]
    g = hq // hkv
    qr = rope(q, p, theta)
    out = np.empty((hq, d), dtype=np.float64)
    for h in range(hq):
        kv = h // g
        s = scale * (np.asarray(k_rot[:, kv, :], dtype=np.float64) @ qr[h])
        e = np.exp(s - s.max())
        out[h] = (e @ np.asarray(v[:, kv, :], dtype=np.float64)) / e.sum()
    return out


def slot_attention_mass(q: np.ndarray, p: int, k_rot: np.ndarray, scale: float, theta: float) -> np.ndarray:
    """Attention mass each cached key draws from a query at ``p``: for every
    slot of an explicit set of keys already rotated at their own positions (as
    in ``decode_from_slots``), the softmax weight it receives, summed over the
    query heads that share its KV head -- the per-step increment of a token's
    heavy-hitter score (the prefix + heavy-hitter + window reading stated in
    ``h2o_decode_trace``).  q: raw [Hq, D]; k_rot: [n_slots, Hkv, D].
    Returns [n_slots, Hkv] float64; each column sums to Hq / Hkv."""
    q = np.asarray(q, dtype=np.float64)
    hq, d = q.shape
    hkv = k_rot.shape[1]
    g = hq // hkv
    qr = rope(q, p, theta)
    mass = np.zeros((k_rot.shape[0], hkv), dtype=np.float64)
    for h in range(hq):
        kv = h // g
        s = scale * (np.asarray(k_rot[:, kv, :], dtype=np.float64) @ qr[h])
        e = np.exp(s - s.max())
        mass[:, kv] += e / e.sum()
    return mass


def key_positions(nk: int, prefix_len: int, kv_start: int) -> np.ndarray:
    """Absolute positions of a prefill key array: [prefix 0..L-1][chunk from kv_start]."""
    k = np.arange(nk, dtype=np.int64)
    return np.where(k < prefix_len, k, kv_start + (k - prefix_len))


def prefill_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, prefix_len: int, window: int,
                      kv_start: int, scale: float, theta: float, rows=None):
    """Masked attention of a prefill chunk.

    q: raw [T, Hq, D]; k, v: raw [Nk, Hkv, D] with key positions from
    ``key_positions``; query t is key Nk - T + t.  ``rows`` optionally limits
    the evaluation to some query indices.  Returns (out [R, Hq, D],
    lse [R, Hq]) with lse the natural-log sum of exp of the scaled, masked
    scores."""
    q = np.asarray(q, dtype=np.float64)
    t_all, hq, d = q.shape
    nk, hkv, _ = k.shape
    g = hq // hkv
    posk = key_positions(nk, prefix_len, kv_start)
    posq_all = posk[nk - t_all:]
    rows = np.arange(t_all) if rows is None else np.asarray(rows, dtype=np.int64)
    posq = posq_all[rows]
    qr = rope(q[rows], posq[:, None], theta)
    kr = rope(np.asarray(k, dtype=np.float64), posk[:, None], theta)
    v = np.asarray(v, dtype=np.float64)
    mask = visible(posq[:, None], posk[None, :], prefix_len, window)
    out = np.empty((rows.size, hq, d), dtype=np.float64)
    lse = np.empty((rows.size, hq), dtype=np.float64)
    for h in range(hq):
        kv = h // g
        s = scale * (qr[:, h, :] @ kr[:, kv, :].T)
        w, l = _masked_softmax_rows(s, mask)
        out[:, h, :] = w @ v[:, kv, :]
        lse[:, h] = l
    return out, lse


def chunk_prefill_attention(q: np.ndarray, k_hist: np.ndarray, v_hist: np.ndarray, start: int,
                            prefix_len: int, window: int, scale: float, theta: float, rows=None):
    """A chunk of T new tokens continues a trace: query t sits at absolute
    position ``start + t`` and attends, under A(i), to the whole history
    0..start+t -- the earlier trace and the chunk up to itself.  Blog
    "Prefix Sliding 完全拆解", mask section (A(i) for every generated or
    appended token); the case arises when long external content is poured into
    a live trace (the blog's limitations section, multi-turn / tool output).

    q: raw [T, Hq, D]; k_hist, v_hist: raw [start + T, Hkv, D] (positions
    0..start+T-1, hidden ones included).  ``rows`` optionally limits the
    evaluation to some chunk queries.  Returns (out [R, Hq, D], lse [R, Hq])
    in float64."""
    q = np.asarray(q, dtype=np.float64)
    t_all, hq, d = q.shape
    n = start + t_all
    hkv = k_hist.shape[1]
    g = hq // hkv
    rows = np.arange(t_all) if rows is None else np.asarray(rows, dtype=np.int64)
    t_q = rows.size
    posq = start + rows
    posk = np.arange(n, dtype=np.int64)
    qr = rope(q[rows], posq[:, None], theta)
    kr = rope(np.asarray(k_hist[:n], dtype=np.float64), posk[:, None], theta)
    v = np.asarray(v_hist[:n], dtype=np.float64)
    mask = visible(posq[:, None], posk[None, :], prefix_len, window)
    out = np.empty((t_q, hq, d), dtype=np.float64)
    lse = np.empty((t_q, hq), dtype=np.float64)
    for h in range(hq):
        kv = h // g
        w, l = _masked_softmax_rows(scale * (qr[:, h, :] @ kr[:, kv, :].T), mask)
        out[:, h, :] = w @ v[:, kv, :]
        lse[:, h] = l
    return out, lse


def prefill_attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, d_out: np.ndarray,
                               prefix_len: int, window: int, kv_start: int, scale: float, theta: float):
    """Gradients of the masked prefill attention with respect to its raw
    inputs, for an upstream gradient ``d_out`` [T, Hq, D] (the truncated-backprop
    trainer of the blog's section "超长 rollouts 的反向传播：截断回传" back-propagates
    through the same masked attention; its loss mask only decides which rows
    of d_out are non-zero).

    Chain rule written out, per query head h with KV head g:
      S = scale * Q' K'^T (masked), P = softmax(S), O = P V
      dV_g += P^T dO;  dP = dO V^T;  dS = P * (dP - rowsum(P * dP))
      dQ' = scale * dS K';  dK'_g += scale * dS^T Q'
    and since Q' = R(pos) Q with R orthogonal, dQ = R(pos)^T dQ' (the rotation
    by -pos), likewise dK.  Returns (dq [T, Hq, D], dk [Nk, Hkv, D],
    dv [Nk, Hkv, D]) in float64."""
    q = np.asarray(q, dtype=np.float64)
    t_q, hq, d = q.shape
    nk, hkv, _ = k.shape
    g = hq // hkv
    posk = key_positions(nk, prefix_len, kv_start)
    posq = posk[nk - t_q:]
    qr = rope(q, posq[:, None], theta)
    kr = rope(np.asarray(k, dtype=np.float64), posk[:, None], theta)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(d_out, dtype=np.float64)
    mask = visible(posq[:, None], posk[None, :], prefix_len, window)
    dqr = np.zeros_like(qr)
    dkr = np.zeros_like(kr)
    dv = np.zeros_like(v)
    for h in range(hq):
        kv = h // g
        p, _ = _masked_softmax_rows(scale * (qr[:, h, :] @ kr[:, kv, :].T), mask)
        dv[:, kv, :] += p.T @ do[:, h, :]
        dp = do[:, h, :] @ v[:, kv, :].T
        ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
        dqr[:, h, :] = scale * (ds @ kr[:, kv, :])
        dkr[:, kv, :] += scale * (ds.T @ qr[:, h, :])
    dq = rope(dqr, -posq[:, None], theta)
    dk = rope(dkr, -posk[:, None], theta)
    return dq, dk, dv


def prefill_attention_backward_sampled(q: np.ndarray, k: np.ndarray, v: np.ndarray, d_out: np.ndarray,
                                       prefix_len: int, window: int, kv_start: int, scale: float, theta: float,
                                       kv_head: int, q_rows, k_rows, block: int = 512):
    """Selected rows of ``prefill_attention_backward`` at sizes where the full
    evaluation does not fit: dq rows ``q_rows`` of the query heads of KV head
    ``kv_head``, and dk / dv rows ``k_rows`` of that KV head.  The same chain
    rule, evaluated for those rows only; the per-query softmax statistics the
    key rows need are formed ``block`` queries at a time (each query row still
    over every key, masked).  Returns (dq [len(q_rows), G, D],
    dk [len(k_rows), D], dv [len(k_rows), D])."""
    q = np.asarray(q, dtype=np.float64)
    t_q, hq, d = q.shape
    nk, hkv, _ = k.shape
    g = hq // hkv
    heads = range(kv_head * g, (kv_head + 1) * g)
    posk = key_positions(nk, prefix_len, kv_start)
    posq = posk[nk - t_q:]
    kr = rope(np.asarray(k[:, kv_head], dtype=np.float64), posk, theta)
    vv = np.asarray(v[:, kv_head], dtype=np.float64)
    do = np.asarray(d_out, dtype=np.float64)
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    dq = np.zeros((q_rows.size, g, d))
    dkr = np.zeros((k_rows.size, d))
    dv = np.zeros((k_rows.size, d))
    for gi, h in enumerate(heads):
        qr = rope(q[:, h], posq, theta)
        for b0 in range(0, t_q, block):
            rows = np.arange(b0, min(t_q, b0 + block))
            mask = visible(posq[rows][:, None], posk[None, :], prefix_len, window)
            p, _ = _masked_softmax_rows(scale * (qr[rows] @ kr.T), mask)
            dp = do[rows, h] @ vv.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dv += p[:, k_rows].T @ do[rows, h]
            dkr += scale * (ds[:, k_rows].T @ qr[rows])
            sel = np.nonzero(np.isin(q_rows, rows))[0]
            for i in sel:
                dq[i, gi] = scale * (ds[q_rows[i] - b0] @ kr)
        dq[:, gi] = rope(dq[:, gi], -posq[q_rows], theta)
    return dq, rope(dkr, -posk[k_rows], theta), dv


# --------------------------------------------------------------------------
# prefill tile plan by element enumeration
# --------------------------------------------------------------------------
def tile_plan(t_q: int, nk: int, prefix_len: int, window: int, kv_start: int, bm: int, bn: int
              ) -> List[Tuple[int, int, int]]:
    """Every (q_tile, k_tile) of the BM x BN grid that holds at least one
    visible in-range (query, key) pair, in (q_tile, k_tile) order, with kind
    KIND_FULL when all BM*BN pairs exist and are visible, else KIND_PARTIAL."""
    posk = key_positions(nk, prefix_len, kv_start)
    posq = posk[nk - t_q:]
    n_qt = -(-t_q // bm)
    n_kt = -(-nk // bn)
    plan = []
    for qt in range(n_qt):
        q0, q1 = qt * bm, min(t_q, (qt + 1) * bm)
        vis = visible(posq[q0:q1, None], posk[None, :], prefix_len, window)  # [rows, nk]
        for kt in range(n_kt):
            k0, k1 = kt * bn, min(nk, (kt + 1) * bn)
            cnt = int(vis[:, k0:k1].sum())
            if cnt == 0:
                continue
            plan.append((qt, kt, KIND_FULL if cnt == bm * bn else KIND_PARTIAL))
    return plan


def visible_pairs(t_q: int, nk: int, prefix_len: int, window: int, kv_start: int) -> int:
    """Total visible (query, key) pairs of a prefill, by enumeration."""
    posk = key_positions(nk, prefix_len, kv_start)
    posq = posk[nk - t_q:]
    total = 0
    for s in range(0, t_q, 1024):
        total += int(visible(posq[s:s + 1024, None], posk[None, :], prefix_len, window).sum())
    return total
