"""Plants plausible mistakes in the oracle (on the CPU, through monkeypatching)
and checks that the pins catch each one."""
import numpy as np
import pytest

import oracle
import oracle.prefix_sliding as ops
from tests import test_oracle_pins as pins

PIN_CHECKS = [
    lambda: pins.test_visible_count_closed_form(3, 2),
    lambda: pins.test_visible_count_closed_form(16, 64),
    lambda: pins.test_pages_max_resident_tokens(),
    lambda: pins.test_prefill_reduces_to_reference_attention(40, 3, "full-prefix"),
    lambda: pins.test_prefill_reduces_to_reference_attention(3, 6, "ps"),
    lambda: pins.test_decode_reduces_to_reference_attention(4, 9),
    lambda: pins.test_decode_with_rope_matches_reference_on_complex_rotation(),
    lambda: pins.test_gqa_head_map_is_consecutive(),
    lambda: pins.test_rope_two_dims_is_plane_rotation(),
    lambda: pins.test_rope_frequencies_and_pairing(),
    lambda: pins.test_tile_plan_hand_worked_cases(),
    lambda: pins.test_zero_query_gives_mean_of_visible_values(4, 6),
    lambda: pins.test_chunk_reduces_to_reference_attention(3, 6, 25, 12),
    lambda: pins.test_chunk_rows_match_decode_with_rotation(),
    lambda: pins.test_chunk_zero_query_gives_mean_of_visible_values(3, 5, 40),
    lambda: pins.test_backward_matches_central_differences(3, 4, 3, 10000.0),
    lambda: pins.test_backward_matches_torch_autograd(4, 5),
    lambda: pins.test_backward_invariants_and_loss_mask_structure(),
    lambda: pins.test_reset_pe_numbering_hand_worked(),
    lambda: pins.test_reset_pe_against_explicit_rotation(),
    lambda: pins.test_reset_pe_reduces_to_continue_pe(3, 4, 20),
    lambda: pins.test_h2o_admission_hand_worked(),
    lambda: pins.test_h2o_zero_query_trace_hand_worked(),
    lambda: pins.test_h2o_reduces_to_prefix_sliding_and_full_attention(3, 5),
    lambda: pins.test_h2o_trace_invariants(),
    lambda: pins.test_slot_attention_mass_closed_forms(),
    lambda: pins.test_slot_attention_mass_against_outputs_and_trace_increments(),
]


def _window_off_by_one(pq, pk, L, W):
    pq, pk = np.asarray(pq), np.asarray(pk)
    return (pk <= pq) & ((pk < L) | (pk >= pq - W))


def _prefix_not_causal(pq, pk, L, W):
    pq, pk = np.asarray(pq), np.asarray(pk)
    return (pk < L) | ((pk <= pq) & (pk > pq - W))


def _prefix_inclusive(pq, pk, L, W):
    pq, pk = np.asarray(pq), np.asarray(pk)
    return (pk <= pq) & ((pk <= L) | (pk > pq - W))


def _rope_sign_flip(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    if not theta:
        return x.copy()
    d = x.shape[-1]
    h = d // 2
    f = float(theta) ** (-2.0 * np.arange(h) / d)
    a = np.asarray(pos, dtype=np.float64)[..., None] * f
    c, s = np.cos(a), np.sin(a)
    return np.concatenate([x[..., :h] * c + x[..., h:] * s, x[..., h:] * c - x[..., :h] * s], axis=-1)


def _rope_wrong_freq(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    if not theta:
        return x.copy()
    d = x.shape[-1]
    h = d // 2
    f = float(theta) ** (-1.0 * np.arange(h) / d)
    a = np.asarray(pos, dtype=np.float64)[..., None] * f
    c, s = np.cos(a), np.sin(a)
    return np.concatenate([x[..., :h] * c - x[..., h:] * s, x[..., h:] * c + x[..., :h] * s], axis=-1)


def _decode_interleaved_gqa(q, k_hist, v_hist, p, L, W, scale, theta):
    # maps query head h to KV head h % Hkv instead of h // G
    hkv = k_hist.shape[1]
    out = np.empty_like(np.asarray(q, dtype=np.float64))
    for h in range(q.shape[0]):
        kk = k_hist[:, [h % hkv], :]
        vv = v_hist[:, [h % hkv], :]
        out[h] = ORIG_DECODE(q[[h]], kk, vv, p, L, W, scale, theta)[0]
    return out


ORIG_DECODE = ops.decode_attention
ORIG_CHUNK = ops.chunk_prefill_attention


def _chunk_forgets_trace(q, k_hist, v_hist, start, L, W, scale, theta):
    # attends to the chunk alone, as if it started a new sequence
    return ORIG_CHUNK(q, k_hist[start:], v_hist[start:], 0, L, W, scale, theta)


def _chunk_query_one_early(q, k_hist, v_hist, start, L, W, scale, theta):
    # query t placed at start + t - 1 (its own key falls outside its view)
    s = max(start - 1, 0)
    return ORIG_CHUNK(q, k_hist[:s + q.shape[0]], v_hist[:s + q.shape[0]], s, L, W, scale, theta)

def _backward_with(bug):
    def f(q, k, v, d_out, L, W, kv_start, scale, theta):
        q = np.asarray(q, dtype=np.float64)
        t_q, hq, d = q.shape
        nk, hkv, _ = k.shape
        g = hq // hkv
        posk = ops.key_positions(nk, L, kv_start)
        posq = posk[nk - t_q:]
        qr, kr = ops.rope(q, posq[:, None], theta), ops.rope(k, posk[:, None], theta)
        mask = ops.visible(posq[:, None], posk[None, :], L, W)
        dqr, dkr, dv = np.zeros_like(qr), np.zeros_like(kr), np.zeros_like(np.asarray(v, dtype=np.float64))
        for h in range(hq):
            kv = h // g
            p, _ = ops._masked_softmax_rows(scale * (qr[:, h] @ kr[:, kv].T), mask)
            dv[:, kv] += p.T @ d_out[:, h]
            dp = d_out[:, h] @ np.asarray(v, dtype=np.float64)[:, kv].T
            ds = p * dp if bug == "no-rowsum" else p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dqr[:, h] = scale * (ds @ kr[:, kv])
            dkr[:, kv] += scale * (ds.T @ qr[:, h])
        if bug == "no-unrotate":
            return dqr, dkr, dv
        return ops.rope(dqr, -posq[:, None], theta), ops.rope(dkr, -posk[:, None], theta), dv
    return f


def _reset_pe_window_from_l_plus_one(p, L, W):
    vis = ops.visible_positions(p, L, W)
    pre, win = vis[vis < L], vis[vis >= L]
    return vis, np.concatenate([pre, L + 1 + np.arange(win.size, dtype=np.int64)])


def _reset_pe_not_renumbered(q, k_hist, v_hist, p, L, W, scale, theta):
    return ORIG_DECODE(q, k_hist, v_hist, p, L, W, scale, theta)


def _h2o_admit_on_tie(heavy_pos, heavy_score, cand_pos, cand_score, capacity):
    n = sum(1 for x in heavy_pos if x >= 0)
    if n < capacity:
        return n, -1
    m = min(range(capacity), key=lambda i: (heavy_score[i], heavy_pos[i]))
    if cand_score >= heavy_score[m]:
        return m, int(heavy_pos[m])
    return -1, int(cand_pos)


def _h2o_evict_newest(heavy_pos, heavy_score, cand_pos, cand_score, capacity):
    n = sum(1 for x in heavy_pos if x >= 0)
    if n < capacity:
        return n, -1
    m = min(range(capacity), key=lambda i: (heavy_score[i], -heavy_pos[i]))
    if cand_score > heavy_score[m]:
        return m, int(heavy_pos[m])
    return -1, int(cand_pos)


def _mass_with(bug):
    def f(q, p, k_rot, scale, theta):
        q = np.asarray(q, dtype=np.float64)
        hq, d = q.shape
        hkv = k_rot.shape[1]
        g = hq // hkv
        qr = q if bug == "unrotated-query" else ops.rope(q, p, theta)
        mass = np.zeros((k_rot.shape[0], hkv))
        for h in range(hq):
            kv = h % hkv if bug == "interleaved" else h // g
            s = scale * (k_rot[:, kv, :] @ qr[h])
            e = np.exp(s - s.max())
            mass[:, kv] += e / e.sum()
        return mass
    return f


MUTANTS = {
    "window-off-by-one": ("visible", _window_off_by_one),
    "prefix-not-causal": ("visible", _prefix_not_causal),
    "prefix-inclusive": ("visible", _prefix_inclusive),
    "rope-sign-flip": ("rope", _rope_sign_flip),
    "rope-wrong-frequency": ("rope", _rope_wrong_freq),
    "gqa-interleaved": ("decode_attention", _decode_interleaved_gqa),
    "chunk-forgets-trace": ("chunk_prefill_attention", _chunk_forgets_trace),
    "chunk-query-one-early": ("chunk_prefill_attention", _chunk_query_one_early),
    "backward-no-rowsum": ("prefill_attention_backward", _backward_with("no-rowsum")),
    "backward-no-unrotate": ("prefill_attention_backward", _backward_with("no-unrotate")),
    "reset-pe-window-from-L+1": ("reset_pe_positions", _reset_pe_window_from_l_plus_one),
    "reset-pe-not-renumbered": ("decode_attention_reset_pe", _reset_pe_not_renumbered),
    "h2o-admit-on-tie": ("h2o_admit", _h2o_admit_on_tie),
    "h2o-evict-newest": ("h2o_admit", _h2o_evict_newest),
    "mass-unrotated-query": ("slot_attention_mass", _mass_with("unrotated-query")),
    "mass-interleaved-heads": ("slot_attention_mass", _mass_with("interleaved")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ops, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    caught = 0
    for check in PIN_CHECKS:
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin caught mutant {name}"
