"""A CPU model of the bf16 backward's rounding, used to measure the error floor
that any bf16-operand implementation of the masked attention backward carries.

TEST INFRASTRUCTURE, NOT AN ORACLE.  The float64 oracle
(``oracle.prefill_attention_backward``) defines the gradients; this module
evaluates the same chain rule with the operands rounded to bf16 where a
bf16 matrix-core pipeline must round them, and float32 everywhere else:

  * the rotated keys K' and the rotated queries with the softmax scale and
    log2(e) folded in (Q'') are bf16 (they are MFMA operands);
  * P = exp2(Q'' K'^T - lse2) and dS = P (dP - Di) are formed in float32 and
    rounded to bf16 before they enter the dV, dK and dQ products;
  * dP = dO V^T, every product accumulation, Di = rowsum(dO * O) and the
    back-rotation by -position are float32; the outputs are rounded to bf16.

The forward output O and LSE it consumes are the oracle's, rounded to bf16 /
float32 (an ideal forward).  Its distance to the oracle is the floor below
which no kernel with these rounding points can go; the GPU tests hold the
kernel to max(1e-2, 1.25 x that floor).  It shares nothing with the HIP
path and is only imported by tests."""
from __future__ import annotations

import math

import numpy as np

import oracle
import synth

LOG2E = 1.4426950408889634


def _bf(x, on=True):
    return synth.round_to(x, "bf16") if on else np.asarray(x, dtype=np.float64)


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _operands(q, k, posq, posk, scale, theta, rnd):
    kr = _f32(_bf(oracle.rope(k, posk[:, None], theta), rnd))
    qs = _f32(_bf(oracle.rope(q, posq[:, None], theta) * (scale * LOG2E), rnd))
    return qs, kr


def backward(q, k, v, o, d_out, lse, prefix_len, window, kv_start, scale, theta, bf16=True):
    """Gradients (dq [T, Hq, D], dk, dv [Nk, Hkv, D], float64 holding bf16 values)
    of the masked prefill.  q, k, v, d_out: raw inputs (bf16 values); o: forward
    output [T, Hq, D] (bf16 values); lse: natural-log LSE [T, Hq].  bf16=False
    skips every rounding (the same chain rule in float32 throughout)."""
    t_q, hq, d = q.shape
    nk, hkv, _ = k.shape
    g = hq // hkv
    posk = oracle.key_positions(nk, prefix_len, kv_start)
    posq = posk[nk - t_q:]
    rnd = bf16
    qs, kr = _operands(np.asarray(q, np.float64), np.asarray(k, np.float64), posq, posk, scale, theta, rnd)
    vv, do = _f32(v), _f32(d_out)
    lse2 = _f32(np.asarray(lse, np.float64) * LOG2E)
    di = (do * _f32(o)).sum(axis=-1, dtype=np.float32)
    mask = oracle.visible(posq[:, None], posk[None, :], prefix_len, window)
    dqr = np.zeros((t_q, hq, d), np.float32)
    dkr = np.zeros((nk, hkv, d), np.float32)
    dvv = np.zeros((nk, hkv, d), np.float32)
    for h in range(hq):
        kv = h // g
        s = qs[:, h] @ kr[:, kv].T
        p = np.where(mask, np.exp2(s - lse2[:, h:h + 1]), np.float32(0)).astype(np.float32)
        dp = do[:, h] @ vv[:, kv].T
        ds = (p * (dp - di[:, h:h + 1])).astype(np.float32)
        pb, dsb = _f32(_bf(p, rnd)), _f32(_bf(ds, rnd))
        dvv[:, kv] += pb.T @ do[:, h]
        dkr[:, kv] += np.float32(math.log(2.0)) * (dsb.T @ qs[:, h])
        dqr[:, h] = np.float32(scale) * (dsb @ kr[:, kv])
    dq = _bf(oracle.rope(dqr.astype(np.float64), -posq[:, None], theta), rnd)
    dk = _bf(oracle.rope(dkr.astype(np.float64), -posk[:, None], theta), rnd)
    return dq, dk, _bf(dvv.astype(np.float64), rnd)


def backward_sampled(q, k, v, d_out, prefix_len, window, kv_start, scale, theta, kv_head, q_rows, k_rows,
                     block=512):
    """Selected rows of ``backward`` at sizes where the full evaluation does not
    fit (same selection as ``oracle.prefill_attention_backward_sampled``): dq
    rows ``q_rows`` of the query heads of ``kv_head`` [len(q_rows), G, D], dk / dv
    rows ``k_rows`` of that KV head [len(k_rows), D].  O and LSE of every query
    row of the group come from the oracle's forward, ``block`` rows at a time."""
    t_q, hq, d = q.shape
    nk, hkv, _ = k.shape
    g = hq // hkv
    heads = list(range(kv_head * g, (kv_head + 1) * g))
    posk = oracle.key_positions(nk, prefix_len, kv_start)
    posq = posk[nk - t_q:]
    kr = _f32(_bf(oracle.rope(np.asarray(k[:, kv_head], np.float64), posk, theta)))
    vv = _f32(v[:, kv_head])
    q_rows = np.asarray(q_rows, dtype=np.int64)
    k_rows = np.asarray(k_rows, dtype=np.int64)
    dq = np.zeros((q_rows.size, g, d), np.float32)
    dkr = np.zeros((k_rows.size, d), np.float32)
    dvv = np.zeros((k_rows.size, d), np.float32)
    for b0 in range(0, t_q, block):
        rows = np.arange(b0, min(t_q, b0 + block))
        o, lse = oracle.prefill_attention(q[:, heads], k[:, kv_head:kv_head + 1], v[:, kv_head:kv_head + 1],
                                          prefix_len, window, kv_start, scale, theta, rows=rows)
        mask = oracle.visible(posq[rows][:, None], posk[None, :], prefix_len, window)
        for gi, h in enumerate(heads):
            qs = _f32(_bf(oracle.rope(np.asarray(q[rows, h], np.float64), posq[rows], theta) * (scale * LOG2E)))
            do = _f32(d_out[rows, h])
            lse2 = _f32(lse[:, gi] * LOG2E)
            di = (do * _f32(_bf(o[:, gi]))).sum(axis=-1, dtype=np.float32)
            s = qs @ kr.T
            p = np.where(mask, np.exp2(s - lse2[:, None]), np.float32(0)).astype(np.float32)
            ds = (p * ((do @ vv.T) - di[:, None])).astype(np.float32)
            pb, dsb = _f32(_bf(p)), _f32(_bf(ds))
            dvv += pb[:, k_rows].T @ do
            dkr += np.float32(math.log(2.0)) * (dsb[:, k_rows].T @ qs)
            for i in np.nonzero(np.isin(q_rows, rows))[0]:
                dq[i, gi] = np.float32(scale) * (dsb[q_rows[i] - b0] @ kr)
    dq64 = np.stack([oracle.rope(dq[:, gi].astype(np.float64), -posq[q_rows], theta) for gi in range(g)], axis=1)
    return _bf(dq64), _bf(oracle.rope(dkr.astype(np.float64), -posk[k_rows], theta)), _bf(dvv.astype(np.float64))


def errors(got, want):
    """(worst row error against max(row max-norm, a tenth of the largest), error
    against the tensor's max-norm): the two gradient metrics of the tests."""
    g = np.asarray(got, dtype=np.float64).reshape(-1, want.shape[-1])
    w = np.asarray(want, dtype=np.float64).reshape(-1, want.shape[-1])
    big = np.abs(w).max()
    row = (np.abs(g - w).max(axis=1) / np.maximum(np.abs(w).max(axis=1), 0.1 * big)).max()
    return float(row), float(np.abs(g - w).max() / big)
