"""GPU parity of the masked prefill backward (ps_prefill_attn_backward) against
the float64 oracle (oracle.prefill_attention_backward), through the C ABI.

The forward output and LSE handed to the backward come from the oracle
(rounded to the kernel dtype), so the check isolates the backward kernels; one
test also runs the GPU forward into the GPU backward.

Tolerances (derived from the arithmetic; the pages fix none for gradients).
In bf16 the scaled, rotated queries and keys are bf16, so a score carries an
absolute error of about 2^-9 times its magnitude (a few units in log2 scale):
each probability is off by a few tenths of a percent.  The softmax gradient
dS = P (dP - Di) sums to zero over a row, so these per-probability errors do
not cancel -- they survive at that relative size against the terms, not
against the (smaller) result.  With the bf16 rounding of P and dS on top, a
gradient tensor is held to 2e-2 of its largest row's max-norm, and each row to
5e-2 of the larger of its own max-norm and a tenth of the largest (rows whose
exact gradient nearly cancels have no meaningful relative error).  The fp32
debug path: 1e-5 for both.  Rows that no gradient can reach (a zero upstream
row; keys no query with a non-zero upstream row sees) must be exactly zero."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import normwise_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu

BF16_ROW_TOL, BF16_TENSOR_TOL = 5e-2, 2e-2
F32_ROW_TOL, F32_TENSOR_TOL = 1e-5, 1e-5


@pytest.fixture(scope="module")
def ps():
    require_gpu()
    import bounded_kv_cache_amd as ps
    return ps


def _errs(got, want):
    """(worst row error against max(row max-norm, 0.1 * largest), error against the tensor's max-norm)"""
    g = np.asarray(got, dtype=np.float64).reshape(-1, want.shape[-1])
    w = np.asarray(want, dtype=np.float64).reshape(-1, want.shape[-1])
    big = np.abs(w).max()
    row = (np.abs(g - w).max(axis=1) / np.maximum(np.abs(w).max(axis=1), 0.1 * big)).max()
    return float(row), float(np.abs(g - w).max() / big)


def _structural_zero_rows(do, L, W, ks, nk):
    """dq rows with a zero upstream row; dk / dv rows of keys that no query with
    a non-zero upstream row can see (per KV head: any query head of the group)."""
    t_q = do.shape[0]
    live_q = np.abs(do).max(axis=-1) > 0                       # [T, Hq]
    posk = oracle.key_positions(nk, L, ks)
    posq = posk[nk - t_q:]
    vis = oracle.visible(posq[:, None], posk[None, :], L, W)   # [T, Nk]
    return ~live_q, vis, live_q


def _run(ps, dtype, hq, hkv, d, L, W, ks, T, chunk, batch=1, seed=0, loss_rows=None):
    dt_name = "bf16" if dtype == "bf16" else "f32"
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16 if dtype == "bf16" else ps.PS_F32, 10000.0, 1 / math.sqrt(d))
    nk = L + chunk
    rs = lambda tensor, b, n, h: synth.round_to(synth.normal((n, h, d), seed, 8, tensor, b), dt_name)
    q = np.stack([rs(synth.T_Q, b, T, hq) for b in range(batch)])
    k = np.stack([rs(synth.T_K, b, nk, hkv) for b in range(batch)])
    v = np.stack([rs(synth.T_V, b, nk, hkv) for b in range(batch)])
    do = np.stack([rs(synth.T_MISC, b, T, hq) for b in range(batch)])
    if loss_rows is not None:            # the trainer's loss mask: only the last rows carry gradient
        do[:, :T - loss_rows] = 0.0
    scale = 1 / math.sqrt(d)
    outs, lses, wants = [], [], []
    for b in range(batch):
        o, l = oracle.prefill_attention(q[b], k[b], v[b], L, W, ks, scale, 10000.0)
        outs.append(synth.round_to(o, dt_name))
        lses.append(l.T.astype(np.float32))            # [Hq, T]
        wants.append(oracle.prefill_attention_backward(q[b], k[b], v[b], do[b], L, W, ks, scale, 10000.0))
    dq = torch.full((batch, T, hq, d), float("nan"), dtype=tdt, device="cuda")
    dk = torch.full((batch, nk, hkv, d), float("nan"), dtype=tdt, device="cuda")
    dv = torch.full((batch, nk, hkv, d), float("nan"), dtype=tdt, device="cuda")
    ps.ps_prefill_attn_backward(attn, W, L, ks, to_dev(q, tdt), to_dev(k, tdt), to_dev(v, tdt),
                                to_dev(np.stack(outs), tdt), to_dev(do, tdt),
                                torch.from_numpy(np.ascontiguousarray(np.stack(lses))).cuda(), dq, dk, dv)
    torch.cuda.synchronize()
    got = [x.float().cpu().numpy() for x in (dq, dk, dv)]
    row_tol, ten_tol = (BF16_ROW_TOL, BF16_TENSOR_TOL) if dtype == "bf16" else (F32_ROW_TOL, F32_TENSOR_TOL)
    worst = {}
    for b in range(batch):
        for name, g, w in zip(("dq", "dk", "dv"), got, wants[b]):
            assert np.isfinite(g[b]).all(), name
            r, tn = _errs(g[b], w)
            worst[name] = max(worst.get(name, (0, 0))[0], r), max(worst.get(name, (0, 0))[1], tn)
            assert r <= row_tol and tn <= ten_tol, (name, b, r, tn)
        dead_q, vis, live_q = _structural_zero_rows(do[b], L, W, ks, nk)
        assert np.all(got[0][b][dead_q] == 0.0)
        g = hq // hkv
        for kv in range(hkv):
            seen = (vis[:, :, None] & live_q[:, None, kv * g:(kv + 1) * g]).any(axis=(0, 2))
            assert np.all(got[1][b][~seen, kv] == 0.0) and np.all(got[2][b][~seen, kv] == 0.0)
    print("backward errors (row, tensor):", worst, flush=True)
    return worst


CASES = [
    # hq, hkv, d, L, W, kv_start, T, chunk, batch
    (8, 2, 128, 20, 64, 500, 300, 300, 2),        # queries = the chunk, band + pinned keys
    (4, 1, 64, 16, 64, 16, 216, 200, 1),          # queries reach into the prefix (T = Nk)
    (28, 4, 128, 100, 256, 5000, 400, 400, 1),    # truncated-backprop shape, small
    (8, 2, 128, 0, 1 << 30, 0, 257, 257, 1),      # full causal comparator, ragged tail
    (16, 2, 128, 37, 130, 37, 190, 300, 1),       # queries are the last 190 of 300 chunk keys
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_bf16_matches_oracle(ps, case):
    hq, hkv, d, L, W, ks, T, chunk, batch = CASES[case]
    print(f"backward bf16 case {case}: Hq={hq} Hkv={hkv} D={d} L={L} W={W} kv_start={ks} T={T} chunk={chunk}",
          flush=True)
    _run(ps, "bf16", hq, hkv, d, L, W, ks, T, chunk, batch, seed=case)


@pytest.mark.parametrize("case", [0, 1, 4])
def test_backward_fp32_matches_oracle(ps, case):
    hq, hkv, d, L, W, ks, T, chunk, batch = CASES[case]
    print(f"backward fp32 case {case}", flush=True)
    _run(ps, "f32", hq, hkv, d, L, W, ks, T, chunk, batch, seed=20 + case)


def test_backward_loss_mask_on_last_window(ps):
    # the trainer's rule: 4W tokens in, loss on the last W -> gradient rows only there
    W = 64
    print("backward loss mask", flush=True)
    _run(ps, "bf16", 8, 2, 128, 24, W, 1000, 4 * W, 4 * W, 1, seed=7, loss_rows=W)


def test_forward_then_backward_pipeline(ps):
    # the product path: the GPU forward's output and LSE feed the GPU backward
    hq, hkv, d, L, W, ks, T, chunk = 28, 4, 128, 100, 512, 9000, 640, 700
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16)
    nk = L + chunk
    rs = lambda tensor, n, h: synth.round_to(synth.normal((n, h, d), 3, 8, tensor, 0), "bf16")
    q, k, v, do = rs(synth.T_Q, T, hq), rs(synth.T_K, nk, hkv), rs(synth.T_V, nk, hkv), rs(synth.T_MISC, T, hq)
    qd, kd, vd, dod = (to_dev(x[None], torch.bfloat16) for x in (q, k, v, do))
    out = torch.empty_like(qd)
    lse = torch.empty((1, hq, T), dtype=torch.float32, device="cuda")
    ps.ps_prefill_attn(attn, W, L, ks, qd, kd, vd, out, lse=lse)
    dq, dk, dv = torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd)
    ps.ps_prefill_attn_backward(attn, W, L, ks, qd, kd, vd, out, dod, lse, dq, dk, dv)
    torch.cuda.synchronize()
    want = oracle.prefill_attention_backward(q, k, v, do, L, W, ks, 1 / math.sqrt(d), 10000.0)
    for name, g, w in zip(("dq", "dk", "dv"), (dq, dk, dv), want):
        r, tn = _errs(g[0].float().cpu().numpy(), w)
        print(name, r, tn, flush=True)
        assert r <= BF16_ROW_TOL and tn <= BF16_TENSOR_TOL, (name, r, tn)
