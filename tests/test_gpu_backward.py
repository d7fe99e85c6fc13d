"""GPU parity of the masked prefill backward (ps_prefill_attn_backward) against
the float64 oracle (oracle.prefill_attention_backward), through the C ABI.

The forward output and LSE handed to the backward come from the oracle
(rounded to the kernel dtype), so the check isolates the backward kernels; one
test also runs the GPU forward into the GPU backward.

Tolerances.  The pages fix none for gradients; the contract's bf16 bound is
1e-2.  Two metrics per gradient tensor: the largest row error against the
larger of the row's max-norm and a tenth of the tensor's (rows whose exact
gradient nearly cancels have no meaningful relative error), and the largest
error against the tensor's max-norm.  A bf16 pipeline cannot reach 1e-2 on
every input: tests/bf16_backward_model.py evaluates the same chain rule with
the operands rounded to bf16 where the kernels round them (rotated query and
key, P and dS; float32 elsewhere) on exact forward statistics, and its
distance to the oracle -- the floor -- exceeds 1e-2 on some of these cases
(tests/test_bf16_backward_floor.py shows it comes from the rounded query and
key).  Each case therefore holds the kernel to max(1e-2, 1.25 x the floor
measured on that case's own inputs), per tensor and metric; a floor above
1.5e-2 fails the test (the model would be wrong).  The fp32 debug path: 1e-5
for both.  Rows that no gradient can reach (a zero upstream row; keys no query
with a non-zero upstream row sees) must be exactly zero."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import bf16_backward_model as model
from tests.gpu_common import normwise_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu

BF16_TOL, FLOOR_FACTOR, FLOOR_MAX = 1e-2, 1.25, 1.5e-2
F32_ROW_TOL, F32_TENSOR_TOL = 1e-5, 1e-5


def bf16_tolerances(floor_row, floor_tensor):
    """max(1e-2, 1.25 x the bf16 model's floor) for each metric."""
    assert floor_row <= FLOOR_MAX and floor_tensor <= FLOOR_MAX, (floor_row, floor_tensor)
    return max(BF16_TOL, FLOOR_FACTOR * floor_row), max(BF16_TOL, FLOOR_FACTOR * floor_tensor)


@pytest.fixture(scope="module")
def ps():
    require_gpu()
    import bounded_kv_cache_amd as ps
    return ps


_errs = model.errors


def _structural_zero_rows(do, L, W, ks, nk):
    """dq rows with a zero upstream row; dk / dv rows of keys that no query with
    a non-zero upstream row can see (per KV head: any query head of the group)."""
    t_q = do.shape[0]
    live_q = np.abs(do).max(axis=-1) > 0                       # [T, Hq]
    posk = oracle.key_positions(nk, L, ks)
    posq = posk[nk - t_q:]
    vis = oracle.visible(posq[:, None], posk[None, :], L, W)   # [T, Nk]
    return ~live_q, vis, live_q


def _run(ps, dtype, hq, hkv, d, L, W, ks, T, chunk, batch=1, seed=0, loss_rows=None, keep_ds=None):
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
    outs, lses, wants, floors = [], [], [], []
    for b in range(batch):
        o, l = oracle.prefill_attention(q[b], k[b], v[b], L, W, ks, scale, 10000.0)
        outs.append(synth.round_to(o, dt_name))
        lses.append(l.T.astype(np.float32))            # [Hq, T]
        wants.append(oracle.prefill_attention_backward(q[b], k[b], v[b], do[b], L, W, ks, scale, 10000.0))
        if dtype == "bf16":   # what an ideal bf16 pipeline reaches on these inputs
            ideal = model.backward(q[b], k[b], v[b], outs[-1], do[b], lses[-1].T, L, W, ks, scale, 10000.0)
            floors.append([_errs(x, w) for x, w in zip(ideal, wants[-1])])
    dq = torch.full((batch, T, hq, d), float("nan"), dtype=tdt, device="cuda")
    dk = torch.full((batch, nk, hkv, d), float("nan"), dtype=tdt, device="cuda")
    dv = torch.full((batch, nk, hkv, d), float("nan"), dtype=tdt, device="cuda")
    ps.ps_prefill_attn_backward(attn, W, L, ks, to_dev(q, tdt), to_dev(k, tdt), to_dev(v, tdt),
                                to_dev(np.stack(outs), tdt), to_dev(do, tdt),
                                torch.from_numpy(np.ascontiguousarray(np.stack(lses))).cuda(), dq, dk, dv,
                                keep_ds=keep_ds)
    torch.cuda.synchronize()
    got = [x.float().cpu().numpy() for x in (dq, dk, dv)]
    worst = {}
    for b in range(batch):
        for i, (name, g, w) in enumerate(zip(("dq", "dk", "dv"), got, wants[b])):
            assert np.isfinite(g[b]).all(), name
            r, tn = _errs(g[b], w)
            if dtype == "bf16":
                row_tol, ten_tol = bf16_tolerances(*floors[b][i])
                print(f"{name} batch {b}: error (row, tensor) ({r:.4f}, {tn:.4f}), bf16 floor "
                      f"({floors[b][i][0]:.4f}, {floors[b][i][1]:.4f})", flush=True)
            else:
                row_tol, ten_tol = F32_ROW_TOL, F32_TENSOR_TOL
            worst[name] = max(worst.get(name, (0, 0))[0], r), max(worst.get(name, (0, 0))[1], tn)
            assert r <= row_tol and tn <= ten_tol, (name, b, r, tn, row_tol, ten_tol)
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


@pytest.mark.parametrize("keep_ds", [True, False], ids=["kept_ds", "recomputed_ds"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_backward_bf16_matches_oracle(ps, case, keep_ds):
    # kept_ds: the dk/dv pass stores its dS tiles and the dq pass reads them;
    # recomputed_ds: the dq pass forms S and dP again (workspace without the dS room)
    hq, hkv, d, L, W, ks, T, chunk, batch = CASES[case]
    print(f"backward bf16 case {case} keep_ds={keep_ds}: Hq={hq} Hkv={hkv} D={d} L={L} W={W} kv_start={ks} "
          f"T={T} chunk={chunk}", flush=True)
    _run(ps, "bf16", hq, hkv, d, L, W, ks, T, chunk, batch, seed=case, keep_ds=keep_ds)


@pytest.mark.parametrize("case", [0, 3, 4])
def test_backward_kept_ds_agrees_with_recomputed(ps, case):
    # the two dq paths share the dk/dv pass: dk and dv are bitwise equal; dq may
    # differ where an fp32 sum in another order rounds a dS element differently
    hq, hkv, d, L, W, ks, T, chunk, batch = CASES[case]
    print(f"backward kept vs recomputed dS, case {case}", flush=True)
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    nk = L + chunk
    g = torch.Generator(device="cuda").manual_seed(40 + case)
    q = torch.randn((batch, T, hq, d), generator=g, device="cuda").bfloat16()
    k = torch.randn((batch, nk, hkv, d), generator=g, device="cuda").bfloat16()
    v = torch.randn((batch, nk, hkv, d), generator=g, device="cuda").bfloat16()
    do = torch.randn_like(q)
    out = torch.empty_like(q)
    lse = torch.empty((batch, hq, T), dtype=torch.float32, device="cuda")
    ps.ps_prefill_attn(attn, W, L, ks, q, k, v, out, lse=lse)
    res = []
    for keep in (True, False):
        grads = [torch.empty_like(x) for x in (q, k, v)]
        ps.ps_prefill_attn_backward(attn, W, L, ks, q, k, v, out, do, lse, *grads, keep_ds=keep)
        res.append([x.float() for x in grads])
    torch.cuda.synchronize()
    assert torch.equal(res[0][1], res[1][1]) and torch.equal(res[0][2], res[1][2])
    dq_k, dq_r = res[0][0], res[1][0]
    diff = float((dq_k - dq_r).norm() / dq_r.norm())
    print("dq relative (Frobenius) difference between the paths:", diff, flush=True)
    assert diff <= 2e-3, diff


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
    scale = 1 / math.sqrt(d)
    want = oracle.prefill_attention_backward(q, k, v, do, L, W, ks, scale, 10000.0)
    o_ref, l_ref = oracle.prefill_attention(q, k, v, L, W, ks, scale, 10000.0)
    ideal = model.backward(q, k, v, synth.round_to(o_ref, "bf16"), do, l_ref.astype(np.float32), L, W, ks, scale,
                           10000.0)
    for name, g, w, x in zip(("dq", "dk", "dv"), (dq, dk, dv), want, ideal):
        r, tn = _errs(g[0].float().cpu().numpy(), w)
        fr, ft = _errs(x, w)
        print(name, r, tn, "floor", fr, ft, flush=True)
        row_tol, ten_tol = bf16_tolerances(fr, ft)
        assert r <= row_tol and tn <= ten_tol, (name, r, tn, row_tol, ten_tol)
