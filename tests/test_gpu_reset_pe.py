"""GPU parity of Reset-PE decode against oracle.decode_attention_reset_pe,
through the C ABI, in both implementations: pe_mode PS_PE_RESET (cache filled
exactly as for Continue PE; only the scoring of prefix slots changes) and
PS_PE_RESET_RECOMPUTE (keys cached un-rotated and re-rotated at their
renumbered positions before every decode call; contiguous caches only).
Prefix lengths that are not multiples of 32 put the prefix end inside a key
chunk (scored with both query rotations in the first mode)."""
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
    return (synth.history(seed, cfg_id, synth.T_K, seq, 0, 0, n, hkv, d, std, dtype),
            synth.history(seed, cfg_id, synth.T_V, seq, 0, 0, n, hkv, d, std, dtype))


MODES = ["reset", "recompute"]


def _mode(ps, name):
    return ps.PS_PE_RESET if name == "reset" else ps.PS_PE_RESET_RECOMPUTE


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("splits", [1, 3])
def test_reset_pe_tiny_fp32_autoregressive(ps, splits, mode):
    c = synth.C1_DECODE
    attn = ps.AttnSpec(c.hq, c.hkv, c.dim, ps.PS_F32, c.rope_theta, 1 / math.sqrt(c.dim), pe_mode=_mode(ps, mode))
    cache = ps.CacheSpec(window=c.window, slot_capacity=128)
    steps = 400
    k, v = _hist(0, c.cfg_id, 0, steps, c.hkv, c.dim, c.kv_std, "f32")
    q = synth.history(0, c.cfg_id, synth.T_Q, 0, 0, 0, steps, c.hq, c.dim, c.q_std, "f32")
    kc, vc = new_cache(ps, attn, cache, 1)
    kd, vd, qd = to_dev(k, torch.float32), to_dev(v, torch.float32), to_dev(q, torch.float32)
    pl = torch.tensor([c.prefix], dtype=torch.int32, device="cuda")
    pos_all = torch.arange(steps, dtype=torch.int64, device="cuda")
    out = torch.empty((steps, c.hq, c.dim), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(ps.ps_decode_workspace_size(attn, cache, 1, splits), 1), dtype=torch.uint8, device="cuda")
    for p in range(steps):
        ps.ps_kv_append(attn, cache, kc, vc, pl, pos_all[p:p + 1], kd[p:p + 1].reshape(1, 1, c.hkv, c.dim),
                        vd[p:p + 1].reshape(1, 1, c.hkv, c.dim))
        ps.ps_decode_attn(attn, cache, kc, vc, pl, pos_all[p:p + 1], qd[p:p + 1], out[p:p + 1], num_splits=splits,
                          workspace=ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for p in range(steps):
        want = oracle.decode_attention_reset_pe(q[p], k, v, p, c.prefix, c.window, 1 / math.sqrt(c.dim),
                                                c.rope_theta)
        worst = max(worst, normwise_err(got[p], want))
    assert worst <= F32_TOL, worst


CASES = [  # (prefix, window, query positions)
    (5, 40, [0, 3, 44, 45, 46, 200, 1000]),
    (0, 33, [0, 32, 33, 34, 500]),
    (64, 64, [63, 127, 128, 129, 4000]),
    (100, 4096, [4195, 4196, 9000, 131072]),
    (37, 200, [10, 236, 237, 238, 5000]),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_reset_pe_bf16_small(ps, case, paged, mode):
    if paged and mode == "recompute":
        pytest.skip("the re-rotating mode takes contiguous caches only (PS_UNSUPPORTED, checked on the host)")
    L, W, positions = CASES[case]
    hq, hkv, d = 16, 2, 128
    n = len(positions)
    cap = -(-(L + W) // 64) * 64
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d), pe_mode=_mode(ps, mode))
    bt, num_pages = (None, 0)
    if paged:
        bt, num_pages = paged_table(n, cap // 64, seed=case)
    cache = ps.CacheSpec(window=W, slot_capacity=cap, page_size=64 if paged else 0, num_pages=num_pages)
    kc, vc = new_cache(ps, attn, cache, n)
    hist = [_hist(4, 70 + case, s, positions[s] + 1, hkv, d, 0.5, "bf16") for s in range(n)]
    fill_ring(ps, attn, cache, kc, vc, [L] * n, [p - 1 for p in positions], [h[0] for h in hist],
              [h[1] for h in hist], block_table=bt)
    kn = np.stack([h[0][p] for h, p in zip(hist, positions)])[:, None]
    vn = np.stack([h[1][p] for h, p in zip(hist, positions)])[:, None]
    pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
    pos = torch.tensor(positions, dtype=torch.int64, device="cuda")
    ps.ps_kv_append(attn, cache, kc, vc, pl, pos, to_dev(kn, torch.bfloat16), to_dev(vn, torch.bfloat16),
                    block_table=bt)
    q = np.stack([synth.query(4, 70 + case, s, 0, 0, hq, d, 1.0, "bf16") for s in range(n)])
    qd = to_dev(q, torch.bfloat16)
    for splits in sorted({sp for sp in (1, 2, 3, 0) if sp <= cap // 32}):
        out = torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda")
        ps.ps_decode_attn(attn, cache, kc, vc, pl, pos, qd, out, block_table=bt, num_splits=splits)
        got = out.float().cpu().numpy()
        for s in range(n):
            want = oracle.decode_attention_reset_pe(q[s], hist[s][0], hist[s][1], positions[s], L, W,
                                                    1 / math.sqrt(d), 10000.0)
            err = normwise_err(got[s], want)
            assert err <= BF16_TOL, (splits, s, positions[s], err)
