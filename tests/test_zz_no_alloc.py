"""ps_decode_step_noalloc (split partials in the library's static device
scratch, no workspace, nothing allocated) against ps_decode_step with a
workspace, through the C ABI: two calls in a row, the second with fewer
sequences, each bit-identical to the workspace entry point on a twin ring
(same kernels, same split count) and within the bf16 bound of the oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_common import BF16_TOL, fill_ring, new_cache, normwise_err, require_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    require_gpu()
    import bounded_kv_cache_amd as ps
    return ps


@pytest.mark.parametrize("splits", [3, 0])
def test_noalloc_step_matches_workspace_step(ps, splits):
    hq, hkv, d, L, W = 16, 2, 128, 37, 1000
    cap = -(-(L + W) // 64) * 64
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    cache = ps.CacheSpec(window=W, slot_capacity=cap)
    print(f"noalloc step: splits {splits}", flush=True)
    for call, starts in enumerate(([1500, 2048, 40, 999, 1037, 5000], [777, 3001, 12])):
        n = len(starts)
        hist = [(synth.history(6, 500 + call, synth.T_K, s, 0, 0, starts[s] + 1, hkv, d, 0.5, "bf16"),
                 synth.history(6, 500 + call, synth.T_V, s, 0, 0, starts[s] + 1, hkv, d, 0.5, "bf16"))
                for s in range(n)]
        q = np.stack([synth.query(6, 500 + call, s, 0, 0, hq, d, 1.0, "bf16") for s in range(n)])
        rings = [new_cache(ps, attn, cache, n) for _ in range(2)]
        for kc, vc in rings:
            fill_ring(ps, attn, cache, kc, vc, [L] * n, [p - 1 for p in starts], [h[0] for h in hist],
                      [h[1] for h in hist])
        pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
        pos = torch.tensor(starts, dtype=torch.int64, device="cuda")
        qd = to_dev(q, torch.bfloat16)
        kn = to_dev(np.stack([hist[s][0][starts[s]] for s in range(n)])[:, None], torch.bfloat16)
        vn = to_dev(np.stack([hist[s][1][starts[s]] for s in range(n)])[:, None], torch.bfloat16)
        outs = [torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
        ps.ps_decode_step(attn, cache, rings[0][0], rings[0][1], pl, pos, qd, kn, vn, outs[0], num_splits=splits)
        ps.ps_decode_step_noalloc(attn, cache, rings[1][0], rings[1][1], pl, pos, qd, kn, vn, outs[1],
                                  num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), call
        assert torch.equal(rings[0][0].view(torch.int16), rings[1][0].view(torch.int16))
        assert torch.equal(rings[0][1].view(torch.int16), rings[1][1].view(torch.int16))
        got = outs[1].float().cpu().numpy()
        for s in range(n):
            want = oracle.decode_attention(q[s], hist[s][0], hist[s][1], starts[s], L, W, 1 / math.sqrt(d), 10000.0)
            assert normwise_err(got[s], want) <= BF16_TOL, (call, s)
