"""The decode step captured in a HIP graph (torch.cuda.CUDAGraph over the
library's launches on the capturing stream): every replay, with new inputs
copied in and eager work and synchronisations between replays, must give
bit-for-bit what the same calls give eagerly on a twin cache (same kernels,
same inputs).  The library allocates nothing, sets no memory with memset and
never synchronises, so a serving loop can capture whole decode steps."""
import math

import numpy as np
import pytest
import torch

from tests.gpu_common import require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ps():
    require_gpu()
    import bounded_kv_cache_amd as ps
    return ps


@pytest.mark.parametrize("mode,splits", [("decode", 1), ("decode", 3), ("step", 1), ("step", 3), ("heavy", 1),
                                         ("heavy", 2)])
def test_graph_replays_match_eager(ps, mode, splits):
    n, hq, hkv, d, L, W, H, layers, p0 = 6, 16, 2, 128, 10, 64, 24, 3, 200
    attn = ps.AttnSpec(hq, hkv, d, ps.PS_BF16, 10000.0, 1 / math.sqrt(d))
    cap = -(-(L + W + (H if mode == "heavy" else 0)) // 64) * 64
    cache = ps.CacheSpec(window=W, slot_capacity=cap)
    g = torch.Generator(device="cuda").manual_seed(7)
    ks, vs = ps.cache_shapes(attn, cache, n)
    pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
    # twin caches (graph / eager), filled with the same history through the bulk append
    hist_k = (torch.randn((n, p0, hkv, d), generator=g, device="cuda") * 0.5).bfloat16()
    hist_v = (torch.randn((n, p0, hkv, d), generator=g, device="cuda") * 0.5).bfloat16()
    caches = []
    for _ in range(2):
        per_layer = []
        for _ in range(layers):
            kc = torch.zeros(ks, dtype=torch.bfloat16, device="cuda")
            vc = torch.zeros(vs, dtype=torch.bfloat16, device="cuda")
            ps.ps_kv_append(attn, cache, kc, vc, pl, torch.zeros(n, dtype=torch.int64, device="cuda"), hist_k, hist_v)
            st = ps.HeavyState.new(attn, cache, n, H) if mode == "heavy" else None
            per_layer.append((kc, vc, st))
        caches.append(per_layer)
    if mode == "heavy":
        ws_need = ps.ps_heavy_workspace_size(attn, cache, n, splits)
    else:
        ws_need = ps.ps_decode_workspace_size(attn, cache, n, splits)
    ws = [torch.empty(max(ws_need, 1), dtype=torch.uint8, device="cuda") for _ in range(2)]
    q = [torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    kn = [torch.empty((n, 1, hkv, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    vn = [torch.empty((n, 1, hkv, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
    outs = [[torch.empty((n, hq, d), dtype=torch.bfloat16, device="cuda") for _ in range(layers)] for _ in range(2)]
    pos = [torch.full((n,), p0, dtype=torch.int64, device="cuda") for _ in range(2)]

    def step(c):
        for li in range(layers):
            kc, vc, st = caches[c][li]
            if mode == "heavy":
                ps.ps_heavy_decode_step(attn, cache, H, kc, vc, pl, pos[c], q[li], kn[li], vn[li], outs[c][li], st,
                                        num_splits=splits, workspace=ws[c])
            elif mode == "step":
                ps.ps_decode_step(attn, cache, kc, vc, pl, pos[c], q[li], kn[li], vn[li], outs[c][li],
                                  num_splits=splits, workspace=ws[c])
            else:
                ps.ps_kv_append(attn, cache, kc, vc, pl, pos[c], kn[li], vn[li])
                ps.ps_decode_attn(attn, cache, kc, vc, pl, pos[c], q[li], outs[c][li], num_splits=splits,
                                  workspace=ws[c])
        pos[c].add_(1)

    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(0)
    torch.cuda.synchronize()
    replays = 40 if mode == "heavy" else 6   # heavy: fill the heavy sets (24 slots), then replace members
    for r in range(replays):
        for li in range(layers):
            q[li].copy_(torch.randn((n, hq, d), generator=g, device="cuda").bfloat16())
            kn[li].copy_((torch.randn((n, 1, hkv, d), generator=g, device="cuda") * 0.5).bfloat16())
            vn[li].copy_((torch.randn((n, 1, hkv, d), generator=g, device="cuda") * 0.5).bfloat16())
        graph.replay()
        torch.cuda.synchronize()
        step(1)
        torch.cuda.synchronize()
        for li in range(layers):
            a_, b_ = outs[0][li].view(torch.int16), outs[1][li].view(torch.int16)
            assert torch.equal(a_, b_), (r, li)
        assert torch.equal(pos[0], pos[1])
    for li in range(layers):
        for x, y in zip(caches[0][li][:2], caches[1][li][:2]):
            assert torch.equal(x.view(torch.int16), y.view(torch.int16)), li
        if mode == "heavy":
            s0, s1 = caches[0][li][2], caches[1][li][2]
            assert torch.equal(s0.score, s1.score) and torch.equal(s0.heavy_count, s1.heavy_count)
            assert int(s0.heavy_count.min()) > 0
    assert np.isfinite(outs[0][0].float().cpu().numpy()).all()
