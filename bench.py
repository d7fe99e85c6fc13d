#!/usr/bin/env python3
"""Benchmark of the Prefix Sliding hot path on one MI355X.

Workload (default): decode at position 131072 with a 100-token prefix and a
4096-token window -- 256 sequences, 28 layers, Hq=16, Hkv=2, head_dim=128,
bf16 (a Qwen3-1.7B attention geometry).  One step = for every layer,
ps_decode_step: append the new token's K/V (RoPE at its absolute position)
into the ring and run split-KV decode attention over it, one launch.  Timed:
K steps after W warm-up steps, inputs resident in HBM, positions advancing by
one per step.

Printed (one JSON line): whole-job decode tok/s, the roofline of the decode
step kernel (algorithmic HBM bytes per launch / average launch time,
against 8 TB/s), the float64 CPU oracle timed on a bounded sample of the
same workload, the masked prefill kernel (truncated-backprop chunk: 8 x 8192
queries behind a 100-token prefix, W=2048, Hq=28, Hkv=4) in TFLOP/s against
the 2.5 PFLOP/s bf16 MFMA peak, the chunk prefill that reads the ring (64
rings at 32768, a 2048-token chunk each), and the full-attention decode
comparator at the same position.  Next to the published peaks it measures
this GPU's own ceilings: HBM read bandwidth of a plain streaming read (the
library's probe), torch's copy bandwidth, and the bf16 rate of the vendor GEMM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "prefix-sliding decode-attn tok/s & HBM GB/s %peak, W=4096 @128K pos"
COUNTERS = os.path.join(ROOT, "profiles", "decode_bf16_128k_w4096_counters.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--window", type=int, default=4096)
    ap.add_argument("--position", type=int, default=131072)
    ap.add_argument("--num-seqs", type=int, default=256)
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--splits", type=int, default=0, help="decode splits (0: library's automatic choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-full", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the decode position sweep (flatness)")
    ap.add_argument("--no-extra", action="store_true", help="skip the other decode workloads")
    ap.add_argument("--no-chunk", action="store_true", help="skip the chunk prefill that reads the ring")
    ap.add_argument("--no-backward", action="store_true", help="skip the masked prefill backward")
    ap.add_argument("--no-heavy", action="store_true", help="skip prefix + heavy hitters + window decoding")
    ap.add_argument("--only", choices=["decode", "prefill", "chunk", "backward", "heavy", "batch-sweep"],
                    default=None,
                    help="run only one leg (for profiling); the JSON line then carries that leg only")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="run one device-to-device copy of BYTES first (reference for HBM counter scaling)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("decode.hip", "ps_common.h", "ps_internal.h"):
        with open(os.path.join(ROOT, "bounded_kv_cache_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------------- decode
class DecodeBench:
    def __init__(self, ps, torch, num_seqs, layers, window, prefix, position, splits, pool=16, seed=0):
        self.ps, self.torch = ps, torch
        self.n, self.layers, self.splits = num_seqs, layers, splits
        self.attn = ps.AttnSpec(16, 2, 128, ps.PS_BF16, 10000.0, 1 / math.sqrt(128))
        cap = -(-min(prefix + window, position + 4096) // 64) * 64
        self.cache = ps.CacheSpec(window=window, slot_capacity=cap)
        self.prefix, self.position, self.window = prefix, position, window
        g = torch.Generator(device="cuda").manual_seed(seed)
        ks, vs = ps.cache_shapes(self.attn, self.cache, num_seqs)
        self.k = [torch.empty(ks, dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
        self.v = [torch.empty(vs, dtype=torch.bfloat16, device="cuda") for _ in range(layers)]
        self.pl = torch.full((num_seqs,), prefix, dtype=torch.int32, device="cuda")
        # rings hold A(position - 1): prefix tokens, then the last window tokens, appended in bulk
        n_pre = min(prefix, position)
        w_start = max(prefix, position - window)
        n_win = position - w_start
        chunk = max(n_pre, n_win, 1)
        kn = (torch.randn((num_seqs, chunk, 2, 128), generator=g, device="cuda") * 0.5).bfloat16()
        vn = (torch.randn((num_seqs, chunk, 2, 128), generator=g, device="cuda") * 0.5).bfloat16()
        for li in range(layers):
            if n_pre:
                ps.ps_kv_append(self.attn, self.cache, self.k[li], self.v[li], self.pl,
                                torch.zeros(num_seqs, dtype=torch.int64, device="cuda"),
                                kn[:, :n_pre].contiguous(), vn[:, :n_pre].contiguous())
            if n_win:
                ps.ps_kv_append(self.attn, self.cache, self.k[li], self.v[li], self.pl,
                                torch.full((num_seqs,), w_start, dtype=torch.int64, device="cuda"),
                                kn[:, :n_win].contiguous(), vn[:, :n_win].contiguous())
        del kn, vn
        self.pool = pool
        self.q = [torch.randn((num_seqs, 16, 128), generator=g, device="cuda").bfloat16() for _ in range(pool)]
        self.kn = [(torch.randn((num_seqs, 1, 2, 128), generator=g, device="cuda") * 0.5).bfloat16()
                   for _ in range(pool)]
        self.vn = [(torch.randn((num_seqs, 1, 2, 128), generator=g, device="cuda") * 0.5).bfloat16()
                   for _ in range(pool)]
        self.out = torch.empty((num_seqs, 16, 128), dtype=torch.bfloat16, device="cuda")
        ws = ps.ps_decode_workspace_size(self.attn, self.cache, num_seqs, splits)
        self.ws = torch.empty(max(ws, 1), dtype=torch.uint8, device="cuda")
        self.max_steps = 0
        self.pos = None

    def prepare_positions(self, total_steps):
        t = self.torch
        self.pos = [t.full((self.n,), self.position + s, dtype=t.int64, device="cuda") for s in range(total_steps)]

    def step(self, s):
        ps = self.ps
        pos = self.pos[s]
        for li in range(self.layers):
            i = (s * self.layers + li) % self.pool
            ps.ps_decode_step(self.attn, self.cache, self.k[li], self.v[li], self.pl, pos, self.q[i], self.kn[i],
                              self.vn[i], self.out, num_splits=self.splits, workspace=self.ws)

    def decode_only(self, reps, pos):
        ps = self.ps
        for r in range(reps):
            ps.ps_decode_attn(self.attn, self.cache, self.k[0], self.v[0], self.pl, pos, self.q[r % self.pool],
                              self.out, num_splits=self.splits, workspace=self.ws)

    def n_vis(self, p):
        return min(p + 1, self.prefix + self.window)

    def kernel_bytes(self, p):
        """Algorithmic HBM bytes of one decode-attention launch (one layer): the
        visible K/V rows, the queries and the outputs."""
        return self.n * (self.n_vis(p) * 2 * 128 * 2 * 2 + 16 * 128 * 2 * 2)

    def step_kernel_bytes(self, p):
        """Algorithmic HBM bytes of one decode-step launch (one layer): the
        attention's bytes plus the new token's K and V, read and written."""
        return self.kernel_bytes(p) + self.n * 2 * 2 * 128 * 2 * 2

    def release(self):
        self.k.clear()
        self.v.clear()


def timed(torch, fn, iters):
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    fn(iters)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1000.0


def time_decode_steps(bench, torch, steps, warmup, reps=5):
    """The timing protocol: the rings and positions of every layer are
    snapshotted once; each rep restores them (untimed), then runs `steps`
    decode steps (28 ps_decode_step launches each) between two HIP events on
    the launch stream, bracketed by device synchronisation.  One warm-up rep
    (which also runs `warmup` untimed steps first) is discarded; the median of
    `reps` timed reps is returned, with every rep's time."""
    snap_k = [k.clone() for k in bench.k]
    snap_v = [v.clone() for v in bench.v]

    def restore():
        for dst, src in zip(bench.k, snap_k):
            dst.copy_(src)
        for dst, src in zip(bench.v, snap_v):
            dst.copy_(src)
        torch.cuda.synchronize()

    times = []
    for rep in range(reps + 1):
        restore()
        if rep == 0:
            for s in range(warmup):
                bench.step(s)
            torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for s in range(steps):
            bench.step(s)
        end.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        if rep > 0:
            times.append(max(wall, start.elapsed_time(end) / 1000.0))
    restore()
    del snap_k, snap_v
    return sorted(times)[len(times) // 2], times


def run_decode(ps, torch, args, num_seqs=None, position=None, window=None, graph=True):
    n = num_seqs or args.num_seqs
    p0 = position or args.position
    w = window or args.window
    bench = DecodeBench(ps, torch, n, args.layers, w, 100, p0, args.splits)
    bench.prepare_positions(max(args.warmup, args.steps))
    splits = args.splits or ps.ps_decode_num_splits(bench.attn, bench.cache, n)
    med, times = time_decode_steps(bench, torch, args.steps, args.warmup)
    launches = args.steps * bench.layers
    # the dominant kernel: every launch of the timed loop is one decode-step
    # kernel (append fused); its average launch duration is the timed loop's
    # time over its launches (an upper bound: launch gaps are included)
    kt = med / launches
    p_last = p0 + args.steps - 1
    kbytes = bench.step_kernel_bytes(p_last)
    res = {
        "tok_s": n * args.steps / med,
        "ms_per_step": med / args.steps * 1000.0,
        "rep_ms": [t * 1000.0 for t in times],
        "splits": splits,
        "kernel_s": kt,
        "kernel_launches": launches,
        "kernel_bytes": kbytes,
        "n_vis": bench.n_vis(p_last),
    }
    if graph:
        # the same step captured once in a HIP graph (28 decode steps, then the
        # positions advance inside the graph) and replayed: what a serving loop
        # that captures its decode step would see
        gpos = bench.pos[args.steps - 1].clone()

        def graph_step():
            for li in range(bench.layers):
                i = li % bench.pool
                ps.ps_decode_step(bench.attn, bench.cache, bench.k[li], bench.v[li], bench.pl, gpos, bench.q[i],
                                  bench.kn[i], bench.vn[i], bench.out, num_splits=bench.splits, workspace=bench.ws)
            gpos.add_(1)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            graph_step()
        for _ in range(2):
            g.replay()
        g_s = timed(torch, lambda k: [g.replay() for _ in range(k)], args.steps)
        del g
        res["graph_tok_s"] = n * args.steps / g_s
        res["graph_ms_per_step"] = g_s / args.steps * 1000.0
    bench.release()
    del bench
    torch.cuda.empty_cache()
    return res


def run_full_attention(ps, torch, args, steps=2):
    """Full-attention comparator at the same position: the same decode kernel
    with W >= n over a linear cache of the whole history.  One layer's buffer
    (34 GB at 256 x 131073 slots) is launched once per layer."""
    n, p = args.num_seqs, args.position
    attn = ps.AttnSpec(16, 2, 128, ps.PS_BF16, 10000.0, 1 / math.sqrt(128))
    cap = -(-(p + steps + 1) // 64) * 64
    cache = ps.CacheSpec(window=1 << 30, slot_capacity=cap)
    ks, vs = ps.cache_shapes(attn, cache, n)
    k = torch.empty(ks, dtype=torch.bfloat16, device="cuda")
    v = torch.empty(vs, dtype=torch.bfloat16, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(7)
    k.normal_(0.0, 0.5, generator=g)
    v.normal_(0.0, 0.5, generator=g)
    pl = torch.zeros(n, dtype=torch.int32, device="cuda")
    q = torch.randn((n, 16, 128), generator=g, device="cuda").bfloat16()
    kn = (torch.randn((n, 1, 2, 128), generator=g, device="cuda") * 0.5).bfloat16()
    vn = (torch.randn((n, 1, 2, 128), generator=g, device="cuda") * 0.5).bfloat16()
    out = torch.empty((n, 16, 128), dtype=torch.bfloat16, device="cuda")
    splits = ps.ps_decode_num_splits(attn, cache, n)
    ws = torch.empty(max(ps.ps_decode_workspace_size(attn, cache, n, 0), 1), dtype=torch.uint8, device="cuda")
    pos = [torch.full((n,), p + s, dtype=torch.int64, device="cuda") for s in range(steps + 1)]

    def one_step(s):
        for _ in range(args.layers):
            ps.ps_kv_append(attn, cache, k, v, pl, pos[s], kn, vn)
            ps.ps_decode_attn(attn, cache, k, v, pl, pos[s], q, out, workspace=ws)

    one_step(0)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(1, steps + 1):
        one_step(s)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    nbytes = n * ((p + steps) * 2 * 128 * 2 * 2 + 16 * 128 * 4)
    del k, v
    torch.cuda.empty_cache()
    return {"tok_s": n * steps / el, "ms_per_step": el / steps * 1e3, "position": p, "splits": splits,
            "hbm_gbs": nbytes * args.layers * steps / el / 1e9}



SWEEP_POSITIONS = (1024, 2048, 4196, 8192, 16384, 32768, 65536, 131072, 262144)


def run_sweep(ps, torch, num_seqs=256, layers=28, reps=10):
    """Decode-kernel time per layer against query position for Prefix Sliding
    (prefix 100, W=4096), plain sliding window (prefix 0, W=4096) and full
    attention (W >= n), all the same kernel.  tok/s = sequences / (layers x
    per-layer time).  Bounded methods go flat once the position passes L+W."""
    attn = ps.AttnSpec(16, 2, 128, ps.PS_BF16, 10000.0, 1 / math.sqrt(128))
    g = torch.Generator(device="cuda").manual_seed(9)
    q = torch.randn((num_seqs, 16, 128), generator=g, device="cuda").bfloat16()
    out = torch.empty_like(q)
    rows = {}
    for label, prefix, window, cap in (("prefix_sliding", 100, 4096, 4224), ("sliding_window", 0, 4096, 4096),
                                       ("full", 0, 1 << 30, -(-(max(SWEEP_POSITIONS) + 1) // 64) * 64)):
        cache = ps.CacheSpec(window=window, slot_capacity=cap)
        ks, vs = ps.cache_shapes(attn, cache, num_seqs)
        k = torch.empty(ks, dtype=torch.bfloat16, device="cuda").normal_(0, 0.5, generator=g)
        v = torch.empty(vs, dtype=torch.bfloat16, device="cuda").normal_(0, 0.5, generator=g)
        pl = torch.full((num_seqs,), prefix, dtype=torch.int32, device="cuda")
        ws = torch.empty(max(ps.ps_decode_workspace_size(attn, cache, num_seqs, 0), 1), dtype=torch.uint8,
                         device="cuda")
        res = []
        for p in SWEEP_POSITIONS:
            pos = torch.full((num_seqs,), p, dtype=torch.int64, device="cuda")
            run = lambda kk: [ps.ps_decode_attn(attn, cache, k, v, pl, pos, q, out, workspace=ws) for _ in range(kk)]
            run(2)
            t = timed(torch, run, reps) / reps
            n_vis = min(p + 1, prefix + window)
            nbytes = num_seqs * (n_vis * 2 * 128 * 2 * 2 + 16 * 128 * 4)
            res.append({"position": p, "n_vis": n_vis, "us_per_layer": round(t * 1e6, 2),
                        "tok_s": round(num_seqs / (t * layers), 1), "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)})
        rows[label] = res
        del k, v, ws
        torch.cuda.empty_cache()
    return rows


def run_batch_sweep(ps, torch, layers=28, reps=20):
    """Decode-kernel time per layer against the number of sequences at 131072
    (prefix 100, W = 4096), with the library's automatic split count: where
    the kernel reaches its bandwidth plateau as the batch grows."""
    attn = ps.AttnSpec(16, 2, 128, ps.PS_BF16, 10000.0, 1 / math.sqrt(128))
    cache = ps.CacheSpec(window=4096, slot_capacity=4224)
    g = torch.Generator(device="cuda").manual_seed(17)
    p, n_vis = 131072, 4196
    rows = []
    for n in (8, 16, 32, 64, 128, 256, 512, 1024):
        ks, vs = ps.cache_shapes(attn, cache, n)
        k = torch.empty(ks, dtype=torch.bfloat16, device="cuda").normal_(0, 0.5, generator=g)
        v = torch.empty(vs, dtype=torch.bfloat16, device="cuda").normal_(0, 0.5, generator=g)
        q = torch.randn((n, 16, 128), generator=g, device="cuda").bfloat16()
        out = torch.empty_like(q)
        pl = torch.full((n,), 100, dtype=torch.int32, device="cuda")
        pos = torch.full((n,), p, dtype=torch.int64, device="cuda")
        ws = torch.empty(max(ps.ps_decode_workspace_size(attn, cache, n, 0), 1), dtype=torch.uint8, device="cuda")
        run = lambda kk: [ps.ps_decode_attn(attn, cache, k, v, pl, pos, q, out, workspace=ws) for _ in range(kk)]
        run(3)
        t = timed(torch, run, reps) / reps
        nbytes = n * (n_vis * 2 * 128 * 2 * 2 + 16 * 128 * 4)
        rows.append({"num_seqs": n, "splits": ps.ps_decode_num_splits(attn, cache, n), "us_per_layer": round(t * 1e6, 2),
                     "tok_s": round(n / (t * layers), 1), "hbm_gbs": round(nbytes / t / 1e9, 1),
                     "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)})
        del k, v, q, out, ws
        torch.cuda.empty_cache()
    return rows


# ------------------------------------------------------------------------- other decode workloads
def run_decode_extra(ps, torch, layers=28, reps=30):
    """Per-layer decode-kernel time of the other decode workloads (one layer's
    cache each; tok/s assumes `layers` layers of decode attention per token):
    64 sequences at 32768 (W=4096), 256 at 131072 with W=8192, the headline
    workload with Continue PE, with Reset PE scoring and with Reset PE re-rotating
    every visible key before each call (what the scoring identity avoids; the
    cache content is immaterial to the cost), and the ragged paged
    batch of 1024 sequences (positions 1024..262144, prefixes 50..2000)."""
    import numpy as np
    import synth
    out = {}
    for name, n, p, W in (("decode-32768-w4096-64seq", 64, 32768, 4096),
                          ("decode-131072-w8192", 256, 131072, 8192)):
        b = DecodeBench(ps, torch, n, 1, W, 100, p, 0, pool=4)
        pos = torch.full((n,), p, dtype=torch.int64, device="cuda")
        b.decode_only(3, pos)
        t = timed(torch, lambda k: b.decode_only(k, pos), reps) / reps
        out[name] = {"us_per_layer": t * 1e6, "hbm_gbs": b.kernel_bytes(p) / t / 1e9,
                     "hbm_frac": b.kernel_bytes(p) / t / 1e9 / HBM_PEAK_GBS,
                     "tok_s_attention_only": n / (t * layers),
                     "splits": ps.ps_decode_num_splits(b.attn, b.cache, n)}
        b.release()
        del b
        torch.cuda.empty_cache()
    # Reset PE at the headline workload: same cache, prefix slots scored with the renumbered query
    import dataclasses
    b = DecodeBench(ps, torch, 256, 1, 4096, 100, 131072, 0, pool=4)
    pos = torch.full((256,), 131072, dtype=torch.int64, device="cuda")
    for mode, key in ((ps.PS_PE_CONTINUE, "decode-131072-w4096-continue-pe"),
                      (ps.PS_PE_RESET, "decode-131072-w4096-reset-pe"),
                      (ps.PS_PE_RESET_RECOMPUTE, "decode-131072-w4096-reset-pe-recompute")):
        b.attn = dataclasses.replace(b.attn, pe_mode=mode)
        if mode == ps.PS_PE_RESET_RECOMPUTE:   # the re-rotated key copy lives in the workspace
            b.ws = torch.empty(ps.ps_decode_workspace_size(b.attn, b.cache, 256, 0), dtype=torch.uint8,
                               device="cuda")
        b.decode_only(3, pos)
        t = timed(torch, lambda k: b.decode_only(k, pos), reps) / reps
        out[key] = {"us_per_layer": t * 1e6, "hbm_gbs": b.kernel_bytes(131072) / t / 1e9,
                    "hbm_frac": b.kernel_bytes(131072) / t / 1e9 / HBM_PEAK_GBS,
                    "tok_s_attention_only": 256 / (t * layers)}
    b.release()
    del b
    torch.cuda.empty_cache()
    # ragged paged batch
    c = synth.C5_DECODE
    n = c.num_seqs
    pos_np, pre_np = synth.ragged_draws(0, n)
    ring = [min(int(pos_np[s]) + 1, int(pre_np[s]) + c.window) for s in range(n)]
    cap = -(-max(int(pre_np[s]) + c.window for s in range(n)) // 64) * 64
    pages = [-(-r // 64) for r in ring]
    num_pages = int(sum(pages))
    perm = synth.page_permutation(0, num_pages)
    table = np.full((n, cap // 64), -1, dtype=np.int32)
    o = 0
    for s_ in range(n):
        table[s_, :pages[s_]] = perm[o:o + pages[s_]]
        o += pages[s_]
    attn = ps.AttnSpec(16, 2, 128, ps.PS_BF16, 10000.0, 1 / math.sqrt(128))
    cache = ps.CacheSpec(window=c.window, slot_capacity=cap, page_size=64, num_pages=num_pages)
    ks, vs = ps.cache_shapes(attn, cache, n)
    g = torch.Generator(device="cuda").manual_seed(5)
    k = torch.empty(ks, dtype=torch.bfloat16, device="cuda").normal_(0, 0.5, generator=g)
    v = torch.empty(vs, dtype=torch.bfloat16, device="cuda").normal_(0, 0.5, generator=g)
    bt = torch.from_numpy(table).cuda()
    pl = torch.from_numpy(pre_np.astype(np.int32)).cuda()
    pos = torch.from_numpy(pos_np.astype(np.int64)).cuda()
    q = torch.randn((n, 16, 128), generator=g, device="cuda").bfloat16()
    o_ = torch.empty_like(q)
    ws = torch.empty(max(ps.ps_decode_workspace_size(attn, cache, n, 0), 1), dtype=torch.uint8, device="cuda")
    run = lambda kk: [ps.ps_decode_attn(attn, cache, k, v, pl, pos, q, o_, block_table=bt, workspace=ws)
                      for _ in range(kk)]
    run(3)
    t = timed(torch, run, reps) / reps
    nbytes = sum(r * 2 * 128 * 2 * 2 + 16 * 128 * 4 + -(-r // 64) * 4 for r in ring)
    out["decode-ragged-paged-1024seq"] = {"us_per_layer": t * 1e6, "hbm_gbs": nbytes / t / 1e9,
                                          "hbm_frac": nbytes / t / 1e9 / HBM_PEAK_GBS,
                                          "tok_s_attention_only": n / (t * layers),
                                          "mean_n_vis": float(np.mean(ring)),
                                          "splits": ps.ps_decode_num_splits(attn, cache, n)}
    del k, v
    torch.cuda.empty_cache()
    return out

# ------------------------------------------------------------------------- prefill
def median_call_s(torch, fn, reps):
    """Median over `reps` calls of fn(), each between two HIP events on the
    current stream (fn enqueues its launches there)."""
    ts = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(b) / 1000.0)
    return sorted(ts)[len(ts) // 2]


def run_prefill(ps, torch, reps=9, full_causal=True):
    import synth
    out = {}
    for cfg in ([synth.C4_PREFILL, synth.C4_PREFILL_FULL] if full_causal else [synth.C4_PREFILL]):
        attn = ps.AttnSpec(cfg.hq, cfg.hkv, cfg.dim, ps.PS_BF16, cfg.rope_theta, 1 / math.sqrt(cfg.dim))
        g = torch.Generator(device="cuda").manual_seed(11)
        q = torch.randn((cfg.batch, cfg.queries, cfg.hq, cfg.dim), generator=g, device="cuda").bfloat16()
        k = torch.randn((cfg.batch, cfg.nk, cfg.hkv, cfg.dim), generator=g, device="cuda").bfloat16()
        v = torch.randn((cfg.batch, cfg.nk, cfg.hkv, cfg.dim), generator=g, device="cuda").bfloat16()
        o = torch.empty_like(q)
        ws = torch.empty(ps.ps_prefill_workspace_size(attn, cfg.batch, cfg.queries, cfg.nk), dtype=torch.uint8,
                         device="cuda")
        r = reps if cfg is synth.C4_PREFILL else 3
        call = lambda: ps.ps_prefill_attn(attn, cfg.window, cfg.prefix, cfg.kv_start, q, k, v, o, workspace=ws)
        call()
        torch.cuda.synchronize()
        t = median_call_s(torch, call, r)
        if cfg is synth.C4_PREFILL:   # every query sees the prefix and min(t+1, W) chunk keys
            pairs = cfg.prefix * cfg.queries + sum(min(t_ + 1, cfg.window) for t_ in range(cfg.queries))
        else:                         # full causal: query t sits at position Nk - T + t
            pairs = sum(cfg.nk - cfg.queries + t_ + 1 for t_ in range(cfg.queries))
        flops = 4.0 * cfg.dim * pairs * cfg.batch * cfg.hq
        out[cfg.name] = {"ms": t * 1e3, "tflops": flops / t / 1e12, "useful_tflop": flops / 1e12,
                         "mfma_frac": flops / t / 1e12 / BF16_PEAK_TFLOPS}
        del q, k, v, o, ws
        torch.cuda.empty_cache()
    return out


def run_backward(ps, torch, reps=5):
    """Backward of the truncated-backprop forward (8 x 8192 queries, W=2048, Hq=28, Hkv=4): dq, dk, dv from
    the forward's output and LSE.  Useful work: the 5 products of attention backward (S recomputed, dP, dV,
    dQ, dK), 2*D flops each per visible pair and head."""
    import synth
    cfg = synth.C4_PREFILL
    attn = ps.AttnSpec(cfg.hq, cfg.hkv, cfg.dim, ps.PS_BF16, cfg.rope_theta, 1 / math.sqrt(cfg.dim))
    g = torch.Generator(device="cuda").manual_seed(12)
    q = torch.randn((cfg.batch, cfg.queries, cfg.hq, cfg.dim), generator=g, device="cuda").bfloat16()
    k = torch.randn((cfg.batch, cfg.nk, cfg.hkv, cfg.dim), generator=g, device="cuda").bfloat16()
    v = torch.randn((cfg.batch, cfg.nk, cfg.hkv, cfg.dim), generator=g, device="cuda").bfloat16()
    do = torch.randn_like(q)
    o = torch.empty_like(q)
    lse = torch.empty((cfg.batch, cfg.hq, cfg.queries), dtype=torch.float32, device="cuda")
    ps.ps_prefill_attn(attn, cfg.window, cfg.prefix, cfg.kv_start, q, k, v, o, lse=lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # with the dS room the dk/dv pass keeps its dS tiles and dq forms one product instead of three
    extra = ps.ps_prefill_backward_ds_workspace_size(attn, cfg.window, cfg.prefix, cfg.kv_start, cfg.batch,
                                                     cfg.queries, cfg.nk)
    keep_ds = 0 < extra <= torch.cuda.mem_get_info()[0] // 4
    ws = torch.empty(ps.ps_prefill_backward_workspace_size(attn, cfg.batch, cfg.queries, cfg.nk)
                     + (extra if keep_ds else 0), dtype=torch.uint8, device="cuda")

    def call(n_):
        for _ in range(n_):
            ps.ps_prefill_attn_backward(attn, cfg.window, cfg.prefix, cfg.kv_start, q, k, v, o, do, lse, dq, dk, dv,
                                        workspace=ws)
    call(1)
    torch.cuda.synchronize()
    t = median_call_s(torch, lambda: call(1), reps)
    pairs = cfg.prefix * cfg.queries + sum(min(t_ + 1, cfg.window) for t_ in range(cfg.queries))
    flops = 10.0 * cfg.dim * pairs * cfg.batch * cfg.hq
    res = {"workload": cfg.name + "-backward", "ms": t * 1e3, "tflops": flops / t / 1e12,
           "useful_tflop": flops / 1e12, "mfma_frac": flops / t / 1e12 / BF16_PEAK_TFLOPS,
           "executed_products": 5 if keep_ds else 7, "kept_ds": keep_ds, "ds_workspace_bytes": extra if keep_ds else 0}
    del q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


def run_heavy(ps, torch, heavy=512, layers=28, reps=32):
    """Prefix + heavy hitters + window decoding at the headline shape: 256 sequences at 131072, L=100, W=4096,
    512 heavy slots per (sequence, KV head), steady state (heavy set full).  One step per layer = admission of
    the token leaving the window, append, attention over L + W + H keys with the score side output, score
    accumulation.  Reported per layer and as attention-only tok/s over `layers` layers, next to the plain
    Prefix Sliding step (append + attention) on the same cache."""
    n, L, W, p0 = 256, 100, 4096, 131072
    attn = ps.AttnSpec(16, 2, 128, ps.PS_BF16, 10000.0, 1 / math.sqrt(128))
    cap = -(-(L + W + heavy) // 64) * 64
    cache = ps.CacheSpec(window=W, slot_capacity=cap)
    g = torch.Generator(device="cuda").manual_seed(21)
    ks, vs = ps.cache_shapes(attn, cache, n)
    kc = (torch.randn(ks, generator=g, device="cuda") * 0.5).bfloat16()
    vc = (torch.randn(vs, generator=g, device="cuda") * 0.5).bfloat16()
    state = ps.HeavyState.new(attn, cache, n, heavy)
    state.score.uniform_(0.0, 1.0, generator=g)
    state.heavy_count.fill_(heavy)
    state.heavy_pos.copy_(torch.arange(heavy, device="cuda").view(1, 1, heavy) * 37 + 500)
    pl = torch.full((n,), L, dtype=torch.int32, device="cuda")
    q = [torch.randn((n, 16, 128), generator=g, device="cuda").bfloat16() for _ in range(4)]
    kn = (torch.randn((n, 1, 2, 128), generator=g, device="cuda") * 0.5).bfloat16()
    vn = (torch.randn((n, 1, 2, 128), generator=g, device="cuda") * 0.5).bfloat16()
    out = torch.empty((n, 16, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(ps.ps_heavy_workspace_size(attn, cache, n, 0), dtype=torch.uint8, device="cuda")
    wsd = torch.empty(max(ps.ps_decode_workspace_size(attn, cache, n, 0), 1), dtype=torch.uint8, device="cuda")
    positions = [torch.full((n,), p0 + i, dtype=torch.int64, device="cuda") for i in range(2 * reps + 8)]
    cursor = [0]

    def heavy_steps(k_):
        for _ in range(k_):
            ps.ps_heavy_decode_step(attn, cache, heavy, kc, vc, pl, positions[cursor[0]], q[cursor[0] % 4], kn, vn, out,
                                    state, workspace=ws)
            cursor[0] += 1

    def plain_steps(k_):
        for i in range(k_):
            ps.ps_kv_append(attn, cache, kc, vc, pl, positions[i], kn, vn)
            ps.ps_decode_attn(attn, cache, kc, vc, pl, positions[i], q[i % 4], out, workspace=wsd)
    heavy_steps(4)
    t_h = timed(torch, heavy_steps, reps) / reps
    plain_steps(4)
    t_p = timed(torch, plain_steps, reps) / reps
    nvis = L + W + heavy
    kv_bytes = n * nvis * 2 * 128 * 2 * 2
    res = {"workload": f"decode-{p0}-w{W}-heavy{heavy}", "us_per_layer": t_h * 1e6,
           "tok_s_attention_only": n / (t_h * layers), "keys_per_query": nvis,
           "kv_gbs": kv_bytes / t_h / 1e9,
           "plain_prefix_sliding_us_per_layer": t_p * 1e6, "plain_tok_s_attention_only": n / (t_p * layers)}
    del kc, vc, state, ws, wsd
    torch.cuda.empty_cache()
    return res


def run_chunk(ps, torch, reps=5):
    """Chunk continuing live traces (C6): 64 rings at 32768 (L=100, W=4096), a 2048-token chunk each.
    One call = chunk prep (ring gather + rotations), attention, append of the chunk into the rings."""
    import synth
    cfg = synth.C6_CHUNK
    attn = ps.AttnSpec(cfg.hq, cfg.hkv, cfg.dim, ps.PS_BF16, cfg.rope_theta, 1 / math.sqrt(cfg.dim))
    cap = (cfg.prefix + cfg.window + 63) // 64 * 64
    cache = ps.CacheSpec(window=cfg.window, slot_capacity=cap)
    n, T = cfg.num_seqs, cfg.chunk
    g = torch.Generator(device="cuda").manual_seed(13)
    ks, vs = ps.cache_shapes(attn, cache, n)
    kc = (torch.randn(ks, generator=g, device="cuda") * cfg.kv_std).bfloat16()
    vc = (torch.randn(vs, generator=g, device="cuda") * cfg.kv_std).bfloat16()
    q = torch.randn((n, T, cfg.hq, cfg.dim), generator=g, device="cuda").bfloat16()
    kn = (torch.randn((n, T, cfg.hkv, cfg.dim), generator=g, device="cuda") * cfg.kv_std).bfloat16()
    vn = (torch.randn((n, T, cfg.hkv, cfg.dim), generator=g, device="cuda") * cfg.kv_std).bfloat16()
    out = torch.empty_like(q)
    pl = torch.full((n,), cfg.prefix, dtype=torch.int32, device="cuda")
    sp = torch.full((n,), cfg.position, dtype=torch.int64, device="cuda")
    ws = torch.empty(ps.ps_chunk_prefill_workspace_size(attn, cache, n, T), dtype=torch.uint8, device="cuda")

    def call(k_):
        for _ in range(k_):
            ps.ps_chunk_prefill_attn(attn, cache, kc, vc, pl, sp, q, kn, vn, out, workspace=ws)
    call(1)
    torch.cuda.synchronize()
    t = median_call_s(torch, lambda: call(1), reps)
    # every chunk query sits beyond L + W: it sees exactly L + W keys
    pairs = sum(min(cfg.position + t_ + 1, cfg.prefix + cfg.window) for t_ in range(T))
    flops = 4.0 * cfg.dim * pairs * n * cfg.hq
    res = {"workload": cfg.name, "num_seqs": n, "chunk": T, "position": cfg.position, "prefix": cfg.prefix,
           "window": cfg.window, "ms": t * 1e3, "tflops": flops / t / 1e12, "useful_tflop": flops / 1e12,
           "mfma_frac": flops / t / 1e12 / BF16_PEAK_TFLOPS, "tok_s": n * T / t}
    del kc, vc, q, kn, vn, out, ws
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------------- CPU oracle
def _oracle_worker(args):
    idx, position, prefix, window, reps = args
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    import synth
    k = synth.history(0, 3, synth.T_K, idx, 0, 0, position + 1, 2, 128, 0.5, "bf16")
    v = synth.history(0, 3, synth.T_V, idx, 0, 0, position + 1, 2, 128, 0.5, "bf16")
    qs = [synth.query(0, 3, idx, 0, r, 16, 128, 1.0, "bf16") for r in range(reps)]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        for q in qs:
            oracle.decode_attention(q, k, v, position, prefix, window, 1 / math.sqrt(128), 10000.0)
        el = time.perf_counter() - t0
    return reps, el


def run_cpu_baseline(args):
    import concurrent.futures
    import multiprocessing
    host = len(os.sched_getaffinity(0))
    cores = min(host, 16)   # at most 16 worker processes, one per core of the host share that serves one GPU
    reps = 2
    jobs = [(i, args.position, 100, args.window, reps) for i in range(cores)]
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        res = list(ex.map(_oracle_worker, jobs))
    tuples = sum(r[0] for r in res)
    slowest = max(r[1] for r in res)
    tok_s = tuples / slowest / args.layers
    return {"value": tok_s, "unit": "tok/s", "cores": cores, "host_cores": host, "kind": "oracle",
            "sample": f"{tuples} (sequence, layer) decode tuples at position {args.position} over the full "
                      f"un-evicted history, {cores} worker processes x 1 BLAS thread, {reps} tuples each; "
                      f"tok/s = tuples / slowest worker's oracle time / {args.layers} layers",
            "cpu_seconds": sum(r[1] for r in res)}


def _oracle_prefill_worker(args):
    """Full query rows of the C4 prefill (W=2048 behind a 100-token prefix)
    for one slice of rows of each sampled (batch, head) pair."""
    idx, n_pairs, row0, n_rows = args
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle
    import synth
    cfg = synth.C4_PREFILL
    rows = np.arange(row0, row0 + n_rows)
    el = 0.0
    for pair in range(n_pairs):
        q = synth.round_to(synth.normal((cfg.queries, 1, cfg.dim), 0, 4, 100 + pair, 0), "bf16")
        k = synth.round_to(synth.normal((cfg.nk, 1, cfg.dim), 0, 4, 200 + pair, 0), "bf16")
        v = synth.round_to(synth.normal((cfg.nk, 1, cfg.dim), 0, 4, 300 + pair, 0), "bf16")
        with threadpool_limits(1):
            t0 = time.perf_counter()
            oracle.prefill_attention(q, k, v, cfg.prefix, cfg.window, cfg.kv_start, 1 / math.sqrt(cfg.dim),
                                     cfg.rope_theta, rows=rows)
            el += time.perf_counter() - t0
    pairs = sum(cfg.prefix + min(t + 1, cfg.window) for t in rows) * n_pairs
    return pairs, el


def run_cpu_prefill_baseline(cores):
    """The oracle on 4 (batch, head) pairs of the C4 prefill, every query row,
    the rows split evenly over the worker processes."""
    import concurrent.futures
    import multiprocessing
    import synth
    cfg = synth.C4_PREFILL
    n_pairs = 4
    per = -(-cfg.queries // cores)
    jobs = [(i, n_pairs, i * per, min(per, cfg.queries - i * per)) for i in range(cores) if i * per < cfg.queries]
    ctx = multiprocessing.get_context("spawn")
    with concurrent.futures.ProcessPoolExecutor(max_workers=cores, mp_context=ctx) as ex:
        res = list(ex.map(_oracle_prefill_worker, jobs))
    pairs = sum(r[0] for r in res)
    slowest = max(r[1] for r in res)
    return {"value": float(4.0 * cfg.dim * pairs / slowest / 1e12), "unit": "TFLOP/s", "cores": len(jobs),
            "host_cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{n_pairs} (batch, head) pairs of the 8 x 8192-query prefill (W=2048, prefix 100), all "
                      f"{cfg.queries} query rows, split over {len(jobs)} worker processes x 1 BLAS thread; "
                      f"TFLOP/s = 4 D x visible pairs / slowest worker's oracle time",
            "cpu_seconds": sum(r[1] for r in res)}


def measure_ceilings(ps, torch, reps=10):
    """Measured ceilings on this GPU, next to the published peaks: the HBM read
    bandwidth of a plain streaming read (the library's probe over 4 GiB), the
    copy bandwidth of torch's copy kernel (1 GiB read + 1 GiB written), and the
    bf16 rate of the vendor GEMM (torch.matmul, 16384^3)."""
    out = {}
    x = torch.ones(1 << 30, dtype=torch.float32, device="cuda")   # 4 GiB
    ck = torch.zeros(1, dtype=torch.int32, device="cuda")
    ps.ps_read_probe(x, ck)
    t = timed(torch, lambda k: [ps.ps_read_probe(x, ck) for _ in range(k)], reps) / reps
    out["hbm_read_gbs"] = x.numel() * 4 / t / 1e9
    del x
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
    dst = torch.empty_like(src)
    dst.copy_(src)
    t = timed(torch, lambda k: [dst.copy_(src) for _ in range(k)], reps) / reps
    out["torch_copy_gbs"] = 2 * src.numel() * 4 / t / 1e9
    del src, dst
    # the fastest of the shapes and layouts tried (4096^3 .. 32768x8192x8192, B row- or
    # column-major: 1.12-1.60 PFLOP/s): 16384^3 with B column-major (A B^T, B stored [n][k])
    n = 16384
    g = torch.Generator(device="cuda").manual_seed(3)
    a = torch.randn((n, n), generator=g, device="cuda").bfloat16()
    b = torch.randn((n, n), generator=g, device="cuda").bfloat16()
    c = torch.matmul(a, b.t())
    t = timed(torch, lambda k: [torch.matmul(a, b.t(), out=c) for _ in range(k)], reps) / reps
    out["bf16_gemm_tflops"] = 2.0 * n ** 3 / t / 1e12
    out["gemm"] = f"torch.matmul bf16 {n}x{n}x{n}, B column-major"
    del a, b, c
    torch.cuda.empty_cache()
    return out


def load_traffic(kernel_bytes):
    """HBM traffic per launch from the committed counter summary, if it was
    taken on the current kernel source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except OSError:
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    return c.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1 (sharding the path "
                                   "across GPUs is not implemented)"}))
        sys.exit(2)
    # the CPU oracle's worker processes start before anything initialises the GPU
    cpu = cpu_prefill = None
    if not args.no_cpu_baseline:
        cpu = run_cpu_baseline(args)
        print(f"[bench] cpu oracle done: {cpu['value']:.3f} tok/s on {cpu['cores']} cores", file=sys.stderr,
              flush=True)
        if not args.no_prefill:
            cpu_prefill = run_cpu_prefill_baseline(cpu["cores"])
            print(f"[bench] cpu oracle prefill done: {cpu_prefill['value'] * 1e3:.3f} GFLOP/s", file=sys.stderr,
                  flush=True)
    import torch
    import bounded_kv_cache_amd as ps
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)   # a plain elementwise kernel: reads and writes BYTES each
        torch.cuda.synchronize()
        print(f"[bench] copy probe: {args.copy_probe} bytes read and written", file=sys.stderr, flush=True)
        del src, dst
    print(f"[bench] decode: {args.num_seqs} seqs x {args.layers} layers @ {args.position}, W={args.window}",
          file=sys.stderr, flush=True)
    if args.only == "prefill":
        print(json.dumps({"prefill": run_prefill(ps, torch, full_causal=not args.no_full)}))
        return
    if args.only == "chunk":
        print(json.dumps({"chunk_prefill": run_chunk(ps, torch)}))
        return
    if args.only == "backward":
        print(json.dumps({"prefill_backward": run_backward(ps, torch)}))
        return
    if args.only == "batch-sweep":
        print(json.dumps({"decode_batch_sweep": run_batch_sweep(ps, torch)}))
        return
    if args.only == "heavy":
        print(json.dumps({"heavy_hitters": run_heavy(ps, torch)}))
        return
    ceil = measure_ceilings(ps, torch)
    print(f"[bench] ceilings: {ceil}", file=sys.stderr, flush=True)
    dec = run_decode(ps, torch, args)
    print(f"[bench] decode done: {dec['tok_s']:.0f} tok/s, {dec['kernel_s'] * 1e6:.1f} us per launch",
          file=sys.stderr, flush=True)
    if args.only == "decode":
        print(json.dumps({"decode": dec}))
        return
    small = None
    if not args.no_extra:
        small = run_decode(ps, torch, args, num_seqs=64, position=32768, graph=False)
        print(f"[bench] decode 64 seqs @ 32768 done: {small['tok_s']:.0f} tok/s", file=sys.stderr, flush=True)
    prefill = None
    if not args.no_prefill:
        prefill = run_prefill(ps, torch)
        print(f"[bench] prefill done: {prefill}", file=sys.stderr, flush=True)
    backward = None
    if not args.no_backward:
        backward = run_backward(ps, torch)
        print(f"[bench] prefill backward done: {backward['tflops']:.0f} TFLOP/s", file=sys.stderr, flush=True)
    heavy = None
    if not args.no_heavy:
        heavy = run_heavy(ps, torch)
        print(f"[bench] heavy hitters done: {heavy['us_per_layer']:.1f} us/layer", file=sys.stderr, flush=True)
    chunk = None
    if not args.no_chunk:
        chunk = run_chunk(ps, torch)
        print(f"[bench] chunk prefill done: {chunk['tflops']:.0f} TFLOP/s", file=sys.stderr, flush=True)
    sweep = None
    if not args.no_sweep:
        sweep = run_sweep(ps, torch, num_seqs=args.num_seqs, layers=args.layers)
        print(f"[bench] position sweep done", file=sys.stderr, flush=True)
    extra = None
    if not args.no_extra:
        extra = run_decode_extra(ps, torch, layers=args.layers)
        print(f"[bench] other decode workloads done", file=sys.stderr, flush=True)
    full = None
    if not args.no_full:
        full = run_full_attention(ps, torch, args)
        print(f"[bench] full attention done: {full['tok_s']:.0f} tok/s", file=sys.stderr, flush=True)
    achieved = dec["kernel_bytes"] / dec["kernel_s"] / 1e9
    line = {
        "metric": METRIC,
        "value": dec["tok_s"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"decode-{args.position}-w{args.window}", "num_seqs": args.num_seqs,
                   "layers": args.layers, "position": args.position, "prefix": 100, "window": args.window,
                   "hq": 16, "hkv": 2, "head_dim": 128, "splits": dec["splits"]},
        "timing": {"protocol": "rings and positions restored from a snapshot before each rep (untimed); 1 warm-up "
                               "rep discarded; value and ms_per_step are the median of 5 timed reps of `steps` "
                               "steps, each bracketed by HIP events on the launch stream",
                   "rep_ms": dec["rep_ms"]},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(dec["kernel_bytes"]),
                     "kernel": "decode_bf16_kernel (append fused)", "kernel_us": dec["kernel_s"] * 1e6,
                     "kernel_us_source": "median timed rep / launches in it (launch gaps included)",
                     "kernel_launches_timed": dec["kernel_launches"],
                     "bytes_per_launch": dec["kernel_bytes"],
                     "measured_read_gbs": ceil["hbm_read_gbs"], "frac_of_measured_read": achieved / ceil["hbm_read_gbs"]},
        "ceilings": ceil,
        "decode_step_in_hip_graph": {"tok_s": dec["graph_tok_s"], "ms_per_step": dec["graph_ms_per_step"],
                                     "note": "the timed step captured once (28 x ps_decode_step + position "
                                             "advance) and replayed; value is the eager loop"},
        "cpu_baseline": cpu,
        "cpu_baseline_prefill": cpu_prefill,
    }
    if small:
        sb = small["kernel_bytes"] / small["kernel_s"] / 1e9
        line["decode_32768_64seq"] = {
            "workload": "decode-32768-w4096-64seq", "num_seqs": 64, "position": 32768, "window": 4096,
            "layers": args.layers, "tok_s": small["tok_s"], "ms_per_step": small["ms_per_step"],
            "splits": small["splits"], "kernel_us": small["kernel_s"] * 1e6, "hbm_gbs": sb,
            "hbm_frac": sb / HBM_PEAK_GBS, "rep_ms": small["rep_ms"]}
    if prefill:
        c4 = prefill["c4-prefill-7b"]
        line["prefill"] = {"workload": "c4-prefill-7b", "batch": 8, "queries": 8192, "prefix": 100, "window": 2048,
                           "hq": 28, "hkv": 4, "head_dim": 128, "ms": c4["ms"], "tflops": c4["tflops"],
                           "useful_tflop": c4["useful_tflop"],
                           "roofline": {"bound": "mfma", "achieved": c4["tflops"], "peak": BF16_PEAK_TFLOPS,
                                        "unit": "TFLOP/s", "frac": c4["mfma_frac"], "traffic": None,
                                        "kernel": "prefill_prep_kernel + prefill_bf16_kernel (whole call)",
                                        "frac_of_measured_gemm": c4["tflops"] / ceil["bf16_gemm_tflops"]}}
        fc = prefill.get("c4-prefill-7b-full-causal")
        if fc:
            fc["frac_of_measured_gemm"] = fc["tflops"] / ceil["bf16_gemm_tflops"]
            line["prefill_full_causal"] = dict(workload="c4-prefill-7b-full-causal", **fc)
    line["prefill_backward"] = backward
    line["chunk_prefill"] = chunk
    line["heavy_hitters"] = heavy
    line["full_attention"] = full
    if extra:
        line["decode_other_workloads"] = extra
    if sweep:
        line["sweep"] = sweep
    print(json.dumps(line))


if __name__ == "__main__":
    main()
