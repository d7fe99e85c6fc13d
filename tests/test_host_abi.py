"""CPU tests of the native library's host side: it loads, exports every symbol
the header declares, validates arguments before launching anything, sizes
workspaces, and its prefill tile scheduler (compiled for the host) agrees with
the oracle's element enumeration."""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "prefix_sliding.h")


@pytest.fixture(scope="module")
def lib():
    from bounded_kv_cache_amd import _lib
    return _lib.load()


def test_library_exports_every_declared_symbol(lib):
    text = open(HEADER).read()
    names = sorted(set(re.findall(r"\b(ps_[a-z_0-9]+)\s*\(", text)))
    assert "ps_kv_append" in names and "ps_decode_attn" in names and "ps_prefill_attn" in names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "bounded_kv_cache_amd",
                                                                      "libprefix_sliding.so")],
                         capture_output=True, text=True).stdout
    for n in names:
        assert re.search(rf"\bT {n}$", out, re.M), f"{n} not exported with C linkage"


def test_abi_version_and_status_strings(lib):
    assert lib.ps_abi_version() == 9
    assert lib.ps_status_string(0) == b"ok"
    assert lib.ps_status_string(3) == b"workspace too small"


def _descs(hq=16, hkv=2, d=128, dtype=0, theta=10000.0, scale=0.0884, window=4096, page=0, cap=4224, mp=0, npages=0,
           pe=0):
    from bounded_kv_cache_amd import _lib
    return (_lib.AttnDesc(hq, hkv, d, dtype, theta, scale, pe), _lib.CacheDesc(window, page, cap, mp, npages))


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("mut,status", [
    (dict(hq=15), 1), (dict(hkv=0), 1), (dict(hq=34, hkv=2), 2), (dict(d=96), 2), (dict(dtype=7), 2),
    (dict(scale=0.0), 1), (dict(scale=float("nan")), 1), (dict(theta=-1.0), 1), (dict(theta=0.5), 1),
    (dict(window=0), 1), (dict(page=32), 2), (dict(cap=100), 1), (dict(page=64, cap=4224, mp=10, npages=5), 1),
    (dict(page=64, cap=4224, mp=66, npages=0), 1), (dict(pe=3), 1), (dict(pe=-1), 1),
])
def test_decode_validation(lib, mut, status):
    a, c = _descs(**mut)
    st = lib.ps_decode_attn(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1,
                            None, 0, None)
    assert st == status, lib.ps_last_error()
    assert lib.ps_last_error()


def test_decode_null_pointers_and_workspace(lib):
    a, c = _descs()
    assert lib.ps_decode_attn(ctypes.byref(a), ctypes.byref(c), None, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 1,
                              None, 0, None) == 1
    # paged mode without a block table
    a, c = _descs(page=64, mp=66, npages=100)
    assert lib.ps_decode_attn(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 1,
                              None, 0, None) == 1
    a, c = _descs()
    need = lib.ps_decode_workspace_size(ctypes.byref(a), ctypes.byref(c), 4, 3)
    assert need == 4 * 16 * 3 * (128 + 2) * 4
    assert lib.ps_decode_workspace_size(ctypes.byref(a), ctypes.byref(c), 4, 1) == 0
    assert lib.ps_decode_attn(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 3,
                              FAKE, need - 1, None) == 3
    assert "workspace" in lib.ps_last_error().decode()
    # too many splits for the capacity
    assert lib.ps_decode_attn(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 500,
                              FAKE, 1 << 40, None) == 1
    # no sequences: nothing to do
    assert lib.ps_decode_attn(ctypes.byref(a), ctypes.byref(c), None, None, None, None, None, None, None, 0, 1,
                              None, 0, None) == 0


def test_append_validation(lib):
    a, c = _descs()
    assert lib.ps_kv_append(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, None, -1, FAKE, FAKE,
                            2, None, None) == 1
    assert lib.ps_kv_append(ctypes.byref(a), ctypes.byref(c), FAKE, None, None, FAKE, FAKE, None, 1, FAKE, FAKE,
                            2, None, None) == 1
    assert lib.ps_kv_append(ctypes.byref(a), ctypes.byref(c), None, None, None, None, None, None, 0, None, None,
                            2, None, None) == 0
    a, c = _descs(window=-3)
    assert lib.ps_kv_append(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, None, 1, FAKE, FAKE,
                            2, None, None) == 1


@pytest.mark.parametrize("args,status", [
    ((0, 0, 0, 1, 8, 8), 1),        # window 0
    ((4, -1, 0, 1, 8, 8), 1),       # negative prefix
    ((4, 9, 9, 1, 8, 8), 1),        # prefix longer than the key array
    ((4, 4, 2, 1, 8, 8), 1),        # kv_start before the end of the prefix
    ((4, 2, 2, 1, 9, 8), 1),        # more queries than keys
    ((4, 2, 5, 1, 8, 8), 1),        # queries reach into the prefix but positions are not contiguous
])
def test_prefill_validation(lib, args, status):
    a, _ = _descs()
    w, L, start, b, t, nk = args
    st = lib.ps_prefill_attn(ctypes.byref(a), w, L, start, FAKE, FAKE, FAKE, b, t, nk, FAKE, None, FAKE, 1 << 40,
                             None)
    assert st == status, lib.ps_last_error()
    st = lib.ps_prefill_plan(ctypes.byref(a), w, L, start, t, nk, FAKE, 10, FAKE, None)
    assert st == status


def test_prefill_workspace_and_tiles(lib):
    a, _ = _descs(hq=28, hkv=4)
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    assert lib.ps_prefill_tile_shape(ctypes.byref(a), ctypes.byref(bm), ctypes.byref(bn)) == 0
    assert (bm.value, bn.value) == (128, 64)
    need = lib.ps_prefill_workspace_size(ctypes.byref(a), 8, 8192, 8292)
    nkp = -(-8292 // 64) * 64
    assert need == (2 * 8 * 4 * nkp * 128 * 2 + 255) // 256 * 256 + 8192 * 64 * 2 * 4
    assert lib.ps_prefill_attn(ctypes.byref(a), 2048, 100, 98304, FAKE, FAKE, FAKE, 8, 8192, 8292, FAKE, None,
                               FAKE, need - 1, None) == 3
    # the bf16 kernel addresses V^T rows with 32-bit offsets: at most 2^28 keys
    nk = (1 << 28) + 1
    assert lib.ps_prefill_attn(ctypes.byref(a), 2048, 100, nk - 64, FAKE, FAKE, FAKE, 1, 64, nk, FAKE, None,
                               FAKE, 1 << 62, None) == 1
    assert "2^28" in lib.ps_last_error().decode()


# ---------------------------------------------------------------- scheduler (host build) vs oracle
@pytest.fixture(scope="module")
def sched():
    tmp = tempfile.mkdtemp(prefix="ps_sched_")
    so = os.path.join(tmp, "sched_host.so")
    subprocess.run(["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-I",
                    os.path.join(ROOT, "bounded_kv_cache_amd", "csrc"),
                    os.path.join(ROOT, "tests", "host", "sched_host.cpp"), "-o", so], check=True)
    lib = ctypes.CDLL(so)
    lib.ps_host_plan.restype = ctypes.c_int
    lib.ps_host_plan.argtypes = [ctypes.c_int] * 4 + [ctypes.c_longlong, ctypes.c_int, ctypes.c_int,
                                                      ctypes.c_void_p, ctypes.c_int]
    return lib


def _host_plan(sched, T, Nk, L, W, start, bm, bn):
    n = sched.ps_host_plan(T, Nk, L, W, start, bm, bn, None, 0)
    buf = np.zeros((max(n, 1), 3), dtype=np.int32)
    sched.ps_host_plan(T, Nk, L, W, start, bm, bn, buf.ctypes.data, n)
    return [tuple(int(x) for x in r) for r in buf[:n]]


def test_scheduler_matches_oracle_golden(sched):
    import json
    with open(os.path.join(ROOT, "tests", "golden", "tile_plan_small.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        got = _host_plan(sched, c["T"], c["Nk"], c["L"], c["W"], c["kv_start"], c["BM"], c["BN"])
        assert got == oracle.tile_plan(c["T"], c["Nk"], c["L"], c["W"], c["kv_start"], c["BM"], c["BN"])


def test_scheduler_matches_oracle_random(sched):
    rs = np.random.default_rng(0)
    for _ in range(300):
        bm, bn = [(128, 64), (64, 64), (4, 4), (2, 3), (16, 8)][rs.integers(5)]
        L = int(rs.integers(0, 40))
        chunk = int(rs.integers(1, 200))
        nk = L + chunk
        contiguous = rs.random() < 0.4
        if contiguous:
            start = L
            T = int(rs.integers(1, nk + 1))
        else:
            start = L + int(rs.integers(0, 500))
            T = int(rs.integers(1, chunk + 1))
        W = int(rs.integers(1, 300))
        got = _host_plan(sched, T, nk, L, W, start, bm, bn)
        want = oracle.tile_plan(T, nk, L, W, start, bm, bn)
        assert got == want, (T, nk, L, W, start, bm, bn)


def test_scheduler_matches_oracle_truncated_backprop_shape(sched):
    got = _host_plan(sched, 8192, 8292, 100, 2048, 98304, 128, 64)
    assert got == oracle.tile_plan(8192, 8292, 100, 2048, 98304, 128, 64)


def _host_walk(sched, T, Nk, L, W, start, bm, bn):
    n = sched.ps_host_walk(T, Nk, L, W, start, bm, bn, None, 0)
    buf = np.zeros((max(n, 1), 3), dtype=np.int32)
    sched.ps_host_walk(T, Nk, L, W, start, bm, bn, buf.ctypes.data, n)
    return [tuple(int(x) for x in r) for r in buf[:n]]


def test_kernel_walk_is_the_oracle_plan(sched):
    # the attention kernels walk exactly the exported plan: every candidate tile
    # holds a visible pair and gets the oracle's kind (queries reaching far into
    # a long prefix included, where prefix tiles past the queries must not be walked).
    # (64, 128) is the backward's dS tiling: a kept dS tile sits at its key tile's
    # position in the 64-query block's walk, so the walk must be exactly the tiles
    # with a visible pair there too
    sched.ps_host_walk.restype = ctypes.c_int
    sched.ps_host_walk.argtypes = sched.ps_host_plan.argtypes
    cases = [(8192, 8292, 100, 2048, 98304, 128, 64), (300, 300, 250, 40, 250, 128, 64),
             (200, 200, 200, 7, 200, 64, 64), (1000, 1000, 700, 100, 700, 128, 64),
             (8192, 8292, 100, 2048, 98304, 64, 128), (1000, 1000, 700, 100, 700, 64, 128)]
    rs = np.random.default_rng(1)
    for _ in range(300):
        bm, bn = [(128, 64), (64, 64), (4, 4), (2, 3), (16, 8), (64, 128)][rs.integers(6)]
        L = int(rs.integers(0, 300))
        chunk = int(rs.integers(1, 200))
        nk = L + chunk
        if rs.random() < 0.5:
            start, T = L, int(rs.integers(1, nk + 1))
        else:
            start, T = L + int(rs.integers(0, 500)), int(rs.integers(1, chunk + 1))
        cases.append((T, nk, L, int(rs.integers(1, 300)), start, bm, bn))
    for c in cases:
        assert _host_walk(sched, *c) == oracle.tile_plan(*c), c


def test_chunk_prefill_validation_and_workspace(lib):
    a, c = _descs()
    S, T = 3, 100
    nkp = (4224 + T + 63) // 64 * 64
    align = lambda x: (x + 255) // 256 * 256
    need = lib.ps_chunk_prefill_workspace_size(ctypes.byref(a), ctypes.byref(c), S, T)
    assert need == align(2 * S * 2 * nkp * 128 * 2) + align(S * T * 64 * 2 * 4)
    a32, _ = _descs(dtype=1)
    assert lib.ps_chunk_prefill_workspace_size(ctypes.byref(a32), ctypes.byref(c), S, T) == \
        align(2 * S * 2 * nkp * 128 * 4) + align(S * T * 64 * 2 * 4)

    def call(attn=a, cache=c, kc=FAKE, q=FAKE, chunk=T, seqs=S, ws=FAKE, wsb=need, bt=None):
        return lib.ps_chunk_prefill_attn(ctypes.byref(attn), ctypes.byref(cache), kc, FAKE, bt, FAKE, FAKE, chunk,
                                         q, FAKE, FAKE, seqs, FAKE, None, None, ws, wsb, None)

    assert call(wsb=need - 1) == 3
    assert call(ws=None) == 3
    assert call(kc=None) == 1
    assert call(q=None) == 1
    assert call(chunk=-1) == 1
    assert call(seqs=-2) == 1
    assert call(seqs=0) == 0 and call(chunk=0) == 0          # nothing to do, nothing launched
    bad_a, _ = _descs(hq=15)
    assert call(attn=bad_a) == 1
    _, paged = _descs(page=64, mp=66, npages=100)
    assert call(cache=paged) == 1                              # paged cache without a block table
    assert lib.ps_last_error()


def test_backward_validation_and_workspace(lib):
    a, _ = _descs()
    B, T, NK = 2, 300, 420
    nkp, tqp = 512, 320
    al = lambda x: (x + 255) // 256 * 256
    # K' row-major and d-major, V; Q''; lse2 and Di; cos/sin of queries and keys
    want = (3 * al(B * 2 * nkp * 128 * 2) + al(B * 16 * tqp * 128 * 2) + 2 * al(B * 16 * tqp * 4)
            + al(T * 128 * 4) + al(nkp * 128 * 4))
    need = lib.ps_prefill_backward_workspace_size(ctypes.byref(a), B, T, NK)
    assert need == want

    def call(window=64, L=20, ks=500, nq=T, nk=NK, lse=FAKE, dq=FAKE, wsb=need, ws=FAKE):
        return lib.ps_prefill_attn_backward(ctypes.byref(a), window, L, ks, FAKE, FAKE, FAKE, FAKE, FAKE, lse, B, nq, nk,
                                            dq, FAKE, FAKE, ws, wsb, None)
    assert call(wsb=need - 1) == 3
    assert call(lse=None) == 1
    assert call(dq=None) == 1
    assert call(window=0) == 1
    assert call(L=500) == 1                 # prefix longer than the key array
    assert call(ks=10) == 1                 # kv_start before the end of the prefix
    assert call(nq=NK + 1) == 1             # more queries than keys
    assert call(nq=NK, ks=600) == 1         # queries reach into the prefix with a gap
    assert call(nq=0) == 0


@pytest.mark.parametrize("pe", [1, 2])
def test_reset_pe_is_decode_only(lib, pe):
    a, c = _descs(pe=pe)
    # prefill, backward and chunk prefill reject Reset PE before looking at anything else
    assert lib.ps_prefill_attn(ctypes.byref(a), 64, 0, 0, FAKE, FAKE, FAKE, 1, 64, 64, FAKE, None, FAKE, 1 << 30,
                               None) == 2
    assert lib.ps_prefill_attn_backward(ctypes.byref(a), 64, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 64,
                                        FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == 2
    assert lib.ps_chunk_prefill_attn(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, 16, FAKE, FAKE,
                                     FAKE, 1, FAKE, None, None, FAKE, 1 << 30, None) == 2
    assert b"Continue PE" in lib.ps_last_error()
    assert lib.ps_heavy_decode_step(ctypes.byref(a), ctypes.byref(c), 8, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, 4, FAKE, FAKE, FAKE, 1, FAKE, 1 << 30, None) == 2
    # decode accepts it (fails later only on the NULL cache pointer)
    assert lib.ps_decode_attn(ctypes.byref(a), ctypes.byref(c), None, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4, 1,
                              None, 0, None) == 1


def test_reset_pe_recompute_workspace_and_layout(lib):
    al = lambda x: (x + 255) // 256 * 256
    for dtype, elem in ((0, 2), (1, 4)):
        a, c = _descs(pe=2, dtype=dtype, cap=4224)
        for splits, part in ((1, 0), (3, 4 * 16 * 3 * (128 + 2) * 4)):
            need = lib.ps_decode_workspace_size(ctypes.byref(a), ctypes.byref(c), 4, splits)
            assert need == al(part) + al(4 * 8) + al(4224 * 64 * 2 * elem) + al(4 * 2 * 4224 * 128 * elem)
            # too small a workspace is reported before anything runs
            assert lib.ps_decode_attn(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, 4,
                                      splits, FAKE, need - 1, None) == 3
    # contiguous caches only
    a, c = _descs(pe=2, page=64, mp=66, npages=1000)
    assert lib.ps_decode_attn(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 1,
                              FAKE, 1 << 40, None) == 2
    assert b"contiguous" in lib.ps_last_error()


def test_heavy_decode_validation_and_workspace(lib):
    a, c = _descs(cap=4352)
    need = lib.ps_heavy_workspace_size(ctypes.byref(a), ctypes.byref(c), 4, 1)
    al = lambda x: (x + 255) // 256 * 256
    # bf16, one split, statistics within the LDS budget (136 chunks x 8 heads x
    # (32 fp16 + one fp32 max) = 74 KB): the decode kernel keeps them in LDS
    assert need == 0
    # more splits: fp16 s - m per slot and head, one fp32 max per 32-slot chunk, the row sums
    stats = al(4 * 16 * 4352 * 2) + al(4 * 16 * (4352 // 32) * 4) + al(4 * 16 * 4)
    need3 = lib.ps_heavy_workspace_size(ctypes.byref(a), ctypes.byref(c), 4, 3)
    assert need3 == al(4 * 16 * 3 * (128 + 2) * 4) + stats
    # one split but statistics beyond the budget (9216 slots: 288 chunks x 8 x 68 B > 152 KB)
    ab, cb = _descs(cap=9216)
    assert lib.ps_heavy_workspace_size(ctypes.byref(ab), ctypes.byref(cb), 4, 1) == \
        al(4 * 16 * 9216 * 2) + al(4 * 16 * (9216 // 32) * 4) + al(4 * 16 * 4)
    # fp32: the scores themselves, no maxima
    a32, c32 = _descs(cap=4352, dtype=1)
    assert lib.ps_heavy_workspace_size(ctypes.byref(a32), ctypes.byref(c32), 4, 1) == \
        al(4 * 16 * 4352 * 4) + al(4 * 16 * 4)

    def call(attn=a, cache=c, H=128, score=FAKE, hpos=FAKE, ws=FAKE, wsb=need3, splits=3, seqs=4):
        return lib.ps_heavy_decode_step(ctypes.byref(attn), ctypes.byref(cache), H, FAKE, FAKE, None, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, FAKE, seqs, score, FAKE, hpos, splits, ws, wsb, None)
    assert call(wsb=need3 - 1) == 3
    assert call(score=None) == 1
    assert call(hpos=None) == 1
    assert call(hpos=None, H=0) != 1 or lib.ps_last_error()      # no heavy slots: heavy_pos may be NULL
    assert call(H=-1) == 1
    assert call(H=4352 - 4096 + 1) == 1                          # W + H beyond the capacity
    assert call(seqs=0) == 0
    r, _ = _descs(pe=1)
    assert call(attn=r) == 2


def test_read_probe_validation(lib):
    assert lib.ps_read_probe(None, 16, FAKE, None) == 1
    assert lib.ps_read_probe(FAKE, 16, None, None) == 1
    assert lib.ps_read_probe(FAKE, 24, FAKE, None) == 1                       # bytes not a multiple of 16
    assert lib.ps_read_probe(ctypes.c_void_p(0x1008), 16, FAKE, None) == 1    # src not 16-byte aligned
    assert b"aligned" in lib.ps_last_error()
    assert lib.ps_read_probe(FAKE, (1 << 40) + 16, FAKE, None) == 1


def test_automatic_split_count(lib):
    """The split count minimises the waves of one workgroup per CU times the
    share of keys per split (ties: fewer splits); without a GPU the library
    assumes 256 CUs.  At capacity 4224 a split keeps at least 512 keys."""
    a, c = _descs(cap=4224)
    got = [lib.ps_decode_num_splits(ctypes.byref(a), ctypes.byref(c), n) for n in (8, 16, 32, 64, 96, 128, 192, 256,
                                                                                   1024)]
    assert got == [8, 8, 4, 2, 4, 1, 2, 1, 1]
    a, c = _descs(cap=128)
    assert lib.ps_decode_num_splits(ctypes.byref(a), ctypes.byref(c), 1) == 1


def test_decode_step_validation(lib):
    """ps_decode_step checks everything (its own pointers and every decode
    argument) before anything is enqueued, on both the one-launch and the
    two-call paths."""
    for dtype in (0, 1):
        a, c = _descs(dtype=dtype)
        assert lib.ps_decode_step(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, None, FAKE,
                                  FAKE, 4, 1, None, 0, None) == 1                      # k_new NULL
        assert lib.ps_decode_step(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, 4, 3, FAKE, 1, None) == 3                      # workspace too small
        assert lib.ps_decode_step(ctypes.byref(a), ctypes.byref(c), None, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, 4, 1, None, 0, None) == 1                      # cache NULL
        assert lib.ps_decode_step(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                  FAKE, 4, 500, FAKE, 1 << 40, None) == 1              # too many splits
    a, c = _descs(pe=2, page=64, mp=66, npages=1000)
    assert lib.ps_decode_step(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                              FAKE, 4, 1, FAKE, 1 << 40, None) == 2                    # recompute needs contiguous
    a, c = _descs()
    assert lib.ps_decode_step(ctypes.byref(a), ctypes.byref(c), None, None, None, None, None, None, None, None,
                              None, 0, 1, None, 0, None) == 0                          # no sequences


def test_band_full_range_equals_the_classification(sched):
    """The attention kernel marks band tiles fully visible from one closed-form
    index range; it must agree with the general classification on every band
    tile, over random geometries (warm-up, ragged ends, W >= n, tiny tiles)."""
    sched.ps_host_full_range_check.restype = ctypes.c_int
    sched.ps_host_full_range_check.argtypes = [ctypes.c_int] * 4 + [ctypes.c_longlong, ctypes.c_int, ctypes.c_int]
    rng = np.random.default_rng(11)
    total = 0
    for _ in range(400):
        L = int(rng.integers(0, 300))
        T = int(rng.integers(1, 700))
        W = int(rng.choice([1, 2, 7, 33, 64, 100, 257, 1 << 30]))
        start = L + int(rng.integers(0, 500)) if rng.random() < 0.7 else L
        nk = L + (start - L) + T
        bm, bn = [(128, 64), (64, 64), (32, 16), (16, 32)][int(rng.integers(0, 4))]
        n = sched.ps_host_full_range_check(T, nk, L, W, start, bm, bn)
        assert n >= 0, (T, nk, L, W, start, bm, bn)
        total += n
    assert total > 10000


ODD = ctypes.c_void_p(0x1008)   # 8-byte aligned only; never dereferenced


def test_misaligned_element_pointers_are_rejected(lib):
    # element tensors are accessed with 16-byte vector loads and stores: a
    # pointer that is not 16-byte aligned (a view at an odd storage offset) is
    # an invalid argument, reported before anything is launched
    a, c = _descs()
    B = ctypes.byref

    def err(name):
        return f"{name} is not".encode() in lib.ps_last_error()

    assert lib.ps_decode_attn(B(a), B(c), FAKE, FAKE, None, FAKE, FAKE, ODD, FAKE, 4, 1, None, 0, None) == 1
    assert err("q")
    assert lib.ps_decode_attn(B(a), B(c), FAKE, ODD, None, FAKE, FAKE, FAKE, FAKE, 4, 1, None, 0, None) == 1
    assert err("v_cache")
    assert lib.ps_decode_step(B(a), B(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, ODD, FAKE, FAKE, 4, 1, None, 0,
                              None) == 1
    assert err("k_new")
    assert lib.ps_kv_append(B(a), B(c), FAKE, FAKE, None, FAKE, FAKE, None, 1, FAKE, ODD, 2, None, None) == 1
    assert err("v_new")
    assert lib.ps_prefill_attn(B(a), 64, 0, 0, FAKE, FAKE, FAKE, 1, 64, 64, ODD, None, FAKE, 1 << 40, None) == 1
    assert err("out")
    # the LSE is written one float at a time: 4-byte alignment is enough
    assert lib.ps_prefill_attn(B(a), 64, 0, 0, FAKE, FAKE, FAKE, 1, 64, 64, FAKE, ctypes.c_void_p(0x1002), FAKE,
                               1 << 40, None) == 1
    assert err("lse")
    assert lib.ps_prefill_attn_backward(B(a), 64, 0, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 64, 64, FAKE, FAKE,
                                        ODD, FAKE, 1 << 40, None) == 1
    assert err("dv")
    assert lib.ps_chunk_prefill_attn(B(a), B(c), ODD, FAKE, None, FAKE, FAKE, 16, FAKE, FAKE, FAKE, 1, FAKE, None,
                                     None, FAKE, 1 << 40, None) == 1
    assert err("k_cache")
    ah, ch = _descs(cap=4352)
    assert lib.ps_heavy_decode_step(B(ah), B(ch), 8, FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, ODD,
                                    FAKE, FAKE, 1, FAKE, 1 << 30, None) == 1
    assert err("score")


def test_noalloc_step_rejects_what_exceeds_its_static_scratch(lib):
    # ps_decode_step_noalloc keeps the split partials in an 8 MiB static device
    # array: a call whose partials would not fit is refused before anything runs
    a, c = _descs()
    assert lib.ps_decode_noalloc_scratch_bytes() == 8 << 20
    n, splits = 1024, 8   # 1024 sequences x 16 heads x 8 splits x (128 + 2) floats = 68 MB
    assert lib.ps_decode_workspace_size(ctypes.byref(a), ctypes.byref(c), n, splits) > 8 << 20
    st = lib.ps_decode_step_noalloc(ctypes.byref(a), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    FAKE, n, splits, None)
    assert st == 3 and b"scratch" in lib.ps_last_error()
    # the argument checks of ps_decode_step come first
    bad, _ = _descs(hq=15)
    assert lib.ps_decode_step_noalloc(ctypes.byref(bad), ctypes.byref(c), FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, n, splits, None) == 1


def test_backward_ds_workspace_is_the_longest_block_walk(lib, sched):
    # the kept-dS room: one 128-key x 64-query bf16 tile (16 KB) per query head,
    # 64-query block and slot, the slots being the longest walk of 128-key tiles
    # over a 64-query block (the host build of the same scheduling functions)
    sched.ps_host_walk.restype = ctypes.c_int
    sched.ps_host_walk.argtypes = sched.ps_host_plan.argtypes
    f = lib.ps_prefill_backward_ds_workspace_size
    f.restype = ctypes.c_size_t
    f.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                  ctypes.c_int32]
    for hq, hkv, B, T, nk, L, W, ks in [(28, 4, 8, 8192, 8292, 100, 2048, 98304), (16, 2, 2, 300, 420, 20, 64, 500),
                                        (8, 2, 1, 257, 257, 0, 1 << 30, 0), (16, 2, 1, 190, 337, 37, 130, 37)]:
        a, _ = _descs(hq=hq, hkv=hkv)
        walk = _host_walk(sched, T, nk, L, W, ks, 64, 128)
        per_block = {}
        for qb, _kt, _kind in walk:
            per_block[qb] = per_block.get(qb, 0) + 1
        slots = max(per_block.values())
        nqb = (T + 63) // 64
        assert f(ctypes.byref(a), W, L, ks, B, T, nk) == B * hq * nqb * slots * 16384, (T, nk, L, W)
    a32, _ = _descs(dtype=1)
    assert f(ctypes.byref(a32), 64, 20, 500, 2, 300, 420) == 0          # fp32: the dq pass recomputes
    a, _ = _descs()
    assert f(ctypes.byref(a), 0, 20, 500, 2, 300, 420) == 0             # invalid window
