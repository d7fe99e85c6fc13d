// Prefill tile scheduler (host and device).
//
// Blog "Prefix Sliding 完全拆解" (pinghaoyang.com.cn), section
// "Kernel 实现：两层级过滤": tiles with no visible pair are skipped outright,
// tiles that are partly visible get an element mask, and the key loop walks a
// prefix tile range and a window (band) tile range.  Here the two ranges are
// merged (during warm-up they overlap and a straddling tile belongs to both),
// and every candidate is classified in closed form:
//   kind 0  skip     no visible (query, key) pair
//   kind 1  full     every pair of the whole BM x BN tile exists and is visible
//   kind 2  partial  element mask needed
//
// Geometry: key k sits at position k (k < L) or kv_start + (k - L), with
// kv_start >= L; query t is key Nk - T + t.  Callers guarantee that the query
// positions are consecutive (queries are all chunk keys, or kv_start == L).
// Then visibility needs no positions at all: in KEY-INDEX space a query whose
// key index is u sees key k iff
//     k <= u  and  (k < L  or  u - k < W)
// (chunk positions are an affine image of chunk indices; a pinned key is
// always at or before a chunk query).  All scheduling arithmetic is int32.
#pragma once

#include <stdint.h>

namespace ps {

#if defined(__HIPCC__)
#define PS_HD __host__ __device__
#else
#define PS_HD
#endif

struct PrefillGeom {
  int32_t T, Nk, L, W;
  int64_t kv_start;
  int32_t bm, bn;
};

// absolute positions (used for the rotary angle only)
PS_HD inline int64_t pf_key_pos(const PrefillGeom& g, int64_t k) { return k < g.L ? k : g.kv_start + (k - g.L); }
PS_HD inline int64_t pf_query_pos(const PrefillGeom& g, int64_t t) { return pf_key_pos(g, (int64_t)g.Nk - g.T + t); }

PS_HD inline int32_t pf_min(int32_t a, int32_t b) { return a < b ? a : b; }
PS_HD inline int32_t pf_max(int32_t a, int32_t b) { return a > b ? a : b; }

PS_HD inline int32_t pf_num_qtiles(const PrefillGeom& g) { return (g.T + g.bm - 1) / g.bm; }
PS_HD inline int32_t pf_num_ktiles(const PrefillGeom& g) { return (g.Nk + g.bn - 1) / g.bn; }

// element visibility in key-index space (u: the query's key index)
PS_HD inline bool pf_visible(const PrefillGeom& g, int32_t u, int32_t k) {
  return k <= u && (k < g.L || u - k < g.W);
}

// Classify tile (qt, kt) from its corners.
PS_HD inline int pf_classify(const PrefillGeom& g, int32_t qt, int32_t kt) {
  const int32_t t0 = qt * g.bm, t1 = pf_min(g.T, t0 + g.bm) - 1;
  const int32_t k0 = kt * g.bn, k1 = pf_min(g.Nk, k0 + g.bn) - 1;
  if (t0 > t1 || k0 > k1) return 0;
  const int32_t u0 = g.Nk - g.T + t0, u1 = g.Nk - g.T + t1;  // key indices of the first/last query
  bool any = false, all = true;
  if (k0 < g.L) {  // pinned keys [k0, min(k1, L-1)]: visible iff k <= u
    const int32_t b = pf_min(k1, g.L - 1);
    if (k0 <= u1) any = true;
    if (b > u0) all = false;
  }
  if (k1 >= g.L) {  // chunk keys [a, k1]: visible iff u - W < k <= u
    const int32_t a = pf_max(k0, g.L);
    if (a <= u1 && k1 > u0 - g.W) any = true;
    if (!(a > u1 - g.W && k1 <= u0)) all = false;
  }
  if (!any) return 0;
  const bool whole = (t0 + g.bm <= g.T) && (k0 + g.bn <= g.Nk);
  return (all && whole) ? 1 : 2;
}

// Band tiles (k-tiles at or after n_prefix) hold chunk keys only; such a tile
// is fully visible to every query of q-tile qt iff its first key is inside the
// window of the tile's last query and its last key is at or before its first
// query, and both tiles are whole: one range [lo, hi] of k-tile indices (empty
// when lo > hi).  Equal to pf_classify(g, qt, kt) == 1 for every band tile.
struct FullRange {
  int32_t lo, hi;
};
PS_HD inline FullRange pf_band_full_range(const PrefillGeom& g, int32_t qt) {
  FullRange r{0, -1};
  const int32_t t0 = qt * g.bm;
  if (t0 + g.bm > g.T) return r;                      // the q-tile is not whole
  const int32_t u0 = g.Nk - g.T + t0, u1 = u0 + g.bm - 1;
  const int64_t first = (int64_t)u1 - g.W + 1;        // first key the last query sees
  r.lo = first <= 0 ? 0 : (int32_t)((first + g.bn - 1) / g.bn);
  r.hi = pf_min((u0 + 1) / g.bn - 1, g.Nk / g.bn - 1);
  return r;
}

// Candidate k-tiles of q-tile qt: [0, n_prefix) then [band_lo, band_hi]
// (band_lo >= n_prefix; empty when band_lo > band_hi).
struct TileRange {
  int32_t n_prefix, band_lo, band_hi;
};

PS_HD inline TileRange pf_tile_range(const PrefillGeom& g, int32_t qt) {
  TileRange r;
  const int32_t nkt = pf_num_ktiles(g);
  const int32_t n_pre = pf_min((g.L + g.bn - 1) / g.bn, nkt);
  r.band_lo = 1;
  r.band_hi = 0;
  const int32_t t0 = qt * g.bm, t1 = pf_min(g.T, t0 + g.bm) - 1;
  if (t0 > t1) {
    r.n_prefix = 0;
    return r;
  }
  const int32_t u0 = g.Nk - g.T + t0, u1 = g.Nk - g.T + t1;
  // a prefix tile that starts after the tile's last query holds no visible pair
  r.n_prefix = pf_min(n_pre, u1 / g.bn + 1);
  if (g.Nk <= g.L) return r;
  // chunk keys visible to some query of the tile: (u0 - W, u1] intersected with [L, Nk)
  const int32_t lo = pf_max(u0 - g.W + 1 > g.L ? u0 - g.W + 1 : g.L, g.L);
  const int32_t hi = pf_min(u1, g.Nk - 1);
  if (lo > hi) return r;
  r.band_lo = pf_max(lo / g.bn, n_pre);
  r.band_hi = hi / g.bn;
  return r;
}

// The walk of q-tile qt, shared by the attention kernels and the plan export:
// candidates [0, n_cand) are the prefix k-tiles [0, n_prefix) followed by the
// band k-tiles band_lo + (ci - n_prefix).  Every candidate holds a visible
// pair (the prefix range stops at the tile's last query, the band range is
// exact), so the walk is the plan.
struct Walk {
  TileRange tr;
  FullRange full;
  int32_t n_cand;
};

PS_HD inline Walk pf_walk(const PrefillGeom& g, int32_t qt) {
  Walk w;
  w.tr = pf_tile_range(g, qt);
  w.full = pf_band_full_range(g, qt);
  w.n_cand = w.tr.n_prefix + (w.tr.band_hi >= w.tr.band_lo ? w.tr.band_hi - w.tr.band_lo + 1 : 0);
  return w;
}

PS_HD inline int32_t pf_walk_tile(const Walk& w, int32_t ci) {
  return ci < w.tr.n_prefix ? ci : w.tr.band_lo + (ci - w.tr.n_prefix);
}

// Kind of candidate ci (1 full, 2 partial): prefix candidates by the general
// classification, band candidates (chunk keys only) from the fully visible
// range.  A candidate that held no visible pair would be reported partial, so
// a kernel masks it whole rather than skipping its mask.
PS_HD inline int pf_walk_kind(const PrefillGeom& g, int32_t qt, const Walk& w, int32_t ci) {
  if (ci < w.tr.n_prefix) {
    const int k = pf_classify(g, qt, ci);
    return k ? k : 2;
  }
  const int32_t kt = w.tr.band_lo + (ci - w.tr.n_prefix);
  return (kt >= w.full.lo && kt <= w.full.hi) ? 1 : 2;
}

}  // namespace ps
