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
// Geometry: key k sits at position k (k < L) or kv_start + (k - L); query t is
// key Nk - T + t.  Callers guarantee consecutive query positions (queries are
// all chunk keys, or kv_start == L), so the union of the windows of a query
// tile is one interval.
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

PS_HD inline int64_t pf_key_pos(const PrefillGeom& g, int64_t k) { return k < g.L ? k : g.kv_start + (k - g.L); }
PS_HD inline int64_t pf_query_pos(const PrefillGeom& g, int64_t t) { return pf_key_pos(g, (int64_t)g.Nk - g.T + t); }
PS_HD inline int64_t pf_min(int64_t a, int64_t b) { return a < b ? a : b; }
PS_HD inline int64_t pf_max(int64_t a, int64_t b) { return a > b ? a : b; }

PS_HD inline int32_t pf_num_qtiles(const PrefillGeom& g) { return (g.T + g.bm - 1) / g.bm; }
PS_HD inline int32_t pf_num_ktiles(const PrefillGeom& g) { return (g.Nk + g.bn - 1) / g.bn; }

// Classify tile (qt, kt) from the positions at its corners.
PS_HD inline int pf_classify(const PrefillGeom& g, int32_t qt, int32_t kt) {
  const int64_t t0 = (int64_t)qt * g.bm, t1 = pf_min(g.T, t0 + g.bm) - 1;
  const int64_t k0 = (int64_t)kt * g.bn, k1 = pf_min(g.Nk, k0 + g.bn) - 1;
  if (t0 > t1 || k0 > k1) return 0;
  const int64_t pq0 = pf_query_pos(g, t0), pq1 = pf_query_pos(g, t1);
  bool any = false, all = true;
  if (k0 < g.L) {  // pinned keys [k0, min(k1, L-1)]: visible iff key <= query
    const int64_t a = k0, b = pf_min(k1, (int64_t)g.L - 1);
    if (a <= pq1) any = true;
    if (b > pq0) all = false;
  }
  if (k1 >= g.L) {  // chunk keys: visible iff query - W < key <= query
    const int64_t a = pf_key_pos(g, pf_max(k0, g.L)), b = pf_key_pos(g, k1);
    if (a <= pq1 && b > pq0 - g.W) any = true;
    if (!(a > pq1 - g.W && b <= pq0)) all = false;
  }
  if (!any) return 0;
  const bool whole = (t0 + g.bm <= g.T) && (k0 + g.bn <= g.Nk);
  return (all && whole) ? 1 : 2;
}

// Candidate k-tiles of q-tile qt: [0, n_prefix) then [band_lo, band_hi]
// (band_lo >= n_prefix; empty when band_lo > band_hi).
struct TileRange {
  int32_t n_prefix, band_lo, band_hi;
};

PS_HD inline TileRange pf_tile_range(const PrefillGeom& g, int32_t qt) {
  TileRange r;
  const int32_t nkt = pf_num_ktiles(g);
  r.n_prefix = (int32_t)pf_min((g.L + g.bn - 1) / g.bn, nkt);
  r.band_lo = 1;
  r.band_hi = 0;
  const int64_t t0 = (int64_t)qt * g.bm, t1 = pf_min(g.T, t0 + g.bm) - 1;
  if (t0 > t1) return r;
  const int64_t pq0 = pf_query_pos(g, t0), pq1 = pf_query_pos(g, t1);
  const int64_t chunk_last = g.kv_start + (g.Nk - g.L) - 1;  // position of the last chunk key
  const int64_t lo = pf_max(pq0 - g.W + 1, g.kv_start), hi = pf_min(pq1, chunk_last);
  if (g.Nk <= g.L || lo > hi) return r;
  const int64_t k_lo = g.L + (lo - g.kv_start), k_hi = g.L + (hi - g.kv_start);
  r.band_lo = (int32_t)pf_max(k_lo / g.bn, r.n_prefix);
  r.band_hi = (int32_t)(k_hi / g.bn);
  return r;
}

}  // namespace ps
