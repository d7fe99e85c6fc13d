// Host build of the library's prefill tile scheduler (ps_sched.h, compiled with
// g++), so the CPU tests can compare the closed-form schedule with the oracle's
// element enumeration without a GPU.
#include "ps_sched.h"

extern "C" int ps_host_plan(int T, int Nk, int L, int W, long long kv_start, int bm, int bn, int* tiles,
                            int max_tiles) {
  ps::PrefillGeom g{T, Nk, L, W, kv_start, bm, bn};
  int n = 0;
  const int nqt = ps::pf_num_qtiles(g);
  for (int qt = 0; qt < nqt; ++qt) {
    const ps::TileRange r = ps::pf_tile_range(g, qt);
    const int ncand = r.n_prefix + (r.band_hi >= r.band_lo ? r.band_hi - r.band_lo + 1 : 0);
    for (int ci = 0; ci < ncand; ++ci) {
      const int kt = ci < r.n_prefix ? ci : r.band_lo + (ci - r.n_prefix);
      const int kind = ps::pf_classify(g, qt, kt);
      if (!kind) continue;
      if (n < max_tiles) {
        tiles[3 * n] = qt;
        tiles[3 * n + 1] = kt;
        tiles[3 * n + 2] = kind;
      }
      ++n;
    }
  }
  return n;
}

extern "C" int ps_host_classify_all(int T, int Nk, int L, int W, long long kv_start, int bm, int bn, int* kinds) {
  ps::PrefillGeom g{T, Nk, L, W, kv_start, bm, bn};
  const int nqt = ps::pf_num_qtiles(g), nkt = ps::pf_num_ktiles(g);
  for (int qt = 0; qt < nqt; ++qt)
    for (int kt = 0; kt < nkt; ++kt) kinds[qt * nkt + kt] = ps::pf_classify(g, qt, kt);
  return nqt * nkt;
}


// For every band tile of every q-tile: 1 when pf_band_full_range contains it
// and pf_classify calls it fully visible, 2 when neither, -1 on disagreement.
extern "C" int ps_host_full_range_check(int T, int Nk, int L, int W, long long kv_start, int bm, int bn) {
  ps::PrefillGeom g{T, Nk, L, W, kv_start, bm, bn};
  const int nqt = ps::pf_num_qtiles(g);
  int checked = 0;
  for (int qt = 0; qt < nqt; ++qt) {
    const ps::TileRange r = ps::pf_tile_range(g, qt);
    const ps::FullRange f = ps::pf_band_full_range(g, qt);
    for (int kt = r.band_lo; kt <= r.band_hi; ++kt) {
      const bool full = ps::pf_classify(g, qt, kt) == 1;
      if (full != (kt >= f.lo && kt <= f.hi)) return -1;
      ++checked;
    }
  }
  return checked;
}

// The attention kernels' walk, candidate by candidate (pf_walk / pf_walk_tile /
// pf_walk_kind): every candidate with the kind the kernel uses for it.  Equal to
// the oracle's element-enumerated plan when no candidate is empty and every
// kind is right.
extern "C" int ps_host_walk(int T, int Nk, int L, int W, long long kv_start, int bm, int bn, int* tiles,
                            int max_tiles) {
  ps::PrefillGeom g{T, Nk, L, W, kv_start, bm, bn};
  int n = 0;
  const int nqt = ps::pf_num_qtiles(g);
  for (int qt = 0; qt < nqt; ++qt) {
    const ps::Walk w = ps::pf_walk(g, qt);
    for (int ci = 0; ci < w.n_cand; ++ci) {
      if (n < max_tiles) {
        tiles[3 * n] = qt;
        tiles[3 * n + 1] = ps::pf_walk_tile(w, ci);
        tiles[3 * n + 2] = ps::pf_walk_kind(g, qt, w, ci);
      }
      ++n;
    }
  }
  return n;
}
