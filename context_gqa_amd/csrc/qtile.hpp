// Key range of a query tile (forward and dQ kernels).
//
// A query tile is kFwdBM consecutive rows of one KV head's group, row index
// = local token * G + head-in-group, so it covers a short run of local
// tokens.  Each token's allowed keys form the interval [dstart(p), p]; the
// tile visits the key tiles covering the union of those intervals.  When the
// tile straddles the rank's two chunks the union can be two intervals, one
// per chunk, and only their key tiles are visited.
#pragma once
#include "common.hpp"

namespace dmgqa {

struct QTileKeys {
  int a0, na;    // first key tile and count of the first run
  int b0, nb;    // second run (nb == 0 if none)
  int min_pos;   // smallest query position in the tile
  int max_lo;    // largest document start among the tile's positions
};

template <int BM, int BN>
__device__ __forceinline__ QTileKeys qtile_keys(int row0, const int32_t* ds, const Geo& g) {
  const int nrows = g.Sq * g.G;
  const int tokf = row0 / g.G;
  const int tokl = (min(row0 + BM, nrows) - 1) / g.G;
  const int pf = local_pos(tokf, g.c, g.cp, g.rank);
  const int pl = local_pos(tokl, g.c, g.cp, g.rank);
  QTileKeys r;
  r.min_pos = pf;
  r.max_lo = ds[pl];
  int a_lo = ds[pf], a_hi, b_lo = 0, b_hi = -1;
  if (tokf < g.c && tokl >= g.c) {
    a_hi = local_pos(g.c - 1, g.c, g.cp, g.rank);
    b_lo = ds[local_pos(g.c, g.c, g.cp, g.rank)];
    b_hi = pl;
  } else {
    a_hi = pl;
  }
  r.a0 = a_lo / BN;
  int a1 = a_hi / BN;
  r.b0 = 0;
  r.nb = 0;
  if (b_hi >= b_lo) {
    const int b0 = b_lo / BN, b1 = b_hi / BN;
    if (b0 <= a1 + 1) {
      a1 = max(a1, b1);
    } else {
      r.b0 = b0;
      r.nb = b1 - b0 + 1;
    }
  }
  r.na = a1 - r.a0 + 1;
  return r;
}

// The same for interval masks with explicit ends (query position p reaches
// keys ds[p] .. dh[p]-1, both non-decreasing in p, keys indexed apart from
// the queries): the runs end at the last key of the run's last token, and
// min_pos holds the smallest last key of the tile's rows.
template <int BM, int BN>
__device__ __forceinline__ QTileKeys qtile_keys_iv(int row0, const int32_t* ds,
                                                   const int32_t* dh, const Geo& g) {
  const int nrows = g.Sq * g.G;
  const int tokf = row0 / g.G;
  const int tokl = (min(row0 + BM, nrows) - 1) / g.G;
  const int pf = local_pos(tokf, g.c, g.cp, g.rank);
  const int pl = local_pos(tokl, g.c, g.cp, g.rank);
  QTileKeys r;
  r.min_pos = dh[pf] - 1;
  r.max_lo = ds[pl];
  int a_lo = ds[pf], a_hi, b_lo = 0, b_hi = -1;
  if (tokf < g.c && tokl >= g.c) {
    a_hi = dh[local_pos(g.c - 1, g.c, g.cp, g.rank)] - 1;
    b_lo = ds[local_pos(g.c, g.c, g.cp, g.rank)];
    b_hi = dh[pl] - 1;
  } else {
    a_hi = dh[pl] - 1;
  }
  r.a0 = a_lo / BN;
  int a1 = a_hi / BN;
  r.b0 = 0;
  r.nb = 0;
  if (b_hi >= b_lo) {
    const int b0 = b_lo / BN, b1 = b_hi / BN;
    if (b0 <= a1 + 1) {
      a1 = max(a1, b1);
    } else {
      r.b0 = b0;
      r.nb = b1 - b0 + 1;
    }
  }
  r.na = a1 - r.a0 + 1;
  return r;
}

}  // namespace dmgqa
