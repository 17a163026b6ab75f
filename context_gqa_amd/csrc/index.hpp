// Index arithmetic of the attention kernels: the chunk map of a CP rank, the
// key tiles a query tile visits (and which of them need the mask), the query
// rows that reach a key tile or a key, and the dS stash blocks of a key tile.
//
// Plain integer code with no HIP dependence: the kernels compile it for the
// GPU, and the host index tests compile it with a C++ compiler and check
// every result bit for bit against the explicit mask.
//
// The mask these functions serve (the pages' document mask with the causal
// mask of a decoder, "Paper notes: The Llama 3 Herd of Models", "Two
// architectural choices"; the CP chunk map of "The Llama 3 Herd of Models",
// section 3.3.2) is an interval of keys per query position p:
//   causal interval masks  keys ds[p] .. p        (ds = document start, or
//                                                  any non-decreasing lo)
//   explicit ends (cross)  keys ds[p] .. dh[p]-1  (ds, dh non-decreasing)
// and, per key t, the query positions that reach it form the run
//   [t, dend[t])  (causal)   or   [kfirst[t], dend[t])  (explicit ends).
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define DMGQA_HD __host__ __device__ __forceinline__
#else
#define DMGQA_HD inline
#endif

namespace dmgqa {

// Forward and dQ kernels: 128 query rows (tokens x group heads) per
// workgroup, 64 keys per step.
constexpr int kFwdBM = 128;
constexpr int kFwdBN = 64;
// dK/dV kernel: 128 keys per work item, query rows streamed 64 at a time.
constexpr int kDkdvBN = 128;
constexpr int kDkdvBM = 64;
// dS stash: blocks of kStashRows query rows (aligned within each KV head's
// row index tok*G + head) x kDkdvBN keys of one key tile, bf16.
constexpr int kStashRows = 32;

DMGQA_HD int imin(int a, int b) { return a < b ? a : b; }
DMGQA_HD int imax(int a, int b) { return a > b ? a : b; }

// Per-call geometry shared by every kernel.
struct Geo {
  int B, S, Skv, Hq, Hkv, G, Sq, c, cp, rank;
  int g_log2;        // log2(G) if G is a power of two, else -1
  unsigned g_magic;  // ceil(2^32 / G) for G >= 2 (see div_small)
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
};

// Global position of local row j (chunk layout of the rank: chunk `rank`,
// then chunk 2*cp-1-rank, each c tokens in ascending order).
DMGQA_HD int local_pos(int j, int c, int cp, int rank) {
  return j < c ? rank * c + j : (2 * cp - 1 - rank) * c + (j - c);
}

// Key range of a query tile (forward and dQ kernels).
//
// A query tile is BM consecutive rows of one KV head's group, row index =
// local token * G + head-in-group, so it covers a short run of local
// tokens.  Each token's allowed keys form an interval; the tile visits the
// BN-key tiles covering the union of those intervals.  When the tile
// straddles the rank's two chunks the union can be two intervals, one per
// chunk, and only their key tiles are visited (merged into one run when they
// touch).
struct QTileKeys {
  int a0, na;    // first key tile and count of the first run
  int b0, nb;    // second run (nb == 0 if none)
  int min_pos;   // smallest last key among the tile's rows
  int max_lo;    // largest first key among the tile's rows
};

// Shared by both mask forms: `last(p)` is the last key of position p.
template <int BM, int BN, class Last>
DMGQA_HD QTileKeys qtile_keys_by(int row0, const int32_t* ds, const Geo& g, Last last) {
  const int nrows = g.Sq * g.G;
  const int tokf = row0 / g.G;
  const int tokl = (imin(row0 + BM, nrows) - 1) / g.G;
  const int pf = local_pos(tokf, g.c, g.cp, g.rank);
  const int pl = local_pos(tokl, g.c, g.cp, g.rank);
  QTileKeys r;
  r.min_pos = last(pf);
  r.max_lo = ds[pl];
  int a_lo = ds[pf], a_hi, b_lo = 0, b_hi = -1;
  if (tokf < g.c && tokl >= g.c) {
    a_hi = last(local_pos(g.c - 1, g.c, g.cp, g.rank));
    b_lo = ds[local_pos(g.c, g.c, g.cp, g.rank)];
    b_hi = last(pl);
  } else {
    a_hi = last(pl);
  }
  r.a0 = a_lo / BN;
  int a1 = a_hi / BN;
  r.b0 = 0;
  r.nb = 0;
  if (b_hi >= b_lo) {
    const int b0 = b_lo / BN, b1 = b_hi / BN;
    if (b0 <= a1 + 1) {
      a1 = imax(a1, b1);
    } else {
      r.b0 = b0;
      r.nb = b1 - b0 + 1;
    }
  }
  r.na = a1 - r.a0 + 1;
  return r;
}

// Causal interval masks: position p reaches keys ds[p] .. p.
template <int BM, int BN>
DMGQA_HD QTileKeys qtile_keys(int row0, const int32_t* ds, const Geo& g) {
  return qtile_keys_by<BM, BN>(row0, ds, g, [](int p) { return p; });
}

// Explicit ends: position p reaches keys ds[p] .. dh[p]-1 (both
// non-decreasing in p, keys indexed apart from the queries).
template <int BM, int BN>
DMGQA_HD QTileKeys qtile_keys_iv(int row0, const int32_t* ds, const int32_t* dh, const Geo& g) {
  return qtile_keys_by<BM, BN>(row0, ds, g, [dh](int p) { return dh[p] - 1; });
}

// Key tile [t0, t0+BN) needs no mask for any row of the tile: every row's
// interval contains it (the rows' first keys are at most max_lo and their
// last keys at least min_pos).
DMGQA_HD bool qtile_full(const QTileKeys& kr, int t0, int BN) {
  return kr.max_lo <= t0 && t0 + BN - 1 <= kr.min_pos;
}

// Local token ranges whose positions fall in [p0, p1): at most one range in
// each of the rank's two chunks, [a0, a0+na) and [b0, b0+nb) (b0 >= c).
DMGQA_HD void token_ranges(int p0, int p1, const Geo& g, int& a0, int& na, int& b0, int& nb) {
  const int baseA = g.rank * g.c;
  const int baseB = (2 * g.cp - 1 - g.rank) * g.c;
  const int la = imin(imax(p0 - baseA, 0), g.c), ha = imin(imax(p1 - baseA, 0), g.c);
  const int lb = imin(imax(p0 - baseB, 0), g.c), hb = imin(imax(p1 - baseB, 0), g.c);
  a0 = la; na = imax(0, ha - la);
  b0 = g.c + lb; nb = imax(0, hb - lb);
}

// Query tokens that reach key tile kt (kDkdvBN keys): the positions
// [first reaching position of its first key, one past the last of its last
// key) -- both ends non-decreasing in the key, so the union over the tile's
// keys is that one range.  The first reaching position of key t is t itself
// for the causal masks (kfirst_b null), else kfirst_b[t].
DMGQA_HD void key_tile_tokens(const int32_t* kfirst_b, const int32_t* dend_b, int kt,
                              const Geo& g, int& a0, int& na, int& b0, int& nb) {
  const int t0 = kt * kDkdvBN;
  const int tl = imin(t0 + kDkdvBN - 1, g.Skv - 1);
  const int p1 = dend_b[tl];
  const int p0 = kfirst_b ? kfirst_b[t0] : t0;
  token_ranges(p0, p1, g, a0, na, b0, nb);
}

// Stash blocks (kStashRows query rows x kDkdvBN keys of dS) of a key tile
// with token runs (a0, na, b0, nb): the tile reaches one contiguous range of
// local tokens [tlo, thi) (when it reaches both chunks the first part runs
// to the end of the rank's first chunk and the second starts at the
// beginning of the second), i.e. the query rows [tlo*G, thi*G), which the
// blocks cover aligned to kStashRows.
DMGQA_HD int stash_blocks(int a0, int na, int b0, int nb, const Geo& g) {
  const int tlo = na > 0 ? a0 : b0, thi = nb > 0 ? b0 + nb : a0 + na;
  if (thi <= tlo) return 0;
  return (thi * g.G + kStashRows - 1) / kStashRows - tlo * g.G / kStashRows;
}

// Rows of a dK/dV work item that reach key `key`.  The item's rows are the
// virtual rows [r_begin, r_end) of the tile's row list: token index ti (run
// A then run B, positions increasing) times G plus the head in the group.
// The key is reached by the local tokens with positions in [f, dend[key])
// (f = key for the causal masks, kfirst_b[key] else): a contiguous run
// [ti_lo, ti_hi) of the token list, i.e. virtual rows [G*ti_lo, G*ti_hi),
// clipped here to the item's rows.  Keys at or past Skv reach no row (empty
// range at r_end).  Both ends grow with the key.
DMGQA_HD void key_rows(int key, const int32_t* kfirst_b, const int32_t* dend_b, int a0, int na,
                       int b0, int nb, const Geo& g, int r_begin, int r_end, int& vr_lo,
                       int& vr_hi) {
  vr_lo = r_end;
  vr_hi = r_end;
  if (key >= g.Skv) return;
  const int A = g.rank * g.c + a0;
  const int Bb = (2 * g.cp - 1 - g.rank) * g.c + (b0 - g.c);
  const int e = dend_b[key];
  const int f = kfirst_b ? kfirst_b[key] : key;
  const int ti_lo = imin(imax(f - A, 0), na) + imin(imax(f - Bb, 0), nb);
  const int ti_hi = imin(imax(e - A, 0), na) + imin(imax(e - Bb, 0), nb);
  vr_lo = imin(imax(ti_lo * g.G, r_begin), r_end);
  vr_hi = imin(imax(ti_hi * g.G, r_begin), r_end);
}

}  // namespace dmgqa
