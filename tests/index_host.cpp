// Host build of the kernels' index arithmetic (context_gqa_amd/csrc/index.hpp)
// for the CPU index tests: each entry point evaluates one of its functions
// over a whole rank share and writes the results to caller arrays, which the
// tests compare bit for bit with the explicit mask.  Compiled with g++; no
// HIP.
#include <stdint.h>

#include "../context_gqa_amd/csrc/index.hpp"

using namespace dmgqa;

namespace {

Geo make(int S, int Skv, int Hq, int Hkv, int cp, int rank, int c, int Sq) {
  Geo g{};
  g.B = 1; g.S = S; g.Skv = Skv; g.Hq = Hq; g.Hkv = Hkv; g.G = Hq / Hkv;
  g.Sq = Sq; g.c = c; g.cp = cp; g.rank = rank;
  return g;
}

}  // namespace

extern "C" {

// Query tiles of kFwdBM rows: per tile a0, na, b0, nb, min_pos, max_lo, and,
// for every visited key tile (run A then run B, at most max_visit), its
// first key and the full flag (qtile_full).  bn is 64 (forward) or 128 (dQ
// from the stash).  dh null: causal interval masks.  c, Sq: the chunk
// geometry (c = S / (2 cp), Sq = 2c; for explicit ends c = Sq = S).
// Returns the number of tiles, or -1 if a tile visits more than max_visit.
int idx_qtiles(const int32_t* ds, const int32_t* dh, int S, int Skv, int Hq, int Hkv, int cp,
               int rank, int c, int Sq, int bn, int max_visit, int32_t* head,
               int32_t* visit) {
  const Geo g = make(S, Skv, Hq, Hkv, cp, rank, c, Sq);
  const int nt = (Sq * g.G + kFwdBM - 1) / kFwdBM;
  for (int t = 0; t < nt; ++t) {
    QTileKeys kr;
    if (bn == 64)
      kr = dh ? qtile_keys_iv<kFwdBM, 64>(t * kFwdBM, ds, dh, g)
              : qtile_keys<kFwdBM, 64>(t * kFwdBM, ds, g);
    else
      kr = dh ? qtile_keys_iv<kFwdBM, 128>(t * kFwdBM, ds, dh, g)
              : qtile_keys<kFwdBM, 128>(t * kFwdBM, ds, g);
    int32_t* h = head + 6 * t;
    h[0] = kr.a0; h[1] = kr.na; h[2] = kr.b0; h[3] = kr.nb; h[4] = kr.min_pos; h[5] = kr.max_lo;
    const int n = kr.na + kr.nb;
    if (n > max_visit) return -1;
    for (int it = 0; it < n; ++it) {
      const int t0 = (it < kr.na ? kr.a0 + it : kr.b0 + (it - kr.na)) * bn;
      visit[2 * (t * max_visit + it)] = t0;
      visit[2 * (t * max_visit + it) + 1] = qtile_full(kr, t0, bn) ? 1 : 0;
    }
  }
  return nt;
}

// Key tiles of kDkdvBN keys: per tile a0, na, b0, nb (key_tile_tokens) and
// its stash block count (stash_blocks).  kfirst null: causal.
int idx_key_tiles(const int32_t* kfirst, const int32_t* dend, int S, int Skv, int Hq, int Hkv,
                  int cp, int rank, int c, int Sq, int32_t* out) {
  const Geo g = make(S, Skv, Hq, Hkv, cp, rank, c, Sq);
  const int nkt = (Skv + kDkdvBN - 1) / kDkdvBN;
  for (int kt = 0; kt < nkt; ++kt) {
    int a0, na, b0, nb;
    key_tile_tokens(kfirst, dend, kt, g, a0, na, b0, nb);
    int32_t* o = out + 5 * kt;
    o[0] = a0; o[1] = na; o[2] = b0; o[3] = nb; o[4] = stash_blocks(a0, na, b0, nb, g);
  }
  return nkt;
}

// Per key t (of its tile, all of the tile's rows as one item): the token
// index range [ti_lo, ti_hi) of the tile's token list that reaches the key
// (key_rows, divided back by G).
int idx_key_rows(const int32_t* kfirst, const int32_t* dend, int S, int Skv, int Hq, int Hkv,
                 int cp, int rank, int c, int Sq, int32_t* out) {
  const Geo g = make(S, Skv, Hq, Hkv, cp, rank, c, Sq);
  for (int t = 0; t < Skv; ++t) {
    int a0, na, b0, nb;
    key_tile_tokens(kfirst, dend, t / kDkdvBN, g, a0, na, b0, nb);
    const int rows = (na + nb) * g.G;
    int lo, hi;
    key_rows(t, kfirst, dend, a0, na, b0, nb, g, 0, rows, lo, hi);
    if (lo % g.G != 0 || (hi % g.G != 0 && hi != rows)) return -1;
    out[2 * t] = lo / g.G;
    out[2 * t + 1] = hi / g.G;
  }
  return Skv;
}

// local_pos for every local row.
int idx_local_pos(int c, int cp, int rank, int Sq, int32_t* out) {
  for (int j = 0; j < Sq; ++j) out[j] = local_pos(j, c, cp, rank);
  return Sq;
}

}  // extern "C"
