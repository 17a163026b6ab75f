"""The kernels' index arithmetic (context_gqa_amd/csrc/index.hpp), compiled
for the host with g++, checked bit for bit against the oracle's explicit
mask on every workload, seed 0-4 and listed rank:

* local_pos equals the oracle's chunk map;
* each query tile (128 rows; 64- and 128-key tiles) visits exactly the key
  tiles that hold an allowed pair of its rows (a superset, with explicit
  ends), and calls a tile full (no mask) exactly when every pair of the
  tile's rows and keys is allowed;
* each key tile of the dK/dV schedule lists exactly the local tokens that
  reach one of its keys (a superset, with explicit ends), and its stash
  block count covers exactly their query rows;
* for each key, key_rows gives exactly the tokens that reach it.

The truth side comes from oracle.allowed_mask / interval_mask, reduced per
local token to its first and last allowed key (checked to be an interval);
set equalities are proved from counts plus end points, using that those
first and last keys are non-decreasing along each chunk (also checked).
"""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "index_host.cpp")
KFWD_BM, KDKDV_BN, KSTASH_ROWS = 128, 128, 32
MAX_VISIT = 2048


@pytest.fixture(scope="module")
def idx(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    out = str(tmp_path_factory.mktemp("index") / "libindex_host.so")
    subprocess.run([cxx, "-O2", "-std=c++17", "-shared", "-fPIC", "-Wall", "-Werror", SRC,
                    "-o", out], check=True)
    lib = ctypes.CDLL(out)
    p = ctypes.POINTER(ctypes.c_int32)
    i = ctypes.c_int
    lib.idx_qtiles.argtypes = [p, p] + [i] * 10 + [p, p]
    lib.idx_key_tiles.argtypes = [p, p] + [i] * 8 + [p]
    lib.idx_key_rows.argtypes = [p, p] + [i] * 8 + [p]
    lib.idx_local_pos.argtypes = [i] * 4 + [p]
    for f in (lib.idx_qtiles, lib.idx_key_tiles, lib.idx_key_rows, lib.idx_local_pos):
        f.restype = ctypes.c_int
    return lib


def _p(a):
    if a is None:
        return None
    assert a.dtype == np.int32 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


class Share:
    """One rank's share: geometry, the per-key arrays the kernels read and
    the explicit mask reduced to one allowed-key interval per local token."""

    def __init__(self, S, cp, rank, Hq, Hkv, Skv, pos, mask_rows, ds, dend, kfirst=None,
                 dh=None, c=None, Sq=None):
        self.S, self.cp, self.rank, self.Hq, self.Hkv, self.Skv = S, cp, rank, Hq, Hkv, Skv
        self.G = Hq // Hkv
        self.pos = pos
        self.c = S // (2 * cp) if c is None else c
        self.Sq = pos.size if Sq is None else Sq
        self.ds, self.dend, self.kfirst, self.dh = ds, dend, kfirst, dh
        first = np.empty(pos.size, np.int64)
        last = np.empty(pos.size, np.int64)
        for s in range(0, pos.size, 64):
            M = mask_rows(pos[s:s + 64])
            cnt = M.sum(1)
            assert np.all(cnt > 0), "every local row reaches a key"
            f = np.argmax(M, 1)
            l = Skv - 1 - np.argmax(M[:, ::-1], 1)
            assert np.array_equal(cnt, l - f + 1), "allowed keys of a row form an interval"
            first[s:s + 64] = f
            last[s:s + 64] = l
        self.first, self.last = first, last
        # chunk by chunk, first and last keys do not decrease along the tokens
        for a, b in ((0, self.c), (self.c, self.Sq)):
            assert np.all(np.diff(first[a:b]) >= 0) and np.all(np.diff(last[a:b]) >= 0)

    def geo_args(self):
        return (self.S, self.Skv, self.Hq, self.Hkv, self.cp, self.rank, self.c, self.Sq)


def causal_share(cfg, seed, rank):
    lengths = W.doc_lengths(cfg.doc_kind, cfg.S, seed)
    doc = W.doc_ids_from_lengths(lengths)
    Skv = W.kv_prefix_len(cfg.S, cfg.cp_size, rank)
    pos = oracle.chunk_positions(cfg.S, cfg.cp_size, rank)
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    ends = np.cumsum(lengths)
    dstart = np.repeat(starts, lengths).astype(np.int32)
    dend = np.minimum(np.repeat(ends, lengths), Skv).astype(np.int32)
    if cfg.window is not None:
        lo = W.window_starts(lengths, cfg.window)
        mask_rows = lambda p: oracle.interval_mask(lo, p, Skv)          # noqa: E731
        ds = np.ascontiguousarray(lo[:Skv]).astype(np.int32)
        # one past the last position p with lo[p] <= t
        dend = np.minimum(np.searchsorted(lo, np.arange(Skv), side="right"), Skv)
        dend = np.maximum(dend, np.arange(Skv) + 1).astype(np.int32)
    else:
        mask_rows = lambda p: oracle.allowed_mask(doc, p, Skv)          # noqa: E731
        ds = np.ascontiguousarray(dstart[:Skv])
        dend = np.ascontiguousarray(dend[:Skv])
    return Share(cfg.S, cfg.cp_size, rank, cfg.Hq, cfg.Hkv, Skv, pos, mask_rows, ds, dend)


def cross_share(text, image, Hq, Hkv):
    lo, hi = W.cross_bounds(text, image)
    S, Skv = len(lo), int(sum(image))
    pos = np.arange(S)
    mask_rows = lambda p: oracle.interval_mask(lo, p, Skv, hi)          # noqa: E731
    t = np.arange(Skv)
    kfirst = np.searchsorted(hi, t, side="right").astype(np.int32)     # first p with hi > t
    kend = np.searchsorted(lo, t, side="right").astype(np.int32)       # first p with lo > t
    return Share(S, 1, 0, Hq, Hkv, Skv, pos, mask_rows, lo, kend, kfirst=kfirst, dh=hi,
                 c=S, Sq=S)


# ------------------------------------------------------------------ checks

def qtile_results(idx, sh, bn):
    nt = (sh.Sq * sh.G + KFWD_BM - 1) // KFWD_BM
    head = np.zeros((nt, 6), np.int32)
    visit = np.full((nt, MAX_VISIT, 2), -1, np.int32)
    n = idx.idx_qtiles(_p(sh.ds), _p(sh.dh), *sh.geo_args(), bn, MAX_VISIT, _p(head), _p(visit))
    assert n == nt
    return head, visit


def check_qtiles(sh, bn, head, visit, exact=True):
    """exact: the visited key tiles are exactly those holding an allowed pair
    (the causal forms, whose rows' intervals overlap or touch).  Otherwise
    (explicit ends, where rows of two samples can sit in one tile with a gap
    between their key ranges) a superset; the full / partial class is exact
    either way, so the extra tiles are masked."""
    nkt = (sh.Skv + bn - 1) // bn
    for t in range(head.shape[0]):
        tokf = t * KFWD_BM // sh.G
        tokl = (min(t * KFWD_BM + KFWD_BM, sh.Sq * sh.G) - 1) // sh.G
        f, l = sh.first[tokf:tokl + 1], sh.last[tokf:tokl + 1]
        want = np.zeros(nkt, bool)
        for a, b in zip(f // bn, l // bn):
            want[a:b + 1] = True
        n = head[t, 1] + head[t, 3]
        v = visit[t, :n]
        got = np.zeros(nkt, bool)
        got[v[:, 0] // bn] = True
        assert np.array_equal(v[:, 0] % bn, np.zeros(n, np.int32)), t
        assert len(set(v[:, 0].tolist())) == n, f"tile {t}: a key tile visited twice"
        if exact:
            assert np.array_equal(got, want), f"tile {t}: visited key tiles"
        else:
            assert np.all(got[want]), f"tile {t}: a key tile with allowed pairs is not visited"
        t0 = v[:, 0].astype(np.int64)
        full = (f.max() <= t0) & (t0 + bn - 1 <= l.min())
        assert np.array_equal(v[:, 1].astype(bool), full), f"tile {t}: full / partial"


def key_tile_results(idx, sh):
    nkt = (sh.Skv + KDKDV_BN - 1) // KDKDV_BN
    out = np.zeros((nkt, 5), np.int32)
    assert idx.idx_key_tiles(_p(sh.kfirst), _p(sh.dend), *sh.geo_args(), _p(out)) == nkt
    return out


def _reach_count(sh, k0, k1):
    """Number of local tokens whose allowed interval meets keys [k0, k1]:
    #{first <= k1} - #{last < k0} (each interval is non-empty)."""
    fs, ls = np.sort(sh.first), np.sort(sh.last)
    return np.searchsorted(fs, k1, side="right") - np.searchsorted(ls, k0, side="left")


def _meets(sh, tok, k0, k1):
    return (sh.first[tok] <= k1) & (sh.last[tok] >= k0)


def check_key_tiles(sh, kt_out, exact=True):
    nkt = kt_out.shape[0]
    t0 = np.arange(nkt) * KDKDV_BN
    tl = np.minimum(t0 + KDKDV_BN - 1, sh.Skv - 1)
    want = _reach_count(sh, t0, tl)
    a0, na, b0, nb, blocks = kt_out.T
    assert np.all(na >= 0) and np.all(nb >= 0)
    assert np.all(a0 + na <= sh.c) and np.all((nb == 0) | ((b0 >= sh.c) & (b0 + nb <= sh.Sq)))
    for kt in range(nkt):
        toks = list(range(a0[kt], a0[kt] + na[kt])) + list(range(b0[kt], b0[kt] + nb[kt]))
        if exact:
            # runs of non-decreasing intervals: the end points meet the tile
            # and the counts agree, so the sets are equal
            assert na[kt] + nb[kt] == want[kt], f"key tile {kt}: token count"
            for s, n in ((a0[kt], na[kt]), (b0[kt], nb[kt])):
                if n:
                    assert _meets(sh, np.array([s, s + n - 1]), t0[kt], tl[kt]).all(), kt
        else:
            reach = np.flatnonzero(_meets(sh, np.arange(sh.Sq), t0[kt], tl[kt]))
            assert set(reach.tolist()) <= set(toks), f"key tile {kt}: a reaching token is missing"
        if toks:
            tlo, thi = min(toks), max(toks) + 1
            assert blocks[kt] == -(-thi * sh.G // KSTASH_ROWS) - tlo * sh.G // KSTASH_ROWS, kt
        else:
            assert blocks[kt] == 0, kt


def key_rows_results(idx, sh):
    out = np.zeros((sh.Skv, 2), np.int32)
    assert idx.idx_key_rows(_p(sh.kfirst), _p(sh.dend), *sh.geo_args(), _p(out)) == sh.Skv
    return out


def check_key_rows(sh, kt_out, kr_out):
    t = np.arange(sh.Skv)
    want = _reach_count(sh, t, t)
    lo, hi = kr_out.T
    assert np.all(hi - lo == want), "per-key token counts"
    nz = hi > lo
    t, lo, hi = t[nz], lo[nz], hi[nz]
    a0, na, b0 = (kt_out[t // KDKDV_BN, i] for i in (0, 1, 2))

    def token(ti):        # token index of the tile's list -> local token
        return np.where(ti < na, a0 + ti, b0 + (ti - na))

    # within each run the first and last keys do not decrease, so every
    # token of a list range reaches the key iff the end points of its part
    # in each run do; with the counts equal, the sets are equal
    ends = [(lo, np.ones_like(lo, bool)), (hi - 1, np.ones_like(lo, bool))]
    straddle = (lo < na) & (hi > na)
    ends += [(na - 1, straddle), (na, straddle)]
    for ti, sel in ends:
        assert _meets(sh, token(ti)[sel], t[sel], t[sel]).all(), "per-key tokens reach the key"


CASES = [(name, seed, rank) for name in ("tiny", "llama8b", "tp405b", "tp405b_swa", "short_docs",
                                          "single_doc", "long_cp")
         for seed in range(5) for rank in W.CONFIGS[name].ranks]


@pytest.mark.parametrize("name,seed,rank", CASES, ids=[f"{n}_s{s}_r{r}" for n, s, r in CASES])
def test_index_bit_exact(idx, name, seed, rank):
    cfg = W.CONFIGS[name]
    sh = causal_share(cfg, seed, rank)
    lp = np.zeros(sh.Sq, np.int32)
    assert idx.idx_local_pos(sh.c, sh.cp, sh.rank, sh.Sq, _p(lp)) == sh.Sq
    assert np.array_equal(lp, sh.pos)
    for bn in (64, 128):
        check_qtiles(sh, bn, *qtile_results(idx, sh, bn))
    kt = key_tile_results(idx, sh)
    check_key_tiles(sh, kt)
    check_key_rows(sh, kt, key_rows_results(idx, sh))


CROSS = [("multimodal", *W.cross_lengths(32, 11), 16, 1),
         ("ragged", [13, 29, 41, 9], [77, 190, 61, 230], 8, 2),
         ("unreached_image", [21, 0, 40], [150, 260, 90], 8, 1),
         ("fewer_keys", [100, 60], [20, 30], 16, 1)]


@pytest.mark.parametrize("cid,text,image,Hq,Hkv", CROSS, ids=[c[0] for c in CROSS])
def test_index_cross_bit_exact(idx, cid, text, image, Hq, Hkv):
    sh = cross_share(text, image, Hq, Hkv)
    for bn in (64, 128):
        check_qtiles(sh, bn, *qtile_results(idx, sh, bn), exact=False)
    kt = key_tile_results(idx, sh)
    check_key_tiles(sh, kt, exact=False)
    check_key_rows(sh, kt, key_rows_results(idx, sh))


PLANTS = ["visit", "full", "tile_tokens", "stash_blocks", "key_rows"]


@pytest.mark.parametrize("plant", PLANTS)
def test_planted_index_mistake_is_caught(idx, plant):
    """One wrong bit in any classifier output fails the checks above."""
    sh = causal_share(W.CONFIGS["tp405b"], 3, 0)
    head, visit = qtile_results(idx, sh, 64)
    kt = key_tile_results(idx, sh)
    kr = key_rows_results(idx, sh)
    t = int(np.argmax(head[:, 1] > 3))
    if plant == "visit":
        visit[t, 1, 0] += 64
    elif plant == "full":
        visit[t, 1, 1] ^= 1
    elif plant == "tile_tokens":
        kt[5, 1] -= 1
    elif plant == "stash_blocks":
        kt[5, 4] += 1
    else:
        kr[777, 1] += 1
    with pytest.raises(AssertionError):
        check_qtiles(sh, 64, head, visit)
        check_key_tiles(sh, kt)
        check_key_rows(sh, kt, kr)
