"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments with the documented status before any
HIP call (so none of these calls needs a GPU)."""
import ctypes
import os
import re

import numpy as np
import pytest

import context_gqa_amd as M

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "docmask_gqa.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(docmask_gqa_\w+)\s*\(", text, re.M)))


def test_header_symbols_exported():
    names = declared_functions()
    assert "docmask_gqa_attn_fwd" in names and "docmask_gqa_attn_bwd" in names
    lib = M.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in M.SIGNATURES, n
    assert set(M.SIGNATURES) == set(names)


def test_status_strings():
    assert M.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert M.status_string(s) not in ("ok", "unknown status")
    assert M.status_string(-99) == "unknown status"


def test_workspace_sizes():
    f = M.docmask_gqa_fwd_workspace_size
    b = M.docmask_gqa_bwd_workspace_size
    assert f(1, 8192, 8192, 16, 1, 128, 1) > 0
    assert b(1, 8192, 8192, 16, 1, 128, 1) > f(1, 8192, 8192, 16, 1, 128, 1)
    assert f(0, 8192, 8192, 16, 1, 128, 1) == 0          # empty batch
    assert f(1, 8190, 8190, 16, 1, 128, 4) == 0          # S % (2*cp) != 0 -> invalid -> 0
    assert f(1, 8192, 8192, 16, 3, 128, 1) == 0          # Hq % Hkv != 0
    assert f(1, 8192, 8192, 16, 1, 96, 1) == 0           # unsupported D
    # independent of the document layout, monotone in the key length
    assert f(1, 131072, 102400, 16, 1, 128, 16) <= f(1, 131072, 131072, 16, 1, 128, 16)
    # the minimum backward workspace (no dS stash) is below the full one and
    # above the forward's; both are 0 for the same invalid shapes
    bm = M.docmask_gqa_bwd_workspace_size_min
    for shape in ((1, 8192, 8192, 16, 1, 128, 1), (1, 131072, 131072, 16, 1, 128, 16),
                  (2, 4096, 4096, 32, 8, 64, 2)):
        assert f(*shape) < bm(*shape) < b(*shape)
    assert bm(1, 8190, 8190, 16, 1, 128, 4) == 0 and bm(1, 8192, 8192, 16, 3, 128, 1) == 0
    # the stash reservation is a worst case over document layouts: with one
    # key tile of 128 and 128 query rows it holds all 128 x 128 bf16 scores
    one_tile = (1, 128, 128, 1, 1, 128, 1)
    assert b(*one_tile) - bm(*one_tile) >= 128 * 128 * 2


GiB = 1 << 30
PATH_R, PATH_S, PATH_M = (M.DMGQA_BWD_PATH_RECOMPUTE, M.DMGQA_BWD_PATH_STASH,
                          M.DMGQA_BWD_PATH_MIXED)


@pytest.mark.parametrize("S,cp,Hq,Hkv,D", [(8192, 1, 16, 1, 128), (8192, 1, 32, 8, 128),
                                          (131072, 16, 16, 1, 128), (32768, 4, 16, 1, 128),
                                          (1200, 3, 12, 4, 128), (768, 3, 16, 1, 128),
                                          (1024, 2, 8, 1, 128), (1000, 2, 6, 2, 64)])
def test_bwd_workspace_covers_every_rank(S, cp, Hq, Hkv, D):
    """The size queries take no rank: the full size must give every rank the
    whole stash, whichever Skv from its own prefix to S it passes, and the
    default must give every rank a stash (whole, or with a budget)."""
    b, bm = M.docmask_gqa_bwd_workspace_size, M.docmask_gqa_bwd_workspace_size_min
    bf = M.docmask_gqa_bwd_workspace_size_full
    c = S // (2 * cp)
    for r in range(cp):
        for Skv in sorted({(2 * cp - r) * c, S}):
            shape = (1, S, Skv, Hq, Hkv, D, cp)
            assert bm(*shape) < b(*shape) <= bf(*shape)
            assert M.docmask_gqa_bwd_path(*shape, r, bf(*shape)) == PATH_S, (r, Skv)
            assert M.docmask_gqa_bwd_path(*shape, r, b(*shape)) in (PATH_S, PATH_M), (r, Skv)
            assert M.docmask_gqa_bwd_path(*shape, r, bm(*shape)) == PATH_R
            assert M.docmask_gqa_bwd_path(*shape, r, bm(*shape) - 1) == WS


def test_default_stash_budget():
    """The default backward workspace holds at most a 2 GiB stash plus the
    fp32 partial-dQ buffer; shapes whose worst case fits get all of it."""
    b, bm = M.docmask_gqa_bwd_workspace_size, M.docmask_gqa_bwd_workspace_size_min
    bf = M.docmask_gqa_bwd_workspace_size_full
    tp405b = (1, 8192, 8192, 16, 1, 128, 1)
    assert b(*tp405b) == bf(*tp405b) and M.docmask_gqa_bwd_path(*tp405b, 0, b(*tp405b)) == PATH_S
    for shape in ((1, 131072, 131072, 16, 1, 128, 16), (1, 32768, 32768, 16, 1, 128, 4)):
        dq_part = 8192 * 16 * 128 * 4
        assert b(*shape) <= bm(*shape) + dq_part + 2 * GiB + 256
        assert bf(*shape) > 3 * GiB
        for r in (0, shape[-1] - 1):
            assert M.docmask_gqa_bwd_path(*shape, r, b(*shape)) == PATH_M
    # a workspace with room for the partial-dQ buffer but not one stash block
    # per KV head falls back to recomputing
    shape = (1, 32768, 32768, 16, 1, 128, 4)
    assert M.docmask_gqa_bwd_path(*shape, 0, bm(*shape) + 8192 * 16 * 128 * 4) == PATH_R
    assert M.docmask_gqa_bwd_path(*shape, 0, bm(*shape) + 8192 * 16 * 128 * 4 + 8192) == PATH_M


class _Buf:
    """16-byte aligned host memory standing in for device pointers: every call
    below is rejected before any pointer is dereferenced."""

    def __init__(self, n=4096):
        self.raw = ctypes.create_string_buffer(n + 16)
        a = ctypes.addressof(self.raw)
        self.p = a + (-a) % 16


def _fwd(**kw):
    b = _Buf()
    args = dict(q=b.p, k=b.p, v=b.p, doc=b.p, cu=None, n_docs=0, B=1, S=512, Skv=512, Hq=4,
                Hkv=1, D=64, cp=1, rank=0, scale=0.125, out=b.p, lse=b.p, ws=b.p, wsb=0)
    args.update(kw)
    a = args
    return M.lib().docmask_gqa_attn_fwd(a["q"], a["k"], a["v"], a["doc"], a["cu"], a["n_docs"],
                                        a["B"], a["S"], a["Skv"], a["Hq"], a["Hkv"], a["D"],
                                        a["cp"], a["rank"], a["scale"], a["out"], a["lse"],
                                        a["ws"], a["wsb"], None)


def _bwd(**kw):
    b = _Buf()
    a = dict(q=b.p, k=b.p, v=b.p, out=b.p, dout=b.p, lse=b.p, doc=b.p, cu=None, n_docs=0, B=1,
             S=512, Skv=512, Hq=4, Hkv=1, D=64, cp=1, rank=0, scale=0.125, dq=b.p, dk=b.p,
             dv=b.p, ws=b.p, wsb=0)
    a.update(kw)
    return M.lib().docmask_gqa_attn_bwd(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"],
                                        a["doc"], a["cu"], a["n_docs"], a["B"], a["S"], a["Skv"],
                                        a["Hq"], a["Hkv"], a["D"], a["cp"], a["rank"], a["scale"],
                                        a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], None)


INV, UNS, WS = M.DMGQA_ERR_INVALID_ARG, M.DMGQA_ERR_UNSUPPORTED, M.DMGQA_ERR_WORKSPACE

CASES = [
    (dict(q=None), INV),
    (dict(lse=None), INV),
    (dict(ws=None), INV),
    (dict(rank=1), INV),                       # rank >= cp_size
    (dict(rank=-1), INV),
    (dict(cp=0), INV),
    (dict(S=500, Skv=500, cp=3), INV),          # S % (2*cp) != 0
    (dict(Hq=6, Hkv=4), INV),                   # Hq % Hkv != 0
    (dict(Skv=511), INV),                       # below the needed prefix
    (dict(Skv=513), INV),                       # beyond S
    (dict(S=512, Skv=383, cp=4, rank=1), INV),  # prefix (8-1)*64 = 448 needed
    (dict(doc=None), INV),                      # neither doc_ids nor cu_seqlens
    (dict(cu="same"), INV),                     # both
    (dict(D=96), UNS),
    (dict(D=256), UNS),
    (dict(doc=None, cu="same", B=2, n_docs=3), UNS),   # cu_seqlens with B > 1
    (dict(doc=None, cu="same", n_docs=0), INV),
    (dict(scale=float("nan")), INV),
    (dict(scale=float("inf")), INV),
    (dict(scale=0.0), INV),
    (dict(scale=-0.125), INV),                  # the kernels assume a positive scale
    (dict(scale=-1e-30), INV),
    (dict(B=-1), INV),
    (dict(wsb=0), WS),                          # all valid but workspace too small
]


@pytest.mark.parametrize("kw,want", CASES, ids=[str(c[0]) for c in CASES])
def test_fwd_rejects(kw, want):
    b = _Buf()
    kw = {k: (b.p if v == "same" else v) for k, v in kw.items()}
    assert _fwd(**kw) == want


@pytest.mark.parametrize("kw,want", CASES + [(dict(dout=None), INV), (dict(dk=None), INV)],
                         ids=[str(c[0]) for c in CASES] + ["dout=None", "dk=None"])
def test_bwd_rejects(kw, want):
    b = _Buf()
    kw = {k: (b.p if v == "same" else v) for k, v in kw.items()}
    assert _bwd(**kw) == want


def test_misaligned_pointer_rejected():
    b = _Buf()
    assert _fwd(q=b.p + 2) == INV
    assert _bwd(dq=b.p + 8) == INV


def test_empty_is_noop():
    # nothing to compute: success without touching any pointer
    assert _fwd(B=0, q=None, k=None, v=None, out=None, lse=None, ws=None) == 0
    assert _fwd(S=0, Skv=0, q=None, k=None, v=None, out=None, lse=None, ws=None) == 0
    assert _bwd(B=0, q=None, dq=None, dk=None, dv=None, ws=None) == 0


def test_binding_requires_device_tensors():
    import torch
    q = torch.zeros(1, 512, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 512, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        M.docmask_gqa_attn_fwd(q, k, k, doc_ids=torch.zeros(1, 512, dtype=torch.int32),
                               cp_size=1, cp_rank=0)
    with pytest.raises(TypeError):
        M.docmask_gqa_attn_fwd(q.float(), k, k, doc_ids=torch.zeros(1, 512, dtype=torch.int32),
                               cp_size=1, cp_rank=0)


# ---------------------------------------------------------------- bounds API

def test_doc_bounds_size():
    f = M.docmask_gqa_doc_bounds_size
    # [2, B, Skv] int32 plus two scan aggregates per 1024-position block
    assert f(1, 8192, 8192) == (2 * 8192 + 2 * 8) * 4
    assert f(2, 1000, 700) == (2 * 2 * 700 + 2 * 2 * 1) * 4
    assert f(0, 8, 8) == 0 and f(1, 8, 9) == 0 and f(1, 8, 0) == 0


def _bounds_call(**kw):
    b = _Buf(1 << 16)
    a = dict(doc=b.p, cu=None, n_docs=0, B=1, S=512, Skv=512, out=b.p, nbytes=1 << 16)
    a.update({k: (b.p if v == "same" else v) for k, v in kw.items()})
    return M.lib().docmask_gqa_doc_bounds(a["doc"], a["cu"], a["n_docs"], a["B"], a["S"],
                                          a["Skv"], a["out"], a["nbytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(out=None), INV),
    (dict(doc=None), INV),                                # neither
    (dict(cu="same", n_docs=2), INV),                     # both
    (dict(doc=None, cu="same", n_docs=2, B=2), UNS),      # cu_seqlens with B > 1
    (dict(doc=None, cu="same", n_docs=0), INV),
    (dict(Skv=513), INV),
    (dict(nbytes=100), WS),
])
def test_doc_bounds_rejects(kw, want):
    assert _bounds_call(**kw) == want


def test_bounds_variants_reject():
    b = _Buf()
    L = M.lib()
    common = (1, 512, 512, 4, 1, 64, 1, 0, 0.125)
    # forward: null bounds; misaligned bounds; workspace too small
    assert L.docmask_gqa_attn_fwd_bounds(b.p, b.p, b.p, None, *common, b.p, b.p, b.p, 1 << 12,
                                        None) == INV
    assert L.docmask_gqa_attn_fwd_bounds(b.p, b.p, b.p, b.p + 2, *common, b.p, b.p, b.p,
                                        1 << 12, None) == INV
    assert L.docmask_gqa_attn_fwd_bounds(b.p, b.p, b.p, b.p, *common, b.p, b.p, b.p, 0,
                                        None) == WS
    assert L.docmask_gqa_attn_bwd_bounds(b.p, b.p, b.p, b.p, b.p, b.p, None, *common, b.p, b.p,
                                        b.p, b.p, 1 << 12, None) == INV
    assert L.docmask_gqa_attn_bwd_bounds(b.p, b.p, b.p, b.p, b.p, b.p, b.p, *common, b.p, b.p,
                                        b.p, b.p, 0, None) == WS


# ---------------------------------------------------------------- batch plan API

def test_batch_plan_size():
    f = M.docmask_gqa_batch_plan_size
    # the bounds array, two orders of B * nt query tiles (128 rows), and the
    # bounds scan's aggregates
    nt = 8192 * 16 // 128
    assert f(1, 8192, 8192, 16, 1, 128, 1) == (2 * 8192 + 2 * nt + 2 * 8) * 4
    # rank-independent: Sq = S / cp local tokens, the key prefix given
    nt = (131072 // 16) * 16 // 128
    assert f(1, 131072, 65536, 16, 1, 128, 16) == (2 * 65536 + 2 * nt + 2 * 64) * 4
    # S = 1000, cp = 2: 500 local tokens x 3 heads = 12 tiles per batch row
    assert f(2, 1000, 700, 6, 2, 64, 2) == (2 * 2 * 700 + 2 * 2 * 12 + 2 * 2 * 1) * 4
    # the plan's head is a bounds array
    assert f(1, 8192, 8192, 16, 1, 128, 1) > M.docmask_gqa_doc_bounds_size(1, 8192, 8192)
    assert f(0, 8, 8, 1, 1, 64, 1) == 0 and f(1, 8, 9, 1, 1, 64, 1) == 0
    assert f(1, 8192, 8192, 16, 3, 128, 1) == 0 and f(1, 8192, 8192, 16, 1, 96, 1) == 0


def _plan_call(**kw):
    b = _Buf(1 << 16)
    a = dict(doc=b.p, cu=None, n_docs=0, B=1, S=512, Skv=512, Hq=4, Hkv=1, D=64, cp=1, rank=0,
             out=b.p, nbytes=1 << 16)
    a.update({k: (b.p if v == "same" else v) for k, v in kw.items()})
    return M.lib().docmask_gqa_batch_plan(a["doc"], a["cu"], a["n_docs"], a["B"], a["S"],
                                          a["Skv"], a["Hq"], a["Hkv"], a["D"], a["cp"],
                                          a["rank"], a["out"], a["nbytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(out=None), INV),
    (dict(doc=None), INV),                                # neither
    (dict(cu="same", n_docs=2), INV),                     # both
    (dict(doc=None, cu="same", n_docs=2, B=2), UNS),      # cu_seqlens with B > 1
    (dict(Skv=513), INV),
    (dict(rank=1), INV),                                  # rank out of range
    (dict(Hkv=3), INV),
    (dict(nbytes=100), WS),
])
def test_batch_plan_rejects(kw, want):
    assert _plan_call(**kw) == want


def test_plan_variants_reject():
    b = _Buf()
    L = M.lib()
    common = (1, 512, 512, 4, 1, 64, 1, 0, 0.125)
    assert L.docmask_gqa_attn_fwd_plan(b.p, b.p, b.p, None, *common, b.p, b.p, b.p, 1 << 12,
                                      None) == INV
    assert L.docmask_gqa_attn_fwd_plan(b.p, b.p, b.p, b.p, *common, b.p, b.p, b.p, 0,
                                      None) == WS
    assert L.docmask_gqa_attn_bwd_plan(b.p, b.p, b.p, b.p, b.p, b.p, None, *common, b.p, b.p,
                                      b.p, b.p, 1 << 12, None) == INV
    assert L.docmask_gqa_attn_bwd_plan(b.p, b.p, b.p, b.p, b.p, b.p, b.p, *common, b.p, b.p,
                                      b.p, b.p, 0, None) == WS
    # empty shapes return before reading any pointer
    empty = (0, 512, 512, 4, 1, 64, 1, 0, 0.125)
    assert L.docmask_gqa_attn_fwd_plan(None, None, None, None, *empty, None, None, None, 0,
                                      None) == 0


# ---------------------------------------------------------------- cross-attention forward

def test_cross_workspace_size():
    f = M.lib().docmask_gqa_fwd_cross_workspace_size
    # the tile order: B * ceil(S * G / 128) int32, 256-byte aligned
    assert f(1, 4870, 66775, 16, 1, 128) == -(-(-(-4870 * 16 // 128) * 4) // 256) * 256
    assert f(2, 64, 3000, 4, 4, 64) == 256
    assert f(1, 63, 100, 4, 1, 64) == 256        # any S (no context parallelism)
    assert f(1, 64, 0, 4, 1, 64) == 0            # no keys
    assert f(1, 64, 100, 4, 1, 96) == 0          # D unsupported
    assert f(0, 64, 100, 4, 1, 64) == 0          # empty


def _cross_call(**kw):
    b = _Buf(1 << 16)
    a = dict(q=b.p, k=b.p, v=b.p, lo=b.p, hi=b.p, B=1, S=64, Skv=300, Hq=4, Hkv=1, D=64,
             scale=0.125, out=b.p, lse=b.p, ws=b.p, nbytes=1 << 16)
    a.update(kw)
    return M.lib().docmask_gqa_attn_fwd_cross(a["q"], a["k"], a["v"], a["lo"], a["hi"], a["B"],
                                              a["S"], a["Skv"], a["Hq"], a["Hkv"], a["D"],
                                              a["scale"], a["out"], a["lse"], a["ws"],
                                              a["nbytes"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(lo=None), INV),
    (dict(hi=None), INV),
    (dict(S=-1), INV),
    (dict(Skv=0), INV),
    (dict(Hq=6, Hkv=4), INV),          # Hq % Hkv
    (dict(D=96), UNS),
    (dict(scale=0.0), INV),
    (dict(scale=float("inf")), INV),
    (dict(scale=-0.125), INV),
    (dict(nbytes=4), WS),
    (dict(ws=None), INV),
])
def test_cross_fwd_rejects(kw, want):
    """Every check happens before any HIP call, so these run without a GPU."""
    assert _cross_call(**kw) == want


def test_cross_checker_rejects_sizes():
    L = M.lib()
    assert L.docmask_gqa_check_cross_intervals(None, None, -1, 4, 4, None) == INV
    assert L.docmask_gqa_check_cross_intervals(None, None, 0, 4, 4, None) == 0
    assert L.docmask_gqa_check_cross_intervals(None, None, 1, 4, 4, None) == INV


# ---------------------------------------------------------------- cross-attention backward

def _cross_bwd(**kw):
    b = _Buf(1 << 16)
    a = dict(q=b.p, k=b.p, v=b.p, out=b.p, dout=b.p, lse=b.p, lo=b.p, hi=b.p, B=1, S=63,
             Skv=300, Hq=4, Hkv=1, D=64, scale=0.125, dq=b.p, dk=b.p, dv=b.p, ws=b.p, nbytes=0)
    a.update(kw)
    return M.lib().docmask_gqa_attn_bwd_cross(a["q"], a["k"], a["v"], a["out"], a["dout"],
                                              a["lse"], a["lo"], a["hi"], a["B"], a["S"],
                                              a["Skv"], a["Hq"], a["Hkv"], a["D"], a["scale"],
                                              a["dq"], a["dk"], a["dv"], a["ws"], a["nbytes"],
                                              None)


def test_cross_bwd_workspace_size():
    f = M.lib().docmask_gqa_bwd_cross_workspace_size
    fmin = M.lib().docmask_gqa_bwd_cross_workspace_size_min
    n = fmin(1, 63, 300, 4, 1, 64)
    # the keys' query ranges (2 x Skv int32) come first, then the schedule,
    # the row statistics (2 x S x Hq fp32) and the partial-sum slots
    assert n >= 2 * 300 * 4 + 2 * 63 * 4 * 4
    # the default adds the worst-case dS stash: every one of the 3 key
    # tiles reaching all 63 x 4 query rows (8 blocks of 32 rows, one more
    # for alignment), 32 x 128 bf16 per block
    assert f(1, 63, 300, 4, 1, 64) >= n + 3 * 9 * 32 * 128 * 2
    # past the 2 GiB stash budget: the budget plus the fp32 partial-dQ
    # buffer [B, S, Hq, D]
    big = f(1, 4870, 66775, 16, 1, 128)
    assert (2 << 30) + 4870 * 16 * 128 * 4 <= big - fmin(1, 4870, 66775, 16, 1, 128) \
        <= (2 << 30) + 4870 * 16 * 128 * 4 + (1 << 20)
    assert f(1, 4870, 66775, 16, 1, 128) > f(1, 4870, 6000, 16, 1, 128)
    for g in (f, fmin):
        assert g(0, 63, 300, 4, 1, 64) == 0
        assert g(1, 63, 0, 4, 1, 64) == 0
        assert g(1, 63, 300, 6, 4, 64) == 0


def test_cross_bwd_path():
    """The dQ path a workspace selects for the cross backward: the minimum
    recomputes, the worst-case stash stashes every tile, sizes in between
    (past the partial-dQ buffer) give the mixed path; at the multimodal
    sizes the default (a 2 GiB budget) is the mixed path."""
    f = M.lib().docmask_gqa_bwd_cross_workspace_size
    fmin = M.lib().docmask_gqa_bwd_cross_workspace_size_min
    p = M.docmask_gqa_bwd_cross_path
    small = (1, 63, 300, 4, 1, 64)
    n, full = fmin(*small), f(*small)
    assert p(*small, n) == M.DMGQA_BWD_PATH_RECOMPUTE
    assert p(*small, n - 1) == WS
    assert p(*small, full) == M.DMGQA_BWD_PATH_STASH
    # below the worst case: the partial dQ [1, 63, 4, 64] fp32, then blocks
    dqb = 63 * 4 * 64 * 4
    assert p(*small, n + dqb) == M.DMGQA_BWD_PATH_RECOMPUTE
    assert p(*small, n + dqb + 4096 + 32 * 128 * 2) == M.DMGQA_BWD_PATH_MIXED
    assert p(*small, full - 32 * 128 * 2) == M.DMGQA_BWD_PATH_MIXED
    big = (1, 4870, 66775, 16, 1, 128)
    assert p(*big, f(*big)) == M.DMGQA_BWD_PATH_MIXED
    assert p(*big, fmin(*big)) == M.DMGQA_BWD_PATH_RECOMPUTE
    assert p(1, 63, 300, 6, 4, 64, 1 << 20) == INV
    assert p(1, 0, 300, 4, 1, 64, 0) == M.DMGQA_BWD_PATH_RECOMPUTE


@pytest.mark.parametrize("kw,want", [
    (dict(q=None), INV), (dict(out=None), INV), (dict(dout=None), INV), (dict(lse=None), INV),
    (dict(lo=None), INV), (dict(hi=None), INV), (dict(dq=None), INV), (dict(dk=None), INV),
    (dict(dv=None), INV), (dict(ws=None), INV),
    (dict(S=-1), INV), (dict(Skv=0), INV), (dict(Hq=6, Hkv=4), INV), (dict(D=96), UNS),
    (dict(scale=0.0), INV), (dict(scale=-1.0), INV), (dict(scale=float("nan")), INV),
    (dict(nbytes=16), WS),
])
def test_cross_bwd_rejects(kw, want):
    """Every check happens before any HIP call, so these run without a GPU."""
    kw.setdefault("nbytes", 1 << 16)
    assert _cross_bwd(**kw) == want


def test_cross_bwd_empty_is_noop():
    assert _cross_bwd(B=0, q=None, lo=None, nbytes=0) == 0
    assert _cross_bwd(S=0, nbytes=0) == 0


# ---------------------------------------------------------------- allocation-free forward

def _noalloc(**kw):
    b = _Buf()
    a = dict(q=b.p, k=b.p, v=b.p, doc=b.p, cu=None, n_docs=0, B=1, S=512, Skv=512, Hq=4, Hkv=1,
             D=64, cp=1, rank=0, scale=0.125, out=b.p, lse=b.p)
    a.update(kw)
    return M.lib().docmask_gqa_attn_fwd_noalloc(a["q"], a["k"], a["v"], a["doc"], a["cu"],
                                                a["n_docs"], a["B"], a["S"], a["Skv"], a["Hq"],
                                                a["Hkv"], a["D"], a["cp"], a["rank"], a["scale"],
                                                a["out"], a["lse"], None)


@pytest.mark.parametrize("kw,want", [
    (dict(B=8, S=131072, Skv=131072, Hq=16, Hkv=1, D=128, cp=16), WS),   # beyond 8 MiB
    (dict(scale=-0.5), INV), (dict(scale=0.0), INV), (dict(Hq=6, Hkv=4), INV),
    (dict(S=500, Skv=500, cp=3), INV), (dict(D=96), UNS), (dict(rank=1), INV),
])
def test_noalloc_rejects_before_hip(kw, want):
    """Scalar checks and the scratch limit come before any HIP call."""
    assert _noalloc(**kw) == want


def test_noalloc_empty_is_noop():
    assert _noalloc(B=0, q=None, out=None) == 0
