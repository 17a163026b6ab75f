"""GPU parity of the cross-attention forward and backward (query token p
attends to keys lo[p] .. hi[p]-1, keys indexed apart from the queries)
against the CPU oracle: packed samples of text queries over their own image
tokens, GQA group sizes 1 / 4 / 16, D 64 and 128, batch rows with different
layouts, fewer keys than queries, one image spanning many key tiles, an odd
number of text tokens, an image no text attends to; the interval checker;
every element at the multimodal size."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import context_gqa_amd as M
import oracle
import workloads as W
from tests.gpu_util import compare, host, say

pytestmark = pytest.mark.gpu

# (id, text lengths per batch row, image lengths per batch row, Hq, Hkv, D, seed)
CASES = [
    ("tiny_d64", [[2, 6]], [[10, 30]], 4, 1, 64, 0),
    ("g16_d128", [[30, 50, 18]], [[400, 700, 333]], 16, 1, 128, 1),
    ("g4_hkv2_ragged", [[13, 29, 41, 9]], [[77, 190, 61, 230]], 8, 2, 128, 2),
    ("mha_g1", [[40, 24]], [[130, 515]], 4, 4, 64, 3),
    ("fewer_keys", [[100, 60]], [[20, 30]], 16, 1, 128, 4),
    ("one_long_image", [[64]], [[3000]], 16, 1, 128, 5),
    ("batch2", [[20, 36], [50, 6]], [[300, 150], [99, 351]], 16, 1, 128, 6),
    ("odd_text", [[33, 50, 18]], [[400, 129, 333]], 16, 1, 128, 7),
    ("unreached_image", [[21, 0, 40]], [[150, 260, 90]], 8, 1, 64, 8),
]


def _case(texts, images, Hq, Hkv, D, seed):
    S = sum(texts[0])
    Skv = sum(images[0])
    assert all(sum(t) == S for t in texts) and all(sum(i) == Skv for i in images)
    lo = np.stack([W.cross_bounds(t, i)[0] for t, i in zip(texts, images)])
    hi = np.stack([W.cross_bounds(t, i)[1] for t, i in zip(texts, images)])
    q, k, v, do = W.cross_tensors(len(texts), S, Skv, Hq, Hkv, D, seed, dout=True)
    return lo, hi, q, k, v, do


@pytest.mark.parametrize("cid,texts,images,Hq,Hkv,D,seed", CASES, ids=[c[0] for c in CASES])
def test_cross_fwd_full_oracle(cid, texts, images, Hq, Hkv, D, seed):
    lo, hi, q, k, v, _ = _case(texts, images, Hq, Hkv, D, seed)
    B, S = lo.shape
    Skv = k.shape[1]
    say(f"[cross {cid}] B={B} S={S} Skv={Skv} Hq={Hq} Hkv={Hkv} D={D}")
    lo_d, hi_d = torch.from_numpy(lo).cuda(), torch.from_numpy(hi).cuda()
    assert M.docmask_gqa_check_cross_intervals(lo_d, hi_d, Skv) == 0
    scale = 1.0 / np.sqrt(D)
    out, lse = M.docmask_gqa_attn_fwd_cross(q.cuda(), k.cuda(), v.cuda(), lo_d, hi_d,
                                            softmax_scale=scale)
    torch.cuda.synchronize()
    rout, rlse = oracle.attn_fwd(q, k, v, None, 1, 0, scale, lo=lo, hi=hi)
    compare("out", host(out), rout)
    compare("lse", host(lse), rlse)


ALIGN = 256   # workspace sections are aligned to this many bytes


def _align(x):
    return (x + ALIGN - 1) // ALIGN * ALIGN


def reached_stash_blocks(lo, hi, Skv, G):
    """dS stash blocks (32 query rows x 128 keys) the layout reaches: per
    128-key tile, its reaching queries [first p with hi[p] > t0, first p with
    lo[p] > last key) as query rows x G, in blocks aligned to 32 rows."""
    total = 0
    for b in range(lo.shape[0]):
        for t0 in range(0, Skv, 128):
            tl = min(t0 + 127, Skv - 1)
            p0 = int(np.searchsorted(hi[b], t0, side="right"))
            p1 = int(np.searchsorted(lo[b], tl, side="right"))
            if p1 > p0:
                total += -(-p1 * G // 32) - (p0 * G // 32)
    return total


def bwd_workspace(kind, lo, hi, B, S, Skv, Hq, Hkv, D):
    """'min': no stash (dQ recomputes the scores); 'default': the size query
    (the stash); 'mixed': the minimum, the fp32 partial-dQ buffer and half of
    the stash blocks the layout reaches, so that some key tiles are stashed
    and the rest recomputed (with a single key tile, where the partial-dQ
    buffer alone is as large as the whole stash, that size stashes every
    tile: tiny_d64, fewer_keys)."""
    if kind == "default":
        return None
    n = M.lib().docmask_gqa_bwd_cross_workspace_size_min(B, S, Skv, Hq, Hkv, D)
    if kind == "mixed":
        need = reached_stash_blocks(lo, hi, Skv, Hq // Hkv)
        n += _align(B * S * Hq * D * 4) + max(need // 2, 1) * Hkv * 32 * 128 * 2
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def _cross_fwd_bwd(q, k, v, do, lo, hi, scale, ws="default"):
    lo_d, hi_d = torch.from_numpy(lo).cuda(), torch.from_numpy(hi).cuda()
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    out, lse = M.docmask_gqa_attn_fwd_cross(qd, kd, vd, lo_d, hi_d, softmax_scale=scale)
    B, S, Hq, D = q.shape
    Skv, Hkv = k.shape[1], k.shape[2]
    work = bwd_workspace(ws, lo, hi, B, S, Skv, Hq, Hkv, D)
    nbytes = (M.lib().docmask_gqa_bwd_cross_workspace_size(B, S, Skv, Hq, Hkv, D)
              if work is None else work.numel())
    path = M.docmask_gqa_bwd_cross_path(B, S, Skv, Hq, Hkv, D, nbytes)
    # the smallest mixed workspace (the partial dQ and one block) already
    # holds the worst case when it is one or two blocks: then it stashes
    one_block = (M.lib().docmask_gqa_bwd_cross_workspace_size_min(B, S, Skv, Hq, Hkv, D) +
                 _align(B * S * Hq * D * 4) + Hkv * 32 * 128 * 2)
    mixed_ok = M.docmask_gqa_bwd_cross_path(B, S, Skv, Hq, Hkv, D, one_block) == \
        M.DMGQA_BWD_PATH_MIXED
    want = {"min": (M.DMGQA_BWD_PATH_RECOMPUTE,),
            "mixed": (M.DMGQA_BWD_PATH_MIXED if mixed_ok else M.DMGQA_BWD_PATH_STASH,),
            "default": (M.DMGQA_BWD_PATH_STASH, M.DMGQA_BWD_PATH_MIXED)}[ws]
    assert path in want, (ws, path)
    say(f"  dQ path {path} ({ws} workspace, {nbytes} bytes)")
    dq, dk, dv = M.docmask_gqa_attn_bwd_cross(qd, kd, vd, out, dod, lse, lo_d, hi_d,
                                              softmax_scale=scale, workspace=work)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


@pytest.mark.parametrize("ws", ["default", "min", "mixed"])
@pytest.mark.parametrize("cid,texts,images,Hq,Hkv,D,seed", CASES, ids=[c[0] for c in CASES])
def test_cross_bwd_full_oracle(cid, texts, images, Hq, Hkv, D, seed, ws):
    """Every element of the backward against the oracle, on each way of
    forming dQ (stash, recompute, mixed); image tokens no text token attends
    to get exactly zero dk / dv."""
    lo, hi, q, k, v, do = _case(texts, images, Hq, Hkv, D, seed)
    B, S = lo.shape
    Skv = k.shape[1]
    say(f"[cross bwd {cid} ws={ws}] B={B} S={S} Skv={Skv} Hq={Hq} Hkv={Hkv} D={D}")
    scale = 1.0 / np.sqrt(D)
    out, lse, dq, dk, dv = _cross_fwd_bwd(q, k, v, do, lo, hi, scale, ws)
    rdq, rdk, rdv, rout, rlse = oracle.attn_bwd(q, k, v, do, None, 1, 0, scale,
                                                return_fwd=True, lo=lo, hi=hi)
    compare("out", host(out), rout)
    compare("lse", host(lse), rlse)
    compare("dq", host(dq), rdq)
    compare("dk", host(dk), rdk)
    compare("dv", host(dv), rdv)
    t = np.arange(Skv)
    for b in range(B):
        reached = ((t[None, :] >= lo[b][:, None]) & (t[None, :] < hi[b][:, None])).any(0)
        unreached = torch.from_numpy(~reached).cuda()
        assert torch.all(dk[b, unreached] == 0) and torch.all(dv[b, unreached] == 0)
        if cid == "unreached_image":
            assert not reached.all()


def test_cross_bwd_multimodal_elementwise():
    """32 samples of 100-199 text tokens against 1200-3000 image tokens each
    (an odd text total), 16 query heads on 1 KV head, d = 128: every element
    of out, lse, dq, dk and dv against the oracle."""
    text, image = W.cross_lengths(32, seed=11)
    lo, hi = W.cross_bounds(text, image)
    S, Skv = sum(text), sum(image)
    q, k, v, do = W.cross_tensors(1, S, Skv, 16, 1, 128, seed=12, dout=True)
    say(f"[cross bwd multimodal] S={S} Skv={Skv}")
    scale = 1.0 / np.sqrt(128)
    rdq, rdk, rdv, rout, rlse = oracle.attn_bwd(q, k, v, do, None, 1, 0, scale,
                                                return_fwd=True, lo=lo[None], hi=hi[None])
    for ws in ("default", "mixed"):
        out, lse, dq, dk, dv = _cross_fwd_bwd(q, k, v, do, lo[None], hi[None], scale, ws)
        tag = f"cross multimodal S={S} Skv={Skv} ws={ws}"
        compare("out", host(out), rout, tag=tag)
        compare("lse", host(lse), rlse, tag=tag)
        compare("dq", host(dq), rdq, tag=tag)
        compare("dk", host(dk), rdk, tag=tag)
        compare("dv", host(dv), rdv, tag=tag)


@pytest.mark.parametrize("ws", ["default", "mixed", "min"])
def test_cross_deterministic(ws):
    """Two calls on the same inputs give bit-identical out, lse, dq, dk and
    dv on each dQ path (the split dK/dV items are summed in a fixed order),
    at the multimodal size."""
    text, image = W.cross_lengths(32, seed=13)
    lo, hi = W.cross_bounds(text, image)
    S, Skv = sum(text), sum(image)
    q, k, v, do = W.cross_tensors(1, S, Skv, 16, 1, 128, seed=14, dout=True)
    say(f"[cross deterministic ws={ws}] S={S} Skv={Skv}")
    scale = 1.0 / np.sqrt(128)
    a = _cross_fwd_bwd(q, k, v, do, lo[None], hi[None], scale, ws)
    b = _cross_fwd_bwd(q, k, v, do, lo[None], hi[None], scale, ws)
    for x, y, n in zip(a, b, ("out", "lse", "dq", "dk", "dv")):
        assert torch.equal(x, y), n


def test_check_cross_intervals():
    lo, hi = W.cross_bounds([3, 5, 4], [10, 2, 7])
    Skv = 19
    good = (torch.from_numpy(lo[None]).cuda(), torch.from_numpy(hi[None]).cuda())
    assert M.docmask_gqa_check_cross_intervals(*good, Skv) == 0
    bad = []
    x = hi.copy(); x[4] = lo[4]                      # empty interval
    bad.append((lo, x))
    x = hi.copy(); x[-1] = Skv + 1                   # past the keys
    bad.append((lo, x))
    x = lo.copy(); x[6] = x[5] - 1                   # decreasing start
    bad.append((x, hi))
    x = lo.copy(); x[0] = -1
    bad.append((x, hi))
    for l, h in bad:
        assert M.docmask_gqa_check_cross_intervals(torch.from_numpy(l[None]).cuda(),
                                                   torch.from_numpy(h[None]).cuda(), Skv) == 1


def test_cross_fwd_multimodal_sampled():
    """32 samples of 100-199 text tokens against 1200-3000 image tokens
    each, 16 query heads on 1 KV head, d = 128: sampled rows against the
    oracle's per-row form."""
    text, image = W.cross_lengths(32, seed=11)
    lo, hi = W.cross_bounds(text, image)
    S, Skv = sum(text), sum(image)
    q, k, v = W.cross_tensors(1, S, Skv, 16, 1, 128, seed=12)
    say(f"[cross multimodal] S={S} Skv={Skv} (odd text total: {S % 2 == 1})")
    scale = 1.0 / np.sqrt(128)
    out, lse = M.docmask_gqa_attn_fwd_cross(q.cuda(), k.cuda(), v.cuda(),
                                            torch.from_numpy(lo[None]).cuda(),
                                            torch.from_numpy(hi[None]).cuda(), softmax_scale=scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    rng = np.random.default_rng(0)
    ends = np.cumsum(text)
    rows = sorted({0, S - 1, int(ends[0]) - 1, int(ends[0]), *rng.integers(0, S, 12).tolist()})
    ro, rl = oracle.attn_fwd_rows(q, k, v, None, 1, 0, scale, 0, rows, lo=lo[None], hi=hi[None])
    compare("out[rows]", host(out[0, rows]), ro)
    compare("lse[rows]", host(lse[0, rows]), rl)
