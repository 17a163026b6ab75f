"""GPU parity of causal interval masks -- query position p attends to keys
lo[p] .. p -- against the CPU oracle: sliding windows inside documents,
arbitrary non-decreasing window starts, CP ranks, batch rows with different
masks, both backward paths; the bounds builder bit-exact against a host
computation and against the document-bounds builder."""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import context_gqa_amd as M
import oracle
import workloads as W
from tests.gpu_util import EXPECT_PATH, bwd_workspace_bytes, compare, host, say
from tests.test_gpu_parity import _cfg, _rng_lengths

pytestmark = pytest.mark.gpu


def window_lo(lengths, wn):
    """Sliding window of wn keys inside documents: max(document start, p - wn + 1)."""
    starts = np.repeat(np.concatenate([[0], np.cumsum(lengths)[:-1]]), lengths)
    p = np.arange(sum(lengths))
    return np.maximum(starts, p - wn + 1).astype(np.int32)


def random_lo(S, seed, max_back=300):
    """A non-decreasing window start with 0 <= lo[p] <= p and irregular steps."""
    rng = np.random.default_rng(seed)
    p = np.arange(S)
    lo = np.maximum.accumulate(np.maximum(p - rng.integers(0, max_back, S), 0))
    return np.minimum(lo, p).astype(np.int32)


def dend_from_lo(lo, Skv):
    """One past the last query position p with lo[p] <= t, capped at Skv."""
    t = np.arange(Skv)
    return np.minimum(np.searchsorted(lo, t, side="right"), Skv).astype(np.int32)


# (id, config, seed, rank, lengths per batch row, mask per batch row: window
# length or "random")
CASES = [
    ("win1_tiny", W.CONFIGS["tiny"], 0, 0, None, [1]),
    ("win37_g16_d128", _cfg("a", 1024, 1, 16, 1, 128), 1, 0, [_rng_lengths(1024, 1, 500, 1)], [37]),
    ("win200_cp2_r0", _cfg("b", 2048, 2, 8, 2, 128), 2, 0, [_rng_lengths(2048, 1, 900, 2)], [200]),
    ("win200_cp2_r1", _cfg("b", 2048, 2, 8, 2, 128), 2, 1, [_rng_lengths(2048, 1, 900, 2)], [200]),
    ("win64_ragged_g3_d64_cp2_r1", _cfg("c", 1000, 2, 6, 2, 64), 3, 1,
     [_rng_lengths(1000, 1, 200, 3)], [64]),
    ("random_g16_d128", _cfg("d", 1024, 1, 16, 1, 128), 4, 0, [[1024]], ["random"]),
    ("random_cp3_r2_g3", _cfg("e", 1200, 3, 12, 4, 128), 5, 2, [[1200]], ["random"]),
    ("batch2_cp3_r1_g16", _cfg("f", 768, 3, 16, 1, 128, B=2), 6, 1,
     [_rng_lengths(768, 1, 300, 6), _rng_lengths(768, 50, 700, 7)], [50, 300]),
    ("g1_mha_d64_win129", _cfg("g", 640, 1, 4, 4, 64), 8, 0, [_rng_lengths(640, 1, 250, 8)], [129]),
]


def _case(cfg, seed, rank, lengths, masks):
    if lengths is None:
        lengths = [W.doc_lengths(cfg.doc_kind, cfg.S, seed + 1000 * b) for b in range(cfg.B)]
    if cfg.B != len(lengths):
        cfg = dataclasses.replace(cfg, B=len(lengths))
    case = W.make_case(cfg, seed, rank, lengths=lengths)
    lo = np.stack([window_lo(l, m) if m != "random" else random_lo(cfg.S, seed + 17 * b)
                   for b, (l, m) in enumerate(zip(lengths, masks))])
    return case, lo


def _run(case, lo, ws):
    cfg = case.cfg
    q, k, v, do = (x.cuda() for x in (case.q, case.k, case.v, case.dout))
    bounds = M.docmask_gqa_interval_bounds(torch.from_numpy(lo).cuda(), Skv=case.Skv)
    out, lse = M.docmask_gqa_attn_fwd(q, k, v, cp_size=cfg.cp_size, cp_rank=case.rank,
                                      softmax_scale=case.scale, bounds=bounds)
    n = bwd_workspace_bytes(case, ws)
    if n < 0:
        pytest.skip("no budgeted-stash workspace for this shape")
    B, Sq, Hq, D = case.q.shape
    path = M.docmask_gqa_bwd_path(B, cfg.S, case.Skv, Hq, cfg.Hkv, D, cfg.cp_size, case.rank, n)
    assert path in EXPECT_PATH[ws], (ws, path)
    ws_t = torch.empty(max(n, 1), dtype=torch.uint8, device=q.device)
    dq, dk, dv = M.docmask_gqa_attn_bwd(q, k, v, out, do, lse, cp_size=cfg.cp_size,
                                        cp_rank=case.rank, softmax_scale=case.scale,
                                        bounds=bounds, workspace=ws_t)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


@pytest.mark.parametrize("ws", ["default", "mixed", "recompute"])
@pytest.mark.parametrize("cid,cfg,seed,rank,lengths,masks", CASES, ids=[c[0] for c in CASES])
def test_interval_small_full_oracle(cid, cfg, seed, rank, lengths, masks, ws):
    case, lo = _case(cfg, seed, rank, lengths, masks)
    say(f"[{cid} {ws}] B={case.cfg.B} S={case.cfg.S} cp={case.cfg.cp_size} rank={rank} "
        f"Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} Skv={case.Skv} masks={masks}")
    assert M.docmask_gqa_check_intervals(torch.from_numpy(lo).cuda()) == 0
    out, lse, dq, dk, dv = _run(case, lo, ws)
    rdq, rdk, rdv, rout, rlse = oracle.attn_bwd(case.q, case.k, case.v, case.dout, None,
                                                case.cfg.cp_size, rank, case.scale,
                                                return_fwd=True, lo=lo)
    compare("out", host(out), rout)
    compare("lse", host(lse), rlse)
    compare("dq", host(dq), rdq)
    compare("dk", host(dk), rdk)
    compare("dv", host(dv), rdv)
    # keys that no local query reaches (explicit mask) get exactly zero
    pos = oracle.chunk_positions(case.cfg.S, case.cfg.cp_size, rank)
    for b in range(case.cfg.B):
        reached = oracle.interval_mask(lo[b], pos, case.Skv).any(0)
        assert torch.all(dk[b, torch.from_numpy(~reached).cuda()] == 0)
        assert torch.all(dv[b, torch.from_numpy(~reached).cuda()] == 0)


def test_interval_bounds_bit_exact():
    """The builder's two arrays equal lo and the host's searchsorted end, and
    for lo = document starts the document-bounds builder's output."""
    B, S, Skv = 2, 3000, 2900
    lo = np.stack([random_lo(S, 1), window_lo(_rng_lengths(S, 1, 700, 2), 250)])
    bounds = M.docmask_gqa_interval_bounds(torch.from_numpy(lo).cuda(), Skv=Skv)
    got = bounds[: 2 * B * Skv].cpu().numpy().reshape(2, B, Skv)
    for b in range(B):
        assert np.array_equal(got[0, b], lo[b, :Skv])
        assert np.array_equal(got[1, b], dend_from_lo(lo[b], Skv))
    lengths = [_rng_lengths(S, 1, 500, 3), _rng_lengths(S, 20, 900, 4)]
    starts = np.stack([window_lo(l, S + 1) for l in lengths])   # window longer than S: doc starts
    doc = torch.from_numpy(np.stack([W.doc_ids_from_lengths(l) for l in lengths])).cuda()
    a = M.docmask_gqa_interval_bounds(torch.from_numpy(starts).cuda(), Skv=Skv)
    d = M.docmask_gqa_doc_bounds(doc, B=B, S=S, Skv=Skv)
    assert torch.equal(a[: 2 * B * Skv], d[: 2 * B * Skv])


def test_check_intervals():
    S = 100
    good = random_lo(S, 3)
    assert M.docmask_gqa_check_intervals(torch.from_numpy(good[None]).cuda()) == 0
    ahead = good.copy(); ahead[10] = 11             # lo[p] > p
    down = good.copy(); down[50] = down[49] - 1 if down[49] > 0 else -1   # decreasing (or < 0)
    neg = good.copy(); neg[0] = -1
    for bad in (ahead, down, neg):
        assert M.docmask_gqa_check_intervals(torch.from_numpy(bad[None]).cuda()) == 1


@pytest.mark.parametrize("name,rank,wn,ws", [("tp405b", 0, 2048, "default"),
                                             ("tp405b", 0, 300, "recompute"),
                                             ("tp405b", 0, 1024, "mixed"),
                                             ("long_cp", 7, 4096, "default")])
def test_interval_full_size_elementwise(name, rank, wn, ws):
    """At the workloads' full sizes, with a sliding window of wn keys inside
    the documents: every element of out, lse, dq, dk and dv against the
    oracle's full tensors."""
    cfg = W.CONFIGS[name]
    case = W.make_case(cfg, 0, rank)
    lo = window_lo(case.lengths[0], wn)[None]
    say(f"[{name} rank {rank} window {wn} {ws}] S={cfg.S} cp={cfg.cp_size} Skv={case.Skv}")
    out, lse, dq, dk, dv = _run(case, lo, ws)
    rdq, rdk, rdv, rout, rlse = oracle.attn_bwd(case.q, case.k, case.v, case.dout, None,
                                                cfg.cp_size, rank, case.scale, return_fwd=True,
                                                lo=lo)
    tag = f"{name} window {wn} rank {rank} {ws}"
    compare("out", host(out), rout, tag=tag)
    compare("lse", host(lse), rlse, tag=tag)
    compare("dq", host(dq), rdq, tag=tag)
    compare("dk", host(dk), rdk, tag=tag)
    compare("dv", host(dv), rdv, tag=tag)
