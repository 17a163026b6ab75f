"""HIP-graph capture of the forward + backward calls (the benchmark replays
one graph per input): every replay, with eager work and synchronisations
between replays, must reproduce the eager results bit for bit (the kernels
are deterministic), including the persistent dK/dV kernel's work counter,
which the scheduling kernel resets on the device in each call."""
from __future__ import annotations

import pytest
import torch

import context_gqa_amd as M
import workloads as W
from gpu_util import say

pytestmark = pytest.mark.gpu


def _buffers(case, d):
    B, Sq, Hq, D = case.q.shape
    cfg = case.cfg
    S = Sq * cfg.cp_size
    t = dict(out=torch.empty_like(d["q"]), lse=torch.empty(B, Sq, Hq, dtype=torch.float32,
                                                           device=d["q"].device),
             dq=torch.empty_like(d["q"]),
             dk=torch.empty(d["k"].shape, dtype=torch.float32, device=d["q"].device),
             dv=torch.empty(d["k"].shape, dtype=torch.float32, device=d["q"].device))
    t["wsf"] = torch.empty(max(1, M.docmask_gqa_fwd_workspace_size(B, S, case.Skv, Hq, cfg.Hkv, D,
                                                                   cfg.cp_size)),
                           dtype=torch.uint8, device=d["q"].device)
    t["wsb"] = torch.empty(max(1, M.docmask_gqa_bwd_workspace_size(B, S, case.Skv, Hq, cfg.Hkv, D,
                                                                   cfg.cp_size)),
                           dtype=torch.uint8, device=d["q"].device)
    return t


def _step(case, d, t):
    cfg = case.cfg
    M.docmask_gqa_attn_fwd(d["q"], d["k"], d["v"], doc_ids=d["doc"], cp_size=cfg.cp_size,
                           cp_rank=case.rank, softmax_scale=case.scale, out=t["out"],
                           lse=t["lse"], workspace=t["wsf"])
    M.docmask_gqa_attn_bwd(d["q"], d["k"], d["v"], t["out"], d["dout"], t["lse"],
                           doc_ids=d["doc"], cp_size=cfg.cp_size, cp_rank=case.rank,
                           softmax_scale=case.scale, dq=t["dq"], dk=t["dk"], dv=t["dv"],
                           workspace=t["wsb"])


@pytest.mark.parametrize("name,seed,rank", [("tp405b", 1, 0), ("short_docs", 0, 2)])
def test_graph_replay_matches_eager(name, seed, rank):
    case = W.make_case(W.CONFIGS[name], seed, rank)
    say(f"graph replay: {name} seed {seed} rank {rank}")
    d = dict(q=case.q.cuda(), k=case.k.cuda(), v=case.v.cuda(), dout=case.dout.cuda(),
             doc=torch.from_numpy(case.doc_ids).cuda())
    t = _buffers(case, d)
    _step(case, d, t)
    torch.cuda.synchronize()
    ref = {k: t[k].clone() for k in ("out", "lse", "dq", "dk", "dv")}

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _step(case, d, t)
    torch.cuda.synchronize()
    for rep in range(3):
        for k in ref:                      # poison the outputs eagerly
            t[k].fill_(float("nan"))
        junk = torch.randn(1024, 1024, device="cuda") @ torch.randn(1024, 1024, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(t[k], ref[k]), f"replay {rep}: {k} differs from the eager result"
        del junk
