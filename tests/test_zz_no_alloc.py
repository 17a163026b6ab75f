"""The allocation-free forward, docmask_gqa_attn_fwd_noalloc, called through
the C ABI: two calls in a row on one GPU, the second with a smaller input,
each equal bit for bit to docmask_gqa_attn_fwd with a caller workspace on
the same inputs (the same kernels and bounds: that entry point is the
reference here), and the small one also within the parity bounds of the
oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import context_gqa_amd as M
import oracle
import workloads as W
from tests.gpu_util import compare, host, say

pytestmark = pytest.mark.gpu


def _noalloc_call(case, q, k, v, doc, out, lse):
    B, Sq, Hq, D = q.shape
    cfg = case.cfg
    stream = torch.cuda.current_stream().cuda_stream
    return M.lib().docmask_gqa_attn_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), doc.data_ptr(), None, 0, B, cfg.S, case.Skv,
        Hq, cfg.Hkv, D, cfg.cp_size, case.rank, case.scale, out.data_ptr(), lse.data_ptr(),
        stream)


@pytest.mark.parametrize("cases", [[("long_cp", 0, 7), ("tiny", 1, 0)],
                                   [("tp405b", 3, 0), ("short_docs", 2, 1)]])
def test_noalloc_forward_matches_workspace_forward(cases):
    for name, seed, rank in cases:
        cfg = W.CONFIGS[name]
        case = W.make_case(cfg, seed, rank)
        say(f"[noalloc {name} seed {seed} rank {rank}] S={cfg.S} Skv={case.Skv}")
        q, k, v = case.q.cuda(), case.k.cuda(), case.v.cuda()
        doc = torch.from_numpy(case.doc_ids).cuda()
        out = torch.full_like(q, float("nan"))
        lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
        assert _noalloc_call(case, q, k, v, doc, out, lse) == M.DMGQA_OK
        ref_out, ref_lse = M.docmask_gqa_attn_fwd(q, k, v, doc_ids=doc, cp_size=cfg.cp_size,
                                                  cp_rank=rank, softmax_scale=case.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        if name == "tiny":
            rout, rlse = oracle.attn_fwd(case.q, case.k, case.v, case.doc_ids, cfg.cp_size, rank,
                                         case.scale)
            compare("out", host(out), rout)
            compare("lse", host(lse), rlse)


def test_noalloc_rejects_beyond_scratch():
    """A forward whose workspace exceeds the fixed scratch is refused before
    any HIP call (8 batch rows of the 131072-token share)."""
    cfg = W.CONFIGS["long_cp"]
    B, c = 8, cfg.S // (2 * cfg.cp_size)
    q = torch.empty(B, 2 * c, cfg.Hq, cfg.D, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(B, cfg.S, cfg.Hkv, cfg.D, dtype=torch.bfloat16, device="cuda")
    doc = torch.zeros(B, cfg.S, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    rc = M.lib().docmask_gqa_attn_fwd_noalloc(
        q.data_ptr(), k.data_ptr(), k.data_ptr(), doc.data_ptr(), None, 0, B, cfg.S, cfg.S,
        cfg.Hq, cfg.Hkv, cfg.D, cfg.cp_size, 0, 0.088, out.data_ptr(), lse.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert rc == M.DMGQA_ERR_WORKSPACE
