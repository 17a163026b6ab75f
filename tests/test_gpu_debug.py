"""DMGQA_DEBUG=1: every call validates its masking input with the
synchronous checkers and refuses a violated precondition before launching
anything; valid inputs run as usual."""
import numpy as np
import pytest
import torch

import context_gqa_amd as M

pytestmark = pytest.mark.gpu


@pytest.fixture
def debug(monkeypatch):
    monkeypatch.setenv("DMGQA_DEBUG", "1")


def _qkv(S=256, Hq=4, Hkv=1, D=64):
    g = torch.Generator().manual_seed(0)
    q = (torch.randn(1, S, Hq, D, generator=g) * 0.5).to(torch.bfloat16).cuda()
    k = (torch.randn(1, S, Hkv, D, generator=g) * 0.5).to(torch.bfloat16).cuda()
    v = (torch.randn(1, S, Hkv, D, generator=g) * 0.5).to(torch.bfloat16).cuda()
    return q, k, v


def _status(fn):
    try:
        fn()
    except M.DocmaskGQAError as e:
        return e.status
    return M.DMGQA_OK


def test_debug_refuses_bad_doc_ids(debug):
    q, k, v = _qkv()
    good = torch.from_numpy(np.repeat(np.arange(4, dtype=np.int32), 64)[None]).cuda()
    bad = good.clone()
    bad[0, 192:] = 0                      # id 0 appears again after ids 1 and 2
    kw = dict(cp_size=1, cp_rank=0)
    assert _status(lambda: M.docmask_gqa_attn_fwd(q, k, v, good, **kw)) == M.DMGQA_OK
    assert _status(lambda: M.docmask_gqa_attn_fwd(q, k, v, bad, **kw)) == M.DMGQA_ERR_INVALID_ARG
    out, lse = M.docmask_gqa_attn_fwd(q, k, v, good, **kw)
    dout = torch.ones_like(out)
    assert _status(lambda: M.docmask_gqa_attn_bwd(q, k, v, out, dout, lse, bad, **kw)) == \
        M.DMGQA_ERR_INVALID_ARG
    assert _status(lambda: M.docmask_gqa_doc_bounds(bad, B=1, S=256, Skv=256)) == \
        M.DMGQA_ERR_INVALID_ARG
    assert _status(lambda: M.docmask_gqa_batch_plan(bad, B=1, S=256, Skv=256, Hq=4, Hkv=1, D=64,
                                                    cp_size=1, cp_rank=0)) == \
        M.DMGQA_ERR_INVALID_ARG
    torch.cuda.synchronize()


def test_debug_refuses_bad_cu_seqlens(debug):
    q, k, v = _qkv()
    good = torch.tensor([0, 100, 256], dtype=torch.int32).cuda()
    bad = torch.tensor([0, 100, 100, 256], dtype=torch.int32).cuda()   # not increasing
    kw = dict(cp_size=1, cp_rank=0)
    assert _status(lambda: M.docmask_gqa_attn_fwd(q, k, v, cu_seqlens=good, **kw)) == M.DMGQA_OK
    assert _status(lambda: M.docmask_gqa_attn_fwd(q, k, v, cu_seqlens=bad, **kw)) == \
        M.DMGQA_ERR_INVALID_ARG
    torch.cuda.synchronize()


def test_debug_refuses_bad_intervals(debug):
    lo = torch.zeros(1, 256, dtype=torch.int32)
    lo[0, 100] = 101                      # lo[p] > p
    assert _status(lambda: M.docmask_gqa_interval_bounds(lo.cuda(), Skv=256)) == \
        M.DMGQA_ERR_INVALID_ARG
    q, k, v = _qkv()
    lo_x = torch.zeros(1, 256, dtype=torch.int32).cuda()
    hi_x = torch.full((1, 256), 200, dtype=torch.int32).cuda()
    hi_x[0, 10] = 0                       # hi <= lo
    assert _status(lambda: M.docmask_gqa_attn_fwd_cross(q, k, v, lo_x, hi_x)) == \
        M.DMGQA_ERR_INVALID_ARG
    torch.cuda.synchronize()
