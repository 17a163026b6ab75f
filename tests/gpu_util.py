"""Helpers of the GPU parity tests: run a workload through the C ABI and
compare with the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import context_gqa_amd as M
import workloads as W

ATOL = 2e-2    # max-abs bound against fp64 (the stated parity tolerance)
RTOL_L2 = 5e-3  # relative L2 bound against fp64


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(case: W.Case, use_cu: bool = False):
    d = dict(q=case.q.cuda(), k=case.k.cuda(), v=case.v.cuda(), dout=case.dout.cuda())
    if use_cu:
        d["cu_seqlens"] = torch.from_numpy(case.cu_seqlens).cuda()
    else:
        d["doc_ids"] = torch.from_numpy(case.doc_ids).cuda()
    return d


def gpu_fwd(case: W.Case, d, use_cu=False):
    kw = {"cu_seqlens": d["cu_seqlens"]} if use_cu else {"doc_ids": d["doc_ids"]}
    return M.docmask_gqa_attn_fwd(d["q"], d["k"], d["v"], cp_size=case.cfg.cp_size,
                                  cp_rank=case.rank, softmax_scale=case.scale, **kw)


def gpu_bwd(case: W.Case, d, out, lse, use_cu=False, ws="stash"):
    """ws = "stash": the workspace the library asks for (dS stash path);
    "recompute": the minimum workspace (dQ recomputes S, P and dP)."""
    kw = {"cu_seqlens": d["cu_seqlens"]} if use_cu else {"doc_ids": d["doc_ids"]}
    if ws == "recompute":
        B, Sq, Hq, D = case.q.shape
        n = M.docmask_gqa_bwd_workspace_size_min(B, Sq * case.cfg.cp_size, case.Skv, Hq,
                                                 case.cfg.Hkv, D, case.cfg.cp_size)
        kw["workspace"] = torch.empty(max(n, 1), dtype=torch.uint8, device=d["q"].device)
    else:
        assert ws == "stash", ws
    return M.docmask_gqa_attn_bwd(d["q"], d["k"], d["v"], out, d["dout"], lse,
                                  cp_size=case.cfg.cp_size, cp_rank=case.rank,
                                  softmax_scale=case.scale, **kw)


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(name: str, got, ref, atol=ATOL, rtol=RTOL_L2):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got))
    say(f"  {name}: max-abs {mx:.3e}  rel-L2 {rel:.3e}")
    assert mx <= atol, f"{name}: max-abs {mx} > {atol}"
    assert rel <= rtol, f"{name}: rel-L2 {rel} > {rtol}"
    return mx, rel


def doc_start_end(lengths):
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    ends = np.cumsum(lengths)
    return np.repeat(starts, lengths), np.repeat(ends, lengths)


def local_positions(S, cp, r):
    c = S // (2 * cp)
    return np.concatenate([np.arange(r * c, (r + 1) * c),
                           np.arange((2 * cp - 1 - r) * c, (2 * cp - r) * c)])
