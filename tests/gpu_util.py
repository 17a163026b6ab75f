"""Helpers of the GPU parity tests: run a workload through the C ABI and
compare with the CPU oracle."""
from __future__ import annotations

import json
import os
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


WS_KINDS = ("default", "full", "mixed", "recompute")


def bwd_workspace_bytes(case: W.Case, ws: str) -> int:
    """Backward workspace size for each way of forming dQ:
    "default": what docmask_gqa_bwd_workspace_size asks for (the whole dS
    stash, or a 2 GiB stash budget for the long shapes);
    "full": the whole worst-case stash;
    "mixed": the minimum, the partial-dQ buffer and a stash of about a third
    of the worst case, so that some key tiles are stashed and the rest
    recomputed;
    "recompute": the minimum (no stash)."""
    B, Sq, Hq, D = case.q.shape
    args = (B, Sq * case.cfg.cp_size, case.Skv, Hq, case.cfg.Hkv, D, case.cfg.cp_size)
    bm = M.docmask_gqa_bwd_workspace_size_min(*args)
    if ws == "recompute":
        return bm
    if ws == "default":
        return M.docmask_gqa_bwd_workspace_size(*args)
    bf = M.docmask_gqa_bwd_workspace_size_full(*args)
    if ws == "full":
        return bf
    assert ws == "mixed", ws
    per_block = case.cfg.Hkv * 32 * 128 * 2
    dq_part = (B * Sq * Hq * D * 4 + 255) // 256 * 256
    # a third of the worst case, less if the partial-dQ buffer and that
    # stash together would already hold the rank's whole stash
    blocks = max(1, (bf - bm) // per_block // 3)
    while blocks >= 1:
        n = bm + dq_part + blocks * per_block
        if M.docmask_gqa_bwd_path(*args, case.rank, n) == M.DMGQA_BWD_PATH_MIXED:
            return n
        blocks //= 2
    return -1


EXPECT_PATH = {"full": (M.DMGQA_BWD_PATH_STASH,), "mixed": (M.DMGQA_BWD_PATH_MIXED,),
               "recompute": (M.DMGQA_BWD_PATH_RECOMPUTE,),
               "default": (M.DMGQA_BWD_PATH_STASH, M.DMGQA_BWD_PATH_MIXED)}
# which of these kernels each path launches (the recomputing dQ of the key
# tiles past the stash budget; the separate partial-sum reduce, which the
# stash paths run inside the dQ-from-stash launch)
PATH_KERNELS = {M.DMGQA_BWD_PATH_STASH: set(),
                M.DMGQA_BWD_PATH_MIXED: {"bwd_dq_rest"},
                M.DMGQA_BWD_PATH_RECOMPUTE: {"bwd_reduce"}}


def gpu_bwd(case: W.Case, d, out, lse, use_cu=False, ws="default"):
    """Backward through the C ABI with the workspace of kind `ws` (see
    bwd_workspace_bytes); checks that the library takes the expected dQ path
    (its path query, and the kernels that actually launched)."""
    kw = {"cu_seqlens": d["cu_seqlens"]} if use_cu else {"doc_ids": d["doc_ids"]}
    B, Sq, Hq, D = case.q.shape
    n = bwd_workspace_bytes(case, ws)
    if n < 0:
        import pytest
        pytest.skip("no workspace between the minimum and the whole stash selects the "
                    "budgeted stash for this shape")
    path = M.docmask_gqa_bwd_path(B, Sq * case.cfg.cp_size, case.Skv, Hq, case.cfg.Hkv, D,
                                  case.cfg.cp_size, case.rank, n)
    assert path in EXPECT_PATH[ws], (ws, path)
    kw["workspace"] = torch.empty(max(n, 1), dtype=torch.uint8, device=d["q"].device)
    torch.cuda.synchronize()
    M.docmask_gqa_timing_enable(True)
    try:
        res = M.docmask_gqa_attn_bwd(d["q"], d["k"], d["v"], out, d["dout"], lse,
                                     cp_size=case.cfg.cp_size, cp_rank=case.rank,
                                     softmax_scale=case.scale, **kw)
        ran = M.docmask_gqa_kernel_times()
    finally:
        M.docmask_gqa_timing_enable(False)
    watched = set().union(*PATH_KERNELS.values())
    launched = {k for k in watched if ran.get(k, (0.0, 0))[1] > 0}
    assert launched == PATH_KERNELS[path], (ws, path, ran)
    assert ran.get("bwd_dkdv", (0.0, 0))[1] == 1 and ran.get("bwd_dq", (0.0, 0))[1] == 1, ran
    return res


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(name: str, got, ref, atol=ATOL, rtol=RTOL_L2, tag=None):
    """Element-wise comparison against the oracle within the stated bounds.
    With DMGQA_PARITY_LOG set, each comparison is appended to that file as
    one JSON line (tag, output, max-abs, rel-L2, element count)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    nrm = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got))
    say(f"  {name}: max-abs {mx:.3e}  rel-L2 {rel:.3e}")
    log = os.environ.get("DMGQA_PARITY_LOG")
    if log and tag is not None:
        with open(log, "a") as f:
            f.write(json.dumps({"case": tag, "out": name, "max_abs": mx, "rel_l2": rel,
                                "n": int(got.size)}) + "\n")
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
