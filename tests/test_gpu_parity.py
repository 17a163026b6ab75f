"""GPU parity: the HIP library (called through the C ABI) against the CPU
fp64 oracle on the same seeded inputs.

Tolerance (floating point): max-abs <= 2e-2 and relative L2 <= 5e-3 against
fp64 for out, lse, dq, dk, dv.  Index work (chunk map, document mask) is
checked bit-exactly with q = 0, where every allowed score is equal and
exp(lse) is the exact number of allowed keys.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import context_gqa_amd as M
import oracle
import workloads as W
from tests.gpu_util import (compare, dev, doc_start_end, gpu_bwd, gpu_fwd, host,
                            local_positions, say)

pytestmark = pytest.mark.gpu


def _rng_lengths(S, lo, hi, seed):
    rng = np.random.default_rng(seed)
    out = []
    while sum(out) < S:
        out.append(int(min(rng.integers(lo, hi + 1), S - sum(out))))
    return out


def _cfg(name, S, cp, Hq, Hkv, D, B=1, vs=0.5):
    return W.Config(name, S, cp, tuple(range(cp)), Hq, Hkv, D, "single", vs, True, B=B)


# (id, config, seed, rank, lengths per batch row or None, Skv or None)
SMALL = [(f"tiny_seed{s}", W.CONFIGS["tiny"], s, 0, None, None) for s in range(5)] + [
    ("cp2_g4_d128_r0", _cfg("a", 2048, 2, 8, 2, 128), 1, 0, [_rng_lengths(2048, 1, 400, 1)], None),
    ("cp2_g4_d128_r1", _cfg("a", 2048, 2, 8, 2, 128), 1, 1, [_rng_lengths(2048, 1, 400, 1)], None),
    ("ragged_g3_d64_r0", _cfg("b", 1000, 2, 6, 2, 64), 2, 0, [_rng_lengths(1000, 1, 200, 2)], None),
    ("ragged_g3_d64_r1", _cfg("b", 1000, 2, 6, 2, 64), 2, 1, [_rng_lengths(1000, 1, 200, 2)], None),
    ("ragged_g3_d128_cp3_r2", _cfg("c", 1200, 3, 12, 4, 128), 3, 2, [_rng_lengths(1200, 30, 500, 3)], None),
    ("batch2_cp3_g16_r0", _cfg("d", 768, 3, 16, 1, 128, B=2), 4, 0,
     [_rng_lengths(768, 1, 300, 4), _rng_lengths(768, 50, 700, 5)], None),
    ("batch2_cp3_g16_r2", _cfg("d", 768, 3, 16, 1, 128, B=2), 4, 2,
     [_rng_lengths(768, 1, 300, 4), _rng_lengths(768, 50, 700, 5)], None),
    ("single_doc_2k_g8", _cfg("e", 2048, 1, 8, 1, 128), 5, 0, [[2048]], None),
    ("unit_docs_cp2_r1", _cfg("f", 512, 2, 4, 1, 64), 6, 1, [[1] * 512], None),
    ("extra_kv_rows_cp2_r1", _cfg("g", 1024, 2, 8, 1, 128), 7, 1, [_rng_lengths(1024, 100, 600, 7)], 1024),
    ("g1_mha_d64", _cfg("h", 640, 1, 4, 4, 64), 8, 0, [_rng_lengths(640, 1, 250, 8)], None),
]


def _small_case(cfg, seed, rank, lengths, Skv):
    if lengths is not None and cfg.B != len(lengths):
        cfg = dataclasses.replace(cfg, B=len(lengths))
    return W.make_case(cfg, seed, rank, Skv=Skv, lengths=lengths)


_small_ref = {}


@pytest.mark.parametrize("ws", ["default", "mixed", "recompute"])
@pytest.mark.parametrize("cid,cfg,seed,rank,lengths,Skv", SMALL, ids=[c[0] for c in SMALL])
def test_small_full_oracle(cid, cfg, seed, rank, lengths, Skv, ws):
    """Every output element against the oracle, for each way the backward
    forms dQ: the whole dS stash (default for these sizes), a stash with a
    budget of about a third of the worst case (key tiles past it recomputed)
    and no stash."""
    case = _small_case(cfg, seed, rank, lengths, Skv)
    say(f"[{cid} {ws}] B={case.cfg.B} S={case.cfg.S} cp={case.cfg.cp_size} rank={rank} "
        f"Hq={cfg.Hq} Hkv={cfg.Hkv} D={cfg.D} Skv={case.Skv}")
    d = dev(case)
    out, lse = gpu_fwd(case, d)
    dq, dk, dv = gpu_bwd(case, d, out, lse, ws=ws)
    torch.cuda.synchronize()
    if cid not in _small_ref:
        _small_ref.clear()
        _small_ref[cid] = oracle.attn_bwd(case.q, case.k, case.v, case.dout, case.doc_ids,
                                          case.cfg.cp_size, rank, case.scale, return_fwd=True)
    rdq, rdk, rdv, rout, rlse = _small_ref[cid]
    compare("out", host(out), rout)
    compare("lse", host(lse), rlse)
    compare("dq", host(dq), rdq)
    compare("dk", host(dk), rdk)
    compare("dv", host(dv), rdv)
    # key rows that no local query reaches (explicit mask) are exactly zero
    for b in range(case.cfg.B):
        pos = oracle.chunk_positions(case.cfg.S, case.cfg.cp_size, rank)
        reached = oracle.allowed_mask(case.doc_ids[b], pos, case.Skv).any(0)
        assert torch.all(dk[b, torch.from_numpy(~reached).cuda()] == 0)
        assert torch.all(dv[b, torch.from_numpy(~reached).cuda()] == 0)


def test_cu_seqlens_matches_doc_ids():
    cfg = _cfg("a", 2048, 2, 8, 2, 128)
    case = W.make_case(cfg, 1, 1, lengths=[_rng_lengths(2048, 1, 400, 1)])
    d = dev(case)
    dc = dict(d, cu_seqlens=torch.from_numpy(case.cu_seqlens).cuda())
    a = gpu_fwd(case, d)
    b = gpu_fwd(case, dc, use_cu=True)
    ga = gpu_bwd(case, d, *a)
    gb = gpu_bwd(case, dc, *b, use_cu=True)
    for x, y in zip(a + ga, b + gb):
        assert torch.equal(x, y)


def test_check_docs_entry_points():
    import context_gqa_amd as M
    ok = torch.tensor([[0, 0, 1, 1, 1, 2], [7, 7, 3, 3, 5, 5]], dtype=torch.int32).cuda()
    bad = torch.tensor([[0, 0, 1, 0, 2, 2]], dtype=torch.int32).cuda()
    assert M.docmask_gqa_check_docs(ok) == 0
    assert M.docmask_gqa_check_docs(bad) == 1
    assert M.docmask_gqa_check_cu_seqlens(torch.tensor([0, 2, 5, 6], dtype=torch.int32).cuda(), 6) == 0
    assert M.docmask_gqa_check_cu_seqlens(torch.tensor([0, 2, 2, 6], dtype=torch.int32).cuda(), 6) == 1


def test_empty_inputs():
    import context_gqa_amd as M
    q = torch.empty(0, 8, 4, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(0, 8, 1, 64, dtype=torch.bfloat16, device="cuda")
    doc = torch.empty(0, 8, dtype=torch.int32, device="cuda")
    out, lse = M.docmask_gqa_attn_fwd(q, k, k, doc_ids=doc, cp_size=1, cp_rank=0)
    assert out.shape == q.shape and lse.shape == (0, 8, 4)


# ----------------------------------------------------------- full sizes

# Every output element of every listed configuration, rank and seed against
# the oracle's full tensors, for the backward's dQ paths: the five headline
# seeds of the 405B share, every rank of each workload's rank list.
FULL_ELEMENTWISE = (
    [("llama8b", 0, 0, ws) for ws in ("default", "recompute")] +
    [("tp405b", s, 0, ws) for s in range(5) for ws in ("default", "recompute")] +
    [("long_cp", 0, r, ws) for r in (0, 7) for ws in ("default", "full", "recompute")] +
    [("short_docs", 0, r, ws) for r in range(4) for ws in ("default", "full", "recompute")] +
    [("single_doc", 0, r, ws) for r in range(4) for ws in ("default", "recompute")])

_full_ref = {}


def _full_reference(name, seed, rank, case):
    key = (name, seed, rank)
    if key not in _full_ref:
        _full_ref.clear()
        _full_ref[key] = oracle.attn_bwd(case.q, case.k, case.v, case.dout, case.doc_ids,
                                         case.cfg.cp_size, rank, case.scale, return_fwd=True)
    return _full_ref[key]


@pytest.mark.parametrize("name,seed,rank,ws", FULL_ELEMENTWISE,
                         ids=[f"{n}_s{s}_r{r}_{w}" for n, s, r, w in FULL_ELEMENTWISE])
def test_full_size_elementwise(name, seed, rank, ws):
    cfg = W.CONFIGS[name]
    case = W.make_case(cfg, seed, rank, full=_full_tensors(name, seed))
    say(f"[{name} seed {seed} rank {rank} {ws}] S={cfg.S} cp={cfg.cp_size} Hq={cfg.Hq} "
        f"Hkv={cfg.Hkv} D={cfg.D} Skv={case.Skv} docs={len(case.lengths[0])}")
    d = dev(case)
    out, lse = gpu_fwd(case, d)
    dq, dk, dv = gpu_bwd(case, d, out, lse, ws=ws)
    torch.cuda.synchronize()
    rdq, rdk, rdv, rout, rlse = _full_reference(name, seed, rank, case)
    tag = f"{name} seed {seed} rank {rank} {ws}"
    compare("out", host(out), rout, tag=tag)
    compare("lse", host(lse), rlse, tag=tag)
    compare("dq", host(dq), rdq, tag=tag)
    compare("dk", host(dk), rdk, tag=tag)
    compare("dv", host(dv), rdv, tag=tag)


# Sampled extras: rows and keys picked at chunk edges and document starts.
FULL = [("tp405b", 0, "default"), ("long_cp", 7, "default"), ("short_docs", 2, "default"),
        ("single_doc", 3, "recompute")]

_full_cache = {}


def _full_tensors(name, seed):
    key = (name, seed)
    if key not in _full_cache:
        _full_cache.clear()
        _full_cache[key] = W.full_tensors(W.CONFIGS[name], seed)
    return _full_cache[key]


def _sample_rows(case, n_random=20, seed=0):
    S, cp, r = case.cfg.S, case.cfg.cp_size, case.rank
    c = S // (2 * cp)
    pos = local_positions(S, cp, r)
    start, _ = doc_start_end(case.lengths[0])
    rows = {0, 1, c - 1, c, c + 1, 2 * c - 1}
    # rows at document starts inside the local positions
    firsts = np.flatnonzero(start[pos] == pos)
    rows.update(firsts[:8].tolist())
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, 2 * c, n_random).tolist())
    return sorted(rows)


def _sample_kv(case, max_reach=128, anchors=3, run=4, seed=0):
    """Key positions whose reaching local rows are few, so the oracle can
    afford those rows' full forward: a few anchor keys with small reach and
    the next keys of the same document (whose reaching rows are a subset),
    plus a few unreachable keys."""
    S, cp, r = case.cfg.S, case.cfg.cp_size, case.rank
    pos = local_positions(S, cp, r)
    start, end = doc_start_end(case.lengths[0])
    t = np.arange(case.Skv)
    sp = np.sort(pos)
    reach = np.searchsorted(sp, np.minimum(end[t], case.Skv), side="left") - \
        np.searchsorted(sp, t, side="left")
    ok = np.flatnonzero((reach > 0) & (reach <= max_reach))
    zero = np.flatnonzero(reach == 0)
    rng = np.random.default_rng(seed)
    pick = set()
    for a in (rng.choice(ok, min(anchors, ok.size), replace=False) if ok.size else []):
        for x in range(int(a), min(int(a) + run, case.Skv)):
            if end[x] == end[a]:
                pick.add(x)
    z = rng.choice(zero, min(4, zero.size), replace=False) if zero.size else np.array([], int)
    return sorted(pick), sorted(z.tolist())


def anchors_budget(case):
    return 3 * 128


@pytest.mark.parametrize("name,rank,ws", FULL, ids=[f"{n}_r{r}_{w}" for n, r, w in FULL])
def test_full_size_sampled(name, rank, ws):
    cfg = W.CONFIGS[name]
    case = W.make_case(cfg, 0, rank, full=_full_tensors(name, 0))
    say(f"[{name} rank {rank} {ws}] S={cfg.S} cp={cfg.cp_size} Hq={cfg.Hq} Hkv={cfg.Hkv} "
        f"D={cfg.D} Skv={case.Skv} docs={len(case.lengths[0])}")
    d = dev(case)
    out, lse = gpu_fwd(case, d)
    dq, dk, dv = gpu_bwd(case, d, out, lse, ws=ws)
    torch.cuda.synchronize()
    for nm, t in (("out", out), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert torch.isfinite(t.float()).all(), nm
    rows = _sample_rows(case)
    ro, rl = oracle.attn_fwd_rows(case.q, case.k, case.v, case.doc_ids, cfg.cp_size, rank,
                                  case.scale, 0, rows)
    compare("out[rows]", host(out[0, rows]), ro)
    compare("lse[rows]", host(lse[0, rows]), rl)
    rdq = oracle.attn_bwd_rows(case.q, case.k, case.v, case.dout, case.doc_ids, cfg.cp_size,
                               rank, case.scale, 0, rows)
    compare("dq[rows]", host(dq[0, rows]), rdq)
    kv, zero = _sample_kv(case)
    if kv:
        rdk, rdv = oracle.attn_bwd_kv_rows(case.q, case.k, case.v, case.dout, case.doc_ids,
                                           cfg.cp_size, rank, case.scale, 0, kv,
                                           max_query_rows=anchors_budget(case))
        compare("dk[kv]", host(dk[0, kv]), rdk)
        compare("dv[kv]", host(dv[0, kv]), rdv)
    if zero:
        assert torch.all(dk[0, zero] == 0) and torch.all(dv[0, zero] == 0)


@pytest.mark.parametrize("name,rank", [("long_cp", 7), ("short_docs", 2), ("tp405b", 0),
                                       ("llama8b", 0)])
def test_mask_bit_exact_q_zero(name, rank):
    """q = 0: every allowed score is 0, so exp(lse) is exactly the number of
    allowed keys of the row, for every row and head, and out is the mean of
    the allowed value rows."""
    cfg = W.CONFIGS[name]
    case = W.make_case(cfg, 0, rank, full=_full_tensors(name, 0))
    say(f"[q=0 {name} rank {rank}]")
    d = dev(case)
    d["q"] = torch.zeros_like(d["q"])
    out, lse = gpu_fwd(case, d)
    torch.cuda.synchronize()
    pos = local_positions(cfg.S, cfg.cp_size, rank)
    start, _ = doc_start_end(case.lengths[0])
    count = (pos - start[pos] + 1).astype(np.int64)
    got = np.rint(np.exp(lse[0].double().cpu().numpy())).astype(np.int64)
    assert np.array_equal(got, np.broadcast_to(count[:, None], got.shape))
    rows = _sample_rows(case, n_random=8)
    v = case.v[0].double().numpy()
    G = cfg.Hq // cfg.Hkv
    ref = np.stack([np.stack([v[start[pos[j]]:pos[j] + 1, h // G].mean(0) for h in range(cfg.Hq)])
                    for j in rows])
    compare("out(q=0)[rows]", host(out[0, rows]), ref)


def test_deterministic():
    name = "tp405b"
    case = W.make_case(W.CONFIGS[name], 0, 0, full=_full_tensors(name, 0))
    d = dev(case)
    a = gpu_fwd(case, d)
    ga = gpu_bwd(case, d, *a)
    b = gpu_fwd(case, d)
    gb = gpu_bwd(case, d, *b)
    for x, y in zip(a + ga, b + gb):
        assert torch.equal(x, y)


def test_cp_split_equals_unsplit_on_gpu():
    """Every CP rank's share run in turn on one GPU, scattered to global
    positions, equals the CP=1 run; dK/dV summed over ranks equal CP=1's."""
    cfg = dataclasses.replace(W.CONFIGS["short_docs"], S=8192)
    lengths = [W.doc_lengths("uniform64_1024", 8192, 11)]
    full = W.full_tensors(cfg, 11)
    one = W.make_case(dataclasses.replace(cfg, cp_size=1, ranks=(0,)), 11, 0, full=full,
                      lengths=lengths)
    d1 = dev(one)
    o1, l1 = gpu_fwd(one, d1)
    q1, k1, v1 = gpu_bwd(one, d1, o1, l1)
    o = torch.empty_like(o1); l = torch.empty_like(l1); dq = torch.empty_like(q1)
    dk = torch.zeros_like(k1); dv = torch.zeros_like(v1)
    for r in range(cfg.cp_size):
        case = W.make_case(cfg, 11, r, full=full, lengths=lengths)
        d = dev(case)
        orr, lr = gpu_fwd(case, d)
        qr, kr, vr = gpu_bwd(case, d, orr, lr)
        pos = torch.from_numpy(local_positions(cfg.S, cfg.cp_size, r)).cuda()
        o[0, pos] = orr[0]; l[0, pos] = lr[0]; dq[0, pos] = qr[0]
        dk[:, :case.Skv] += kr; dv[:, :case.Skv] += vr
    torch.cuda.synchronize()
    compare("out cp4 vs cp1", host(o), host(o1))
    compare("lse cp4 vs cp1", host(l), host(l1))
    compare("dq cp4 vs cp1", host(dq), host(q1))
    compare("dk sum vs cp1", host(dk), host(k1))
    compare("dv sum vs cp1", host(dv), host(v1))


@pytest.mark.parametrize("name,seed,rank,use_cu", [("tiny", 0, 0, False), ("tiny", 1, 0, True),
                                                   ("short_docs", 0, 2, False),
                                                   ("short_docs", 1, 0, False),
                                                   ("tp405b", 1, 0, True),
                                                   ("long_cp", 0, 7, False)])
def test_bounds_path_matches_doc_path(name, seed, rank, use_cu):
    """docmask_gqa_doc_bounds equals the host's document starts / ends
    (bit-exact, ends capped at Skv), and the *_bounds calls reproduce the
    doc_ids calls bit for bit (same kernels, same bounds).  Skv from 512 to
    131072 keys (short_docs rank 0: 32768, a multiple of the scan block)."""
    cfg = W.CONFIGS[name]
    case = W.make_case(cfg, seed, rank)
    say(f"[bounds {name} seed {seed} rank {rank} cu={use_cu}]")
    d = dev(case, use_cu=use_cu)
    B, Sq, Hq, D = case.q.shape
    S = Sq * cfg.cp_size
    kw = {"cu_seqlens": d["cu_seqlens"]} if use_cu else {"doc_ids": d["doc_ids"]}
    bounds = M.docmask_gqa_doc_bounds(**kw, B=B, S=S, Skv=case.Skv)
    torch.cuda.synchronize()
    got = bounds[:2 * B * case.Skv].view(2, B, case.Skv).cpu().numpy()
    for b in range(B):
        start, end = doc_start_end(case.lengths[b])
        assert np.array_equal(got[0, b], start[:case.Skv])
        assert np.array_equal(got[1, b], np.minimum(end[:case.Skv], case.Skv))
    out_a, lse_a = gpu_fwd(case, d, use_cu=use_cu)
    out_b, lse_b = M.docmask_gqa_attn_fwd(d["q"], d["k"], d["v"], cp_size=cfg.cp_size,
                                          cp_rank=rank, softmax_scale=case.scale, bounds=bounds)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    if cfg.backward or name == "tiny":
        ga = gpu_bwd(case, d, out_a, lse_a, use_cu=use_cu)
        gb = M.docmask_gqa_attn_bwd(d["q"], d["k"], d["v"], out_a, d["dout"], lse_a,
                                    cp_size=cfg.cp_size, cp_rank=rank, softmax_scale=case.scale,
                                    bounds=bounds)
        torch.cuda.synchronize()
        for x, y in zip(ga, gb):
            assert torch.equal(x, y)


PLAN_CASES = [
    # (id, config, seed, rank, lengths or None, use_cu): document ids and
    # cu_seqlens, B = 1 and 2, Skv from 512 to 102400 keys, D 64 and 128
    ("tiny", W.CONFIGS["tiny"], 0, 0, None, False),
    ("tp405b", W.CONFIGS["tp405b"], 3, 0, None, False),
    ("short_docs_r0", W.CONFIGS["short_docs"], 1, 0, None, False),
    ("short_docs_r3", W.CONFIGS["short_docs"], 2, 3, None, False),
    ("ragged_g3_d64_r1", _cfg("b", 1000, 2, 6, 2, 64), 2, 1, [_rng_lengths(1000, 1, 200, 2)],
     False),
    ("tiny_cu", W.CONFIGS["tiny"], 1, 0, None, True),
    ("batch2_cp3_g16_r2", _cfg("d", 768, 3, 16, 1, 128, B=2), 4, 2,
     [_rng_lengths(768, 1, 300, 4), _rng_lengths(768, 50, 700, 5)], False),
    ("long_cp_r7", W.CONFIGS["long_cp"], 0, 7, None, False),
]


@pytest.mark.parametrize("cid,cfg,seed,rank,lengths,use_cu", PLAN_CASES,
                         ids=[c[0] for c in PLAN_CASES])
def test_plan_path_matches_doc_path(cid, cfg, seed, rank, lengths, use_cu):
    """docmask_gqa_batch_plan: its bounds equal the host's document starts /
    ends (bit-exact), both orders are permutations of the (batch row, query
    tile) items, and the *_plan calls reproduce the doc_ids calls bit for
    bit (the order only decides which workgroup computes a tile)."""
    case = _small_case(cfg, seed, rank, lengths, None) if lengths else W.make_case(cfg, seed, rank)
    say(f"[plan {cid} seed {seed} rank {rank} cu={use_cu}]")
    d = dev(case, use_cu=use_cu)
    B, Sq, Hq, D = case.q.shape
    S = Sq * case.cfg.cp_size
    Hkv = case.cfg.Hkv
    kw = {"cu_seqlens": d["cu_seqlens"]} if use_cu else {"doc_ids": d["doc_ids"]}
    plan = M.docmask_gqa_batch_plan(**kw, B=B, S=S, Skv=case.Skv, Hq=Hq, Hkv=Hkv, D=D,
                                    cp_size=case.cfg.cp_size, cp_rank=rank)
    torch.cuda.synchronize()
    p = plan.cpu().numpy()
    got = p[:2 * B * case.Skv].reshape(2, B, case.Skv)
    for b in range(B):
        start, end = doc_start_end(case.lengths[b])
        assert np.array_equal(got[0, b], start[:case.Skv])
        assert np.array_equal(got[1, b], np.minimum(end[:case.Skv], case.Skv))
    G = Hq // Hkv
    nt = (Sq * G + 127) // 128
    n_items = B * nt
    pos = local_positions(S, case.cfg.cp_size, rank)
    for k, bn in enumerate((64, 128)):   # forward order, dQ order
        o = p[2 * B * case.Skv + k * n_items:2 * B * case.Skv + (k + 1) * n_items]
        assert np.array_equal(np.sort(o), np.arange(n_items))
        # heaviest first: the number of bn-key tiles a query tile's rows
        # reach (the union over its tokens of [start, p]) never grows along
        # the order (costs past the last sort class share it)
        cost = np.empty(n_items, dtype=np.int64)
        for x in range(n_items):
            b, t = divmod(x, nt)
            toks = np.unique(np.arange(128 * t, min(128 * t + 128, Sq * G)) // G)
            pp = pos[toks]
            st = got[0, b][pp]
            tiles = set()
            for a, z in zip(st // bn, pp // bn):
                tiles.update(range(a, z + 1))
            cost[x] = min(len(tiles), 4095)
        assert np.all(np.diff(cost[o]) <= 0), f"order {k} not heaviest first"

    out_a, lse_a = gpu_fwd(case, d, use_cu=use_cu)
    out_b, lse_b = M.docmask_gqa_attn_fwd(d["q"], d["k"], d["v"], cp_size=case.cfg.cp_size,
                                          cp_rank=rank, softmax_scale=case.scale, plan=plan)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    if case.cfg.backward or cid.startswith("tiny"):
        ga = gpu_bwd(case, d, out_a, lse_a, use_cu=use_cu)
        gb = M.docmask_gqa_attn_bwd(d["q"], d["k"], d["v"], out_a, d["dout"], lse_a,
                                    cp_size=case.cfg.cp_size, cp_rank=rank,
                                    softmax_scale=case.scale, plan=plan)
        torch.cuda.synchronize()
        for x, y in zip(ga, gb):
            assert torch.equal(x, y)
