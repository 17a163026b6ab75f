"""Checks that pin the CPU oracle to facts outside itself.

Each check raises AssertionError on failure.  They take the oracle module as
an argument so that tests can also run them against an oracle with a planted
mistake and confirm that the mistake is caught.

Sources of the facts:
* chunk rule and equal causal work -- "The Llama 3 Herd of Models", section
  3.3.2 (context parallelism), and the guided reading of Herd section 3.3
  ("Context parallelism and FSDP": 2*CP chunks give every GPU equal work under
  the causal mask);
* document mask = attention run on each document alone -- "Paper notes: The
  Llama 3 Herd of Models", "Two architectural choices";
* softmax rows sum to one, online/standard attention equivalence --
  "Training Infrastructure and Systems", "Online softmax";
* library special cases -- torch.nn.functional.scaled_dot_product_attention
  in float64 on the CPU, an implementation independent of the oracle;
* gradients -- central finite differences and torch.autograd in float64.
"""
from __future__ import annotations

import math

import numpy as np
import torch
import torch.nn.functional as F

import workloads as W


def _rand(shape, seed, scale=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * scale


def _case(S, cp, Hq, Hkv, D, lengths, seed=0, B=1, scale_v=0.7):
    assert sum(lengths) == S
    doc = np.stack([W.doc_ids_from_lengths(lengths)] * B)
    q_full = _rand((B, S, Hq, D), seed, scale_v)
    k_full = _rand((B, S, Hkv, D), seed + 1, scale_v)
    v_full = _rand((B, S, Hkv, D), seed + 2, 1.0)
    do_full = _rand((B, S, Hq, D), seed + 3, 1.0)
    return doc, q_full, k_full, v_full, do_full


def _doc_start_from_lengths(lengths):
    """Start position of each token's document, from the lengths alone."""
    starts = np.concatenate([[0], np.cumsum(lengths)[:-1]])
    return np.repeat(starts, lengths)


def _local(x, S, cp, r):
    return W.take_local_rows(x, S, cp, r)


# -------------------------------------------------------------------------

def check_chunk_permutation(orc):
    for S, cp in [(8, 1), (8, 2), (24, 2), (48, 3), (64, 4), (512, 16)]:
        allpos = np.concatenate([orc.chunk_positions(S, cp, r) for r in range(cp)])
        assert np.array_equal(np.sort(allpos), np.arange(S)), (S, cp)
        assert allpos.size == S


def check_causal_equal_work(orc):
    """Single document: every rank's allowed pairs equal S*c + c."""
    for S, cp in [(16, 2), (48, 3), (64, 4), (256, 8), (1024, 4)]:
        c = S // (2 * cp)
        doc = np.zeros((1, S), dtype=np.int32)
        for r in range(cp):
            n = int(orc.allowed_counts(doc, cp, r, S).sum())
            assert n == S * c + c, (S, cp, r, n, S * c + c)


def check_causal_equal_work_single_doc_full():
    """The 32768-token, CP=4 single-document shape: 134,221,824 per rank."""
    S, cp = 32768, 4
    c = S // (2 * cp)
    assert S * c + c == 134_221_824


def check_interval_rule(orc):
    """Allowed count of each local row = p - doc_start(p) + 1."""
    rng = np.random.default_rng(5)
    for S, cp in [(96, 2), (240, 3), (512, 4)]:
        lengths = []
        while sum(lengths) < S:
            lengths.append(int(min(rng.integers(1, 40), S - sum(lengths))))
        doc = W.doc_ids_from_lengths(lengths)[None]
        start = _doc_start_from_lengths(lengths)
        for r in range(cp):
            c = S // (2 * cp)
            pos = np.concatenate([np.arange(r * c, (r + 1) * c),
                                  np.arange((2 * cp - 1 - r) * c, (2 * cp - r) * c)])
            Skv = (2 * cp - r) * c
            got = orc.allowed_counts(doc, cp, r, Skv)[0]
            assert np.array_equal(got, pos - start[pos] + 1), (S, cp, r)


def check_q_zero(orc):
    """q = 0 makes every allowed score equal: lse = ln(count) and out is the
    mean of the allowed value rows."""
    S, cp, Hq, Hkv, D = 64, 2, 4, 2, 8
    lengths = [5, 20, 1, 30, 8]
    doc, q, k, v, _ = _case(S, cp, Hq, Hkv, D, lengths, seed=11)
    start = _doc_start_from_lengths(lengths)
    c = S // (2 * cp)
    for r in range(cp):
        Skv = (2 * cp - r) * c
        ql = np.zeros((1, 2 * c, Hq, D))
        out, lse = orc.attn_fwd(ql, k[:, :Skv], v[:, :Skv], doc, cp, r, 0.3, threads=1)
        pos = np.concatenate([np.arange(r * c, (r + 1) * c),
                              np.arange((2 * cp - 1 - r) * c, (2 * cp - r) * c)])
        for j, p in enumerate(pos):
            cnt = p - start[p] + 1
            for h in range(Hq):
                g = h // (Hq // Hkv)
                assert abs(lse[0, j, h] - math.log(cnt)) < 1e-12
                ref = v[0, start[p]:p + 1, g].mean(0)
                assert np.max(np.abs(out[0, j, h] - ref)) < 1e-12


def check_softmax_rows(orc):
    """Rows of P sum to one, P is zero off the mask, and
    ln P + lse reproduces scale * <q, k> on the mask."""
    S, cp, Hq, Hkv, D = 48, 2, 4, 1, 16
    lengths = [10, 3, 25, 10]
    doc, q, k, v, _ = _case(S, cp, Hq, Hkv, D, lengths, seed=3)
    start = _doc_start_from_lengths(lengths)
    scale = 1 / math.sqrt(D)
    c = S // (2 * cp)
    for r in range(cp):
        Skv = (2 * cp - r) * c
        ql = _local(q, S, cp, r)
        P = orc.attn_probs(ql, k[:, :Skv], doc, cp, r, scale)
        _, lse = orc.attn_fwd(ql, k[:, :Skv], v[:, :Skv], doc, cp, r, scale, threads=1)
        assert np.max(np.abs(P.sum(-1) - 1.0)) < 1e-12
        pos = np.concatenate([np.arange(r * c, (r + 1) * c),
                              np.arange((2 * cp - 1 - r) * c, (2 * cp - r) * c)])
        for j, p in enumerate(pos):
            allowed = np.zeros(Skv, dtype=bool)
            allowed[start[p]:p + 1] = True
            assert np.all(P[0, j, :, ~allowed] == 0.0)
            for h in range(Hq):
                s = scale * np.dot(k[0, :Skv][allowed, 0], ql[0, j, h])
                assert np.max(np.abs(np.log(P[0, j, h, allowed]) + lse[0, j, h] - s)) < 1e-10


def _sdpa_full(q, k, v, mask, scale):
    """torch SDPA in float64; q [B,S,Hq,D], k/v [B,S,Hkv,D] (numpy),
    mask [S,S] bool (True = attend).  K/V heads are repeat-interleaved."""
    G = q.shape[2] // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    out = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale)
    return out.permute(0, 2, 1, 3).numpy()


def _docmask_from_lengths(lengths):
    S = sum(lengths)
    m = np.zeros((S, S), dtype=bool)
    o = 0
    for L in lengths:
        m[o:o + L, o:o + L] = np.tril(np.ones((L, L), dtype=bool))
        o += L
    return m


def check_per_document(orc):
    """CP=1: the document-masked result equals plain causal attention run on
    each document alone (positions rebased), via torch SDPA is_causal=True."""
    S, Hq, Hkv, D = 80, 4, 2, 16
    lengths = [13, 1, 40, 26]
    doc, q, k, v, do = _case(S, 1, Hq, Hkv, D, lengths, seed=21)
    scale = 1 / math.sqrt(D)
    out, lse = orc.attn_fwd(q, k, v, doc, 1, 0, scale, threads=1)
    dq, dk, dv = orc.attn_bwd(q, k, v, do, doc, 1, 0, scale, threads=1)
    G = Hq // Hkv
    o = 0
    for L in lengths:
        sl = slice(o, o + L)
        qt = torch.from_numpy(q[:, sl]).permute(0, 2, 1, 3).clone().requires_grad_(True)
        kt = torch.from_numpy(k[:, sl]).permute(0, 2, 1, 3).clone().requires_grad_(True)
        vt = torch.from_numpy(v[:, sl]).permute(0, 2, 1, 3).clone().requires_grad_(True)
        ref = F.scaled_dot_product_attention(qt, kt.repeat_interleave(G, 1), vt.repeat_interleave(G, 1),
                                             is_causal=True, scale=scale)
        assert np.max(np.abs(out[:, sl] - ref.detach().permute(0, 2, 1, 3).numpy())) < 1e-12
        (ref * torch.from_numpy(do[:, sl]).permute(0, 2, 1, 3)).sum().backward()
        assert np.max(np.abs(dq[:, sl] - qt.grad.permute(0, 2, 1, 3).numpy())) < 1e-11
        assert np.max(np.abs(dk[:, sl] - kt.grad.permute(0, 2, 1, 3).numpy())) < 1e-11
        assert np.max(np.abs(dv[:, sl] - vt.grad.permute(0, 2, 1, 3).numpy())) < 1e-11
        # lse from torch.logsumexp of the causal scores of this document
        s = torch.einsum("bhld,bhmd->bhlm", qt.detach(), kt.detach().repeat_interleave(G, 1)) * scale
        s = s.masked_fill(~torch.tril(torch.ones(L, L, dtype=torch.bool)), float("-inf"))
        ref_lse = torch.logsumexp(s, -1).permute(0, 2, 1).numpy()
        assert np.max(np.abs(lse[:, sl] - ref_lse)) < 1e-12
        o += L


def check_sdpa_explicit_mask(orc):
    """CP ranks of a multi-document sequence equal the rank's rows of full
    SDPA with an explicit block-diagonal causal mask."""
    S, cp, Hq, Hkv, D = 96, 3, 6, 2, 8
    lengths = [7, 30, 2, 41, 16]
    doc, q, k, v, _ = _case(S, cp, Hq, Hkv, D, lengths, seed=31)
    scale = 0.37
    ref = _sdpa_full(q, k, v, _docmask_from_lengths(lengths), scale)
    c = S // (2 * cp)
    for r in range(cp):
        Skv = (2 * cp - r) * c
        out, _ = orc.attn_fwd(_local(q, S, cp, r), k[:, :Skv], v[:, :Skv], doc, cp, r, scale, threads=1)
        assert np.max(np.abs(out - _local(ref, S, cp, r))) < 1e-12, r


def check_gqa_vs_mha(orc):
    """GQA equals MHA with each KV head repeated over its group; dK/dV equal
    the sums over the repeated heads."""
    S, cp, Hq, Hkv, D = 48, 2, 6, 2, 8
    lengths = [20, 28]
    doc, q, k, v, do = _case(S, cp, Hq, Hkv, D, lengths, seed=41)
    G = Hq // Hkv
    for r in range(cp):
        c = S // (2 * cp)
        Skv = (2 * cp - r) * c
        ql, dol = _local(q, S, cp, r), _local(do, S, cp, r)
        kk, vv = k[:, :Skv], v[:, :Skv]
        km, vm = np.repeat(kk, G, axis=2), np.repeat(vv, G, axis=2)
        o1, l1 = orc.attn_fwd(ql, kk, vv, doc, cp, r, 0.5, threads=1)
        o2, l2 = orc.attn_fwd(ql, km, vm, doc, cp, r, 0.5, threads=1)
        assert np.max(np.abs(o1 - o2)) < 1e-13 and np.max(np.abs(l1 - l2)) < 1e-13
        dq1, dk1, dv1 = orc.attn_bwd(ql, kk, vv, dol, doc, cp, r, 0.5, threads=1)
        dq2, dk2, dv2 = orc.attn_bwd(ql, km, vm, dol, doc, cp, r, 0.5, threads=1)
        assert np.max(np.abs(dq1 - dq2)) < 1e-12
        B, Skv_, _, D_ = dk2.shape
        assert np.max(np.abs(dk1 - dk2.reshape(B, Skv_, Hkv, G, D_).sum(3))) < 1e-12
        assert np.max(np.abs(dv1 - dv2.reshape(B, Skv_, Hkv, G, D_).sum(3))) < 1e-12


def check_cp_split(orc):
    """Scattering every rank's rows to their global positions reproduces the
    CP=1 result; dK and dV summed over ranks equal the CP=1 gradients."""
    S, Hq, Hkv, D = 96, 4, 2, 8
    lengths = [11, 35, 4, 46]
    doc, q, k, v, do = _case(S, 1, Hq, Hkv, D, lengths, seed=51)
    scale = 0.4
    o_ref, l_ref = orc.attn_fwd(q, k, v, doc, 1, 0, scale, threads=1)
    dq_ref, dk_ref, dv_ref = orc.attn_bwd(q, k, v, do, doc, 1, 0, scale, threads=1)
    for cp in (2, 3, 4, 6):
        c = S // (2 * cp)
        o = np.full_like(o_ref, np.nan); l = np.full_like(l_ref, np.nan); dq = np.full_like(dq_ref, np.nan)
        dk = np.zeros_like(dk_ref); dv = np.zeros_like(dv_ref)
        for r in range(cp):
            Skv = (2 * cp - r) * c
            ql, dol = _local(q, S, cp, r), _local(do, S, cp, r)
            pos = orc.chunk_positions(S, cp, r)
            o_r, l_r = orc.attn_fwd(ql, k[:, :Skv], v[:, :Skv], doc, cp, r, scale, threads=1)
            dq_r, dk_r, dv_r = orc.attn_bwd(ql, k[:, :Skv], v[:, :Skv], dol, doc, cp, r, scale, threads=1)
            o[:, pos] = o_r; l[:, pos] = l_r; dq[:, pos] = dq_r
            dk[:, :Skv] += dk_r; dv[:, :Skv] += dv_r
        assert np.max(np.abs(o - o_ref)) < 1e-12, cp
        assert np.max(np.abs(l - l_ref)) < 1e-12, cp
        assert np.max(np.abs(dq - dq_ref)) < 1e-12, cp
        assert np.max(np.abs(dk - dk_ref)) < 1e-12, cp
        assert np.max(np.abs(dv - dv_ref)) < 1e-12, cp


def check_finite_differences(orc, n_samples=24):
    """Central differences of L = sum(dO * out) on tiny fp64 inputs
    (S=24, CP=2, Hq=4, Hkv=2, D=8, documents [7, 9, 8]): relative error of
    the sampled gradient entries <= 1e-6."""
    S, cp, Hq, Hkv, D = 24, 2, 4, 2, 8
    lengths = [7, 9, 8]
    doc, q, k, v, do = _case(S, cp, Hq, Hkv, D, lengths, seed=61)
    scale = 1 / math.sqrt(D)
    h = 1e-6
    rng = np.random.default_rng(7)
    c = S // (2 * cp)
    for r in range(cp):
        Skv = (2 * cp - r) * c
        ql, dol = _local(q, S, cp, r).copy(), _local(do, S, cp, r)
        kk, vv = k[:, :Skv].copy(), v[:, :Skv].copy()
        dq, dk, dv = orc.attn_bwd(ql, kk, vv, dol, doc, cp, r, scale, threads=1)

        def loss(qx, kx, vx):
            o, _ = orc.attn_fwd(qx, kx, vx, doc, cp, r, scale, threads=1)
            return float((o * dol).sum())

        for name, arr, grad in (("q", ql, dq), ("k", kk, dk), ("v", vv, dv)):
            idx = [tuple(rng.integers(0, s) for s in arr.shape) for _ in range(n_samples)]
            fd = []
            an = []
            for ix in idx:
                old = arr[ix]
                arr[ix] = old + h
                lp = loss(ql, kk, vv)
                arr[ix] = old - h
                lm = loss(ql, kk, vv)
                arr[ix] = old
                fd.append((lp - lm) / (2 * h))
                an.append(grad[ix])
            fd, an = np.array(fd), np.array(an)
            err = np.linalg.norm(fd - an) / max(np.linalg.norm(an), 1e-30)
            assert err <= 1e-6, (name, r, err)


def check_autograd(orc):
    """dq/dk/dv equal torch.autograd through an explicitly masked softmax in
    float64 (written with torch ops on the whole sequence)."""
    S, cp, Hq, Hkv, D = 64, 2, 4, 1, 16
    lengths = [9, 22, 33]
    doc, q, k, v, do = _case(S, cp, Hq, Hkv, D, lengths, seed=71)
    scale = 0.25
    G = Hq // Hkv
    mask = torch.from_numpy(_docmask_from_lengths(lengths))
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    kr = kt.repeat_interleave(G, dim=2)
    vr = vt.repeat_interleave(G, dim=2)
    s = torch.einsum("bshd,bthd->bhst", qt, kr) * scale
    s = s.masked_fill(~mask, float("-inf"))
    p = torch.softmax(s, -1)
    o = torch.einsum("bhst,bthd->bshd", p, vr)
    c = S // (2 * cp)
    for r in range(cp):
        Skv = (2 * cp - r) * c
        pos = torch.from_numpy(np.concatenate([np.arange(r * c, (r + 1) * c),
                                               np.arange((2 * cp - 1 - r) * c, (2 * cp - r) * c)]))
        dol = _local(do, S, cp, r)
        for t in (qt, kt, vt):
            t.grad = None
        (o[:, pos] * torch.from_numpy(dol)).sum().backward(retain_graph=True)
        dq, dk, dv = orc.attn_bwd(_local(q, S, cp, r), k[:, :Skv], v[:, :Skv], dol, doc, cp, r, scale, threads=1)
        assert np.max(np.abs(dq - qt.grad[:, pos].numpy())) < 1e-11
        assert np.max(np.abs(dk - kt.grad[:, :Skv].numpy())) < 1e-11
        assert np.max(np.abs(dv - vt.grad[:, :Skv].numpy())) < 1e-11
        assert np.all(kt.grad[:, Skv:].numpy() == 0)


def check_window(orc):
    """Column-windowed and full-width forms agree."""
    S, cp, Hq, Hkv, D = 256, 2, 4, 2, 16
    lengths = [40, 100, 3, 113]
    doc, q, k, v, do = _case(S, cp, Hq, Hkv, D, lengths, seed=81)
    for r in range(cp):
        c = S // (2 * cp)
        Skv = (2 * cp - r) * c
        args = (_local(q, S, cp, r), k[:, :Skv], v[:, :Skv], _local(do, S, cp, r), doc, cp, r, 0.3)
        a = orc.attn_bwd(*args, window=True, threads=2, return_fwd=True)
        b = orc.attn_bwd(*args, window=False, threads=1, return_fwd=True)
        for x, y in zip(a, b):
            assert np.max(np.abs(x - y)) < 1e-12


def check_sampled_forms(orc):
    """The per-row and per-key forms equal the full forward/backward."""
    S, cp, Hq, Hkv, D = 128, 2, 8, 2, 16
    lengths = [17, 50, 1, 60]
    doc, q, k, v, do = _case(S, cp, Hq, Hkv, D, lengths, seed=91, B=2)
    doc[1] = W.doc_ids_from_lengths([64, 64])
    scale = 0.3
    for r in range(cp):
        c = S // (2 * cp)
        Skv = (2 * cp - r) * c
        ql, dol = _local(q, S, cp, r), _local(do, S, cp, r)
        kk, vv = k[:, :Skv], v[:, :Skv]
        out, lse = orc.attn_fwd(ql, kk, vv, doc, cp, r, scale, threads=1)
        dq, dk, dv = orc.attn_bwd(ql, kk, vv, dol, doc, cp, r, scale, threads=1)
        rows = [0, 5, c - 1, c, 2 * c - 1]
        kvr = [0, 16, 17, Skv - 1, Skv // 2]
        for b in range(2):
            o2, l2 = orc.attn_fwd_rows(ql, kk, vv, doc, cp, r, scale, b, rows)
            assert np.max(np.abs(o2 - out[b, rows])) < 1e-12
            assert np.max(np.abs(l2 - lse[b, rows])) < 1e-12
            dq2 = orc.attn_bwd_rows(ql, kk, vv, dol, doc, cp, r, scale, b, rows)
            assert np.max(np.abs(dq2 - dq[b, rows])) < 1e-12
            dk2, dv2 = orc.attn_bwd_kv_rows(ql, kk, vv, dol, doc, cp, r, scale, b, kvr)
            assert np.max(np.abs(dk2 - dk[b, kvr])) < 1e-12
            assert np.max(np.abs(dv2 - dv[b, kvr])) < 1e-12


def _window_lo(lengths, Wn):
    """lo[p] of a sliding window of Wn keys inside documents, from the lengths."""
    p = np.arange(sum(lengths))
    return np.maximum(_doc_start_from_lengths(lengths), p - Wn + 1)


def _band_docmask(lengths, Wn):
    """Explicit [S, S] mask: same document, causal, at most Wn keys back."""
    m = _docmask_from_lengths(lengths)
    i = np.arange(m.shape[0])
    return m & (i[None, :] > i[:, None] - Wn)


def check_interval_brute(orc):
    """interval_mask is lo[p] <= t <= p, and the row counts are p - lo[p] + 1."""
    g = np.random.default_rng(5)
    S, Skv = 40, 40
    lo = np.minimum(np.maximum.accumulate(g.integers(0, S, S)), np.arange(S))
    pos = np.arange(S)
    M = orc.interval_mask(lo, pos, Skv)
    for p in range(S):
        for t in range(Skv):
            assert M[p, t] == (lo[p] <= t <= p)
    cnt = orc.allowed_counts(None, 1, 0, Skv, lo=lo[None])
    assert np.array_equal(cnt[0], pos - lo + 1)


def check_interval_sliding_window(orc):
    """A sliding window of W keys inside documents (lo = max(document start,
    p - W + 1)) equals full-sequence attention with an explicit band mask,
    forward through torch SDPA and backward through torch.autograd, both in
    float64, on every CP rank."""
    S, cp, Hq, Hkv, D = 96, 2, 4, 2, 8
    lengths = [11, 40, 1, 44]
    Wn = 7
    doc, q, k, v, do = _case(S, cp, Hq, Hkv, D, lengths, seed=41)
    lo = _window_lo(lengths, Wn)[None]
    scale = 0.3
    mask = _band_docmask(lengths, Wn)
    ref = _sdpa_full(q, k, v, mask, scale)
    G = Hq // Hkv
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    sc = torch.einsum("bshd,bthd->bhst", qt, kt.repeat_interleave(G, dim=2)) * scale
    pr = torch.softmax(sc.masked_fill(~torch.from_numpy(mask), float("-inf")), -1)
    o = torch.einsum("bhst,bthd->bshd", pr, vt.repeat_interleave(G, dim=2))
    c = S // (2 * cp)
    for r in range(cp):
        Skv = (2 * cp - r) * c
        ql, dol = _local(q, S, cp, r), _local(do, S, cp, r)
        out, _ = orc.attn_fwd(ql, k[:, :Skv], v[:, :Skv], None, cp, r, scale, threads=1, lo=lo)
        assert np.max(np.abs(out - _local(ref, S, cp, r))) < 1e-12, r
        pos = torch.from_numpy(orc.chunk_positions(S, cp, r))
        for t in (qt, kt, vt):
            t.grad = None
        (o[:, pos] * torch.from_numpy(dol)).sum().backward(retain_graph=True)
        dq, dk, dv = orc.attn_bwd(ql, k[:, :Skv], v[:, :Skv], dol, None, cp, r, scale,
                                  threads=1, lo=lo)
        assert np.max(np.abs(dq - qt.grad[:, pos].numpy())) < 1e-11
        assert np.max(np.abs(dk - kt.grad[:, :Skv].numpy())) < 1e-11
        assert np.max(np.abs(dv - vt.grad[:, :Skv].numpy())) < 1e-11


def check_interval_is_document_mask(orc):
    """lo = first position of each document gives the document-masked result."""
    S, cp, Hq, Hkv, D = 64, 2, 4, 1, 8
    lengths = [5, 30, 29]
    doc, q, k, v, do = _case(S, cp, Hq, Hkv, D, lengths, seed=51)
    lo = _doc_start_from_lengths(lengths)[None]
    c = S // (2 * cp)
    for r in range(cp):
        Skv = (2 * cp - r) * c
        args = (_local(q, S, cp, r), k[:, :Skv], v[:, :Skv], _local(do, S, cp, r))
        a = orc.attn_bwd(*args, doc, cp, r, 0.4, threads=1, return_fwd=True)
        b = orc.attn_bwd(*args, None, cp, r, 0.4, threads=1, return_fwd=True, lo=lo)
        for x, y in zip(a, b):
            assert np.max(np.abs(x - y)) == 0.0


def _cross_case(text, image, Hq, Hkv, D, seed):
    """Text queries against the image tokens of their own sample: lo / hi of
    every text token (its sample's image span) and random tensors; the keys
    are indexed on their own (Skv = all image tokens)."""
    istart = np.concatenate([[0], np.cumsum(image)[:-1]])
    lo = np.repeat(istart, text)
    hi = np.repeat(istart + np.asarray(image), text)
    S, Skv = sum(text), sum(image)
    q = _rand((1, S, Hq, D), seed, 0.7)
    k = _rand((1, Skv, Hkv, D), seed + 1, 0.7)
    v = _rand((1, Skv, Hkv, D), seed + 2, 1.0)
    do = _rand((1, S, Hq, D), seed + 3, 1.0)
    return lo[None], hi[None], q, k, v, do


def check_cross_brute(orc):
    """With hi, interval_mask is lo[p] <= t < hi[p] over keys indexed on
    their own, and the row counts are hi - lo."""
    g = np.random.default_rng(7)
    S, Skv = 30, 50
    lo = np.sort(g.integers(0, Skv - 1, S))
    hi = np.maximum(np.sort(g.integers(1, Skv + 1, S)), lo + 1)
    pos = np.arange(S)
    M = orc.interval_mask(lo, pos, Skv, hi)
    for p in range(S):
        for t in range(Skv):
            assert M[p, t] == (lo[p] <= t < hi[p])
    cnt = orc.allowed_counts(None, 1, 0, Skv, lo=lo[None], hi=hi[None])
    assert np.array_equal(cnt[0], hi - lo)


def check_cross_attention(orc):
    """Text queries attending to every image token of their own sample (lo,
    hi = the sample's image span, more keys than queries) equal float64
    attention with the explicit block mask: output and log-sum-exp directly,
    gradients through torch.autograd; the per-row and per-key sampled forms
    agree with the full ones.  An even and an odd number of text tokens
    (cross-attention is not split over CP ranks, so any count is valid)."""
    _cross_attention_case(orc, [4, 7, 3, 2], [13, 5, 21, 9])
    _cross_attention_case(orc, [4, 7, 3, 3], [13, 5, 21, 9])


def _cross_attention_case(orc, text, image):
    Hq, Hkv, D = 4, 2, 8
    lo, hi, q, k, v, do = _cross_case(text, image, Hq, Hkv, D, seed=61)
    S, Skv, G, scale = sum(text), sum(image), Hq // Hkv, 0.35
    mask = np.zeros((S, Skv), dtype=bool)
    for p in range(S):
        mask[p, lo[0, p]:hi[0, p]] = True
    qt = torch.from_numpy(q).requires_grad_(True)
    kt = torch.from_numpy(k).requires_grad_(True)
    vt = torch.from_numpy(v).requires_grad_(True)
    sc = torch.einsum("bshd,bthd->bhst", qt, kt.repeat_interleave(G, dim=2)) * scale
    sc = sc.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.einsum("bhst,bthd->bshd", torch.softmax(sc, -1), vt.repeat_interleave(G, dim=2))
    lse_ref = torch.logsumexp(sc, -1).permute(0, 2, 1).detach().numpy()
    (o * torch.from_numpy(do)).sum().backward()
    dq, dk, dv, out, lse = orc.attn_bwd(q, k, v, do, None, 1, 0, scale, threads=1,
                                        return_fwd=True, lo=lo, hi=hi)
    fo, fl = orc.attn_fwd(q, k, v, None, 1, 0, scale, threads=1, lo=lo, hi=hi)
    o_ref = o.detach().numpy()
    for x in (out, fo):
        assert np.max(np.abs(x - o_ref)) < 1e-12
    for x in (lse, fl):
        assert np.max(np.abs(x - lse_ref)) < 1e-12
    assert np.max(np.abs(dq - qt.grad.numpy())) < 1e-11
    assert np.max(np.abs(dk - kt.grad.numpy())) < 1e-11
    assert np.max(np.abs(dv - vt.grad.numpy())) < 1e-11
    rows = [0, 5, S - 1]
    ro, rl = orc.attn_fwd_rows(q, k, v, None, 1, 0, scale, 0, rows, lo=lo, hi=hi)
    assert np.max(np.abs(ro - out[0, rows])) < 1e-12
    assert np.max(np.abs(rl - lse[0, rows])) < 1e-12
    rdq = orc.attn_bwd_rows(q, k, v, do, None, 1, 0, scale, 0, rows, lo=lo, hi=hi)
    assert np.max(np.abs(rdq - dq[0, rows])) < 1e-12
    kv = [0, 14, Skv - 1]
    rdk, rdv = orc.attn_bwd_kv_rows(q, k, v, do, None, 1, 0, scale, 0, kv, lo=lo, hi=hi)
    assert np.max(np.abs(rdk - dk[0, kv])) < 1e-12
    assert np.max(np.abs(rdv - dv[0, kv])) < 1e-12


def check_cross_causal_special_case(orc):
    """hi[p] = p + 1 is the causal interval: the same results as lo alone,
    on every CP rank."""
    S, cp, Hq, Hkv, D = 64, 2, 4, 2, 8
    lengths = [9, 23, 32]
    doc, q, k, v, do = _case(S, cp, Hq, Hkv, D, lengths, seed=71)
    lo = _window_lo(lengths, 6)[None]
    hi = (np.arange(S) + 1)[None]
    c = S // (2 * cp)
    for r in range(cp):
        Skv = (2 * cp - r) * c
        args = (_local(q, S, cp, r), k[:, :Skv], v[:, :Skv], _local(do, S, cp, r))
        a = orc.attn_bwd(*args, None, cp, r, 0.4, threads=1, return_fwd=True, lo=lo)
        b = orc.attn_bwd(*args, None, cp, r, 0.4, threads=1, return_fwd=True, lo=lo, hi=hi)
        for x, y in zip(a, b):
            assert np.max(np.abs(x - y)) == 0.0


ALL_CHECKS = [
    check_chunk_permutation, check_causal_equal_work, check_interval_rule,
    check_q_zero, check_softmax_rows, check_per_document,
    check_sdpa_explicit_mask, check_gqa_vs_mha, check_cp_split,
    check_finite_differences, check_autograd, check_window,
    check_sampled_forms, check_interval_brute, check_interval_sliding_window,
    check_interval_is_document_mask, check_cross_brute, check_cross_attention,
    check_cross_causal_special_case,
]
