"""The CPU oracle against what the pages and the mathematics fix."""
import json
import os

import numpy as np
import pytest

import oracle
import oracle.attention as OA
import workloads as W
from tests import oracle_checks as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("check", C.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(OA)


def test_single_doc_pair_count_closed_form():
    C.check_causal_equal_work_single_doc_full()


@pytest.mark.slow
def test_single_doc_pair_count_full_shape():
    """The 32768-token, CP=4 single-document workload: every rank has
    S*c + c = 134,221,824 allowed pairs per head, counted from the mask."""
    doc = np.zeros((1, 32768), dtype=np.int32)
    for r in range(4):
        Skv = W.kv_prefix_len(32768, 4, r)
        assert int(OA.allowed_counts(doc, 4, r, Skv, block=1024).sum()) == 134_221_824


def test_pages_chunk_examples():
    """Worked chunk assignments from tests/golden/pages_facts.json."""
    facts = json.load(open(os.path.join(GOLDEN, "pages_facts.json")))
    for ex in facts["chunk_assignment"]["examples"]:
        S, cp = ex["S"], ex["cp"]
        c = S // (2 * cp)
        for r, chunks in enumerate(ex["chunks_per_rank"]):
            pos = OA.chunk_positions(S, cp, r)
            want = np.concatenate([np.arange(j * c, (j + 1) * c) for j in chunks])
            assert np.array_equal(pos, want)


# --- planted mistakes: each must make at least one pin fail -----------------

_ORIG = {n: getattr(OA, n) for n in ("chunk_positions", "_backward_block", "_softmax_block")}

def _mut_strict_causal(doc, pos, Skv):
    t = np.arange(Skv)
    return (t[None, :] < pos[:, None]) & (doc[:Skv][None, :] == doc[pos][:, None])


def _mut_causal_only(doc, pos, Skv):
    t = np.arange(Skv)
    return t[None, :] <= pos[:, None]


def _mut_chunks(S, cp, r):
    c = S // (2 * cp)
    j = (cp + r) % (2 * cp)
    return np.concatenate([np.arange(r * c, (r + 1) * c), np.arange(j * c, (j + 1) * c)])


def _mut_chunks_order(S, cp, r):
    return np.sort(_ORIG['chunk_positions'](S, cp, r))[::-1].copy()


def _mut_no_D(P, o, qb, kw, vw, dob, scale):
    n, G, D = qb.shape
    Wd = kw.shape[0]
    dP = (dob.reshape(n * G, D) @ vw.T).reshape(n, G, Wd)
    dS = P * dP
    return (scale * (dS.reshape(n * G, Wd) @ kw).reshape(n, G, D),
            scale * (dS.reshape(n * G, Wd).T @ qb.reshape(n * G, D)),
            P.reshape(n * G, Wd).T @ dob.reshape(n * G, D))


def _mut_dk_no_scale(P, o, qb, kw, vw, dob, scale):
    dq, dk, dv = _ORIG['_backward_block'](P, o, qb, kw, vw, dob, scale)
    return dq, dk / scale, dv


def _mut_dv_transposed(P, o, qb, kw, vw, dob, scale):
    dq, dk, dv = _ORIG['_backward_block'](P, o, qb, kw, vw, dob, scale)
    n, G, D = qb.shape
    return dq, dk, dv * 0.0 + (P.reshape(n * G, -1).T @ o.reshape(n * G, D))


def _mut_heads_strided(g, G):
    return slice(g, None, max(1, G))


def _mut_interval_open_lo(lo, pos, Skv, hi=None):
    t = np.arange(Skv)
    end = pos + 1 if hi is None else np.asarray(hi)[pos]
    return (t[None, :] > np.asarray(lo)[pos][:, None]) & (t[None, :] < end[:, None])


def _mut_interval_hi_inclusive(lo, pos, Skv, hi=None):
    t = np.arange(Skv)
    end = pos if hi is None else np.asarray(hi)[pos]
    return (t[None, :] >= np.asarray(lo)[pos][:, None]) & (t[None, :] <= end[:, None])


def _mut_softmax_no_scale(qb, kw, vw, M, scale):
    return _ORIG['_softmax_block'](qb, kw, vw, M, 1.0)


MUTATIONS = {
    "strict_causal": ("allowed_mask", _mut_strict_causal),
    "causal_only": ("allowed_mask", _mut_causal_only),
    "wrong_second_chunk": ("chunk_positions", _mut_chunks),
    "chunks_reversed": ("chunk_positions", _mut_chunks_order),
    "no_D_term": ("_backward_block", _mut_no_D),
    "dk_missing_scale": ("_backward_block", _mut_dk_no_scale),
    "dv_uses_out": ("_backward_block", _mut_dv_transposed),
    "heads_strided": ("_group_heads", _mut_heads_strided),
    "softmax_no_scale": ("_softmax_block", _mut_softmax_no_scale),
    "interval_open_lo": ("interval_mask", _mut_interval_open_lo),
    "interval_hi_inclusive": ("interval_mask", _mut_interval_hi_inclusive),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    orig = getattr(OA, attr)
    monkeypatch.setattr(OA, attr, fn)
    failures = 0
    for check in C.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(OA)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failures += 1
    monkeypatch.setattr(OA, attr, orig)
    assert failures > 0, f"planted mistake {name} passed every pin"
