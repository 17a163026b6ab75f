"""CPU fp64 oracle for document-masked causal GQA attention on one
context-parallel (CP) rank -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU
baseline leg may import this module.  The GPU library never calls it, and it
shares no code with the GPU library.

What it computes, and where the pages state it:

* Chunk assignment -- "The Llama 3 Herd of Models", section 3.3.2,
  "Context parallelism for long sequences": the sequence is cut into 2*CP
  equal chunks and rank i holds chunk i and chunk 2*CP-1-i.  The same rule is
  restated in "Scaling Llama 3 Training with Efficient Parallelism
  Strategies" (review), section on CP implementation details.
* All-gather CP attention -- same section of the Herd paper: K and V of the
  whole sequence are gathered first, then the attention output is computed
  for the rank's local query chunks.  Here the gathered K/V arrive as input.
* Document mask -- "Paper notes: The Llama 3 Herd of Models", "Two
  architectural choices": tokens do not attend across document boundaries;
  the model is a causal decoder ("full causal mask" in Herd section 3.3.2).
  Reading used here: key t is allowed for query position p iff t <= p and
  doc(t) == doc(p).
* Interval masks -- "Scaling Llama 3 Training with Efficient Parallelism
  Strategies" (review), section "Context Parallelism (CP)", implementation
  details and Figure 7: with the whole K/V gathered, a rank can apply any
  attention mask (causal, document, CP-document are drawn).  The form
  supported here is a causal mask with a per-position window start: key t is
  allowed for query position p iff lo[p] <= t <= p (lo given per position;
  the document mask is lo = first position of p's document).  Every
  function below takes either doc_ids or lo.
* Non-causal intervals -- the same page, section on pipeline parallelism
  for multimodal training (Figure 5 and its second challenge): the
  cross-attention layers take image sequences of 1.2K-3K tokens next to text
  of under 200 tokens.  Reading used here (the page gives no mask): text
  query p attends to every image token of its own sample, i.e. an interval
  with an exclusive end not tied to the position, lo[p] <= t < hi[p], over
  keys indexed independently of the queries.  Every function below that
  takes lo also takes hi; without hi the end is p (inclusive).
* GQA -- Herd section 3.3.2 and "Paper notes", "Two architectural choices":
  groups of query heads share one key/value head.  Reading used here:
  contiguous groups, query head h uses KV head h // (Hq // Hkv).
* Attention itself -- "Training Infrastructure and Systems", section
  "FlashAttention: never write the score matrix": scores S = Q K^T, softmax
  over each row, output P V; the per-row max m and sum l are kept for the
  backward pass.  This oracle is the plain "standard attention" of that
  section, not the tiled one: each row's full set of allowed scores is formed
  and normalised at once.  The softmax scale (never stated on the pages) is an
  explicit argument, normally 1/sqrt(D).  The saved statistic is
  lse = m + ln(l), one fp64 number per row.
* Backward -- the pages only say that the backward pass recomputes the scores
  (same section, "Tiling").  The gradients are the textbook chain rule of
  softmax attention: D = <dO, O>, dP = dO V^T, dS = P * (dP - D),
  dQ = scale * dS K, dK = scale * dS^T Q, dV = P^T dO, with dK/dV summed over
  all query heads of the KV group.

Every function works in float64.  Rows are processed in blocks, and each
block's columns may be restricted to the span where its explicit mask has any
allowed entry (`window=True`).  That is exact: every column outside the span
is masked for every row of the block, so its probability is exactly 0.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from typing import List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "chunk_positions", "query_positions", "allowed_mask", "interval_mask", "allowed_counts", "attn_probs",
    "attn_fwd", "attn_bwd", "attn_fwd_rows", "attn_bwd_rows",
    "attn_bwd_kv_rows", "to_f64",
]


def to_f64(x) -> np.ndarray:
    """Upcast a numpy array or a CPU torch tensor (any float dtype) to fp64."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    return x.detach().to("cpu").double().numpy()


def chunk_positions(S: int, cp_size: int, cp_rank: int) -> np.ndarray:
    """Global positions of the rank's local rows: chunk `cp_rank`, then chunk
    2*cp_size-1-cp_rank, each in ascending order (Herd section 3.3.2, CP).
    The chunk length is S / (2*cp_size); S must divide evenly."""
    if S % (2 * cp_size) != 0:
        raise ValueError("S must be a multiple of 2*cp_size")
    if not 0 <= cp_rank < cp_size:
        raise ValueError("cp_rank out of range")
    c = S // (2 * cp_size)
    first = np.arange(cp_rank * c, (cp_rank + 1) * c, dtype=np.int64)
    j = 2 * cp_size - 1 - cp_rank
    second = np.arange(j * c, (j + 1) * c, dtype=np.int64)
    return np.concatenate([first, second])


def query_positions(S: int, cp_size: int, cp_rank: int, hi=None) -> np.ndarray:
    """Positions of the local query rows.  With hi (the cross-attention form)
    and cp_size 1 the rows are the S query tokens in order, for any S: the
    multimodal cross-attention of "Scaling Llama 3 Training with Efficient
    Parallelism Strategies" (pipeline parallelism for multimodal training)
    is not split over context-parallel ranks.  For even S that is the same
    as the chunk map with one rank.  Otherwise the chunk map."""
    if hi is not None and cp_size == 1 and cp_rank == 0:
        return np.arange(S, dtype=np.int64)
    return chunk_positions(S, cp_size, cp_rank)


def allowed_mask(doc: np.ndarray, pos: np.ndarray, Skv: int) -> np.ndarray:
    """Explicit boolean mask M[i, t] for query positions `pos` over keys
    t in [0, Skv): causal (t <= p) and same document (doc[t] == doc[p])."""
    t = np.arange(Skv, dtype=np.int64)
    same_doc = doc[:Skv][None, :] == doc[pos][:, None]
    causal = t[None, :] <= pos[:, None]
    return causal & same_doc


def interval_mask(lo: np.ndarray, pos: np.ndarray, Skv: int,
                  hi: Optional[np.ndarray] = None) -> np.ndarray:
    """Explicit boolean mask M[i, t] for query positions `pos` over keys
    t in [0, Skv): lo[p] <= t <= p, or with `hi` (exclusive ends, not tied
    to the position) lo[p] <= t < hi[p]."""
    t = np.arange(Skv, dtype=np.int64)
    end = pos + 1 if hi is None else np.asarray(hi)[pos]
    return (t[None, :] >= np.asarray(lo)[pos][:, None]) & (t[None, :] < end[:, None])


def _masks(doc_ids, lo, hi=None):
    """The mask source: (array [B, S], fn(b, positions, Skv) -> explicit mask)."""
    if (doc_ids is None) == (lo is None):
        raise ValueError("pass exactly one of doc_ids / lo")
    if hi is not None and lo is None:
        raise ValueError("hi needs lo")
    if lo is not None:
        arr = np.asarray(lo)
        if hi is None:
            return arr, lambda b, p, Skv: interval_mask(arr[b], p, Skv)
        harr = np.asarray(hi)
        if harr.shape != arr.shape:
            raise ValueError("lo and hi must have the same shape")
        if np.any(harr <= arr):
            raise ValueError("every query needs at least one key (lo < hi)")
        return arr, lambda b, p, Skv: interval_mask(arr[b], p, Skv, harr[b])
    arr = np.asarray(doc_ids)
    return arr, lambda b, p, Skv: allowed_mask(arr[b], p, Skv)


def allowed_counts(doc_ids: Optional[np.ndarray], cp_size: int, cp_rank: int, Skv: int,
                   block: int = 256, lo: Optional[np.ndarray] = None,
                   hi: Optional[np.ndarray] = None) -> np.ndarray:
    """Number of allowed keys of every local row, counted from the explicit
    mask.  doc_ids (or lo, and optionally hi): [B, S].  Returns int64 [B, Sq]."""
    arr, mask = _masks(doc_ids, lo, hi)
    B, S = arr.shape
    pos = query_positions(S, cp_size, cp_rank, hi)
    out = np.zeros((B, pos.size), dtype=np.int64)
    for b in range(B):
        for s in range(0, pos.size, block):
            out[b, s:s + block] = mask(b, pos[s:s + block], Skv).sum(1)
    return out


def _window(M: np.ndarray, window: bool) -> Tuple[int, int]:
    if not window:
        return 0, M.shape[1]
    cols = np.flatnonzero(M.any(0))
    if cols.size == 0:
        return 0, 0
    return int(cols[0]), int(cols[-1]) + 1


def _softmax_block(qb: np.ndarray, kw: np.ndarray, vw: np.ndarray,
                   M: np.ndarray, scale: float):
    """Standard attention for one block.  qb [n, G, D], kw/vw [W, D],
    M [n, W].  Returns P [n, G, W], out [n, G, D], lse [n, G]."""
    n, G, D = qb.shape
    W = kw.shape[0]
    s = scale * (qb.reshape(n * G, D) @ kw.T).reshape(n, G, W)
    s = np.where(M[:, None, :], s, -np.inf)
    m = s.max(axis=-1)
    e = np.exp(s - m[..., None])
    l = e.sum(axis=-1)
    P = e / l[..., None]
    out = (P.reshape(n * G, W) @ vw).reshape(n, G, D)
    lse = m + np.log(l)
    return P, out, lse


def _group_heads(g: int, G: int) -> slice:
    """Query heads served by KV head g: the contiguous group g*G .. g*G+G-1."""
    return slice(g * G, (g + 1) * G)


def _backward_block(P, o, qb, kw, vw, dob, scale):
    """Chain rule of softmax attention for one block.  P [n,G,W], o/qb/dob
    [n,G,D], kw/vw [W,D].  Returns dq [n,G,D], dk/dv partial sums [W,D]."""
    n, G, D = qb.shape
    W = kw.shape[0]
    Dr = (dob * o).sum(-1)                                     # D = <dO, O>
    dP = (dob.reshape(n * G, D) @ vw.T).reshape(n, G, W)       # dO V^T
    dS = P * (dP - Dr[..., None])                              # P * (dP - D)
    dqb = scale * (dS.reshape(n * G, W) @ kw).reshape(n, G, D)
    dkw = scale * (dS.reshape(n * G, W).T @ qb.reshape(n * G, D))
    dvw = P.reshape(n * G, W).T @ dob.reshape(n * G, D)
    return dqb, dkw, dvw


def _threads(threads: Optional[int]) -> int:
    if threads is not None:
        return max(1, int(threads))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _blocks(n_rows: int, G: int, W_max: int, target_elems: int = 1 << 22) -> int:
    """Rows per block so that a block's score matrix stays near target size."""
    per_row = max(1, G * max(W_max, 1))
    return int(max(1, min(n_rows, 64, target_elems // per_row)))


def _run(tasks, fn, threads: int):
    if threads <= 1 or len(tasks) <= 1:
        return [fn(t) for t in tasks]
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    if threadpool_limits is not None:
        with threadpool_limits(limits=1, user_api="blas"):
            with ThreadPoolExecutor(max_workers=threads) as ex:
                return list(ex.map(fn, tasks))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, tasks))


def _check(q, k, doc_ids, cp_size, cp_rank, hi=None):
    B, Sq, Hq, D = q.shape
    Bk, Skv, Hkv, Dk = k.shape
    S = doc_ids.shape[1]
    if Bk != B or Dk != D or doc_ids.shape[0] != B:
        raise ValueError("shape mismatch")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    pos = query_positions(S, cp_size, cp_rank, hi)
    if pos.size != Sq:
        raise ValueError("q must hold 2*S/(2*cp_size) local rows")
    if hi is None:
        if Skv > S or Skv <= int(pos.max()):
            raise ValueError("K/V must cover every position a local row can reach")
    elif int(np.max(np.asarray(hi)[:, pos])) > Skv:
        raise ValueError("K/V must cover every key a local row can reach")
    return B, Sq, Hq, D, Skv, Hkv, Hq // Hkv, pos


def attn_probs(q, k, doc_ids, cp_size: int, cp_rank: int, softmax_scale: float,
               lo=None, hi=None):
    """Explicit probability matrix P [B, Sq, Hq, Skv] (small cases only)."""
    q = to_f64(q); k = to_f64(k)
    arr, mask = _masks(doc_ids, lo, hi)
    B, Sq, Hq, D, Skv, Hkv, G, pos = _check(q, k, arr, cp_size, cp_rank, hi)
    P = np.zeros((B, Sq, Hq, Skv))
    for b in range(B):
        M = mask(b, pos, Skv)
        for g in range(Hkv):
            hs = _group_heads(g, G)
            p, _, _ = _softmax_block(q[b, :, hs], k[b, :, g], k[b, :, g], M, softmax_scale)
            P[b, :, hs] = p
    return P


def attn_fwd(q, k, v, doc_ids, cp_size: int, cp_rank: int, softmax_scale: float,
             window: bool = True, threads: Optional[int] = None, lo=None, hi=None):
    """Forward.  q [B,Sq,Hq,D] (local rows), k/v [B,Skv,Hkv,D] (gathered,
    global order), doc_ids [B,S] (or lo [B,S]).  Returns out [B,Sq,Hq,D],
    lse [B,Sq,Hq]."""
    q = to_f64(q); k = to_f64(k); v = to_f64(v)
    arr, mask = _masks(doc_ids, lo, hi)
    B, Sq, Hq, D, Skv, Hkv, G, pos = _check(q, k, arr, cp_size, cp_rank, hi)
    out = np.zeros((B, Sq, Hq, D))
    lse = np.zeros((B, Sq, Hq))
    nb = _blocks(Sq, G, Skv if not window else min(Skv, 16384))
    tasks = [(b, g, s) for b in range(B) for g in range(Hkv) for s in range(0, Sq, nb)]

    def work(t):
        b, g, s = t
        e = min(s + nb, Sq)
        M = mask(b, pos[s:e], Skv)
        lo, hi = _window(M, window)
        hs = _group_heads(g, G)
        _, o, l = _softmax_block(q[b, s:e, hs], k[b, lo:hi, g], v[b, lo:hi, g],
                                 M[:, lo:hi], softmax_scale)
        return t, o, l

    for (b, g, s), o, l in _run(tasks, work, _threads(threads)):
        e = min(s + nb, Sq)
        hs = _group_heads(g, G)
        out[b, s:e, hs] = o
        lse[b, s:e, hs] = l
    return out, lse


def attn_bwd(q, k, v, dout, doc_ids, cp_size: int, cp_rank: int,
             softmax_scale: float, window: bool = True,
             threads: Optional[int] = None, return_fwd: bool = False, lo=None, hi=None):
    """Backward.  Recomputes P and the oracle's own fp64 output, then applies
    the chain rule.  Returns dq [B,Sq,Hq,D], dk/dv [B,Skv,Hkv,D] (rows that no
    local query reaches are exactly 0); with return_fwd also out and lse."""
    q = to_f64(q); k = to_f64(k); v = to_f64(v); dout = to_f64(dout)
    arr, mask = _masks(doc_ids, lo, hi)
    B, Sq, Hq, D, Skv, Hkv, G, pos = _check(q, k, arr, cp_size, cp_rank, hi)
    dq = np.zeros((B, Sq, Hq, D))
    dk = np.zeros((B, Skv, Hkv, D))
    dv = np.zeros((B, Skv, Hkv, D))
    out = np.zeros((B, Sq, Hq, D)) if return_fwd else None
    lse = np.zeros((B, Sq, Hq)) if return_fwd else None
    scale = softmax_scale
    nb = _blocks(Sq, G, Skv if not window else min(Skv, 16384))
    tasks = [(b, g, s) for b in range(B) for g in range(Hkv) for s in range(0, Sq, nb)]

    def work(t):
        b, g, s = t
        e = min(s + nb, Sq)
        n = e - s
        M = mask(b, pos[s:e], Skv)
        lo, hi = _window(M, window)
        hs = _group_heads(g, G)
        qb = q[b, s:e, hs]
        kw = k[b, lo:hi, g]
        vw = v[b, lo:hi, g]
        dob = dout[b, s:e, hs]
        P, o, l = _softmax_block(qb, kw, vw, M[:, lo:hi], scale)
        dqb, dkw, dvw = _backward_block(P, o, qb, kw, vw, dob, scale)
        return t, lo, hi, dqb, dkw, dvw, o, l

    # dK/dV partial sums are added in task order, so the result is
    # deterministic for a given thread count and block size.
    for (b, g, s), lo, hi, dqb, dkw, dvw, o, l in _run(tasks, work, _threads(threads)):
        e = min(s + nb, Sq)
        hs = _group_heads(g, G)
        dq[b, s:e, hs] = dqb
        dk[b, lo:hi, g] += dkw
        dv[b, lo:hi, g] += dvw
        if return_fwd:
            out[b, s:e, hs] = o
            lse[b, s:e, hs] = l
    if return_fwd:
        return dq, dk, dv, out, lse
    return dq, dk, dv


# --- sampled forms for workloads too large for the full oracle ---------------

def _row_stats(q, k, v, mask_b, pos_rows, scale, G, g):
    """out, lse, window per single row (all G heads of KV group g); mask_b
    gives the explicit mask of query positions over the keys."""
    res = []
    Skv = k.shape[0]
    for p, qr in zip(pos_rows, q):
        M = mask_b(np.array([p]), Skv)
        lo, hi = _window(M, True)
        P, o, l = _softmax_block(qr[None], k[lo:hi, g], v[lo:hi, g], M[:, lo:hi], scale)
        res.append((lo, hi, P[0], o[0], l[0]))
    return res


def attn_fwd_rows(q, k, v, doc_ids, cp_size: int, cp_rank: int,
                  softmax_scale: float, b: int, rows: Sequence[int], lo=None, hi=None):
    """out [n, Hq, D] and lse [n, Hq] of selected local rows of batch b.
    Each row is computed on its own, exactly as in attn_fwd."""
    q = to_f64(q[b:b + 1]); k = to_f64(k[b:b + 1]); v = to_f64(v[b:b + 1])
    hi = None if hi is None else np.asarray(hi)[b:b + 1]
    arr, mask = _masks(None if doc_ids is None else np.asarray(doc_ids)[b:b + 1],
                       None if lo is None else np.asarray(lo)[b:b + 1], hi)
    _, Sq, Hq, D, Skv, Hkv, G, pos = _check(q, k, arr, cp_size, cp_rank, hi)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((rows.size, Hq, D)); lse = np.zeros((rows.size, Hq))
    for g in range(Hkv):
        hs = _group_heads(g, G)
        for i, (lo, hi, P, o, l) in enumerate(
                _row_stats(q[0, rows][:, hs], k[0], v[0], lambda p, n: mask(0, p, n), pos[rows],
                           softmax_scale, G, g)):
            out[i, hs] = o
            lse[i, hs] = l
    return out, lse


def attn_bwd_rows(q, k, v, dout, doc_ids, cp_size: int, cp_rank: int,
                  softmax_scale: float, b: int, rows: Sequence[int], lo=None, hi=None):
    """dq [n, Hq, D] of selected local rows of batch b (each row's dq needs
    only that row's own probabilities and output)."""
    q = to_f64(q[b:b + 1]); k = to_f64(k[b:b + 1]); v = to_f64(v[b:b + 1])
    dout = to_f64(dout[b:b + 1])
    hi = None if hi is None else np.asarray(hi)[b:b + 1]
    arr, mask = _masks(None if doc_ids is None else np.asarray(doc_ids)[b:b + 1],
                       None if lo is None else np.asarray(lo)[b:b + 1], hi)
    _, Sq, Hq, D, Skv, Hkv, G, pos = _check(q, k, arr, cp_size, cp_rank, hi)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, Hq, D))
    for g in range(Hkv):
        hs = _group_heads(g, G)
        stats = _row_stats(q[0, rows][:, hs], k[0], v[0], lambda p, n: mask(0, p, n), pos[rows],
                           softmax_scale, G, g)
        for i, (lo, hi, P, o, l) in enumerate(stats):
            do = dout[0, rows[i], hs]                      # [G, D]
            Dr = (do * o).sum(-1)
            dP = do @ v[0, lo:hi, g].T                     # [G, W]
            dS = P * (dP - Dr[:, None])
            dq[i, hs] = softmax_scale * dS @ k[0, lo:hi, g]
    return dq


def attn_bwd_kv_rows(q, k, v, dout, doc_ids, cp_size: int, cp_rank: int,
                     softmax_scale: float, b: int, kv_rows: Sequence[int],
                     max_query_rows: Optional[int] = None, lo=None, hi=None):
    """dk, dv [n, Hkv, D] at selected key positions of batch b.  Every local
    row that reaches one of those keys gets its full forward (lse and output)
    computed first, as attn_bwd does; then the keys' columns of dS and P are
    summed over those rows and all heads of the group."""
    q = to_f64(q[b:b + 1]); k = to_f64(k[b:b + 1]); v = to_f64(v[b:b + 1])
    dout = to_f64(dout[b:b + 1])
    doc_b = None if doc_ids is None else np.asarray(doc_ids)[b:b + 1]
    lo_b = None if lo is None else np.asarray(lo)[b:b + 1]
    hi_b = None if hi is None else np.asarray(hi)[b:b + 1]
    arr, mask = _masks(doc_b, lo_b, hi_b)
    _, Sq, Hq, D, Skv, Hkv, G, pos = _check(q, k, arr, cp_size, cp_rank, hi_b)
    kv_rows = np.asarray(kv_rows, dtype=np.int64)
    # Which local rows reach any selected key: explicit mask, row blocks.
    reach = np.zeros(Sq, dtype=bool)
    for s in range(0, Sq, 512):
        M = mask(0, pos[s:s + 512], Skv)
        reach[s:s + 512] = M[:, kv_rows].any(1)
    rows = np.flatnonzero(reach)
    if max_query_rows is not None and rows.size > max_query_rows:
        raise ValueError(f"{rows.size} query rows reach the selected keys "
                         f"(limit {max_query_rows})")
    out, lse = attn_fwd_rows(q, k, v, doc_b, cp_size, cp_rank, softmax_scale, 0, rows, lo=lo_b,
                             hi=hi_b)
    dk = np.zeros((kv_rows.size, Hkv, D)); dv = np.zeros((kv_rows.size, Hkv, D))
    if rows.size == 0:
        return dk, dv
    M = mask(0, pos[rows], Skv)[:, kv_rows]                    # [n, T]
    for g in range(Hkv):
        hs = _group_heads(g, G)
        qr = q[0, rows][:, hs]                                   # [n, G, D]
        dor = dout[0, rows][:, hs]
        kt = k[0, kv_rows, g]                                    # [T, D]
        vt = v[0, kv_rows, g]
        s = softmax_scale * np.einsum("ngd,td->ngt", qr, kt)
        P = np.where(M[:, None, :], np.exp(s - lse[:, hs][..., None]), 0.0)
        Dr = (dor * out[:, hs]).sum(-1)
        dP = np.einsum("ngd,td->ngt", dor, vt)
        dS = P * (dP - Dr[..., None])
        dk[:, g] = softmax_scale * np.einsum("ngt,ngd->td", dS, qr)
        dv[:, g] = np.einsum("ngt,ngd->td", P, dor)
    return dk, dv
