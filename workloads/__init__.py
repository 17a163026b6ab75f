"""Seeded synthetic inputs for document-masked causal GQA attention on one
context-parallel (CP) rank.

This module only *draws data*: document lengths, per-token document ids,
bf16 tensors, and the rank-local row layout in which a caller hands its
query rows to an attention call.  It holds none of the attention arithmetic;
both the CPU oracle and the GPU library receive exactly what it returns.

Workload shapes follow the Llama 3 pre-training setting described in
"The Llama 3 Herd of Models", section 3.3.2 (context parallelism: the input
is cut into 2*CP chunks and rank i holds chunks i and 2*CP-1-i; GQA with few
KV heads; a document mask over packed documents) and the ISCA'25 review
"Scaling Llama 3 Training with Efficient Parallelism Strategies" (CP section:
8K and 128K sequences, document mask).  Meta's document-length statistics are
not public, so document lengths are drawn from the stated distributions
below (a stand-in for the training corpus).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

__all__ = [
    "Config", "CONFIGS", "doc_lengths", "doc_ids_from_lengths",
    "cu_seqlens_from_lengths", "full_tensors", "take_local_rows", "Case",
    "make_case", "chunk_len", "kv_prefix_len", "window_starts",
]


@dataclass(frozen=True)
class Config:
    name: str
    S: int                 # total sequence length (all CP ranks together)
    cp_size: int
    ranks: Tuple[int, ...]  # the CP ranks whose share is run
    Hq: int
    Hkv: int
    D: int
    doc_kind: str          # how document lengths are drawn (see doc_lengths)
    value_scale: float     # q/k/v ~ N(0,1) * value_scale; dout ~ N(0,1)
    backward: bool
    B: int = 1
    description: str = ""
    # sliding window: query position p attends to keys
    # max(document start, p - window + 1) .. p (None: the document mask)
    window: Optional[int] = None


# The five workloads (plus the single-document variant of the last one).
CONFIGS: Dict[str, Config] = {
    "tiny": Config("tiny", 512, 1, (0,), 4, 1, 64, "three_cuts", 1.0, False,
                   description="S=512, CP=1, 4 Q heads / 1 KV head, d=64, "
                               "3 documents, forward only"),
    "llama8b": Config("llama8b", 8192, 1, (0,), 32, 8, 128, "geometric2048", 0.5, True,
                      description="8B-like layer: S=8192, CP=1, 32/8 heads, d=128, "
                                  "geometric document lengths (mean 2048)"),
    "tp405b": Config("tp405b", 8192, 1, (0,), 16, 1, 128, "lognormal1024", 0.5, True,
                     description="405B TP=8 per-GPU share: S=8192, CP=1, 16/1 heads, "
                                 "d=128, lognormal lengths (median 1024, sigma 1)"),
    "long_cp": Config("long_cp", 131072, 16, (0, 7), 16, 1, 128, "lognormal16384", 0.5, True,
                      description="long-context CP share: S=131072, CP=16, ranks 0 and 7, "
                                  "16/1 heads, d=128, lognormal lengths (median 16K)"),
    "short_docs": Config("short_docs", 32768, 4, (0, 1, 2, 3), 16, 1, 128, "uniform64_1024", 0.5, True,
                         description="short-document stress: S=32768, CP=4, all ranks, "
                                     "16/1 heads, d=128, lengths uniform in [64, 1024]"),
    "single_doc": Config("single_doc", 32768, 4, (0, 1, 2, 3), 16, 1, 128, "single", 0.5, True,
                         description="same shape as short_docs with one document "
                                     "(pure causal mask)"),
    "tp405b_swa": Config("tp405b_swa", 8192, 1, (0,), 16, 1, 128, "lognormal1024", 0.5, True,
                         description="405B TP=8 per-GPU share with a sliding window of 1024 "
                                     "keys inside the documents (interval mask)",
                         window=1024),
}


def _fill(S: int, draw: Callable[[], float]) -> List[int]:
    """Append max(1, int(draw())) until the lengths reach S; the last
    document is truncated so the lengths sum to exactly S."""
    out: List[int] = []
    total = 0
    while total < S:
        n = max(1, int(draw()))
        n = min(n, S - total)
        out.append(n)
        total += n
    return out


def doc_lengths(kind: str, S: int, seed: int) -> List[int]:
    """Seeded document lengths summing to S."""
    rng = np.random.default_rng(seed)
    if kind == "three_cuts":
        cuts = sorted(int(x) for x in rng.choice(np.arange(1, S), 2, replace=False))
        return [cuts[0], cuts[1] - cuts[0], S - cuts[1]]
    if kind == "geometric2048":
        return _fill(S, lambda: rng.geometric(1.0 / 2048))
    if kind == "lognormal1024":
        return _fill(S, lambda: round(rng.lognormal(math.log(1024), 1.0)))
    if kind == "lognormal16384":
        return _fill(S, lambda: round(rng.lognormal(math.log(16384), 1.0)))
    if kind == "uniform64_1024":
        return _fill(S, lambda: rng.integers(64, 1025))
    if kind == "single":
        return [S]
    raise ValueError(f"unknown document-length kind {kind!r}")


def doc_ids_from_lengths(lengths: List[int]) -> np.ndarray:
    """Per-token document index (int32), documents numbered 0,1,2,... in order."""
    return np.repeat(np.arange(len(lengths), dtype=np.int32),
                     np.asarray(lengths, dtype=np.int64)).astype(np.int32)


def window_starts(lengths: List[int], window: int) -> np.ndarray:
    """Per-position first allowed key of a sliding window of `window` keys
    inside documents: max(document start, p - window + 1) (int32)."""
    starts = np.repeat(np.concatenate([[0], np.cumsum(lengths)[:-1]]),
                       np.asarray(lengths, dtype=np.int64))
    p = np.arange(int(sum(lengths)))
    return np.maximum(starts, p - window + 1).astype(np.int32)


def cu_seqlens_from_lengths(lengths: List[int]) -> np.ndarray:
    """Cumulative document offsets [0, l0, l0+l1, ..., S] (int32)."""
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def chunk_len(S: int, cp_size: int) -> int:
    return S // (2 * cp_size)


def kv_prefix_len(S: int, cp_size: int, cp_rank: int) -> int:
    """Length of the gathered K/V prefix that the rank's rows can reach:
    the end of its later chunk, (2*CP - rank) * chunk."""
    return (2 * cp_size - cp_rank) * chunk_len(S, cp_size)


def full_tensors(cfg: Config, seed: int, dtype=None):
    """q, k, v, dout for the whole sequence, drawn in that order from one
    CPU torch.Generator seeded with `seed`, as fp32 N(0,1), scaled, then
    rounded to bf16 (round-to-nearest-even).  Shapes: q/dout [B,S,Hq,D],
    k/v [B,S,Hkv,D]."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    B, S = cfg.B, cfg.S
    q = torch.randn(B, S, cfg.Hq, cfg.D, generator=g, dtype=torch.float32)
    k = torch.randn(B, S, cfg.Hkv, cfg.D, generator=g, dtype=torch.float32)
    v = torch.randn(B, S, cfg.Hkv, cfg.D, generator=g, dtype=torch.float32)
    dout = torch.randn(B, S, cfg.Hq, cfg.D, generator=g, dtype=torch.float32)
    s = cfg.value_scale
    if s != 1.0:
        q.mul_(s); k.mul_(s); v.mul_(s)
    out_dtype = torch.bfloat16 if dtype is None else dtype
    return q.to(out_dtype), k.to(out_dtype), v.to(out_dtype), dout.to(out_dtype)


def cross_lengths(n: int, seed: int, text=(100, 200), image=(1200, 3000)):
    """Per-sample text and image token counts of a cross-attention batch:
    uniform in [text[0], text[1]) and [image[0], image[1]] (the multimodal
    sizes of "Scaling Llama 3 Training with Efficient Parallelism
    Strategies": image 1.2K-3K tokens, text under 200)."""
    rng = np.random.default_rng(seed)
    t = rng.integers(text[0], text[1], n)
    im = rng.integers(image[0], image[1] + 1, n)
    return t.tolist(), im.tolist()


def cross_bounds(text: List[int], image: List[int]):
    """lo, hi (int32 [S]) of every text token: the image span of its sample
    when the samples' text and image tokens are packed in order."""
    istart = np.concatenate([[0], np.cumsum(image)[:-1]])
    lo = np.repeat(istart, text).astype(np.int32)
    hi = np.repeat(istart + np.asarray(image), text).astype(np.int32)
    return lo, hi


def cross_tensors(B: int, S: int, Skv: int, Hq: int, Hkv: int, D: int, seed: int,
                  value_scale: float = 0.5, dout: bool = False):
    """q [B,S,Hq,D] and k, v [B,Skv,Hkv,D], drawn in that order from one CPU
    torch.Generator seeded with `seed` as fp32 N(0,1), scaled, rounded to
    bf16; with dout, also the output gradient [B,S,Hq,D] drawn next as
    unscaled N(0,1) (as for the self-attention workloads)."""
    import torch
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    q = torch.randn(B, S, Hq, D, generator=g, dtype=torch.float32) * value_scale
    k = torch.randn(B, Skv, Hkv, D, generator=g, dtype=torch.float32) * value_scale
    v = torch.randn(B, Skv, Hkv, D, generator=g, dtype=torch.float32) * value_scale
    res = (q.to(torch.bfloat16), k.to(torch.bfloat16), v.to(torch.bfloat16))
    if dout:
        do = torch.randn(B, S, Hq, D, generator=g, dtype=torch.float32)
        res = res + (do.to(torch.bfloat16),)
    return res


def take_local_rows(x, S: int, cp_size: int, cp_rank: int):
    """The rank-local row layout used by the attention calls: along dim 1,
    the rank's first chunk (chunk cp_rank) followed by its second chunk
    (chunk 2*cp_size-1-cp_rank), each in ascending position order."""
    c = chunk_len(S, cp_size)
    a = x[:, cp_rank * c:(cp_rank + 1) * c]
    j = 2 * cp_size - 1 - cp_rank
    b = x[:, j * c:(j + 1) * c]
    if isinstance(x, np.ndarray):
        return np.concatenate([a, b], axis=1)
    import torch
    return torch.cat([a, b], dim=1).contiguous()


@dataclass
class Case:
    cfg: Config
    seed: int
    rank: int
    lengths: List[List[int]]      # per batch entry
    doc_ids: np.ndarray           # int32 [B, S]
    cu_seqlens: Optional[np.ndarray]  # int32 [n_docs+1] (B == 1 only)
    q: "object"                   # bf16 [B, Sq, Hq, D]   (torch CPU)
    k: "object"                   # bf16 [B, Skv, Hkv, D]
    v: "object"
    dout: "object"                # bf16 [B, Sq, Hq, D]
    Skv: int
    scale: float = field(default=0.0)
    lo: Optional[np.ndarray] = None  # int32 [B, S] window starts (windowed configs)

    @property
    def Sq(self) -> int:
        return 2 * chunk_len(self.cfg.S, self.cfg.cp_size)


def make_case(cfg: Config, seed: int, rank: int, Skv: Optional[int] = None,
              full=None, lengths: Optional[List[List[int]]] = None) -> Case:
    """Everything one rank's attention call receives.  `full` may pass
    tensors already drawn by full_tensors(cfg, seed) to share them between
    ranks; `lengths` may fix the document lengths of each batch row."""
    if lengths is None:
        lengths = [doc_lengths(cfg.doc_kind, cfg.S, seed + 1000 * b) for b in range(cfg.B)]
    doc_ids = np.stack([doc_ids_from_lengths(l) for l in lengths])
    cu = cu_seqlens_from_lengths(lengths[0]) if cfg.B == 1 else None
    q, k, v, dout = full if full is not None else full_tensors(cfg, seed)
    if Skv is None:
        Skv = kv_prefix_len(cfg.S, cfg.cp_size, rank)
    ql = take_local_rows(q, cfg.S, cfg.cp_size, rank)
    dl = take_local_rows(dout, cfg.S, cfg.cp_size, rank)
    lo = (np.stack([window_starts(l, cfg.window) for l in lengths])
          if cfg.window is not None else None)
    return Case(cfg, seed, rank, lengths, doc_ids, cu, ql,
                k[:, :Skv].contiguous(), v[:, :Skv].contiguous(), dl, Skv,
                scale=1.0 / math.sqrt(cfg.D), lo=lo)
