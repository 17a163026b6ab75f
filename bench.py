#!/usr/bin/env python3
"""Benchmark of document-masked causal GQA attention (forward + backward) for
one context-parallel rank on one MI355X.

A step is one pass of the whole hot path -- forward call then backward call
of the C-ABI library -- over one seed's synthetic input.  The timed steps
cycle over the seeds (all inputs resident in HBM before timing starts).
`value` is useful TFLOP/s over the timed steps: useful FLOPs count
4*D (forward) + 8*D (backward) per allowed (query, key) pair per query head,
excluding recomputation as model-FLOPs utilisation does ("Training
Infrastructure and Systems", "Model FLOPs Utilization").

    python bench.py [--steps K] [--warmup W] [--workload tp405b]

Prints one JSON line.  Only one GPU is used; --gpus N with N > 1 exits.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np

# MI355X published dense MFMA peak for bf16: 256 CUs x 2.4 GHz x 4096 flop/clk/CU.
PEAK_BF16_TFLOPS = 256 * 2.4e9 * 4096 / 1e12
PEAK_HBM_GBS = 8000.0


def local_positions(S: int, cp: int, r: int) -> np.ndarray:
    c = S // (2 * cp)
    return np.concatenate([np.arange(r * c, (r + 1) * c),
                           np.arange((2 * cp - 1 - r) * c, (2 * cp - r) * c)])


def allowed_pairs(lengths, S: int, cp: int, r: int, window=None) -> int:
    """Allowed (query, key) pairs of the rank's local rows (per query head):
    each local position p may attend to its document's keys start(p)..p
    (with a sliding window: the last `window` of them)."""
    starts = np.repeat(np.concatenate([[0], np.cumsum(lengths)[:-1]]), lengths)
    pos = local_positions(S, cp, r)
    lo = starts[pos] if window is None else np.maximum(starts[pos], pos - window + 1)
    return int((pos - lo + 1).sum())


def useful_flops(pairs: int, Hq: int, D: int, backward: bool) -> dict:
    """Useful FLOPs split by the kernel that does each product:
    forward Q K^T and P V (4D per pair-head); dQ kernel dS K (2D); dK/dV kernel
    dO V^T, P^T dO and dS^T Q (6D)."""
    ph = pairs * Hq
    f = {"fwd": 4 * D * ph}
    if backward:
        f["bwd_dq"] = 2 * D * ph
        f["bwd_dkdv"] = 6 * D * ph
    f["total"] = sum(f.values())
    return f


def algorithmic_bytes(case, backward: bool) -> int:
    """Minimum HBM bytes of one step: read Q and reachable K/V, write out/lse
    (forward); read Q, out, dO, lse, reachable K/V, write dQ, dK, dV
    (backward, dK/dV fp32 over the whole key prefix)."""
    B, Sq, Hq, D = case.q.shape
    Skv, Hkv = case.k.shape[1], case.k.shape[2]
    q = B * Sq * Hq * D * 2
    kv = 2 * B * Skv * Hkv * D * 2
    lse = B * Sq * Hq * 4
    fwd = q + kv + q + lse
    if not backward:
        return fwd
    bwd = 3 * q + lse + kv + q + 2 * B * Skv * Hkv * D * 4
    return fwd + bwd


COPY_CALIBRATION_BYTES = 512 << 20
# A cold repetition first writes this many bytes, more than the GPU's L2 and
# last-level (Infinity) cache hold, so the step starts without cached inputs.
FLUSH_BYTES = 512 << 20


def _gpu_sysfs_dir():
    """The amdgpu sysfs directory of cuda:0: its PCI address from the device
    properties, else the only GPU listed under /sys/class/drm."""
    import glob
    import torch
    try:
        p = torch.cuda.get_device_properties(0)
        hits = glob.glob("/sys/bus/pci/devices/%04x:%02x:%02x.*" % (
            p.pci_domain_id, p.pci_bus_id, p.pci_device_id))
        hits = [h for h in hits if os.path.exists(os.path.join(h, "pp_dpm_sclk"))]
        if len(hits) == 1:
            return hits[0], None
    except Exception:  # noqa: BLE001 - fall back to the listing below
        pass
    cards = sorted({os.path.realpath(os.path.dirname(f))
                    for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")})
    if len(cards) == 1:
        return cards[0], None
    return None, f"{len(cards)} GPUs with clock files and none matched by PCI address"


def sample_clocks(delay_s: float = 0.5):
    """Current shader, memory and fabric clocks (MHz) of the GPU, read in
    this process from the amdgpu driver's pp_dpm_* files (the current level
    is the line marked '*') delay_s seconds into a phase in which the GPU is
    busy with steps.  Returns a dict, with "error" when unreadable."""
    import re
    time.sleep(delay_s)
    d, err = _gpu_sysfs_dir()
    if d is None:
        return {"error": err}
    res = {"source": d}
    for key in ("sclk", "mclk", "fclk"):
        try:
            with open(os.path.join(d, f"pp_dpm_{key}")) as f:
                txt = f.read()
        except OSError:
            continue
        m = re.search(r"(\d+)\s*Mhz\s*\*", txt, re.IGNORECASE)
        if m:
            res[key + "_mhz"] = int(m.group(1))
    return res if len(res) > 1 else {"error": f"no current level in {d}/pp_dpm_*"}


TRAFFIC_DIR = os.path.join(ROOT, "profiles")


# The sources each measured kernel is compiled from (its .hip file and the
# headers it includes), for kernel_source_hash.
KERNEL_SOURCES = {
    "bwd_dkdv": ("dkdv.hip", "common.hpp", "dma.hpp", "index.hpp", "kernels.hpp"),
    "fwd": ("fwd.hip", "common.hpp", "dma.hpp", "index.hpp", "kernels.hpp"),
    "bwd_dq": ("dqs.hip", "common.hpp", "dma.hpp", "index.hpp", "kernels.hpp",
               "reduce.hpp"),
}


def code_only(text: str) -> str:
    """C++ source without its comments, whitespace runs outside string and
    character literals collapsed to one space (literals kept as written)."""
    out, i, n = [], 0, len(text)

    def space():
        if out and out[-1] != " ":
            out.append(" ")

    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
            space()
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            space()
        elif c.isspace():
            space()
            i += 1
        else:
            out.append(c)
            i += 1
    return "".join(out).strip()


def kernel_source_hash(kernel: str = "bwd_dkdv") -> str:
    """Hash of the code of `kernel`'s sources (comments and layout left
    out): a stored traffic figure is reported only for the kernel it was
    measured on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "context_gqa_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            h.update(name.encode() + b"\0" + code_only(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel`, from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE measurement (profiles/traffic_<kernel>_<workload>.json,
    written by `bench.py --traffic-from-pmc`); None if there is none or the
    kernels have changed since it was taken."""
    path = os.path.join(TRAFFIC_DIR, f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_hash") != kernel_source_hash(kernel):
        return None
    return rec["bytes_per_launch"]


KERNEL_KEYS = {"fwd": "fwd_kernel", "bwd_dq": "bwd_dq_kernel", "bwd_dkdv": "bwd_dkdv_kernel"}


def traffic_from_pmc(fetch_csv: str, write_csv: str, kernel: str, workload: str,
                     command: str) -> dict:
    """HBM bytes per launch of `kernel` from two rocprofv3 --pmc runs of
    `bench.py --copy-calibration` (FETCH_SIZE, then WRITE_SIZE; KiB per
    dispatch), each scaled by the same counter's reading for the
    device-to-device copy of COPY_CALIBRATION_BYTES in the same run."""
    import csv

    def per_dispatch(path, counter):
        ours, copies = [], []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            name = r["Kernel_Name"]
            if KERNEL_KEYS[kernel] in name:
                ours.append(v)
            elif "copy" in name.lower() and "dmgqa" not in name:
                copies.append(v)
        if not ours or not copies:
            raise SystemExit(f"{path}: no {counter} rows for {kernel} or for the copy kernel")
        return sum(ours) / len(ours), max(copies)

    f_k, f_copy = per_dispatch(fetch_csv, "FETCH_SIZE")
    w_k, w_copy = per_dispatch(write_csv, "WRITE_SIZE")
    f_scale = COPY_CALIBRATION_BYTES / (f_copy * 1024)
    w_scale = COPY_CALIBRATION_BYTES / (w_copy * 1024)
    return {"kernel": kernel, "workload": workload,
            "fetch_kib_per_launch": round(f_k, 1), "write_kib_per_launch": round(w_k, 1),
            "copy_bytes": COPY_CALIBRATION_BYTES, "copy_fetch_kib": f_copy,
            "copy_write_kib": w_copy, "fetch_scale": round(f_scale, 4),
            "write_scale": round(w_scale, 4),
            "bytes_per_launch": int(f_k * 1024 * f_scale + w_k * 1024 * w_scale),
            "source_hash": kernel_source_hash(kernel), "command": command}


def cpu_baseline(runs, min_s: float = 10.0, max_s: float = 30.0) -> dict:
    """The CPU oracle (fp64 numpy, all host cores) on the same inputs: whole
    ranks' forward + backward, cycling over the seeds until at least min_s
    seconds of work (stopping before max_s)."""
    import oracle
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    done, flops, t0 = [], 0.0, time.perf_counter()
    i = 0
    while True:
        r = runs[i % len(runs)]
        c = r["case"]
        t1 = time.perf_counter()
        oracle.attn_bwd(c.q, c.k, c.v, c.dout, None if c.lo is not None else c.doc_ids,
                        c.cfg.cp_size, c.rank, c.scale, threads=cores, return_fwd=True,
                        lo=c.lo)
        last = time.perf_counter() - t1
        flops += r["flops"]["total"]
        done.append(c.seed)
        i += 1
        el = time.perf_counter() - t0
        if el >= min_s or el + last > max_s:
            break
    dt = time.perf_counter() - t0
    cfg = runs[0]["case"].cfg
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{cfg.name} rank {runs[0]['case'].rank}: the oracle's whole-rank forward + "
                      f"backward on seeds {done} (same inputs as the GPU steps)"}


def cross_study(args) -> int:
    """Forward and backward of the cross-attention form: 32 packed samples of
    100-199 text tokens against 1200-3000 image tokens each (query token p
    attends to its own sample's image tokens), 16 query heads on 1 KV head,
    d = 128; one JSON line with every seed.  Useful FLOPs as for the main
    line: 4*D per allowed pair and query head forward, 8*D backward."""
    import torch
    import context_gqa_amd as M
    import workloads as W
    seeds = [int(x) for x in args.seeds.split(",") if x != ""]
    res = []
    for seed in seeds:
        text, image = W.cross_lengths(32, seed=seed)
        lo, hi = W.cross_bounds(text, image)
        S, Skv, Hq, Hkv, D = sum(text), sum(image), 16, 1, 128
        q, k, v, do = (x.cuda() for x in W.cross_tensors(1, S, Skv, Hq, Hkv, D, seed=seed + 100,
                                                         dout=True))
        lo_d = torch.from_numpy(lo[None]).cuda()
        hi_d = torch.from_numpy(hi[None]).cuda()
        out = torch.empty_like(q)
        lse = torch.empty(1, S, Hq, dtype=torch.float32, device="cuda")
        dq = torch.empty_like(q)
        dk = torch.empty(k.shape, dtype=torch.float32, device="cuda")
        dv = torch.empty_like(dk)
        wsf = torch.empty(max(M.lib().docmask_gqa_fwd_cross_workspace_size(1, S, Skv, Hq, Hkv, D),
                              1), dtype=torch.uint8, device="cuda")
        # the default workspace holds the dS stash; --stash recompute (or
        # --recompute) gives the minimum, where dQ recomputes the scores
        size_bwd = (M.lib().docmask_gqa_bwd_cross_workspace_size_min
                    if args.recompute or args.stash == "recompute"
                    else M.lib().docmask_gqa_bwd_cross_workspace_size)
        wsb = torch.empty(max(size_bwd(1, S, Skv, Hq, Hkv, D), 1), dtype=torch.uint8,
                          device="cuda")

        def fwd():
            M.docmask_gqa_attn_fwd_cross(q, k, v, lo_d, hi_d, out=out, lse=lse, workspace=wsf)

        def bwd():
            M.docmask_gqa_attn_bwd_cross(q, k, v, out, do, lse, lo_d, hi_d, dq=dq, dk=dk, dv=dv,
                                         workspace=wsb)

        def timed(fn):
            for _ in range(args.warmup):
                fn()
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(args.steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) / args.steps

        fms = timed(fwd)
        bms = timed(bwd)
        pairs = int(np.dot(np.asarray(text, dtype=np.int64), np.asarray(image, dtype=np.int64)))
        ff, bf = 4.0 * D * pairs * Hq, 8.0 * D * pairs * Hq
        res.append({"seed": seed, "S": S, "Skv": Skv, "fwd_ms": round(fms, 4),
                    "bwd_ms": round(bms, 4),
                    "fwd_tflops": round(ff / (fms * 1e-3) / 1e12, 2),
                    "bwd_tflops": round(bf / (bms * 1e-3) / 1e12, 2),
                    "tflops": round((ff + bf) / ((fms + bms) * 1e-3) / 1e12, 2)})
        print(f"cross seed {seed}: S={S} Skv={Skv} fwd {fms:.4f} ms bwd {bms:.4f} ms "
              f"{res[-1]['tflops']} TFLOP/s", file=sys.stderr, flush=True)
    print(json.dumps({"study": "cross-attention forward + backward", "heads": "16/1",
                      "head_dim": 128, "samples": 32, "text": "100-199", "image": "1200-3000",
                      "dq": "recompute" if args.recompute or args.stash == "recompute"
                      else "stash",
                      "steps": args.steps, "warmup": args.warmup, "per_seed": res}))
    return 0


def all_ranks(args) -> int:
    """Per-rank study of one workload on one GPU: every CP rank's share
    (forward with its document bounds, then backward), timed by HIP events
    (median of `--steps` repetitions per rank), with the document mask of
    each seed and with a single document over the whole sequence (pure
    causal mask, same shapes).  Prints one JSON line: per rank the key
    prefix, allowed pairs per head, forward / backward / step times and
    useful TFLOP/s; per mask the slowest / fastest rank ratio of the step
    time and of throughput."""
    import torch
    import context_gqa_amd as M
    import workloads as W
    cfg = W.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    seeds = [int(x) for x in args.seeds.split(",") if x != ""]
    ranks = list(range(cfg.cp_size))
    B, S, Hq, Hkv, D = cfg.B, cfg.S, cfg.Hq, cfg.Hkv, cfg.D
    c = W.chunk_len(S, cfg.cp_size)
    Sq = 2 * c
    f_ws = max(M.docmask_gqa_fwd_workspace_size(B, S, W.kv_prefix_len(S, cfg.cp_size, r), Hq,
                                                 Hkv, D, cfg.cp_size) for r in ranks)
    stash_kind = "recompute" if args.recompute else args.stash
    b_size = {"default": M.docmask_gqa_bwd_workspace_size,
              "full": M.docmask_gqa_bwd_workspace_size_full,
              "recompute": M.docmask_gqa_bwd_workspace_size_min}[stash_kind]
    b_ws = max(b_size(B, S, W.kv_prefix_len(S, cfg.cp_size, r), Hq, Hkv, D, cfg.cp_size)
               for r in ranks)
    wsf = torch.empty(max(1, f_ws), dtype=torch.uint8, device=dev)
    wsb = torch.empty(max(1, b_ws), dtype=torch.uint8, device=dev)
    out = torch.empty(B, Sq, Hq, D, dtype=torch.bfloat16, device=dev)
    dq = torch.empty_like(out)
    lse = torch.empty(B, Sq, Hq, dtype=torch.float32, device=dev)
    dk = torch.empty(B, S, Hkv, D, dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    plan = torch.empty(M.docmask_gqa_batch_plan_size(B, S, S, Hq, Hkv, D, cfg.cp_size) // 4,
                       dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    res = {"study": "per-rank imbalance", "workload": f"{cfg.name}: {cfg.description}",
           "cp_size": cfg.cp_size, "ranks": ranks, "seeds": seeds, "reps": args.steps,
           "backward_workspace": stash_kind, "masks": {}}
    for mask in ("document", "causal"):
        per = []
        for seed in seeds:
            full = W.full_tensors(cfg, seed)
            lengths = None if mask == "document" else [[S] for _ in range(B)]
            qg, kg, vg, dg = (x.to(dev) for x in full)
            for r in ranks:
                case = W.make_case(cfg, seed, r, full=full, lengths=lengths)
                Skv = case.Skv
                q = W.take_local_rows(qg, S, cfg.cp_size, r)
                do = W.take_local_rows(dg, S, cfg.cp_size, r)
                k, v = kg[:, :Skv], vg[:, :Skv]
                doc = torch.from_numpy(case.doc_ids).to(dev)
                dkr, dvr = dk[:, :Skv], dv[:, :Skv]
                pairs = sum(allowed_pairs(l, S, cfg.cp_size, r) for l in case.lengths)
                fl = useful_flops(pairs, Hq, D, cfg.backward)

                def fwd():
                    M.docmask_gqa_batch_plan(doc, B=B, S=S, Skv=Skv, Hq=Hq, Hkv=Hkv, D=D,
                                             cp_size=cfg.cp_size, cp_rank=r, out=plan)
                    M.docmask_gqa_attn_fwd(q, k, v, cp_size=cfg.cp_size, cp_rank=r,
                                           softmax_scale=case.scale, out=out, lse=lse,
                                           workspace=wsf, plan=plan)

                def bwd():
                    if not cfg.backward:
                        return
                    M.docmask_gqa_attn_bwd(q, k, v, out, do, lse, cp_size=cfg.cp_size, cp_rank=r,
                                           softmax_scale=case.scale, dq=dq, dk=dkr, dv=dvr,
                                           workspace=wsb, plan=plan)
                for _ in range(args.warmup):
                    fwd(); bwd()
                ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)]
                      for _ in range(args.steps)]
                for e in ev:
                    e[0].record(stream); fwd(); e[1].record(stream); bwd(); e[2].record(stream)
                torch.cuda.synchronize()
                fw = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
                bw = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
                st = float(np.median([e[0].elapsed_time(e[2]) for e in ev]))
                per.append({"seed": seed, "rank": r, "Skv": Skv, "pairs_per_head": pairs,
                            "fwd_ms": round(fw, 4), "bwd_ms": round(bw, 4), "step_ms": round(st, 4),
                            "tflops": round(fl["total"] / (st * 1e-3) / 1e12, 2)})
                print(f"{mask} seed {seed} rank {r}: {st:.3f} ms, {per[-1]['tflops']} TFLOP/s",
                      file=sys.stderr, flush=True)
            del qg, kg, vg, dg, full
        summ = {}
        for seed in seeds:
            rows = [x for x in per if x["seed"] == seed]
            t = [x["step_ms"] for x in rows]
            f = [x["tflops"] for x in rows]
            summ[str(seed)] = {"slowest_over_fastest_step": round(max(t) / min(t), 3),
                               # a CP group waits for its slowest rank
                               "mean_over_slowest_step": round(float(np.mean(t)) / max(t), 3),
                               "slowest_rank": rows[int(np.argmax(t))]["rank"],
                               "fastest_rank": rows[int(np.argmin(t))]["rank"],
                               "tflops_min": min(f), "tflops_max": max(f),
                               "tflops_all_ranks": round(
                                   sum(x["pairs_per_head"] for x in rows) * Hq
                                   * (12 if cfg.backward else 4) * D
                                   / (sum(t) * 1e-3) / 1e12, 2)}
        res["masks"][mask] = {"per_rank": per, "summary": summ}
    print(json.dumps(res), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # The first few dozen steps after start-up run up to ~10% slower while
    # the GPU's clocks ramp up (measured: 526 TFLOP/s timing 20 steps after 3
    # warm-up steps, 583-591 after 50); the defaults time the steady state.
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="tp405b")
    ap.add_argument("--rank", type=int, default=None, help="CP rank (default: first listed)")
    ap.add_argument("--seeds", default="0,1,2,3,4")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--all-ranks", action="store_true",
                    help="per-rank study instead of the benchmark line: every CP rank of the "
                         "workload, document and single-document masks (see all_ranks)")
    ap.add_argument("--cross", action="store_true",
                    help="forward and backward of the cross-attention form (text queries "
                         "over their own sample's image tokens) instead of the benchmark line")
    ap.add_argument("--no-clocks", action="store_true",
                    help="skip reading the GPU clocks (sysfs) during a busy phase")
    ap.add_argument("--stash", choices=("default", "full", "recompute"), default="default",
                    help="backward workspace: the library's default (the whole dS stash, or a "
                         "2 GiB stash budget for long shares), the whole worst-case stash, "
                         "or the minimum (no stash: dQ recomputes the scores); with --cross "
                         "'full' is the default")
    ap.add_argument("--recompute", action="store_true", help="same as --stash recompute")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run three device-to-device copies of 512 MiB (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--graph", action="store_true",
                    help="replay one captured HIP graph per seed instead of launching eagerly "
                         "(measured slower than eager launches on ROCm 7)")
    ap.add_argument("--traffic-from-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<kernel>_<workload>.json from two "
                         "rocprofv3 --pmc counter files and exit")
    ap.add_argument("--traffic-kernel", default="bwd_dkdv")
    ap.add_argument("--traffic-command", default="")
    args = ap.parse_args(argv)
    if args.traffic_from_pmc:
        import workloads as W
        rec = traffic_from_pmc(*args.traffic_from_pmc, args.traffic_kernel,
                               W.CONFIGS[args.workload].name, args.traffic_command)
        path = os.path.join(TRAFFIC_DIR, f"traffic_{rec['kernel']}_{rec['workload']}.json")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {max(args.gpus, world)}): this "
              "library has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import context_gqa_amd as M
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    M.lib()
    if args.all_ranks:
        return all_ranks(args)
    if args.cross:
        return cross_study(args)
    stash_kind = "recompute" if args.recompute else args.stash
    cfg = W.CONFIGS[args.workload]
    rank = cfg.ranks[0] if args.rank is None else args.rank
    seeds = [int(s) for s in args.seeds.split(",") if s != ""]
    dev = torch.device("cuda:0")

    runs = []
    for seed in seeds:
        case = W.make_case(cfg, seed, rank)
        B, Sq, Hq, D = case.q.shape
        Skv, Hkv = case.Skv, cfg.Hkv
        S = cfg.S
        t = dict(q=case.q.to(dev), k=case.k.to(dev), v=case.v.to(dev), dout=case.dout.to(dev),
                 doc=torch.from_numpy(case.doc_ids).to(dev))
        if case.lo is not None:
            t["lo"] = torch.from_numpy(case.lo).to(dev)
        t["out"] = torch.empty_like(t["q"])
        t["lse"] = torch.empty(B, Sq, Hq, dtype=torch.float32, device=dev)
        t["dq"] = torch.empty_like(t["q"])
        t["dk"] = torch.empty(B, Skv, Hkv, D, dtype=torch.float32, device=dev)
        t["dv"] = torch.empty_like(t["dk"])
        t["wsf"] = torch.empty(max(1, M.docmask_gqa_fwd_workspace_size(B, S, Skv, Hq, Hkv, D,
                                                                      cfg.cp_size)),
                               dtype=torch.uint8, device=dev)
        t["bounds"] = torch.empty(M.docmask_gqa_doc_bounds_size(B, S, Skv) // 4,
                                  dtype=torch.int32, device=dev)
        t["plan"] = torch.empty(M.docmask_gqa_batch_plan_size(B, S, Skv, Hq, Hkv, D,
                                                              cfg.cp_size) // 4,
                                dtype=torch.int32, device=dev)
        wsb_size = {"default": M.docmask_gqa_bwd_workspace_size,
                    "full": M.docmask_gqa_bwd_workspace_size_full,
                    "recompute": M.docmask_gqa_bwd_workspace_size_min}[stash_kind]
        t["wsb"] = torch.empty(max(1, wsb_size(B, S, Skv, Hq, Hkv, D, cfg.cp_size)),
                               dtype=torch.uint8, device=dev)
        pairs = sum(allowed_pairs(l, S, cfg.cp_size, rank, cfg.window) for l in case.lengths)
        runs.append(dict(case=case, t=t, pairs=pairs,
                         flops=useful_flops(pairs, Hq, D, cfg.backward),
                         bytes=algorithmic_bytes(case, cfg.backward)))

    def mask_kw(t):
        return {"bounds": t["bounds"]} if "lo" in t else {"plan": t["plan"]}

    def fwd_part(i):
        """The masking input of seed i's batch, built from doc_ids in every
        step (the batch plan: bounds and query-tile orders; interval masks:
        their bounds), and the forward."""
        r = runs[i % len(runs)]
        t, case = r["t"], r["case"]
        B_, Sq_, Hq_, D_ = t["q"].shape
        if "lo" in t:
            M.docmask_gqa_interval_bounds(t["lo"], Skv=case.Skv, out=t["bounds"])
        else:
            M.docmask_gqa_batch_plan(t["doc"], B=B_, S=cfg.S, Skv=case.Skv, Hq=Hq_,
                                     Hkv=cfg.Hkv, D=D_, cp_size=cfg.cp_size, cp_rank=rank,
                                     out=t["plan"])
        M.docmask_gqa_attn_fwd(t["q"], t["k"], t["v"], cp_size=cfg.cp_size, cp_rank=rank,
                               softmax_scale=case.scale, out=t["out"], lse=t["lse"],
                               workspace=t["wsf"], **mask_kw(t))

    def bwd_part(i):
        r = runs[i % len(runs)]
        t, case = r["t"], r["case"]
        if cfg.backward:
            M.docmask_gqa_attn_bwd(t["q"], t["k"], t["v"], t["out"], t["dout"], t["lse"],
                                   cp_size=cfg.cp_size, cp_rank=rank, softmax_scale=case.scale,
                                   dq=t["dq"], dk=t["dk"], dv=t["dv"], workspace=t["wsb"],
                                   **mask_kw(t))

    def step(i):
        """One step on seed i's inputs, on the current stream: the document
        bounds, then the forward and the backward, both reading them."""
        fwd_part(i)
        bwd_part(i)

    # With --graph each seed's step is captured once into a HIP graph (the
    # library makes no allocation, synchronisation or memset inside a call)
    # and the timed loop replays it.
    for i in range(max(args.warmup, len(runs))):
        step(i)
    torch.cuda.synchronize()
    graphs = None
    if args.graph:
        graphs = []
        for j in range(len(runs)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(j)
            graphs.append(g)
        torch.cuda.synchronize()

    def run_step(i):
        if graphs is None:
            step(i)
        else:
            graphs[i % len(runs)].replay()

    stream = torch.cuda.current_stream()
    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        run_step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = sum(runs[i % len(runs)]["flops"]["total"] for i in range(args.steps))
    value = flops / (ms * 1e-3) / 1e12

    per_seed = []
    for j, r in enumerate(runs):   # per-seed time for the median
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True); b = torch.cuda.Event(enable_timing=True)
        reps = max(3, args.steps // len(runs))
        a.record(stream)
        for _ in range(reps):
            run_step(j)
        b.record(stream)
        torch.cuda.synchronize()
        per_seed.append(r["flops"]["total"] / (a.elapsed_time(b) / reps * 1e-3) / 1e12)

    # Per seed: forward (with the bounds) and backward timed separately by
    # HIP events around each of `reps` back-to-back repetitions (median),
    # warm (inputs possibly cached from the previous repetition) and cold
    # (each repetition preceded by a write of FLUSH_BYTES).
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def seed_detail(j, reps, cold):
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
        for e in ev:
            if cold:
                flush.fill_(1.0)
            e[0].record(stream)
            fwd_part(j)
            e[1].record(stream)
            bwd_part(j)
            e[2].record(stream)
        torch.cuda.synchronize()
        fw = float(np.median([e[0].elapsed_time(e[1]) for e in ev]))
        bw = float(np.median([e[1].elapsed_time(e[2]) for e in ev]))
        st = float(np.median([e[0].elapsed_time(e[2]) for e in ev]))
        return fw, bw, st

    detail = []
    for j, r in enumerate(runs):
        fw, bw, st = seed_detail(j, 20, False)
        cfw, cbw, cst = seed_detail(j, 20, True)
        fl = r["flops"]
        d = {"seed": r["case"].seed, "fwd_ms": round(fw, 4), "bwd_ms": round(bw, 4),
             "step_ms": round(st, 4), "tflops": round(fl["total"] / (st * 1e-3) / 1e12, 2),
             "fwd_tflops": round(fl["fwd"] / (fw * 1e-3) / 1e12, 2),
             "alg_gbps": round(r["bytes"] / (st * 1e-3) / 1e9, 1),
             "cold": {"fwd_ms": round(cfw, 4), "bwd_ms": round(cbw, 4), "step_ms": round(cst, 4),
                      "tflops": round(fl["total"] / (cst * 1e-3) / 1e12, 2)}}
        if cfg.backward:
            d["bwd_tflops"] = round((fl["total"] - fl["fwd"]) / (bw * 1e-3) / 1e12, 2)
        detail.append(d)
    del flush

    # Clocks while the GPU is busy with steps (read from sysfs by a second
    # thread, after the timed measurements so that it cannot disturb them).
    clocks = None
    if not args.no_clocks:
        import threading
        box = {}
        th = threading.Thread(target=lambda: box.update(c=sample_clocks()))
        th.start()
        t_end = time.perf_counter() + 1.5
        i = 0
        while time.perf_counter() < t_end or th.is_alive():
            step(i)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        th.join()
        torch.cuda.synchronize()
        clocks = box.get("c")

    roofline = None
    kernels = {}
    if not args.no_kernel_timing:
        M.docmask_gqa_timing_enable(True)
        torch.cuda.synchronize()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        times = M.docmask_gqa_kernel_times()
        M.docmask_gqa_timing_enable(False)
        kernels = {k: {"avg_us": round(1e3 * v[0] / v[1], 3), "launches": v[1]}
                   for k, v in times.items() if v[1] > 0}
        dom = max((k for k in times if times[k][1] > 0), key=lambda k: times[k][0])
        tot_ms, n = times[dom]
        alg = sum(runs[i % len(runs)]["flops"].get(dom, 0) for i in range(args.steps)) / args.steps
        achieved = alg / (tot_ms / n * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                    "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                    "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None,
                    "avg_launch_us": round(1e3 * tot_ms / n, 3)}

    if roofline is not None:
        roofline["traffic"] = measured_traffic(roofline["kernel"], cfg.name)

    if args.copy_calibration:
        src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(runs)

    res = {
        "metric": "doc-masked GQA attn fwd+bwd useful TFLOP/s; % MI355X bf16 MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: {cfg.description}", "cp_size": cfg.cp_size,
                   "cp_rank": rank, "seq_len": cfg.S, "Hq": cfg.Hq, "Hkv": cfg.Hkv,
                   "head_dim": cfg.D, "global_batch": cfg.B, "seeds": seeds,
                   "parallelism": "one CP rank's share on one GPU",
                   "launch": "hip graph per seed" if args.graph else "eager",
                   "backward": {"default": "default workspace (dS stash, 2 GiB budget)",
                                "full": "whole worst-case dS stash",
                                "recompute": "recompute (minimum workspace)"}[stash_kind],
                   "bwd_path": sorted({M.docmask_gqa_bwd_path(
                       r["case"].cfg.B, cfg.S, r["case"].Skv, cfg.Hq, cfg.Hkv, cfg.D,
                       cfg.cp_size, rank, r["t"]["wsb"].numel()) for r in runs}),
                   "masking": ("sliding window of %d keys inside the documents: interval "
                               "bounds from the window starts once per step" % cfg.window)
                              if cfg.window is not None else
                              "batch plan (document bounds and both query-tile orders) "
                              "from doc_ids once per step, read by the forward and the "
                              "backward"},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "per_seed_tflops": [round(x, 2) for x in per_seed],
        "median_seed_tflops": round(float(np.median(per_seed)), 2),
        "useful_gflop_per_seed": [round(r["flops"]["total"] / 1e9, 2) for r in runs],
        "per_seed": detail,
        "clocks": clocks,
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
