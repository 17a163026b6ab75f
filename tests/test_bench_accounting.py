"""bench.py's FLOP accounting against the oracle's explicit mask."""
import numpy as np
import pytest

import bench
import oracle
import workloads as W


@pytest.mark.parametrize("name,seed", [("tiny", 0), ("tiny", 3), ("tp405b", 0), ("short_docs", 1)])
def test_allowed_pairs_matches_explicit_mask(name, seed):
    cfg = W.CONFIGS[name]
    L = W.doc_lengths(cfg.doc_kind, cfg.S, seed)
    doc = W.doc_ids_from_lengths(L)[None]
    for r in cfg.ranks[:2]:
        Skv = W.kv_prefix_len(cfg.S, cfg.cp_size, r)
        want = int(oracle.allowed_counts(doc, cfg.cp_size, r, Skv).sum())
        assert bench.allowed_pairs(L, cfg.S, cfg.cp_size, r) == want


@pytest.mark.parametrize("name,seed,window,cp,r", [("tp405b_swa", 0, 1024, 1, 0),
                                                  ("tp405b", 2, 37, 1, 0),
                                                  ("short_docs", 1, 200, 4, 3)])
def test_windowed_pairs_match_explicit_interval_mask(name, seed, window, cp, r):
    """The sliding-window count equals the oracle's explicit interval mask
    (keys max(document start, p - window + 1) .. p) built from the same
    window starts as the workload's cases."""
    cfg = W.CONFIGS[name]
    L = W.doc_lengths(cfg.doc_kind, cfg.S, seed)
    lo = W.window_starts(L, window)[None]
    Skv = W.kv_prefix_len(cfg.S, cp, r)
    want = int(oracle.allowed_counts(None, cp, r, Skv, lo=lo).sum())
    assert bench.allowed_pairs(L, cfg.S, cp, r, window) == want


def test_single_doc_pairs_closed_form():
    S, cp = 32768, 4
    for r in range(cp):
        assert bench.allowed_pairs([S], S, cp, r) == 134_221_824


def test_seed0_useful_gflop():
    """Seed-0 useful work of the 405B TP-share workload: 5,359,333 pairs per
    head x 16 heads x 12 x 128 flops = 131.7 GFLOP."""
    cfg = W.CONFIGS["tp405b"]
    L = W.doc_lengths(cfg.doc_kind, cfg.S, 0)
    p = bench.allowed_pairs(L, cfg.S, 1, 0)
    assert p == 5_359_333
    f = bench.useful_flops(p, 16, 128, True)
    assert abs(f["total"] / 1e9 - 131.7) < 0.05
    assert f["fwd"] + f["bwd_dq"] + f["bwd_dkdv"] == f["total"]


def test_score_matrix_bytes_example():
    """The pages' example of the score-matrix size that tiling avoids:
    32 heads x 8192^2 x 2 bytes = 4.3 GB."""
    import json, os
    facts = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_facts.json")))
    f = facts["score_matrix_bytes"]
    assert round(f["heads"] * f["L"] ** 2 * f["bytes_per_elem"] / 1e9, 1) == f["bytes_rounded_GB"]


def test_multi_gpu_request_exits():
    assert bench.main(["--gpus", "2"]) == 2


def test_kernel_hash_follows_code_not_comments():
    """The traffic record's source hash ignores comments and layout, keeps
    string literals (inline assembly) and changes with any code token."""
    c = bench.code_only
    assert c('a /* x */ b // y\n"// s" \'/\' c\n  d') == 'a b "// s" \'/\' c d'
    assert c("x = 1;  // one\n") == c("x   =   1;\n/* no code */")
    assert c("x = 1;") != c("x = 2;")
    assert c('asm("v_mov_b32 %0, %1")') != c('asm("v_mov_b32  %0, %1")')
    assert len(bench.kernel_source_hash("bwd_dkdv")) == 16


def _pmc_csv(path, counter, rows):
    import csv
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_from_pmc_scales_by_the_copy(tmp_path):
    """Per-launch bytes: the kernel's average counter reading (KiB) times
    the factor that maps the copy kernel's reading onto the bytes it moved;
    other kernels and counters are ignored."""
    n = bench.COPY_CALIBRATION_BYTES
    ours = "void dmgqa::bwd_dkdv_kernel<128, true>(unsigned short const*)"
    copy = "__amd_rocclr_copyBuffer"
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the copy reads n bytes but the counter shows 2n (scale 1/2); it
    # writes n bytes and the counter shows n (scale 1)
    _pmc_csv(fetch, "FETCH_SIZE", [(ours, 1000.0), (ours, 1200.0), (copy, 2 * n / 1024),
                                   ("dmgqa::fwd_kernel<128, false>", 9e9)])
    _pmc_csv(write, "WRITE_SIZE", [(ours, 300.0), (ours, 500.0), (copy, n / 1024)])
    rec = bench.traffic_from_pmc(str(fetch), str(write), "bwd_dkdv", "tp405b", "cmd")
    assert rec["fetch_kib_per_launch"] == 1100.0 and rec["write_kib_per_launch"] == 400.0
    assert rec["fetch_scale"] == 0.5 and rec["write_scale"] == 1.0
    assert rec["bytes_per_launch"] == int(1100 * 1024 * 0.5 + 400 * 1024)
    assert rec["source_hash"] == bench.kernel_source_hash("bwd_dkdv")
    _pmc_csv(write, "WRITE_SIZE", [(copy, n / 1024)])
    with pytest.raises(SystemExit):
        bench.traffic_from_pmc(str(fetch), str(write), "bwd_dkdv", "tp405b", "cmd")


def test_measured_traffic_only_for_the_measured_code(tmp_path, monkeypatch):
    """A stored traffic figure is reported while its source hash matches the
    kernel's code, and dropped (None) once the code has changed."""
    import json
    monkeypatch.setattr(bench, "TRAFFIC_DIR", str(tmp_path))
    assert bench.measured_traffic("bwd_dkdv", "tp405b") is None
    rec = {"bytes_per_launch": 12345, "source_hash": bench.kernel_source_hash("bwd_dkdv")}
    (tmp_path / "traffic_bwd_dkdv_tp405b.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("bwd_dkdv", "tp405b") == 12345
    rec["source_hash"] = "0" * 16
    (tmp_path / "traffic_bwd_dkdv_tp405b.json").write_text(json.dumps(rec))
    assert bench.measured_traffic("bwd_dkdv", "tp405b") is None

