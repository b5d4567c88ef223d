"""The mask-quality measurement (recall and retained mass of a block mask against a tile
heatmap) on hand-made rows."""
import numpy as np

import bench
import workloads as W


def test_mask_quality_hand_rows():
    tmax = np.array([[0.9, 0.1, 0.5, 0.2],
                     [0.1, 0.2, 0.3, 0.4]])
    tmass = np.array([[0.6, 0.1, 0.2, 0.1],
                      [0.1, 0.2, 0.3, 0.4]])
    # row 0 keeps blocks {0, 1}; row 1 keeps {3}
    rp = np.array([0, 2, 3])
    ci = np.array([0, 1, 3])
    q = bench.mask_quality(tmax, tmass, rp, ci)
    # row 0: top-2 by max is {0, 2} -> recall 1/2; by mass {0, 2} -> 1/2;
    # retained 0.7 of a best 0.8. Row 1: top-1 is {3} -> recall 1, retained 0.4 of 0.4.
    assert q["recall_max"]["mean"] == 0.75 and q["recall_max"]["min"] == 0.5
    assert q["recall_mass"]["mean"] == 0.75
    assert abs(q["retained_mass"]["mean"] - 0.55) < 1e-9
    assert abs(q["mass_efficiency"]["min"] - 0.875) < 1e-4


def test_mask_quality_ties_rank_lower_index_first():
    tmax = np.array([[0.5, 0.5, 0.5]])
    tmass = np.array([[0.3, 0.3, 0.4]])
    q = bench.mask_quality(tmax, tmass, np.array([0, 1]), np.array([0]))
    assert q["recall_max"]["mean"] == 1.0      # block 0 wins the three-way tie
    assert q["recall_mass"]["mean"] == 0.0     # block 2 holds the most mass


def test_cpu_baseline_walks_heads_within_budget():
    """The CPU baseline leg: whole heads of the oracle's output track until the budget is
    used."""
    from oracle import oracle_plan
    w = W.CONFIGS["tiny_fp32"]
    q, k, v, _ = W.make_inputs(w)
    rp, ci, _ = oracle_plan(W.to_f32(q), W.to_f32(k), w.block_q, w.block_kv, w.topk, w.top_p)
    res = bench.cpu_baseline(w, q, k, v, rp, ci, budget_s=1e9)
    assert res["kind"] == "oracle" and res["value"] > 0 and res["cores"] >= 1
    assert f"heads 0..{w.H - 1}" in res["sample"]
    one = bench.cpu_baseline(w, q, k, v, rp, ci, budget_s=0.0)     # stops after the first head
    assert "heads 0..0" in one["sample"]


def test_more_than_one_gpu_is_refused_before_any_work():
    """--gpus above 1 exits with status 2 and a message, before torch or the library loads."""
    import subprocess
    import sys
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_traffic_needs_the_profiled_kernel_source(tmp_path, monkeypatch):
    """The committed HBM bytes are reported only for the kernel source they were taken on."""
    import json
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps({"w": {"kernel_source_sha256_16": bench.source_hash(),
                                   "hbm_bytes_per_launch": 123}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.traffic_for("w", 1.0) == 123
    assert bench.traffic_for("other", 1.0) is None
    f.write_text(json.dumps({"w": {"kernel_source_sha256_16": "0" * 16, "hbm_bytes_per_launch": 123}}))
    assert bench.traffic_for("w", 1.0) is None


def test_traffic_key_covers_the_compile_flags(monkeypatch):
    """Counters taken on one build of the forward are not reported for another build of the
    same source (a changed instruction schedule changes the kernel)."""
    from block_sparse_attention_05_amd import build as B
    h = bench.source_hash()
    flags = dict(B.SOURCES)
    flags["sparse_fwd_bf16.hip"] = [f for f in flags["sparse_fwd_bf16.hip"] if "sched" not in f and f != "-mllvm"]
    monkeypatch.setattr(B, "SOURCES", flags)
    assert bench.source_hash() != h
