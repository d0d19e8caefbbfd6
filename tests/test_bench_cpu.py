"""Host-side pieces of bench.py: the byte counts behind the metric, the
kernel-code hash that keys the committed counters, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from sparse_attention_kv_dsa_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _window_bytes_by_loop(w):
    total = 0
    for r in range(w.rows):
        g = r // w.row_repeat
        s = 0 if w.row_ks is None else int(w.row_ks[g])
        e = int(w.row_ke[g])
        total += sum(1 for c in range(w.width) if s <= c < e)
    return total * 4


def test_in_window_bytes_counts_columns():
    cases = [workloads.config(1)] + [workloads.random_case(seed) for seed in range(40)]
    for w in cases:
        assert bench.in_window_bytes(w) == _window_bytes_by_loop(w), w.name


def test_algorithmic_bytes_add_bounds_and_out():
    w = workloads.config(1)
    extra = bench.algorithmic_bytes(w) - bench.in_window_bytes(w)
    groups = -(-w.rows // w.row_repeat)
    assert extra == groups * 4 + w.rows * w.topk_blocks * 4


def test_kernel_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    src = open(bench.KERNEL_SRC, encoding="utf-8").read()
    h = bench.kernel_src_hash()
    edited = tmp_path / "edited.hip"
    edited.write_text("// a new comment\n" + src.replace("{\n", "{  /* note */\n\n", 3))
    monkeypatch.setattr(bench, "KERNEL_SRC", str(edited))
    assert bench.kernel_src_hash() == h
    edited.write_text(src.replace("kUnroll = 8", "kUnroll = 4", 1))
    assert bench.kernel_src_hash() != h


def test_traffic_lookup_needs_matching_code_and_plan(monkeypatch):
    """A committed counter record is used only for the kernel code (hash) and
    launch plan it was taken with; otherwise the bench reports null."""
    table = json.load(open(bench.TRAFFIC_JSON))
    assert table
    for workload, rec in table.items():
        monkeypatch.setattr(bench, "kernel_src_hash", lambda: rec["kernel_src_sha256_16"])
        assert bench.traffic_for(workload, rec["plan"]) == rec["bytes_per_launch"]
        assert bench.traffic_for(workload, rec["plan"] + 10) is None
        monkeypatch.setattr(bench, "kernel_src_hash", lambda: "0" * 16)
        assert bench.traffic_for(workload, rec["plan"]) is None
        assert 0.99 < rec["traffic_over_algorithmic"] < 1.2, workload


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]
