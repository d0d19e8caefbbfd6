"""bench.py's JSON line on the GPU: short runs of the tiny workload, of the
decode batch with the long-context decode beside it (per_config), and of
rows after selection, checked for the fields the line promises."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                       capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


@pytest.mark.parametrize("args", [("--config", "1", "--per-config", "none"), ("--op", "lse"),
                                  ("--op", "blockscores"), ("--op", "blockscores", "--keys"),
                                  ("--op", "scores", "--keys")])
def test_bench_line(args):
    d = _run(*args, "--steps", "20", "--warmup", "5", "--cpu-seconds", "0.5",
             "--rotate-bytes", "0.25")
    assert d["n_gpus"] == 1 and d["steps"] == 20 and d["warmup"] == 5
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["parity"] is True
    assert d["higher_is_better"] is True and d["data"] == "synthetic"
    assert "workload" in d["config"]
    roof = d["roofline"]
    assert roof["bound"] == "hbm" and roof["unit"] == "GB/s" and roof["peak"] == 8000.0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-3
    assert "traffic" in roof
    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    ctx = d["context"]
    assert ctx["read_stream_GBps"] > 1000 and ctx["graph_launch_floor_us"] > 0
    rep = d["repeats"]
    assert rep["n"] == 5 and rep["ms_per_step_min"] <= rep["ms_per_step_median"] <= rep["ms_per_step_max"]


def test_bench_per_config():
    d = _run("--config", "2", "--per-config", "4", "--steps", "10", "--warmup", "3",
             "--cpu-seconds", "0.5", "--rotate-bytes", "0.5")
    assert d["config"]["workload"].startswith("decode-64x32768") and d["parity"] is True
    assert d["parity_all"] is True
    (name, pc), = d["per_config"].items()
    assert name.startswith("longctx-decode") and pc["parity"] is True
    assert pc["ms_per_step"] > 0 and pc["plan"] == 4 and pc["input_copies"] >= 2
    assert abs(pc["roofline"]["frac"] - pc["roofline"]["achieved"] / 8000.0) < 1e-3
    assert pc["repeats"]["n"] == 5
