"""The streaming loads read only window columns (CPU, no GPU).

tests/stream_geom_check.cpp includes csrc/stream_geom.h, the header whose
functions the HIP kernels call for every load address, and replays them
for 20000 random rows: start, end, width, row alignment, block size, chunk
and wave count.  It checks that every address lies in the row's window
[max(s, 0), min(e, width)) and that each window column of a block enters
that block's maximum exactly once.
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_kv_dsa_amd", "csrc")


def test_stream_loads_stay_in_window(tmp_path):
    exe = str(tmp_path / "stream_geom_check")
    subprocess.check_call(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-I", CSRC,
                           os.path.join(ROOT, "tests", "stream_geom_check.cpp"), "-o", exe])
    res = subprocess.run([exe, "20000"], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok "), res.stdout
