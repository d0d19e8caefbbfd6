"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle (oracle/oracle.c), built with -fsanitize=address,undefined
  together with tests/sanitize_oracle.c, runs the hand-worked rows and seeded
  random cases of every function (selection, block scores, selection from
  scores and from codes, masking, LSE correction); its results must equal
  those of the regular oracle build.  Every input array is allocated at
  exactly its size, so a read past it is reported.
- libdsa's host code (argument checks, plan and workspace sizing), built by
  hipcc with the sanitizers on the host side only, is driven by
  tests/sanitize_host.cpp over argument values at the edges of their types.
  That driver launches nothing that could run: it refuses to run where a GPU
  is visible.

A sanitizer report makes the driver exit non-zero, which fails the test.
"""
import hashlib
import json
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from sparse_attention_kv_dsa_amd import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "sparse_attention_kv_dsa_amd", "csrc")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def _hex(a):
    return " ".join(f"{v:08x}" for v in np.ascontiguousarray(a, np.float32).reshape(-1).view(np.uint32))


def _ints(a):
    return " ".join(str(int(v)) for v in np.asarray(a).reshape(-1))


def _flat_rows(x, ld):
    """Rows of width x.shape[1] at stride ld, the last row without slack."""
    rows, width = x.shape
    if rows == 0:
        return np.zeros(0, np.float32), np.zeros((0, width), np.float32)
    buf = np.full((rows - 1) * ld + width, np.float32(12345.0))
    view = np.lib.stride_tricks.as_strided(buf, (rows, width), (ld * 4, 4))
    view[...] = x
    return buf, view


def _golden_workloads():
    conv = {"nan": np.nan, "inf": np.inf, "-inf": -np.inf, "-0": -0.0}
    with open(os.path.join(HERE, "golden", "hand_worked.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        width = len(c["logits"][0])
        x = np.array([[conv[v] if isinstance(v, str) else float(v) for v in r] for r in c["logits"]],
                     np.float32).reshape(len(c["logits"]), width)
        ks = None if c["row_ks"] is None else np.array(c["row_ks"], np.int32)
        yield workloads.Workload(c["id"], x, ks, np.array(c["row_ke"], np.int32), c["block_size"],
                                 c["topk"], c["row_repeat"])


def _oracle_cases():
    """(record text, expected output line) for every case."""
    recs = []
    sel = list(_golden_workloads()) + [workloads.random_case(s) for s in range(120)]
    sel += [workloads.many_rows_case(900 + s, 9, 3001 + s, (1, 7, 64)[s % 3], 1 + s % 3, 20)
            for s in range(6)]
    for i, w in enumerate(sel):
        if w.width == 0:
            continue
        ld = w.width + i % 3
        buf, view = _flat_rows(w.logits, ld)
        groups = -(-w.rows // w.row_repeat)
        starts = "" if w.row_ks is None else _ints(w.row_ks[:groups])
        rec = (f"S {w.rows} {w.width} {ld} {w.block_size} {w.row_repeat} {w.topk_blocks} "
               f"{int(w.row_ks is not None)} {1 + i % 3} {starts} {_ints(w.row_ke[:groups])} "
               f"{_hex(buf)}")
        nb = -(-w.width // w.block_size)
        out = np.empty((w.rows, w.topk_blocks), np.int32)
        sc = np.empty((w.rows, nb), np.float32)
        oracle.select_candidate_blocks(view, w.row_ks, w.row_ke, w.topk_blocks, w.block_size, out,
                                       w.row_repeat, scores_out=sc)
        off = oracle.block_scores(view, w.row_ks, w.row_ke, w.block_size, w.row_repeat,
                                  pin_newest=False)
        exp = f"S 0 {_ints(out)} {_hex(sc)} | 0 {_hex(off)}".replace("  ", " ").strip()
        recs.append((rec, exp))
    for seed in range(40):
        w = workloads.random_scores_case(seed, max_rows=12, max_nscore=400)
        rows, n = w.scores.shape
        ld = n + seed % 2
        if rows == 0 or n == 0:
            continue
        buf, view = _flat_rows(w.scores, ld)
        groups = -(-rows // w.row_repeat)
        rec = (f"F {rows} {n} {ld} {w.max_global_blocks} {w.row_repeat} {w.global_block_size} "
               f"{w.topk_blocks} {_ints(w.global_row_ke[:groups])} {_hex(buf)}")
        out = np.empty((rows, w.topk_blocks), np.int32)
        oracle.select_from_scores(view, w.global_row_ke, w.topk_blocks, w.global_block_size,
                                  w.max_global_blocks, out, w.row_repeat)
        exp = f"F 0 {_ints(out)} | 0 {_ints(out)}"
        recs.append((rec, exp))
    rng = np.random.default_rng(44)
    for i in range(16):
        rows, width = int(rng.integers(1, 6)), int(rng.integers(1, 3000))
        B, R, k = int(rng.choice([1, 3, 64])), int(rng.integers(1, 3)), int(rng.integers(0, 9))
        groups = -(-rows // R)
        x = rng.standard_normal((rows, width)).astype(np.float32)
        starts = rng.integers(-5, width, size=groups).astype(np.int32) if i % 2 else None
        ends = rng.integers(-3, width + 9, size=groups).astype(np.int32)
        ldc = k + 1
        cand = rng.integers(-1, -(-width // B) + 2, size=(rows, ldc)).astype(np.int32)
        ld = width + i % 2
        buf, view = _flat_rows(x, ld)
        cflat = cand.reshape(-1)[:(rows - 1) * ldc + k]   # the last row's first k entries
        rec = (f"M {rows} {width} {ld} {B} {R} {k} {int(starts is not None)} {ldc} "
               f"{'' if starts is None else _ints(starts)} {_ints(ends)} {_ints(cflat)} "
               f"{_hex(buf)}")
        exp_buf, exp_view = _flat_rows(x, ld)
        oracle.mask_candidates(exp_view, starts, ends, cand, k, B, R)
        recs.append((rec, f"M 0 {_hex(exp_buf)}"))
    return recs


def _lse_cases():
    out = []
    for N in (1, 3, 70):
        w = workloads.lse_merge(B=3, H=2, D=5, N=N, seed=500 + N)
        w.lses[0, 0, 0] = np.nan
        w.lses[-1, 1, 1] = np.inf
        rank = N - 1
        rec = f"L 3 2 5 {N} {rank} {_hex(w.out)} {_hex(w.lses)}"
        new, lse = oracle.correct_attn_out(w.out, w.lses, rank)
        out.append((rec, lse.reshape(-1), new.reshape(-1)))   # new is [H, B, D]
    return out


def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "sanitize_oracle")
    subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-D_GNU_SOURCE", "-Wall", "-Wextra",
                           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
                           os.path.join(HERE, "sanitize_oracle.c"),
                           os.path.join(ROOT, "oracle", "oracle.c"), "-o", exe, "-lm"])
    cases = _oracle_cases()
    lse = _lse_cases()
    path = tmp_path / "cases.txt"
    path.write_text("\n".join([r for r, _ in cases] + [r for r, _, _ in lse]) + "\n")
    res = subprocess.run([exe, str(path)], capture_output=True, text=True, timeout=600, env=ENV)
    assert res.returncode == 0, res.stderr[-4000:]
    lines = res.stdout.strip().split("\n")
    assert len(lines) == len(cases) + len(lse)
    for (rec, exp), got in zip(cases, lines):
        assert " ".join(got.split()) == " ".join(exp.split()), rec[:80]
    for (rec, exp_lse, exp_new), got in zip(lse, lines[len(cases):]):
        vals = got.split()
        assert vals[:2] == ["L", "0"]
        nums = np.array([float(v) for v in vals[2:]])
        exp = np.concatenate([exp_lse, exp_new])
        assert np.array_equal(nums, exp, equal_nan=True), rec[:40]   # printed with 17 digits


def _host_build():
    """The sanitized host driver, built once per source state (cached)."""
    srcs = [os.path.join(CSRC, "dsa.hip"), os.path.join(CSRC, "stream_geom.h"),
            os.path.join(ROOT, "include", "dsa.h"), os.path.join(HERE, "sanitize_host.cpp")]
    h = hashlib.sha256()
    for s in srcs:
        h.update(open(s, "rb").read())
    exe = os.path.join(tempfile.gettempdir(), f"dsa_sanitize_host_{h.hexdigest()[:16]}")
    if not os.path.exists(exe):
        cmd = [os.environ.get("HIPCC", "/opt/rocm/bin/hipcc"), "--offload-arch=gfx950", "-O1", "-g",
               "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
               "-Xarch_host", "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "include"),
               srcs[0], srcs[3], "-o", exe + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        assert res.returncode == 0, res.stderr[-4000:]
        os.replace(exe + ".tmp", exe)
    return exe


def test_host_code_under_sanitizers():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the driver's fake pointers would reach a kernel")
    exe = _host_build()
    res = subprocess.run([exe], capture_output=True, text=True, timeout=900, env=ENV)
    assert res.returncode == 0, (res.stdout[-3000:], res.stderr[-4000:])
    assert res.stdout.strip().splitlines()[-1].startswith("ok "), res.stdout[-2000:]
