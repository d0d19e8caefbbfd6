#!/usr/bin/env python3
"""Benchmark of DSA candidate-block selection on one MI355X.

A step is one call of dsa_select_candidate_blocks (windowed block max, pin,
top-k, ordered -1 padded store; one launch, or two under the split plan) over
one batch of the chosen synthetic workload, with its inputs already resident
in HBM.
The default workload is the decode batch (64 rows x 32768 columns, block 64,
top-32, row_repeat 2).

Protocol
  * inputs are drawn on the host (sparse_attention_kv_dsa_amd.workloads),
    checked once against the CPU oracle, then copied to M device copies so
    that >= 2 GiB of logits stream between two uses of the same copy (the
    256 MB Infinity Cache would otherwise serve them);
  * W warmup steps, then exactly K steps, captured into a HIP graph (step i
    uses copy i mod M) and replayed between two synchronisations; HIP events
    on the replay stream give the time;
  * value = in-window logits GB/s (algorithmic bytes: only the columns of
    each row's [start, end) window are counted), rows/s beside it;
  * roofline: HBM-bound, achieved = algorithmic bytes per launch / average
    launch duration, against the 8 TB/s MI355X peak; traffic = per-launch HBM
    bytes from rocprofv3 counters (profiles/traffic.json) when they were taken
    on the current kernel source, else null;
  * cpu_baseline: the oracle (plain C, all host cores) on the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "candidate-block selection: logits GB/s (fraction of HBM peak) and rows/s, 1 GPU"
HBM_PEAK_GBPS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "sparse_attention_kv_dsa_amd", "csrc", "dsa.hip")
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="workload (1 tiny, 2 decode, 3 prefill, 4 long-context decode, 5 large prefill)")
    ap.add_argument("--plan", type=int, default=0, choices=[0, 1, 2, 3])
    ap.add_argument("--plan-arg", type=int, default=0,
                    help="plan 1: waves per workgroup; plan 2: blocks per chunk (0: automatic)")
    ap.add_argument("--rotate-bytes", type=float, default=2.0, help="GiB of input copies to rotate over")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget (0: skip)")
    ap.add_argument("--eager", action="store_true", help="launch every step from Python, no graph")
    ap.add_argument("--profile", action="store_true",
                    help="short eager run for rocprofv3: no graph, no oracle timing, no context runs")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain copy of this many MiB (counter scale for rocprofv3 --pmc)")
    return ap.parse_args()


def kernel_src_hash() -> str:
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def in_window_bytes(w) -> int:
    import numpy as np
    r = np.arange(w.rows)
    g = r // w.row_repeat
    s = np.zeros(w.rows, np.int64) if w.row_ks is None else w.row_ks.astype(np.int64)[g]
    e = w.row_ke.astype(np.int64)[g]
    lo, hi = np.maximum(s, 0), np.minimum(e, w.width)
    return int(np.maximum(hi - lo, 0).sum()) * 4


def algorithmic_bytes(w) -> int:
    groups = -(-w.rows // w.row_repeat)
    bounds = groups * 4 * (2 if w.row_ks is not None else 1)
    return in_window_bytes(w) + bounds + w.rows * w.topk_blocks * 4


def traffic_for(workload: str, plan: int):
    """Per-launch HBM bytes from committed rocprofv3 counters, if they match
    the current kernel source and plan; otherwise None."""
    try:
        with open(TRAFFIC_JSON) as fh:
            rec = json.load(fh).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_src_sha256_16") != kernel_src_hash() or rec.get("plan") != plan:
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(w, budget_s: float):
    import numpy as np
    import oracle
    threads = len(os.sched_getaffinity(0))
    out = np.empty((w.rows, w.topk_blocks), dtype=np.int32)
    oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks, w.block_size,
                                   out, w.row_repeat, nthreads=threads)          # warm
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks,
                                       w.block_size, out, w.row_repeat, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 100000:
            break
    per = el / reps
    return {"value": round(in_window_bytes(w) / per / 1e9, 4), "unit": "GB/s",
            "rows_per_s": round(w.rows / per, 1), "cores": threads, "kind": "oracle",
            "sample": f"the whole {w.name} batch ({w.rows} rows), {reps} back-to-back calls "
                      f"in {el:.1f} s, rows split over {threads} threads"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus N > 1 is not supported "
                                   "(rows shard across GPUs with no communication, see DESIGN.md)"}))
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_attention_kv_dsa_amd as dsa
    from sparse_attention_kv_dsa_amd import build as dsa_build
    from sparse_attention_kv_dsa_amd import workloads

    dev = torch.device("cuda:0")
    w = workloads.config(args.config)
    print(f"# workload {w.name}: drawn", file=sys.stderr, flush=True)
    nb = -(-w.width // w.block_size)
    plan, cb = dsa.select_plan(w.rows, w.width, w.block_size, w.topk_blocks)
    if args.plan:
        plan, cb = args.plan, args.plan_arg
    L = dsa.lib()

    ks = None if w.row_ks is None else torch.from_numpy(w.row_ks).to(dev)
    ke = torch.from_numpy(w.row_ke).to(dev)
    mat_bytes = w.logits.nbytes
    copies = max(1, min(512, int(-(-args.rotate_bytes * 2**30 // mat_bytes))))
    if args.profile:
        copies = 1
    host = torch.from_numpy(w.logits)
    xs = [host.to(dev) for _ in range(copies)]
    out = torch.empty((w.rows, w.topk_blocks), dtype=torch.int32, device=dev)
    ws = dsa.Workspace(dev, dsa.select_workspace_bytes(w.rows, w.width, w.block_size,
                                                       w.topk_blocks))
    torch.cuda.synchronize()

    # parity once, before timing
    dsa.select_candidate_blocks(xs[0], ks, ke, w.topk_blocks, w.block_size, out, w.row_repeat,
                                workspace=ws, plan=plan, plan_arg=cb)
    got = out.cpu().numpy()
    parity = None
    if not args.profile or w.rows <= 128:
        import oracle
        exp = np.empty_like(got)
        if w.rows > 512:   # the oracle checks a row sample on the big prefill workloads
            rows = np.linspace(0, w.rows - 1, 64).astype(np.int64)
            sub = workloads.Workload(w.name, np.ascontiguousarray(w.logits[rows]),
                                     None if w.row_ks is None else w.row_ks[rows].copy(),
                                     w.row_ke[rows].copy(), w.block_size, w.topk_blocks, 1)
            exp = np.empty((len(rows), w.topk_blocks), np.int32)
            oracle.select_candidate_blocks(sub.logits, sub.row_ks, sub.row_ke, sub.topk_blocks,
                                           sub.block_size, exp, 1, nthreads=8)
            parity = bool(np.array_equal(got[rows], exp))
        else:
            oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks,
                                           w.block_size, exp, w.row_repeat, nthreads=8)
            parity = bool(np.array_equal(got, exp))
    print(f"# parity vs oracle: {parity}", file=sys.stderr, flush=True)

    vp = ctypes.c_void_p
    ks_p = None if ks is None else ks.data_ptr()

    def launch(i):
        code = L.dsa_select_candidate_blocks_plan(
            xs[i % copies].data_ptr(), w.rows, w.width, w.width, ks_p, ke.data_ptr(),
            w.topk_blocks, w.block_size, w.row_repeat, out.data_ptr(), w.topk_blocks, None, 0,
            ws.buf.data_ptr(), ws.buf.numel(), plan, cb,
            vp(torch.cuda.current_stream(dev).cuda_stream))
        if code:
            raise RuntimeError(f"dsa_select_candidate_blocks: {dsa.status_string(code)}")

    if args.calib_copy_mib:
        calib = ctypes.CDLL(dsa_build.lib_path("libdsa_calib.so"))
        calib.dsa_calib_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
        nbytes = args.calib_copy_mib << 20
        a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        assert calib.dsa_calib_copy(a.data_ptr(), b.data_ptr(), nbytes,
                                    vp(torch.cuda.current_stream(dev).cuda_stream)) == 0
        torch.cuda.synchronize()
        print(f"# calibration copy of {args.calib_copy_mib} MiB done", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    use_graph = not (args.eager or args.profile)
    K, W = args.steps, args.warmup
    if use_graph:
        cap = torch.cuda.Stream(dev)
        graphs = {}
        for name, n in (("warm", W), ("timed", K)):
            g = torch.cuda.CUDAGraph()
            if n:
                with torch.cuda.graph(g, stream=cap):
                    for i in range(n):
                        launch(i)
            graphs[name] = g
        torch.cuda.synchronize()
        if W:
            graphs["warm"].replay()
    else:
        for i in range(W):
            launch(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    if use_graph:
        graphs["timed"].replay()
    else:
        for i in range(K):
            launch(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / K
    print(f"# timed {K} steps: {ms * 1e3:.2f} us/step (wall {wall:.3f} s)", file=sys.stderr,
          flush=True)
    # every launch of the timed region wrote the same ids
    assert np.array_equal(out.cpu().numpy(), got), "timed launches disagree with the checked one"

    win = in_window_bytes(w)
    alg = algorithmic_bytes(w)
    gbps = win / (ms * 1e-3) / 1e9
    achieved = alg / (ms * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(gbps, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": W, "ms_per_step": round(ms, 6), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "width": w.width,
                   "block_size": w.block_size, "topk_blocks": w.topk_blocks,
                   "row_repeat": w.row_repeat, "plan": plan, "plan_arg": cb,
                   "input_copies": copies, "graph": use_graph,
                   "logits_sha256": workloads.sha256(w.logits)[:16]},
        "rows_per_s": round(w.rows / (ms * 1e-3), 1),
        "parity": parity,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for(w.name, plan),
                     "algorithmic_bytes_per_launch": alg, "in_window_bytes": win,
                     "timed": "whole step (both kernels under the split plan)",
                     "kernel": {1: "select_group_rows_kernel", 2: "stream_keys_kernel",
                                3: "select_wave_rows_kernel"}[plan]},
    }

    if not args.profile:
        # context: launch floor and a plain read stream on this GPU
        calib = ctypes.CDLL(dsa_build.lib_path("libdsa_calib.so"))
        calib.dsa_calib_empty.argtypes = [vp]
        calib.dsa_calib_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=torch.cuda.Stream(dev)):
            for _ in range(1000):
                calib.dsa_calib_empty(vp(torch.cuda.current_stream(dev).cuda_stream))
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        floor_us = e0.elapsed_time(e1)          # 1000 launches -> ms == us per launch
        nbytes = 2 << 30
        buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        sink = torch.empty(calib.dsa_calib_read_sink_words(), dtype=torch.int32, device=dev)
        sp = vp(stream.cuda_stream)
        for _ in range(2):
            calib.dsa_calib_read(buf.data_ptr(), nbytes, sink.data_ptr(), sp)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            calib.dsa_calib_read(buf.data_ptr(), nbytes, sink.data_ptr(), sp)
        e1.record(stream)
        torch.cuda.synchronize()
        read_gbps = 5 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del buf
        res["context"] = {"graph_launch_floor_us": round(floor_us, 3),
                          "read_stream_GBps": round(read_gbps, 1),
                          "frac_of_read_stream": round(achieved / read_gbps, 4)}
        if args.cpu_seconds > 0:
            print("# timing the CPU oracle", file=sys.stderr, flush=True)
            res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
