#!/usr/bin/env python3
"""Benchmark of DSA candidate-block selection on one MI355X.

A step is one call of dsa_select_candidate_blocks (windowed block max, pin,
top-k, ordered -1 padded store; one launch, or two under the split plan) over
one batch of a synthetic workload, with its inputs already resident in HBM.
The headline workload is the large packed prefill (8192 rows x 65536
columns, 2 GiB of logits, block 64, top-64), the largest of the five; the
decode batch, the prefill chunk and the long-context decode are timed in the
same run under the same protocol and reported under `per_config`.

Protocol (every workload)
  * inputs are drawn on the host (sparse_attention_kv_dsa_amd.workloads),
    checked once in full against the CPU oracle (every row, ids and scores),
    then copied to M device copies (M = --rotate-bytes / matrix size, at
    least 2);
  * W warmup steps (step i reads copy i mod M), then five timed regions of
    exactly K steps each, every region its own HIP graph replayed between two
    synchronisations; step i of region j reads copy (W + j*K + i) mod M, so
    the copies keep rotating and no timed step re-reads a copy a warmup step
    has just read: the 256 MB Infinity Cache cannot serve them.  HIP events
    on the replay stream time each region; the first region is the reported
    step time, the five give its spread;
  * value = in-window logits GB/s (algorithmic bytes: only the columns of
    each row's [start, end) window are counted), rows/s beside it;
  * roofline: HBM-bound, achieved = algorithmic bytes per launch / average
    step time, against the 8 TB/s MI355X peak; traffic = per-launch HBM
    bytes from rocprofv3 counters (profiles/traffic.json) when they were
    taken on the current kernel source and plan, else null;
  * cpu_baseline: the oracle (plain C, all host cores) on the headline
    workload.
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
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5],
                    help="headline workload (1 tiny, 2 decode, 3 prefill, 4 long-context decode, "
                         "5 large prefill)")
    ap.add_argument("--per-config", default="auto",
                    help="comma list of workloads also timed into per_config ('auto': 2-5 "
                         "without the headline; 'none': no others)")
    ap.add_argument("--plan", type=int, default=0, choices=[0, 1, 2, 3, 4])
    ap.add_argument("--plan-arg", type=int, default=0,
                    help="plan 1: waves per workgroup; plan 2: blocks per chunk (0: automatic)")
    ap.add_argument("--rotate-bytes", type=float, default=4.0,
                    help="GiB of input copies to rotate over (at least two copies)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle time budget (0: skip)")
    ap.add_argument("--eager", action="store_true", help="launch every step from Python, no graph")
    ap.add_argument("--profile", action="store_true",
                    help="short eager run for rocprofv3: no graph, no oracle timing, no context runs")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain copy of this many MiB (counter scale for rocprofv3 --pmc)")
    ap.add_argument("--keys", action="store_true",
                    help="with --op scores / blockscores: the uint32-code variants "
                         "(dsa_select_from_keys / dsa_block_score_keys)")
    ap.add_argument("--op", default="select",
                    choices=["select", "scores", "mask", "lse", "blockscores"],
                    help="select: candidate-block selection (the headline, default); scores: the "
                         "DCP selection from reduced scores; mask: candidate masking; lse: the "
                         "base-2 LSE correction; blockscores: one DCP rank's local block "
                         "scores (pin off)")
    return ap.parse_args()


def kernel_src_hash() -> str:
    """sha256 prefix of the kernel source's code: comments and whitespace are
    dropped first, so editing a comment keeps the committed counters valid.
    (A // inside a string literal would be cut too; the source has none.)"""
    import re
    with open(KERNEL_SRC, encoding="utf-8") as fh:
        text = fh.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    text = re.sub(r"\s+", "", text)
    return hashlib.sha256(text.encode()).hexdigest()[:16]


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
    """The oracle on the whole batch, rows split over every host core the
    process may use (the reported baseline), then on one thread for about a
    third of the budget (beside it)."""
    import numpy as np
    import oracle
    threads = len(os.sched_getaffinity(0))
    out = np.empty((w.rows, w.topk_blocks), dtype=np.int32)

    def timed(nthreads, budget):
        oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks,
                                       w.block_size, out, w.row_repeat, nthreads=nthreads)  # warm
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks,
                                           w.block_size, out, w.row_repeat, nthreads=nthreads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget or reps >= 100000:
                return reps, el

    reps, el = timed(threads, budget_s)
    per = el / reps
    reps1, el1 = timed(1, max(1.0, 0.3 * budget_s))
    per1 = el1 / reps1
    return {"value": round(in_window_bytes(w) / per / 1e9, 4), "unit": "GB/s",
            "rows_per_s": round(w.rows / per, 1), "cores": threads, "kind": "oracle",
            "sample": f"the whole {w.name} batch ({w.rows} rows), {reps} back-to-back calls "
                      f"in {el:.1f} s, rows split over {threads} threads",
            "one_thread": {"value": round(in_window_bytes(w) / per1 / 1e9, 4), "unit": "GB/s",
                           "rows_per_s": round(w.rows / per1, 1), "cores": 1,
                           "sample": f"the same batch, {reps1} calls in {el1:.1f} s, one thread"}}


def _calib_copy(args, dev):
    """One plain device copy of --calib-copy-mib MiB: its hardware read/write
    byte counters give the scale for the kernels' counters."""
    if not args.calib_copy_mib:
        return
    import torch
    from sparse_attention_kv_dsa_amd import build as dsa_build
    vp = ctypes.c_void_p
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


def _stream_context(dev, achieved, kind):
    """This GPU's own ceilings beside a result: the launch floor of an empty
    kernel replayed from a graph, and plain 2 GiB read, fill (write-only) and
    copy streams (libdsa_calib.so).  `achieved` (GB/s) is also given as a
    fraction of the `kind` stream that matches the kernel's traffic."""
    import torch
    from sparse_attention_kv_dsa_amd import build as dsa_build
    vp = ctypes.c_void_p
    calib = ctypes.CDLL(dsa_build.lib_path("libdsa_calib.so"))
    calib.dsa_calib_empty.argtypes = [vp]
    calib.dsa_calib_read.argtypes = [vp, ctypes.c_size_t, vp, vp]
    calib.dsa_calib_fill.argtypes = [vp, ctypes.c_size_t, ctypes.c_uint32, vp]
    calib.dsa_calib_copy.argtypes = [vp, vp, ctypes.c_size_t, vp]
    stream = torch.cuda.current_stream(dev)
    sp = vp(stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
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
    half = nbytes // 2
    calls = {
        "read": (lambda: calib.dsa_calib_read(buf.data_ptr(), nbytes, sink.data_ptr(), sp), nbytes),
        "fill": (lambda: calib.dsa_calib_fill(buf.data_ptr(), nbytes, 0xFF800000, sp), nbytes),
        "copy": (lambda: calib.dsa_calib_copy(buf.data_ptr(), buf.data_ptr() + half, half, sp),
                 2 * half),
    }
    ctx = {"graph_launch_floor_us": round(floor_us, 3)}
    for name, (call, moved) in calls.items():
        for _ in range(2):
            assert call() == 0
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(5):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        ctx[f"{name}_stream_GBps"] = round(5 * moved / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del buf
    ctx[f"frac_of_{kind}_stream"] = round(achieved / ctx[f"{kind}_stream_GBps"], 4)
    return ctx


def _time_steps(launch, K, W, copies, dev, use_graph, regions=5):
    """W warmup steps (step i reads copy i mod copies), then `regions` timed
    regions of exactly K steps (step i of region j reads copy
    (W + j*K + i) mod copies), each region its own HIP graph unless
    use_graph is False (then one eager region).  Returns ms per step of the
    first region; _REPEATS holds every region's."""
    import torch
    stream = torch.cuda.current_stream(dev)
    n_regions = regions if use_graph else 1
    if use_graph:
        cap = torch.cuda.Stream(dev)

        def capture(first, n):
            g = torch.cuda.CUDAGraph()
            if n:
                with torch.cuda.graph(g, stream=cap):
                    for i in range(n):
                        launch((first + i) % copies)
            return g

        warm = capture(0, W)
        timed = [capture(W + j * K, K) for j in range(n_regions)]
        torch.cuda.synchronize()
        if W:
            warm.replay()
    else:
        for i in range(W):
            launch(i % copies)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    times = []
    for j in range(n_regions):
        torch.cuda.synchronize()
        e0.record(stream)
        if use_graph:
            timed[j].replay()
        else:
            for i in range(K):
                launch((W + i) % copies)
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / K)
    _REPEATS[:] = times
    return times[0]


_REPEATS: list = []


def _repeats_field():
    """min / median / max ms per step over the timed region and its repeats."""
    v = sorted(_REPEATS)
    if not v:
        return None
    return {"n": len(v), "ms_per_step_min": round(v[0], 6),
            "ms_per_step_median": round(v[len(v) // 2], 6), "ms_per_step_max": round(v[-1], 6)}


def bench_next(args):
    """The rows after selection (one JSON line each): --op scores | mask | lse."""
    import numpy as np
    import torch

    import sparse_attention_kv_dsa_amd as dsa
    from sparse_attention_kv_dsa_amd import workloads

    dev = torch.device("cuda:0")
    use_graph = not (args.eager or args.profile)
    K, W = args.steps, args.warmup
    threads = len(os.sched_getaffinity(0))
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    if args.op == "scores":
        import oracle
        w = workloads.dcp_prefill_scores()
        rows, nscore = w.scores.shape
        mat = w.scores.nbytes
        copies = 1 if args.profile else max(2, min(512, int(-(-args.rotate_bytes * 2**30 // mat))))
        # --keys: the same scores as uint32 codes (the reduced matrix of the
        # integer-maximum reduce), held in int32 tensors
        host = oracle.score_keys(w.scores).view(np.int32) if args.keys else w.scores
        xs = [torch.from_numpy(host).to(dev) for _ in range(copies)]
        ke = i32(w.global_row_ke)
        out = torch.empty((rows, w.topk_blocks), dtype=torch.int32, device=dev)
        sel = dsa.select_from_keys if args.keys else dsa.select_from_scores
        sel(xs[0], ke, w.topk_blocks, w.global_block_size, w.max_global_blocks, out)
        torch.cuda.synchronize()
        exp = np.empty((rows, w.topk_blocks), np.int32)
        oracle.select_from_scores(w.scores, w.global_row_ke, w.topk_blocks, w.global_block_size,
                                  w.max_global_blocks, exp)
        parity = bool(np.array_equal(out.cpu().numpy(), exp))

        def launch(i):
            sel(xs[i], ke, w.topk_blocks, w.global_block_size, w.max_global_blocks, out)

        live = int((w.global_row_ke > 0).sum())
        read = live * min(nscore, w.max_global_blocks) * 4
        alg = read + rows * 4 + rows * w.topk_blocks * 4
        metric = ("DCP select-from-keys: code GB/s (fraction of HBM peak), 1 GPU" if args.keys
                  else "DCP select-from-scores: score GB/s (fraction of HBM peak), 1 GPU")
        value_bytes, kernel = read, "select_scores_kernel"
        cfg = {"workload": w.name + ("-codes" if args.keys else ""), "rows": rows, "nscore": nscore,
               "max_global_blocks": w.max_global_blocks, "global_block_size": w.global_block_size,
               "topk_blocks": w.topk_blocks, "input_copies": copies}

        def cpu(budget):
            sub = max(1, rows // 16)
            o = np.empty((sub, w.topk_blocks), np.int32)
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.select_from_scores(np.ascontiguousarray(w.scores[:sub]), w.global_row_ke[:sub],
                                          w.topk_blocks, w.global_block_size, w.max_global_blocks, o)
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    break
            per = el / reps
            return {"value": round(sub * min(nscore, w.max_global_blocks) * 4 / per / 1e9, 4),
                    "unit": "GB/s", "cores": 1, "kind": "oracle",
                    "sample": f"the first {sub} rows of {w.name}, {reps} calls in {el:.1f} s, one thread"}
    elif args.op == "mask":
        import oracle
        w = workloads.config(3)
        sel = np.empty((w.rows, w.topk_blocks), np.int32)
        oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks, w.block_size,
                                       sel, w.row_repeat, nthreads=threads)
        copies = 1 if args.profile else max(2, min(512, int(-(-args.rotate_bytes * 2**30 // w.logits.nbytes))))
        xs = [torch.from_numpy(w.logits).to(dev) for _ in range(copies)]
        ks, ke, cd = i32(w.row_ks), i32(w.row_ke), i32(sel)
        dsa.mask_candidates(xs[0], ks, ke, cd, w.topk_blocks, w.block_size, w.row_repeat)
        torch.cuda.synchronize()
        exp = w.logits.copy()
        oracle.mask_candidates(exp, w.row_ks, w.row_ke, sel, w.topk_blocks, w.block_size, 1)
        parity = bool(np.array_equal(xs[0].cpu().numpy().view(np.uint32), exp.view(np.uint32)))
        del exp
        # kept columns: in-window columns of selected blocks (neither read nor written)
        kept = 0
        for r in range(w.rows):
            s, e = int(w.row_ks[r]), int(w.row_ke[r])
            for b in sel[r]:
                if b >= 0:
                    lo, hi = max(s + b * w.block_size, s, 0), min(s + (b + 1) * w.block_size, e, w.width)
                    kept += max(hi - lo, 0)
        kept = int(kept)
        written = (w.rows * w.width - kept) * 4

        def launch(i):
            dsa.mask_candidates(xs[i], ks, ke, cd, w.topk_blocks, w.block_size, w.row_repeat)

        alg = written + w.rows * w.topk_blocks * 4 + w.rows * 8
        metric = "candidate masking: written GB/s (fraction of HBM peak), 1 GPU"
        value_bytes, kernel = written, "mask_candidates_kernel"
        cfg = {"workload": "mask-" + w.name, "rows": w.rows, "width": w.width,
               "block_size": w.block_size, "topk_blocks": w.topk_blocks, "input_copies": copies,
               "kept_columns": kept}

        def cpu(budget):
            sub = 64
            reps, t0 = 0, time.perf_counter()
            while True:
                y = np.ascontiguousarray(w.logits[:sub])
                oracle.mask_candidates(y, w.row_ks[:sub], w.row_ke[:sub], np.ascontiguousarray(sel[:sub]),
                                       w.topk_blocks, w.block_size, 1)
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    break
            per = el / reps
            return {"value": round(written * sub / w.rows / per / 1e9, 4), "unit": "GB/s", "cores": 1,
                    "kind": "oracle",
                    "sample": f"the first {sub} rows of the prefill chunk, {reps} calls in {el:.1f} s, one thread"}
    elif args.op == "blockscores":
        import oracle
        w = workloads.dcp_local_logits()
        nb = -(-w.width // w.block_size)
        copies = 1 if args.profile else max(2, min(512, int(-(-args.rotate_bytes * 2**30 // w.logits.nbytes))))
        xs = [torch.from_numpy(w.logits).to(dev) for _ in range(copies)]
        ks, ke = i32(w.row_ks), i32(w.row_ke)
        threads = max(1, min(16, threads))
        if args.keys:
            sc = torch.empty((w.rows, nb), dtype=torch.int32, device=dev)
            run = dsa.block_score_keys
            exp = oracle.block_score_keys(w.logits, w.row_ks, w.row_ke, w.block_size, 1,
                                          pin_newest=False, nthreads=threads).view(np.uint32)
        else:
            sc = torch.empty((w.rows, nb), dtype=torch.float32, device=dev)
            run = dsa.block_scores
            exp = oracle.block_scores(w.logits, w.row_ks, w.row_ke, w.block_size, 1,
                                      pin_newest=False, nthreads=threads).view(np.uint32)
        run(xs[0], ks, ke, w.block_size, 1, pin_newest=False, out=sc)
        torch.cuda.synchronize()
        parity = bool(np.array_equal(sc.cpu().numpy().view(np.uint32), exp))   # every row
        del exp

        def launch(i):
            run(xs[i], ks, ke, w.block_size, 1, pin_newest=False, out=sc)

        read = in_window_bytes(w)
        written = w.rows * nb * 4
        alg = read + written + w.rows * 8
        metric = ("DCP local block score codes: logits GB/s (fraction of HBM peak), 1 GPU"
                  if args.keys else
                  "DCP local block scores: logits GB/s (fraction of HBM peak), 1 GPU")
        value_bytes, kernel = read, "block_scores_kernel"
        cfg = {"workload": w.name + ("-codes" if args.keys else ""), "rows": w.rows,
               "width": w.width, "block_size": w.block_size,
               "pin_newest": False, "input_copies": copies, "scores_bytes": written}

        def cpu(budget):
            sub = 64
            y = np.ascontiguousarray(w.logits[:sub])
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.block_scores(y, w.row_ks[:sub], w.row_ke[:sub], w.block_size, 1,
                                    pin_newest=False)
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    break
            per = el / reps
            sub_read = in_window_bytes(workloads.Workload(w.name, y, w.row_ks[:sub].copy(),
                                                          w.row_ke[:sub].copy(), w.block_size, 0, 1))
            return {"value": round(sub_read / per / 1e9, 4), "unit": "GB/s", "cores": 1,
                    "kind": "oracle",
                    "sample": f"the first {sub} rows of {w.name}, {reps} calls in {el:.1f} s, one thread"}
    else:
        import oracle
        w = workloads.lse_merge()
        B, H, D = w.out.shape
        N = w.lses.shape[0]
        copies = 1 if args.profile else max(2, min(64, int(-(-args.rotate_bytes * 2**30 // w.out.nbytes))))
        outs = [torch.from_numpy(w.out).to(dev) for _ in range(copies)]
        lses = torch.from_numpy(w.lses).to(dev)
        new = torch.empty((H, B, D), dtype=torch.float32, device=dev)
        lse = torch.empty((B, H), dtype=torch.float32, device=dev)
        dsa.correct_attn_out(outs[0], lses, w.cp_rank, new_output=new, lse=lse)
        torch.cuda.synchronize()
        ref_new, ref_lse = oracle.correct_attn_out(w.out, w.lses, w.cp_rank)
        got = new.cpu().numpy().astype(np.float64)
        parity = bool(np.allclose(got, ref_new, rtol=1e-5, atol=0) and
                      np.allclose(lse.cpu().numpy(), ref_lse, rtol=1e-6, atol=1e-5))
        del ref_new, got

        def launch(i):
            dsa.correct_attn_out(outs[i], lses, w.cp_rank, new_output=new, lse=lse)

        alg = 2 * B * H * D * 4 + N * B * H * 4 + B * H * 4
        metric = "DCP LSE correction: HBM GB/s (fraction of HBM peak), 1 GPU"
        value_bytes, kernel = alg, "correct_attn_out_kernel"
        cfg = {"workload": w.name, "B": B, "H": H, "D": D, "N": N, "input_copies": copies}

        def cpu(budget):
            sub = 8
            reps, t0 = 0, time.perf_counter()
            while True:
                oracle.correct_attn_out(np.ascontiguousarray(w.out[:sub]),
                                        np.ascontiguousarray(w.lses[:, :sub]), w.cp_rank)
                reps += 1
                el = time.perf_counter() - t0
                if el >= budget:
                    break
            per = el / reps
            return {"value": round(alg * sub / B / per / 1e9, 4), "unit": "GB/s", "cores": 1,
                    "kind": "oracle",
                    "sample": f"{sub} of {B} query rows, {reps} calls in {el:.1f} s, one thread"}

    print(f"# {args.op}: parity vs oracle: {parity}", file=sys.stderr, flush=True)
    _calib_copy(args, dev)
    ms = _time_steps(launch, K, W, copies, dev, use_graph)
    print(f"# timed {K} steps: {ms * 1e3:.2f} us/step", file=sys.stderr, flush=True)
    alg, value_bytes = int(alg), int(value_bytes)
    achieved = alg / (ms * 1e-3) / 1e9
    res = {"metric": metric, "value": round(value_bytes / (ms * 1e-3) / 1e9, 2), "unit": "GB/s",
           "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic", "config": dict(cfg, graph=use_graph), "parity": parity,
           "repeats": _repeats_field(),
           "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                        "traffic": traffic_for(cfg["workload"], 0),
                        "algorithmic_bytes_per_launch": alg, "kernel": kernel}}
    if not args.profile:
        res["context"] = _stream_context(dev, achieved, {"scores": "read", "mask": "fill",
                                                          "lse": "copy",
                                                          "blockscores": "read"}[args.op])
    if args.cpu_seconds > 0 and not args.profile:
        print("# timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu(args.cpu_seconds)
    print(json.dumps(res), flush=True)


KERNELS = {1: "select_group_rows_kernel", 2: "stream_keys_kernel", 3: "select_wave_rows_kernel",
           4: "select_pair_rows_kernel"}


def bench_select(cfg, args, dev, use_graph):
    """One selection workload under the protocol above: full parity, timing,
    roofline.  Returns (result dict, workload)."""
    import numpy as np
    import torch

    import oracle
    import sparse_attention_kv_dsa_amd as dsa
    from sparse_attention_kv_dsa_amd import workloads

    w = workloads.config(cfg)
    print(f"# workload {w.name}: drawn", file=sys.stderr, flush=True)
    plan, cb = dsa.select_plan(w.rows, w.width, w.block_size, w.topk_blocks)
    if args.plan and cfg == args.config:
        plan, cb = args.plan, args.plan_arg
    L = dsa.lib()
    K, W = args.steps, args.warmup
    ks = None if w.row_ks is None else torch.from_numpy(w.row_ks).to(dev)
    ke = torch.from_numpy(w.row_ke).to(dev)
    copies = 1 if args.profile else max(2, min(512, int(-(-args.rotate_bytes * 2**30 //
                                                          w.logits.nbytes))))
    host = torch.from_numpy(w.logits)
    xs = [host.to(dev) for _ in range(copies)]
    out = torch.empty((w.rows, w.topk_blocks), dtype=torch.int32, device=dev)
    nb = -(-w.width // w.block_size)
    sc = torch.empty((w.rows, nb), dtype=torch.float32, device=dev)
    ws = dsa.Workspace(dev, dsa.select_workspace_bytes(w.rows, w.width, w.block_size,
                                                       w.topk_blocks))
    torch.cuda.synchronize()

    # parity once, before timing: every row's ids and scores against the oracle
    dsa.select_candidate_blocks(xs[0], ks, ke, w.topk_blocks, w.block_size, out, w.row_repeat,
                                scores_out=sc, workspace=ws, plan=plan, plan_arg=cb)
    got, got_sc = out.cpu().numpy(), sc.cpu().numpy()
    del sc
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    exp = np.empty_like(got)
    exp_sc = np.empty_like(got_sc)
    oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks, w.block_size,
                                   exp, w.row_repeat, scores_out=exp_sc, nthreads=threads)
    parity = bool(np.array_equal(got, exp) and
                  np.array_equal(got_sc.view(np.uint32), exp_sc.view(np.uint32)))
    del exp_sc, got_sc
    print(f"# {w.name}: parity vs oracle (all {w.rows} rows, ids and scores): {parity}",
          file=sys.stderr, flush=True)

    vp = ctypes.c_void_p
    ks_p = None if ks is None else ks.data_ptr()

    def launch(i):
        code = L.dsa_select_candidate_blocks_plan(
            xs[i].data_ptr(), w.rows, w.width, w.width, ks_p, ke.data_ptr(),
            w.topk_blocks, w.block_size, w.row_repeat, out.data_ptr(), w.topk_blocks, None, 0,
            ws.buf.data_ptr(), ws.buf.numel(), plan, cb,
            vp(torch.cuda.current_stream(dev).cuda_stream))
        if code:
            raise RuntimeError(f"dsa_select_candidate_blocks: {dsa.status_string(code)}")

    _calib_copy(args, dev)
    ms = _time_steps(launch, K, W, copies, dev, use_graph)
    print(f"# {w.name}: timed {K} steps: {ms * 1e3:.2f} us/step", file=sys.stderr, flush=True)
    # every launch of the timed regions wrote the checked ids
    assert np.array_equal(out.cpu().numpy(), got), "timed launches disagree with the checked one"
    del xs
    torch.cuda.empty_cache()

    win = in_window_bytes(w)
    alg = algorithmic_bytes(w)
    achieved = alg / (ms * 1e-3) / 1e9
    res = {
        "value": round(win / (ms * 1e-3) / 1e9, 2), "unit": "GB/s", "ms_per_step": round(ms, 6),
        "config": {"workload": w.name, "rows": w.rows, "width": w.width,
                   "block_size": w.block_size, "topk_blocks": w.topk_blocks,
                   "row_repeat": w.row_repeat, "plan": plan, "plan_arg": cb,
                   "input_copies": copies, "graph": use_graph,
                   "logits_sha256": workloads.sha256(w.logits)[:16]},
        "rows_per_s": round(w.rows / (ms * 1e-3), 1),
        "parity": parity,
        "repeats": _repeats_field(),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_for(w.name, plan),
                     "algorithmic_bytes_per_launch": alg, "in_window_bytes": win,
                     "timed": ("whole step (both kernels of the split plan)" if plan == 2
                               else "whole step (one kernel launch)"),
                     "kernel": KERNELS[plan]},
    }
    return res, w


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus N > 1 is not "
                                   "supported (rows would shard across GPUs with no "
                                   "communication between them)"}))
        sys.exit(2)
    if args.op != "select":
        bench_next(args)
        return
    import torch

    dev = torch.device("cuda:0")
    use_graph = not (args.eager or args.profile)
    head, w = bench_select(args.config, args, dev, use_graph)
    others = []
    if args.per_config == "auto":
        others = [c for c in (2, 3, 4, 5) if c != args.config]
    elif args.per_config not in ("", "none"):
        others = [int(c) for c in args.per_config.split(",") if int(c) != args.config]
    per = {}
    for c in others:
        r, _ = bench_select(c, args, dev, use_graph)
        per[r["config"]["workload"]] = dict(
            r["config"], ms_per_step=r["ms_per_step"], value=r["value"], unit=r["unit"],
            rows_per_s=r["rows_per_s"], parity=r["parity"], repeats=r["repeats"],
            roofline={k: r["roofline"][k] for k in ("achieved", "frac", "traffic",
                                                    "algorithmic_bytes_per_launch", "kernel")})
    res = {"metric": METRIC, "value": head["value"], "unit": head["unit"], "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic"}
    res.update({k: head[k] for k in ("config", "rows_per_s", "parity", "repeats", "roofline")})
    res["parity_all"] = bool(head["parity"] and all(v["parity"] for v in per.values()))
    if per:
        res["per_config"] = per
    if not args.profile:
        res["context"] = _stream_context(dev, head["roofline"]["achieved"], "read")
        if args.cpu_seconds > 0:
            print("# timing the CPU oracle", file=sys.stderr, flush=True)
            res["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
