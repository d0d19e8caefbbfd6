"""Pins of the oracle's functions for the steps after candidate selection.

select_from_scores (the DCP branch of _select_candidate_blocks_impl after
the reduce, on the vLLM-fork candidate_blocks.py diff page):
- hand-worked cases (tests/golden/next_hand_worked.json);
- the page's decomposition: split a row's columns over W ranks by token
  index mod W, score every shard with block size B/W and the pin off, take
  the element-wise maximum and select from it with the global ends: the ids
  equal the unsharded selection (start 0, end <= width);
- an independent pure-Python statement on random tiny cases.
mask_candidates (the masking function on the same page):
- hand-worked cases; an independent pure-Python statement;
- composition with the selection: re-scoring the masked logits gives the
  original unpinned score on every selected block and -inf elsewhere.
correct_attn_out (page 3, _correct_attn_cp_out_kernel):
- N = 1 is the identity (factor 1, final LSE = the LSE);
- the factors of all ranks sum to 1;
- partial attention merge: splitting one softmax attention over N chunks,
  each with its own base-2 LSE and normalised output, the corrected
  outputs sum to the unsplit attention output and the final LSE is the
  base-2 LSE of all scores (computed directly here, not by the formula);
- NaN / +inf LSEs are left out, an all -inf set gives -inf and factor 0.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "next_hand_worked.json")
NAN, INF = float("nan"), float("inf")


def _f(v):
    if isinstance(v, str):
        return {"nan": np.nan, "inf": np.inf, "-inf": -np.inf, "-0": -0.0}[v]
    return float(v)


def _golden(section):
    with open(GOLDEN) as fh:
        return json.load(fh)[section]


# ------------------------------------------------------------ select_from_scores

@pytest.mark.parametrize("c", _golden("select_from_scores"), ids=lambda c: c["id"])
def test_select_from_scores_hand_worked(c):
    rows = len(c["scores"])
    width = len(c["scores"][0])
    sc = np.array([[_f(v) for v in r] for r in c["scores"]], np.float32).reshape(rows, width)
    out = np.full((rows, c["k"]), 99, np.int32)
    oracle.select_from_scores(sc, np.array(c["ends"], np.int32), c["k"], c["G"],
                              c["max_global_blocks"], out, c["R"])
    assert out.tolist() == c["out"]


def _py_select_from_scores(scores, ends, k, G, max_global_blocks, R):
    """Independent statement: list the non--inf blocks of the pinned, masked
    row in ranking order (NaN first, value descending, id ascending)."""
    rows = len(scores)
    nblocks = max(max_global_blocks, 1)
    res = []
    for r in range(rows):
        e = ends[r // R]
        full = [(scores[r][b] if b < len(scores[r]) else -INF) for b in range(nblocks)]
        p = min(max((e - 1) // G, 0), nblocks - 1)
        full[p] = INF
        if e <= 0:
            full = [-INF] * nblocks
        keyed = sorted(((0 if math.isnan(v) else 1, 0 if math.isnan(v) else -v, b)
                        for b, v in enumerate(full) if not (v == -INF)))
        ids = [b for _, _, b in keyed][:min(k, nblocks)]
        res.append(ids + [-1] * (k - len(ids)))
    return res


def test_select_from_scores_brute_force():
    rng = np.random.default_rng(11)
    vals = np.array([-1.0, 0.5, 1.0, 2.0, -np.inf, np.inf, np.nan], np.float32)
    for _ in range(400):
        rows = int(rng.integers(1, 5))
        R = int(rng.integers(1, 3))
        nscore = int(rng.integers(0, 9))
        mgb = int(rng.integers(0, 10))
        G = int(rng.integers(1, 6))
        k = int(rng.integers(0, 12))
        sc = vals[rng.integers(0, len(vals), size=(rows, nscore))]
        ends = rng.integers(-3, 60, size=-(-rows // R)).astype(np.int32)
        out = np.full((rows, k), 99, np.int32)
        oracle.select_from_scores(sc, ends, k, G, mgb, out, R)
        exp = _py_select_from_scores(sc.tolist(), ends.tolist(), k, G, mgb, R)
        assert out.tolist() == exp


@pytest.mark.parametrize("W", [2, 4])
def test_select_from_scores_dcp_decomposition(W):
    rng = np.random.default_rng(20 + W)
    for _ in range(60):
        rows = int(rng.integers(1, 6))
        B = W * int(rng.integers(1, 5))
        width = int(rng.integers(1, 200))
        k = int(rng.integers(1, 12))
        x = rng.standard_normal((rows, width)).astype(np.float32)
        x[rng.random((rows, width)) < 0.02] = np.nan
        x[rng.random((rows, width)) < 0.05] = -np.inf
        ends = rng.integers(0, width + 1, size=rows).astype(np.int32)
        nblocks = -(-width // B)
        reduced = np.full((rows, nblocks), -np.inf, np.float32)
        for w in range(W):
            local = np.ascontiguousarray(x[:, w::W])
            lend = np.maximum(0, -(-(ends.astype(np.int64) - w) // W)).astype(np.int32)
            if local.shape[1] == 0:
                continue
            sc = oracle.block_scores(local, None, lend, B // W, 1, pin_newest=False)
            n = min(sc.shape[1], nblocks)
            # NaN-propagating element-wise maximum (the inputs hold no zeros)
            reduced[:, :n] = np.maximum(reduced[:, :n], sc[:, :n])
        got = np.empty((rows, k), np.int32)
        oracle.select_from_scores(reduced, ends, k, B, nblocks, got)
        exp = np.empty((rows, k), np.int32)
        oracle.select_candidate_blocks(x, None, ends, k, B, exp)
        assert np.array_equal(got, exp)


# ------------------------------------------------------------------- masking

@pytest.mark.parametrize("c", _golden("mask"), ids=lambda c: c["id"])
def test_mask_hand_worked(c):
    x = np.array([[_f(v) for v in r] for r in c["logits"]], np.float32)
    exp = np.array([[_f(v) for v in r] for r in c["out"]], np.float32)
    ks = None if c["starts"] is None else np.array(c["starts"], np.int32)
    oracle.mask_candidates(x, ks, np.array(c["ends"], np.int32), np.array(c["cand"], np.int32),
                           c["k"], c["B"], c["R"])
    assert np.array_equal(x, exp, equal_nan=True)


def _py_mask(x, starts, ends, cand, k, B, R):
    y = [list(r) for r in x]
    for r, row in enumerate(y):
        g = r // R
        s = 0 if starts is None else starts[g]
        e = ends[g]
        keep_blocks = {c for c in cand[r][:k] if c >= 0}
        for c in range(len(row)):
            if not (s <= c < e and (c - s) // B in keep_blocks):
                row[c] = -INF
    return y


def test_mask_brute_force():
    rng = np.random.default_rng(12)
    for _ in range(300):
        rows = int(rng.integers(1, 5))
        R = int(rng.integers(1, 3))
        width = int(rng.integers(1, 40))
        B = int(rng.integers(1, 7))
        k = int(rng.integers(0, 6))
        G = -(-rows // R)
        x = rng.standard_normal((rows, width)).astype(np.float32)
        x[rng.random((rows, width)) < 0.05] = np.nan
        starts = None if rng.random() < 0.5 else rng.integers(-3, width, size=G).astype(np.int32)
        ends = rng.integers(-2, width + 4, size=G).astype(np.int32)
        cand = rng.integers(-1, -(-width // B) + 2, size=(rows, max(k, 1))).astype(np.int32)
        exp = np.array(_py_mask(x.tolist(), None if starts is None else starts.tolist(),
                                ends.tolist(), cand.tolist(), k, B, R), np.float32)
        oracle.mask_candidates(x, starts, ends, cand, k, B, R)
        assert np.array_equal(x, exp, equal_nan=True)


def test_mask_after_select_keeps_selected_block_scores():
    rng = np.random.default_rng(13)
    for _ in range(40):
        rows, width, B, k = 4, int(rng.integers(20, 300)), int(rng.integers(1, 9)), 5
        x = rng.standard_normal((rows, width)).astype(np.float32)
        starts = rng.integers(0, width // 2, size=rows).astype(np.int32)
        ends = (starts + rng.integers(1, width // 2 + 1, size=rows)).astype(np.int32)
        sel = np.empty((rows, k), np.int32)
        oracle.select_candidate_blocks(x, starts, ends, k, B, sel)
        before = oracle.block_scores(x, starts, ends, B, 1, pin_newest=False)
        y = x.copy()
        oracle.mask_candidates(y, starts, ends, sel, k, B)
        after = oracle.block_scores(y, starts, ends, B, 1, pin_newest=False)
        for r in range(rows):
            chosen = set(int(b) for b in sel[r] if b >= 0)
            for b in range(after.shape[1]):
                if b in chosen:
                    assert after[r, b] == before[r, b]
                else:
                    assert after[r, b] == -np.inf


# ------------------------------------------------------ LSE correction (page 3)

def test_lse_single_rank_is_identity():
    rng = np.random.default_rng(14)
    out = rng.standard_normal((3, 5, 8)).astype(np.float32)
    lses = (rng.standard_normal((1, 3, 5)) * 10).astype(np.float32)
    new, lse = oracle.correct_attn_out(out, lses, 0)
    assert np.array_equal(new, out.transpose(1, 0, 2).astype(np.float64))
    assert np.array_equal(lse, lses[0].astype(np.float64))


def test_lse_equal_ranks_halve():
    out = np.ones((2, 3, 4), np.float32)
    lses = np.full((2, 2, 3), 5.0, np.float32)
    for rank in range(2):
        new, lse = oracle.correct_attn_out(out, lses, rank)
        assert np.allclose(lse, 6.0, rtol=0, atol=1e-12)
        assert np.allclose(new, 0.5, rtol=0, atol=1e-12)


def test_lse_factors_sum_to_one():
    rng = np.random.default_rng(15)
    N, B, H = 6, 4, 7
    lses = (rng.standard_normal((N, B, H)) * 20).astype(np.float32)
    lses[2, 1, 3] = -np.inf
    ones = np.ones((B, H, 1), np.float32)
    total = sum(oracle.correct_attn_out(ones, lses, n)[0][:, :, 0] for n in range(N))
    assert np.allclose(total, 1.0, rtol=0, atol=1e-12)


def test_lse_merge_equals_unsplit_attention():
    rng = np.random.default_rng(16)
    B, H, D, T, N = 3, 4, 16, 40, 5
    s = rng.standard_normal((B, H, T)) * 4       # base-2 logits
    v = rng.standard_normal((B, H, T, D))
    cuts = np.sort(rng.choice(np.arange(1, T), size=N - 2, replace=False))
    bounds = [0, *cuts.tolist(), T, T]            # the last chunk is empty
    lses = np.empty((N, B, H), np.float32)
    outs = np.zeros((N, B, H, D), np.float32)
    for n in range(N):
        a, b = bounds[n], bounds[n + 1]
        if a == b:
            lses[n] = -np.inf
            continue
        w = np.exp2(s[..., a:b])
        z = w.sum(-1)
        lses[n] = np.log2(z)
        outs[n] = (np.einsum("bht,bhtd->bhd", w, v[..., a:b, :]) / z[..., None])
    # the partial results above are rounded to fp32, as a kernel would hold them
    full_w = np.exp2(s)
    full_lse = np.log2(full_w.sum(-1))
    full_out = np.einsum("bht,bhtd->bhd", full_w, v) / full_w.sum(-1)[..., None]
    merged = np.zeros((H, B, D))
    for n in range(N):
        new, lse = oracle.correct_attn_out(np.ascontiguousarray(outs[n]), lses, n)
        merged += new
        assert np.allclose(lse, full_lse, rtol=0, atol=1e-5)
    assert np.allclose(merged, full_out.transpose(1, 0, 2), rtol=1e-5, atol=1e-5)


def test_lse_special_values():
    out = np.ones((1, 4, 2), np.float32)
    lses = np.array([[[np.nan, np.inf, -np.inf, 3.0]],
                     [[1.0, 2.0, -np.inf, np.nan]]], np.float32)   # [N=2, B=1, H=4]
    new0, lse = oracle.correct_attn_out(out, lses, 0)
    new1, _ = oracle.correct_attn_out(out, lses, 1)
    # head 0: rank 0 NaN is left out -> final = 1, factors (NaN -> 0, 1)
    assert lse[0, 0] == 1.0 and new0[0, 0, 0] == 0.0 and new1[0, 0, 0] == 1.0
    # head 1: rank 0 +inf is left out -> final = 2; rank 0's raw +inf gives +inf - 2 -> 0
    assert lse[0, 1] == 2.0 and new0[1, 0, 0] == 0.0 and new1[1, 0, 0] == 1.0
    # head 2: all -inf -> final -inf, factors 0 (no NaN)
    assert lse[0, 2] == -np.inf and new0[2, 0, 0] == 0.0 and new1[2, 0, 0] == 0.0
    # head 3: only rank 0 counts -> final 3, factors 1 and 0
    assert lse[0, 3] == 3.0 and new0[3, 0, 0] == 1.0 and new1[3, 0, 0] == 0.0


def test_lse_strided_views():
    rng = np.random.default_rng(17)
    out = rng.standard_normal((4, 3, 8)).astype(np.float32)
    lses = (rng.standard_normal((5, 4, 3)) * 5).astype(np.float32)
    big = np.zeros((5, 4, 3, 2), np.float32)
    big[..., 0] = lses
    outv = np.zeros((4, 2, 3, 8), np.float32)
    outv[:, 1] = out
    a = oracle.correct_attn_out(out, lses, 2)
    b = oracle.correct_attn_out(outv[:, 1], big[..., 0], 2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------ mutation battery

import subprocess  # noqa: E402

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS_NEXT = {
    "dcp_pin_skipped_not_clamped": ("if (p > nblocks - 1) p = nblocks - 1;\n    full[p] = INFINITY;",
                                    "if (p <= nblocks - 1) full[p] = INFINITY;"),
    "dcp_end_mask_off": ("if (e <= 0)\n      for (int64_t b = 0; b < nblocks; ++b) full[b] = -INFINITY;", ""),
    "dcp_missing_columns_zero": ("full[b] = b < ncopy ? scores[r * ld_scores + b] : -INFINITY;",
                                 "full[b] = b < ncopy ? scores[r * ld_scores + b] : 0.0f;"),
    "dcp_pin_from_end_not_end_minus_one": ("int64_t p = floor_div(e - 1, global_block_size);",
                                           "int64_t p = floor_div(e, global_block_size);"),
    "mask_window_start_ignored": ("if (c >= s && c < e) {", "if (c < e) {"),
    "mask_k_ignored": ("for (int32_t j = 0; j < topk && !keep; ++j)", "for (int32_t j = 0; j < ld_cand && !keep; ++j)"),
    "mask_absolute_blocks": ("int64_t b = (c - s) / block_size;", "int64_t b = c / block_size;"),
    "lse_natural_exp": ("acc += exp2(l - m);", "acc += exp(l - m);"),
    "lse_max_dropped": ("double final_lse = log2(acc) + m;", "double final_lse = log2(acc);"),
    "lse_max_not_reset": ("if (isinf(m) && m < 0) m = 0.0;", ""),
    "lse_local_not_sanitised": ("if (isnan(d) || (isinf(d) && d > 0)) d = -INFINITY;", ""),
    "lse_wrong_rank": ("double d = (double)lses[rank * l_sn", "double d = (double)lses[0 * l_sn"),
}

_BATTERY = None


def _battery_next():
    """True iff the currently loaded oracle passes every pin of this file."""
    checks = [lambda c=c: test_select_from_scores_hand_worked(c) for c in _golden("select_from_scores")]
    checks += [lambda c=c: test_mask_hand_worked(c) for c in _golden("mask")]
    checks += [test_select_from_scores_brute_force, lambda: test_select_from_scores_dcp_decomposition(2),
               test_mask_brute_force, test_mask_after_select_keeps_selected_block_scores,
               test_lse_single_rank_is_identity, test_lse_equal_ranks_halve,
               test_lse_factors_sum_to_one, test_lse_merge_equals_unsplit_attention,
               test_lse_special_values, test_lse_strided_views]
    for chk in checks:
        try:
            chk()
        except AssertionError:
            return False
    return True


def test_unmodified_oracle_passes_next_battery():
    assert _battery_next()


@pytest.mark.parametrize("name", sorted(MUTANTS_NEXT))
def test_next_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS_NEXT[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / "oracle_mut.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
                           "-pthread", str(path), "-o", str(lib), "-lm"])
    with oracle.use_library(str(lib)):
        assert not _battery_next(), f"mutant {name} survived the pins"
