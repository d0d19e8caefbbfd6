"""Pins of the CPU oracle against things other than itself.

- hand-worked rows (tests/golden/hand_worked.json), worked out by hand from
  the definition on the vLLM-fork candidate_blocks.py diff page;
- an independent brute-force full sort (tests/bruteforce.py) on random and
  hypothesis-generated tiny inputs that force NaN, +-0, +-inf and ties;
- special cases that reduce to a library routine: block size 1 (scores are
  the windowed logits), tie-free NaN-free rows (ids == torch.topk over the
  scores, the page's own composition), numpy's max over reshaped blocks;
- the column-interleave decomposition the page states for its DCP branch
  (max over W shards scored with block size B/W equals the unsharded
  scores), and row_repeat == expanded per-row bounds (repeat_interleave);
- invariants: every finite score is an element of its block, no element of
  the block exceeds it, permuting columns inside a block changes nothing,
  output ids are distinct, in range, valid before -1, scores non-increasing.
"""
import json
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, HealthCheck
from hypothesis import strategies as st

import bruteforce
import oracle
from sparse_attention_kv_dsa_amd import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")
CANON_NAN = 0x7FC00000


def _f(v):
    if isinstance(v, str):
        return {"nan": np.nan, "inf": np.inf, "-inf": -np.inf, "-0": -0.0}[v]
    return float(v)


def _arr(rows, width=None):
    a = np.array([[_f(v) for v in r] for r in rows], dtype=np.float32)
    if width is not None:
        a = a.reshape(len(rows), width)
    return a


def _bits(a):
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = a.view(np.uint32).copy()
    b[np.isnan(a)] = CANON_NAN          # expected NaNs are the canonical one
    return b


def _golden():
    with open(GOLDEN) as fh:
        return json.load(fh)["cases"]


def _case_inputs(c):
    width = len(c["logits"][0])
    logits = _arr(c["logits"], width)
    ks = None if c["row_ks"] is None else np.array(c["row_ks"], dtype=np.int32)
    ke = np.array(c["row_ke"], dtype=np.int32)
    return logits, ks, ke


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["id"])
def test_oracle_hand_worked(case):
    logits, ks, ke = _case_inputs(case)
    B, R, k = case["block_size"], case["row_repeat"], case["topk"]
    out = np.full((logits.shape[0], k), 7, dtype=np.int32)
    nb = -(-logits.shape[1] // B)
    sc = np.full((logits.shape[0], max(nb, 1)), 5.0, dtype=np.float32)
    oracle.select_candidate_blocks(logits, ks, ke, k, B, out, R, scores_out=sc[:, :nb] if nb else None)
    assert out.tolist() == case["out"]
    if logits.shape[1]:
        exp = _arr(case["scores"], nb)
        # raw bits, not canonicalised: the oracle must emit 0x7FC00000 itself
        assert (sc[:, :nb].view(np.uint32) == _bits(exp)).all()
        s_pin = oracle.block_scores(logits, ks, ke, B, R, pin_newest=True)
        s_nopin = oracle.block_scores(logits, ks, ke, B, R, pin_newest=False)
        assert (s_pin.view(np.uint32) == _bits(exp)).all()
        assert (s_nopin.view(np.uint32) == _bits(_arr(case["scores_nopin"], nb))).all()


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["id"])
def test_bruteforce_hand_worked(case):
    """The brute force itself agrees with the hand-worked values."""
    logits, ks, ke = _case_inputs(case)
    B, R, k = case["block_size"], case["row_repeat"], case["topk"]
    assert bruteforce.select(logits.tolist(), ks, ke, k, B, R) == case["out"]
    if logits.shape[1]:
        got = np.array(bruteforce.scores(logits.tolist(), ks, ke, B, R), dtype=np.float32)
        assert (_bits(got) == _bits(_arr(case["scores"], got.shape[1]))).all()


def test_rows_zero_leaves_out_untouched():
    out = np.full((0, 4), 7, dtype=np.int32)
    oracle.select_candidate_blocks(np.zeros((0, 10), np.float32), None,
                                   np.zeros(0, np.int32), 4, 4, out)
    sentinel = np.full((3, 4), 7, dtype=np.int32)
    # topk == 0 writes nothing either
    oracle.select_candidate_blocks(np.ones((3, 10), np.float32), None,
                                   np.full(3, 10, np.int32), 0, 4, sentinel[:, :0])
    assert (sentinel == 7).all()


def _oracle_run(w, nthreads=1):
    out = np.empty((w.rows, w.topk_blocks), dtype=np.int32)
    oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks,
                                   w.block_size, out, w.row_repeat, nthreads=nthreads)
    return out


@pytest.mark.parametrize("seed", range(400))
def test_oracle_vs_bruteforce_random(seed):
    w = workloads.random_case(seed, ld_pad=seed % 3)
    got = _oracle_run(w)
    exp = bruteforce.select(w.logits.tolist(), w.row_ks, w.row_ke, w.topk_blocks,
                            w.block_size, w.row_repeat)
    assert got.tolist() == exp
    sc = oracle.block_scores(w.logits, w.row_ks, w.row_ke, w.block_size, w.row_repeat)
    bf = np.array(bruteforce.scores(w.logits.tolist(), w.row_ks, w.row_ke, w.block_size,
                                    w.row_repeat), dtype=np.float32).reshape(sc.shape)
    assert (sc.view(np.uint32) == _bits(bf)).all()


_vals = st.sampled_from([-1.0, -0.0, 0.0, 1.0, 2.0, float("inf"), float("-inf"), float("nan")])


@st.composite
def _tiny(draw):
    rows = draw(st.integers(1, 6))
    width = draw(st.integers(1, 40))
    B = draw(st.integers(1, 9))
    R = draw(st.integers(1, 3))
    k = draw(st.integers(0, 12))
    g = -(-rows // R)
    logits = np.array(draw(st.lists(_vals, min_size=rows * width, max_size=rows * width)),
                      dtype=np.float32).reshape(rows, width)
    ke = np.array(draw(st.lists(st.integers(0, width + 3), min_size=g, max_size=g)), np.int32)
    ks = None
    if draw(st.booleans()):
        ks = np.array(draw(st.lists(st.integers(-3, width + 2), min_size=g, max_size=g)), np.int32)
    return logits, ks, ke, B, R, k


@settings(max_examples=300, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_tiny())
def test_oracle_vs_bruteforce_hypothesis(case):
    logits, ks, ke, B, R, k = case
    out = np.empty((logits.shape[0], k), dtype=np.int32)
    oracle.select_candidate_blocks(logits, ks, ke, k, B, out, R)
    assert out.tolist() == bruteforce.select(logits.tolist(), ks, ke, k, B, R)


def test_block_size_one_scores_are_windowed_logits():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((5, 37), dtype=np.float32)
    x[1, 3] = np.nan
    x[2, 5] = -0.0
    ks = np.array([0, 3, 10, 0, 36], np.int32)
    ke = np.array([37, 20, 10, 1, 37], np.int32)
    sc = oracle.block_scores(x, ks, ke, 1, 1, pin_newest=False)
    for r in range(5):
        exp = np.full(37, -np.inf, np.float32)
        # block b of row r is the single column ks[r] + b
        n = max(0, ke[r] - ks[r])
        exp[:n] = x[r, ks[r]:ks[r] + n]
        assert (sc[r].view(np.uint32) == _bits(exp)).all()


def test_tie_free_rows_match_torch_topk():
    """On NaN-free, tie-free rows the page's composition torch.topk(scores, k')
    followed by -inf -> -1 gives the same ids in the same order."""
    rng = np.random.default_rng(12)
    for trial in range(30):
        rows, width, B = 7, int(rng.integers(50, 600)), int(rng.integers(1, 40))
        x = rng.permutation(rows * width).astype(np.float32).reshape(rows, width)
        ke = rng.integers(0, width + 1, size=rows).astype(np.int32)
        k = int(rng.integers(1, 40))
        sc = oracle.block_scores(x, None, ke, B, 1, pin_newest=True)
        out = np.empty((rows, k), np.int32)
        oracle.select_candidate_blocks(x, None, ke, k, B, out, 1)
        kk = min(k, sc.shape[1])
        t = torch.topk(torch.from_numpy(sc), kk, dim=-1)
        ids = torch.where(torch.isinf(t.values) & (t.values < 0), -1, t.indices).numpy()
        exp = np.full((rows, k), -1, np.int32)
        exp[:, :kk] = ids
        # several blocks can share the value -inf; all of them become -1
        assert (out == exp).all(), trial


def test_numpy_blockwise_max():
    """NaN-free, +-0-free rows: scores == numpy max over -inf padded blocks."""
    rng = np.random.default_rng(13)
    for B in (1, 3, 4, 7, 64):
        x = rng.standard_normal((6, 333), dtype=np.float32)
        sc = oracle.block_scores(x, None, np.full(6, 333, np.int32), B, 1, pin_newest=False)
        nb = -(-333 // B)
        pad = np.full((6, nb * B), -np.inf, np.float32)
        pad[:, :333] = x
        assert (sc == pad.reshape(6, nb, B).max(axis=2)).all()


def test_row_repeat_equals_expanded_bounds():
    w = workloads.random_case(5, max_rows=9, max_width=120, special=True)
    for R in (1, 2, 3, 4):
        g = -(-w.rows // R)
        rng = np.random.default_rng(R)
        ks = rng.integers(0, w.width, size=g).astype(np.int32)
        ke = rng.integers(0, w.width + 1, size=g).astype(np.int32)
        a = np.empty((w.rows, 5), np.int32)
        b = np.empty((w.rows, 5), np.int32)
        oracle.select_candidate_blocks(w.logits, ks, ke, 5, 3, a, R)
        oracle.select_candidate_blocks(w.logits, np.repeat(ks, R)[:w.rows], np.repeat(ke, R)[:w.rows],
                                       5, 3, b, 1)
        assert (a == b).all()


@pytest.mark.parametrize("W", [2, 4, 8])
def test_column_interleave_decomposition(W):
    """Token t on shard t mod W at local slot t div W; local block size B/W.
    The max over shards of the local (pin-off) scores equals the global
    pin-off scores when W divides B and the start."""
    rng = np.random.default_rng(W)
    rows, width, B = 6, 64 * 9, 16
    vals = workloads.SPECIAL_VALUES
    x = vals[rng.integers(0, len(vals), size=(rows, width))]
    x[:, ::5] = rng.standard_normal((rows, x[:, ::5].shape[1])).astype(np.float32)
    ks = (rng.integers(0, 20, size=rows) * W).astype(np.int32)
    ke = rng.integers(0, width + 1, size=rows).astype(np.int32)
    ref = oracle.block_scores(x, ks, ke, B, 1, pin_newest=False)
    nb = ref.shape[1]
    acc = np.full((rows, nb), -np.inf, np.float32)
    for w in range(W):
        shard = np.ascontiguousarray(x[:, w::W])
        # local bounds: number of owned tokens below start / end
        lks = ((ks - w + W - 1) // W).astype(np.int32)
        lke = ((ke - w + W - 1) // W).astype(np.int32)
        loc = oracle.block_scores(shard, lks, lke, B // W, 1, pin_newest=False)
        n = min(nb, loc.shape[1])
        a, b = acc[:, :n], loc[:, :n]
        both = np.where(np.isnan(a) | np.isnan(b), np.float32(np.nan),
                        np.where((a == b) & (a == 0), np.where(np.signbit(a) & np.signbit(b), a, np.float32(0.0)),
                                 np.maximum(a, b)))
        acc[:, :n] = both
    assert (_bits(acc) == ref.view(np.uint32)).all()


def _check_invariants(w, out, sc):
    rows, width = w.logits.shape
    B = w.block_size
    nb = sc.shape[1]
    for r in range(rows):
        g = r // w.row_repeat
        s = 0 if w.row_ks is None else int(w.row_ks[g])
        e = int(w.row_ke[g])
        p = (e - s - 1) // B if e > s else -1
        for b in range(nb):
            lo, hi = max(s + b * B, s, 0), min(s + (b + 1) * B, e, width)
            blk = w.logits[r, lo:hi] if hi > lo else np.zeros(0, np.float32)
            v = sc[r, b]
            if b == p:
                assert v == np.inf
            elif blk.size == 0:
                assert v == -np.inf
            elif np.isnan(blk).any():
                assert sc[r, b:b + 1].view(np.uint32)[0] == CANON_NAN
            else:
                assert (blk.view(np.uint32) == np.float32(v).view(np.uint32)).any()   # exact
                assert not (blk > v).any()
        ids = [i for i in out[r] if i >= 0]
        assert len(set(ids)) == len(ids) and all(0 <= i < nb for i in ids)
        n = len(ids)
        assert (out[r, n:] == -1).all()
        seq = sc[r, ids]
        for a, b in zip(seq[:-1], seq[1:]):
            assert np.isnan(a) or (not np.isnan(b) and a >= b)


@pytest.mark.parametrize("seed", range(40))
def test_oracle_invariants(seed):
    w = workloads.random_case(seed + 7000, max_rows=5, max_width=300, max_block=70, max_k=20,
                              special=seed % 2 == 0)
    out = _oracle_run(w)
    sc = oracle.block_scores(w.logits, w.row_ks, w.row_ke, w.block_size, w.row_repeat)
    _check_invariants(w, out, sc)
    # permuting columns inside every block (relative to the first row's start) changes nothing
    if w.row_ks is None:
        rng = np.random.default_rng(seed)
        perm = np.arange(w.width)
        for b0 in range(0, w.width, w.block_size):
            seg = perm[b0:b0 + w.block_size]
            rng.shuffle(seg)
        # a permutation that moves an element across the window edge changes the
        # element set, so only permute rows whose window covers whole blocks
        ok = all((int(w.row_ke[r // w.row_repeat]) % w.block_size == 0
                  or int(w.row_ke[r // w.row_repeat]) >= w.width) for r in range(w.rows))
        if ok:
            w2 = workloads.Workload(w.name, np.ascontiguousarray(w.logits[:, perm]), None,
                                    w.row_ke, w.block_size, w.topk_blocks, w.row_repeat)
            assert (_oracle_run(w2) == out).all()


def test_threads_do_not_change_results():
    w = workloads.random_case(3, max_rows=64, max_width=2000, max_block=70, max_k=40,
                              special=False)
    assert (_oracle_run(w, 1) == _oracle_run(w, 7)).all()


def test_tiny_workload_invariants():
    w = workloads.tiny()
    out = _oracle_run(w)
    sc = oracle.block_scores(w.logits, w.row_ks, w.row_ke, w.block_size, w.row_repeat)
    _check_invariants(w, out, sc)
    exp = bruteforce.select(w.logits.tolist(), w.row_ks, w.row_ke, w.topk_blocks,
                            w.block_size, w.row_repeat)
    assert out.tolist() == exp
    assert (out[0] == -1).all()        # the end = 0 row selects nothing
