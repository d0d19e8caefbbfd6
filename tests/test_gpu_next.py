"""GPU parity for the steps after selection, against the CPU oracle.

- dsa_select_from_scores (the DCP branch after its reduce): ids bit-exact on
  random cases (NaN, +-inf, ties, clamped pins, ends <= 0, short and
  truncated score rows, row_repeat) and on the full-size DCP prefill share;
  plus the DCP decomposition run on the GPU (shards scored by
  dsa_block_scores with the pin off, reduced with an element-wise maximum)
  against the unsharded GPU selection.
- dsa_block_score_keys / dsa_select_from_keys (the same DCP steps on
  order-preserving uint32 codes): codes bit-exact on random cases and at
  full size, the selection on random and raw codes, and the DCP
  decomposition reduced by an integer maximum with +-0 and NaN present.
- dsa_mask_candidates: bit-exact against the oracle on random cases (odd
  widths and block sizes, unaligned rows, negative starts) and on the
  prefill chunk masked with its own selection (every row).
- dsa_correct_attn_out: within the fp32 tolerance stated below against the
  oracle's float64 arithmetic, for N up to 70 ranks (more than one pass of
  64 lanes), strided views, special values and the full-size workload.
Expected values come only from oracle/.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_kv_dsa_amd as dsa
from sparse_attention_kv_dsa_amd import workloads
from bound_rows import bound_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
HOST_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _say(*a):
    print(*a, flush=True)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


# ------------------------------------------------------------ select_from_scores

def _gpu_sfs(w, ld_pad=0):
    rows, nscore = w.scores.shape
    sc = torch.full((rows, nscore + ld_pad), 12345.0, dtype=torch.float32, device=DEV)
    sc[:, :nscore] = torch.from_numpy(w.scores).to(DEV)
    out = torch.full((rows, w.topk_blocks + 2), 777, dtype=torch.int32, device=DEV)
    dsa.select_from_scores(sc[:, :nscore], _i32(w.global_row_ke), w.topk_blocks,
                           w.global_block_size, w.max_global_blocks, out[:, :w.topk_blocks],
                           w.row_repeat)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert (got[:, w.topk_blocks:] == 777).all(), "wrote past topk_blocks"
    return got[:, :w.topk_blocks]


def _oracle_sfs(w):
    exp = np.empty((w.scores.shape[0], w.topk_blocks), np.int32)
    oracle.select_from_scores(w.scores, w.global_row_ke, w.topk_blocks, w.global_block_size,
                              w.max_global_blocks, exp, w.row_repeat)
    return exp


def test_select_from_scores_random_cases():
    for seed in range(60):
        w = workloads.random_scores_case(seed)
        got = _gpu_sfs(w, ld_pad=seed % 3)
        exp = _oracle_sfs(w)
        assert np.array_equal(got, exp), (seed, w.scores.shape, w.max_global_blocks, w.topk_blocks)


def test_select_from_scores_random_many_rows():
    """Random DCP cases at up to 9000 rows: the narrow workgroups and the
    occupancy the kernel is held to at many rows give the oracle's ids."""
    for seed in range(24):
        w = workloads.random_scores_case(50_000 + seed, max_rows=(600, 3000, 9000)[seed % 3],
                                         max_nscore=2500)
        got = _gpu_sfs(w)
        exp = _oracle_sfs(w)
        assert np.array_equal(got, exp), (seed, w.scores.shape, w.max_global_blocks, w.topk_blocks)


def test_select_from_scores_full_size():
    w = workloads.dcp_prefill_scores()
    _say("select_from_scores", w.name)
    got = _gpu_sfs(w)
    assert np.array_equal(got, _oracle_sfs(w))


def test_select_from_scores_repeats_identical():
    """The two-wave rows of the full-size DCP share (no barrier between
    clearing a row's select state and its select) give the oracle's ids on
    every one of 12 back-to-back calls, at k = 64 (128 group maxima) and at
    k = 32 (64 group maxima, the split rank)."""
    base = workloads.dcp_prefill_scores()
    for k in (64, 32):
        w = workloads.ScoresWorkload(f"{base.name}-k{k}", base.scores, base.global_row_ke,
                                     base.global_block_size, base.max_global_blocks, k,
                                     base.row_repeat)
        exp = _oracle_sfs(w)
        sc = torch.from_numpy(w.scores).to(DEV)
        ke = _i32(w.global_row_ke)
        outs = [torch.empty((sc.shape[0], k), dtype=torch.int32, device=DEV) for _ in range(12)]
        for o in outs:  # back to back on one stream
            dsa.select_from_scores(sc, ke, k, w.global_block_size, w.max_global_blocks, o,
                                   w.row_repeat)
        torch.cuda.synchronize()
        for i, o in enumerate(outs):
            assert np.array_equal(o.cpu().numpy(), exp), (k, i)


@pytest.mark.parametrize("rows,k", [(200, 7), (700, 64), (3000, 64), (3000, 300)])
def test_select_from_scores_row_counts(rows, k):
    """The workgroup width follows the row count (16, 4 or 2 waves per row):
    every width gives the oracle's ids, on scores with heavy ties, NaN, -inf,
    rows whose global end is <= 0 and ends past the last block."""
    rng = np.random.default_rng(rows + k)
    nscore, G = 1024, 64
    x = (np.rint(rng.uniform(-4, 4, size=(rows, nscore)) * 8) / 8).astype(np.float32)
    x[rng.random((rows, nscore)) < 1e-3] = np.nan
    x[rng.random((rows, nscore)) < 2e-2] = -np.inf
    ends = rng.integers(-G, (nscore + 2) * G, size=rows).astype(np.int32)
    w = workloads.ScoresWorkload(f"rows-{rows}-k{k}", x, ends, G, nscore, k, 1)
    got = _gpu_sfs(w, ld_pad=rows % 3)
    assert np.array_equal(got, _oracle_sfs(w))


@pytest.mark.parametrize("rows,n", [(100, 1024), (100, 1500), (600, 1024), (600, 1000),
                                    (600, 1500)])
def test_select_from_scores_bound_paths(rows, n):
    """Rows built around the candidate bound (bound_rows): every path of the
    bound search (128 groups for 32 < k <= 64, 64 groups below) and the
    exact fallback, with the rows' keys held in registers (up to 8 per lane)
    or in LDS, on scores and on their codes."""
    x = bound_rows(rows, n, rows + n)
    G = 16
    rng = np.random.default_rng(n)
    ends = np.full(rows, n * G, np.int32)   # most rows pin their last block
    short = rng.random(rows) < 0.3
    ends[short] = rng.integers(1, n * G, size=int(short.sum()))
    for k in (64, 40, 32, 16):   # 128 groups, then 64
        w = workloads.ScoresWorkload(f"bound-{rows}x{n}-k{k}", x, ends, G, n, k, 1)
        exp = _oracle_sfs(w)
        got = _gpu_sfs(w)
        assert np.array_equal(got, exp), ("scores", rows, n, k)
        codes = oracle.score_keys(x)
        expk = np.empty((rows, k), np.int32)
        oracle.select_from_keys(codes, ends, k, G, n, expk, 1)
        assert np.array_equal(expk, exp)
        kd = torch.from_numpy(codes.view(np.int32)).to(DEV)
        out = torch.full((rows, k), 777, dtype=torch.int32, device=DEV)
        dsa.select_from_keys(kd, _i32(ends), k, G, n, out, 1)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), exp), ("codes", rows, n, k)


@pytest.mark.parametrize("W", [2, 4, 8])
def test_dcp_decomposition_on_gpu(W):
    rng = np.random.default_rng(40 + W)
    rows, width, B, k = 24, 20000, 64, 32
    x = (np.rint(rng.standard_normal((rows, width)) * 4) / 4).astype(np.float32)
    x[rng.random((rows, width)) < 0.2] *= -0.0            # +0 and -0 side by side
    x[rng.random((rows, width)) < 1e-4] = np.nan
    ends = rng.integers(0, width + 1, size=rows).astype(np.int32)
    ends[0] = 0
    xd = torch.from_numpy(x).to(DEV)
    nblocks = -(-width // B)
    reduced = torch.full((rows, nblocks), -float("inf"), dtype=torch.float32, device=DEV)
    for wr in range(W):
        local = xd[:, wr::W].contiguous()
        lend = np.maximum(0, -(-(ends.astype(np.int64) - wr) // W)).astype(np.int32)
        sc = dsa.block_scores(local, None, _i32(lend), B // W, 1, pin_newest=False)
        n = min(sc.shape[1], nblocks)
        # torch.maximum propagates NaN; which zero it keeps for -0 vs +0 is
        # not specified, but the ranking treats them alike (ids compared only)
        reduced[:, :n] = torch.maximum(reduced[:, :n], sc[:, :n])
    got = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    dsa.select_from_scores(reduced, _i32(ends), k, B, nblocks, got)
    ref = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    dsa.select_candidate_blocks(xd, None, _i32(ends), k, B, ref)
    torch.cuda.synchronize()
    exp = np.empty((rows, k), np.int32)
    oracle.select_candidate_blocks(x, None, ends, k, B, exp)
    assert np.array_equal(got.cpu().numpy(), exp)
    assert np.array_equal(ref.cpu().numpy(), exp)


def test_dcp_local_scores_full_size():
    """One DCP rank's local block scores (pin off) at the size the bench
    times: 8192 rows of 8192 local columns, blocks of 8; every score of
    every row bit for bit, and -inf past every row's window."""
    w = workloads.dcp_local_logits()
    _say("dcp local scores", w.name)
    x = torch.from_numpy(w.logits).to(DEV)
    sc = dsa.block_scores(x, _i32(w.row_ks), _i32(w.row_ke), w.block_size, 1, pin_newest=False)
    got = sc.cpu().numpy()
    exp = oracle.block_scores(w.logits, w.row_ks, w.row_ke, w.block_size, 1, pin_newest=False,
                              nthreads=HOST_THREADS)
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))
    nb = got.shape[1]
    last = -(-(w.row_ke.astype(np.int64) - w.row_ks) // w.block_size)   # blocks with a column
    col = np.arange(nb)[None, :]
    assert np.all(np.isneginf(got[col >= last[:, None]]))


# --------------------------------------------- uint32 score codes (DCP reduce)

_SIGN = -2 ** 31


def _codes_max(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """Unsigned maximum of two code tensors held as int32 bit patterns:
    flipping the sign bit makes signed order the codes' unsigned order."""
    return torch.maximum(a ^ _SIGN, b ^ _SIGN) ^ _SIGN


def _np_codes(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("pin", [True, False])
def test_block_score_keys_random(pin):
    for i in range(60):
        w = workloads.random_case(700 + i, max_rows=9, max_width=3000, max_block=300,
                                  special=i % 2 == 0)
        x = torch.from_numpy(w.logits).to(DEV)
        ks = None if w.row_ks is None else _i32(w.row_ks)
        got = dsa.block_score_keys(x, ks, _i32(w.row_ke), w.block_size, w.row_repeat,
                                   pin_newest=pin)
        torch.cuda.synchronize()
        exp = oracle.block_score_keys(w.logits, w.row_ks, w.row_ke, w.block_size, w.row_repeat,
                                      pin_newest=pin)
        assert np.array_equal(_np_codes(got), exp), i


@pytest.mark.parametrize("B", [4, 8, 16, 32, 64, 128, 256])
def test_block_scores_every_vector_block_size(B):
    """Every block size of the vector path (16 to 1024 bytes per block, one
    to 64 lanes per block; from 128 on the lanes of a block span rows of 16
    and combine through row broadcasts), as fp32 scores and as codes, pin on
    and off, unaligned windows and starts, few rows (chunks) and many (whole
    rows): bit-exact against the oracle."""
    for seed, rows, width in ((B, 40, 9000 + B), (B + 1, 1030, 2 * B * 37 + 5)):
        w = workloads.many_rows_case(900 + seed, rows, width, B, 1 + seed % 2)
        x = torch.from_numpy(w.logits).to(DEV)
        ks = None if w.row_ks is None else _i32(w.row_ks)
        for pin in (True, False):
            got = dsa.block_scores(x, ks, _i32(w.row_ke), B, w.row_repeat, pin_newest=pin)
            exp = oracle.block_scores(w.logits, w.row_ks, w.row_ke, B, w.row_repeat,
                                      pin_newest=pin, nthreads=HOST_THREADS)
            assert np.array_equal(got.cpu().numpy().view(np.uint32), exp.view(np.uint32)), \
                (B, rows, width, pin)
            got = dsa.block_score_keys(x, ks, _i32(w.row_ke), B, w.row_repeat, pin_newest=pin)
            exp = oracle.block_score_keys(w.logits, w.row_ks, w.row_ke, B, w.row_repeat,
                                          pin_newest=pin, nthreads=HOST_THREADS)
            assert np.array_equal(_np_codes(got), exp), (B, rows, width, pin, "codes")


def test_block_score_keys_full_size():
    """One DCP rank's local scores at the benchmarked size as codes: every
    code of every row equals the oracle's."""
    w = workloads.dcp_local_logits()
    x = torch.from_numpy(w.logits).to(DEV)
    got = dsa.block_score_keys(x, _i32(w.row_ks), _i32(w.row_ke), w.block_size, 1,
                               pin_newest=False)
    exp = oracle.block_score_keys(w.logits, w.row_ks, w.row_ke, w.block_size, 1,
                                  pin_newest=False, nthreads=HOST_THREADS)
    assert np.array_equal(_np_codes(got), exp)


def test_select_from_keys_random_cases():
    """Codes of the random DCP score cases, and raw uint32 codes of every
    range (the codes of NaNs with other payloads and signs included)."""
    for seed in range(60):
        w = workloads.random_scores_case(seed)
        rows = w.scores.shape[0]
        codes = oracle.score_keys(w.scores)
        if seed % 3 == 2 and codes.size:   # any uint32 at all in a third of the cells
            g = np.random.default_rng(seed)
            pick = g.random(codes.shape) < 0.3
            codes[pick] = g.integers(0, 2 ** 32, size=int(pick.sum()), dtype=np.uint64)
        exp = np.empty((rows, w.topk_blocks), np.int32)
        oracle.select_from_keys(codes, w.global_row_ke, w.topk_blocks, w.global_block_size,
                                w.max_global_blocks, exp, w.row_repeat)
        kd = torch.from_numpy(codes.view(np.int32)).to(DEV)
        out = torch.full((rows, w.topk_blocks), 777, dtype=torch.int32, device=DEV)
        dsa.select_from_keys(kd, _i32(w.global_row_ke), w.topk_blocks, w.global_block_size,
                             w.max_global_blocks, out, w.row_repeat)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), exp), seed


@pytest.mark.parametrize("W", [2, 4, 8])
def test_dcp_decomposition_keys_on_gpu(W):
    """The page's DCP branch on one GPU with exact integer codes: each of W
    shards (token t on shard t mod W) scored by dsa_block_score_keys at
    block size B/W with the pin off, reduced by an unsigned maximum, equals
    the oracle's codes of the unsharded pin-off scores bit for bit (+0 and
    -0 side by side, NaN), and dsa_select_from_keys then gives the oracle's
    unsharded selection."""
    rng = np.random.default_rng(80 + W)
    rows, width, B, k = 24, 20000, 64, 32
    x = (np.rint(rng.standard_normal((rows, width)) * 4) / 4).astype(np.float32)
    x[rng.random((rows, width)) < 0.3] *= -0.0
    x[rng.random((rows, width)) < 1e-4] = np.nan
    x[5, :] = -0.0
    x[6, 128:192] = 0.0
    x[6, 150] = -0.0
    ends = rng.integers(0, width + 1, size=rows).astype(np.int32)
    ends[0] = 0
    ends[5] = ends[6] = width
    xd = torch.from_numpy(x).to(DEV)
    nblocks = -(-width // B)
    red = torch.full((rows, nblocks), oracle.score_key(float("-inf")), dtype=torch.int32,
                     device=DEV)                      # the code of -inf, 0x007FFFFF
    for wr in range(W):
        local = xd[:, wr::W].contiguous()
        lend = np.maximum(0, -(-(ends.astype(np.int64) - wr) // W)).astype(np.int32)
        kc = dsa.block_score_keys(local, None, _i32(lend), B // W, 1, pin_newest=False)
        n = min(kc.shape[1], nblocks)
        red[:, :n] = _codes_max(red[:, :n], kc.view(torch.int32)[:, :n])
    got_codes = _np_codes(red)
    exp_codes = oracle.block_score_keys(x, None, ends, B, 1, pin_newest=False)
    assert np.array_equal(got_codes, exp_codes)
    assert got_codes[5, 0] == oracle.score_key(-0.0) and got_codes[6, 2] == oracle.score_key(0.0)
    got = torch.empty((rows, k), dtype=torch.int32, device=DEV)
    dsa.select_from_keys(red, _i32(ends), k, B, nblocks, got)
    torch.cuda.synchronize()
    exp = np.empty((rows, k), np.int32)
    oracle.select_candidate_blocks(x, None, ends, k, B, exp)
    assert np.array_equal(got.cpu().numpy(), exp)


# ------------------------------------------------------------------- masking

def _dev_rows(x, ld_pad, offset):
    rows, width = x.shape
    ld = width + ld_pad
    flat = torch.full((offset + rows * ld,), 4242.0, dtype=torch.float32, device=DEV)
    view = flat[offset:offset + rows * ld].view(rows, ld)
    view[:, :width].copy_(torch.from_numpy(x))
    return flat, view[:, :width]


@pytest.mark.parametrize("seed", range(12))
def test_mask_random_cases(seed):
    rng = np.random.default_rng(500 + seed)
    for _ in range(6):
        rows = int(rng.integers(1, 12))
        R = int(rng.integers(1, 3))
        width = int(rng.integers(1, 20000))
        B = int(rng.choice([1, 3, 4, 7, 16, 64, 100, 128]))
        k = int(rng.integers(0, 40)) if rng.random() < 0.7 else int(rng.integers(60, 130))
        groups = -(-rows // R)
        x = rng.standard_normal((rows, width)).astype(np.float32)
        x[rng.random((rows, width)) < 1e-3] = np.nan
        starts = None if rng.random() < 0.3 else rng.integers(-5, width, size=groups).astype(np.int32)
        ends = rng.integers(-3, width + 50, size=groups).astype(np.int32)
        nb = -(-width // B) + 2
        cand = rng.integers(-1, nb, size=(rows, max(k, 1) + 1)).astype(np.int32)
        ld_pad, offset = int(rng.integers(0, 5)), int(rng.integers(0, 4))
        flat, xd = _dev_rows(x, ld_pad, offset)
        before = flat.clone()
        dsa.mask_candidates(xd, None if starts is None else _i32(starts), _i32(ends),
                            _i32(cand), k, B, R)
        torch.cuda.synchronize()
        exp = x.copy()
        oracle.mask_candidates(exp, starts, ends, cand, k, B, R)
        got = xd.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), exp.view(np.uint32)), (seed, rows, width, B, k)
        # nothing outside the rows' first `width` columns was written
        changed = (flat != before) & ~(torch.isnan(flat) & torch.isnan(before))
        mask = torch.zeros_like(changed)
        mask[offset:offset + rows * (width + ld_pad)].view(rows, width + ld_pad)[:, :width] = True
        assert not (changed & ~mask).any()


def test_mask_prefill_chunk_with_its_selection():
    w = workloads.config(3)
    sel = np.empty((w.rows, w.topk_blocks), np.int32)
    oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks, w.block_size,
                                   sel, w.row_repeat, nthreads=HOST_THREADS)
    xd = torch.from_numpy(w.logits).to(DEV)
    dsa.mask_candidates(xd, _i32(w.row_ks), _i32(w.row_ke), _i32(sel), w.topk_blocks,
                        w.block_size, w.row_repeat)
    torch.cuda.synchronize()
    exp = w.logits.copy()
    oracle.mask_candidates(exp, w.row_ks, w.row_ke, sel, w.topk_blocks, w.block_size, 1)
    got = xd.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))


# ------------------------------------------------------ LSE correction (page 3)

def _lse_tol(ref_new, ref_lse, lses, rank):
    """fp32 kernel vs float64 oracle.  final = log2(sum 2^(l-m)) + m carries
    about (N + 4) float ulps of relative error from the exp2 terms, the sum
    and log2, plus the roundings of l - m and + m (|m|, |final| times 2^-23
    each); the factor 2^d then has relative error ln2 * |error of d|, with d
    = local - final adding one more rounding of |d|; the product out *
    factor adds one ulp.  Bounds below take twice those terms."""
    N = lses.shape[0]
    eps = 2.0 ** -23
    local = lses[rank].astype(np.float64)
    fin = np.where(np.isfinite(ref_lse), np.abs(ref_lse), 0.0)
    big = np.maximum(fin, np.where(np.isfinite(local), np.abs(local), 0.0))
    tol_lse = 2 * ((N + 4) * eps * 1.5 + 2 * eps * fin)
    tol_d = tol_lse + 2 * eps * (big + fin)
    rel = np.log(2.0) * tol_d + 2 * eps
    return tol_lse, rel


def _check_lse(out_np, lses_np, rank, new, lse):
    ref_new, ref_lse = oracle.correct_attn_out(out_np, lses_np, rank)
    tol_lse, rel = _lse_tol(ref_new, ref_lse, lses_np, rank)
    lse_np = lse.cpu().numpy().astype(np.float64)
    same_inf = np.isinf(ref_lse) & (lse_np == ref_lse)
    with np.errstate(invalid="ignore"):   # -inf - -inf where both are -inf
        close = np.abs(lse_np - ref_lse) <= tol_lse
    assert (same_inf | close).all()
    new_np = new.cpu().numpy().astype(np.float64)
    bound = rel.T[:, :, None] * np.abs(ref_new) + 1e-37
    assert (np.abs(new_np - ref_new) <= bound).all()


@pytest.mark.parametrize("N", [1, 2, 8, 64, 70])
def test_lse_random(N):
    w = workloads.lse_merge(B=7, H=5, D=36, N=N, seed=310 + N)
    for rank in sorted({0, N // 2, N - 1}):
        out = torch.from_numpy(w.out).to(DEV)
        lses = torch.from_numpy(w.lses).to(DEV)
        new, lse = dsa.correct_attn_out(out, lses, rank)
        torch.cuda.synchronize()
        _check_lse(w.out, w.lses, rank, new, lse)


@pytest.mark.parametrize("D", [4, 260, 1028, 1500])
def test_lse_vector_lengths(D):
    """D-vectors shorter than one 256-column pass of the wave's float4
    loads, with a partial last pass, and several passes long, for N <= 64
    (one pass of LSE lanes) and N > 64 (two)."""
    for N in (3, 65):
        w = workloads.lse_merge(B=3, H=2, D=D, N=N, seed=400 + D + N)
        rank = N - 1
        new, lse = dsa.correct_attn_out(torch.from_numpy(w.out).to(DEV),
                                        torch.from_numpy(w.lses).to(DEV), rank)
        torch.cuda.synchronize()
        _check_lse(w.out, w.lses, rank, new, lse)


def test_lse_strided_and_special_values():
    rng = np.random.default_rng(77)
    B, H, D, N = 6, 4, 64, 5
    out = rng.standard_normal((B, H, D)).astype(np.float32)
    lses = (rng.standard_normal((N, B, H)) * 6).astype(np.float32)
    lses[0, 0, 0] = np.nan
    lses[1, 0, 1] = np.inf
    lses[:, 1, 2] = -np.inf
    lses[2, 2, 3] = np.nan
    big = torch.zeros((N, B, H, 2), dtype=torch.float32, device=DEV)
    big[..., 1] = torch.from_numpy(lses).to(DEV)
    outv = torch.zeros((B, 2, H, D), dtype=torch.float32, device=DEV)
    outv[:, 0] = torch.from_numpy(out).to(DEV)
    newv = torch.zeros((H, 2 * B, D + 3), dtype=torch.float32, device=DEV)
    for rank in range(N):
        new, lse = dsa.correct_attn_out(outv[:, 0], big[..., 1], rank,
                                        new_output=newv[:, ::2, 1:D + 1])
        torch.cuda.synchronize()
        _check_lse(out, lses, rank, new, lse)
        assert torch.isfinite(new).all()


def test_lse_full_size():
    w = workloads.lse_merge()
    _say("lse", w.name)
    out = torch.from_numpy(w.out).to(DEV)
    lses = torch.from_numpy(w.lses).to(DEV)
    new, lse = dsa.correct_attn_out(out, lses, w.cp_rank)
    torch.cuda.synchronize()
    bs = np.arange(0, w.out.shape[0], 17)
    sub_out = np.ascontiguousarray(w.out[bs])
    sub_l = np.ascontiguousarray(w.lses[:, bs])
    _check_lse(sub_out, sub_l, w.cp_rank, new[:, bs], lse[bs])
