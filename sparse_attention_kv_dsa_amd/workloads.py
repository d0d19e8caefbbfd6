"""Seeded synthetic inputs for DSA candidate-block selection.

This module only draws inputs; it holds none of the selection arithmetic.
Both the GPU path's tests/benchmark and the CPU oracle's tests take their
inputs from here, so the two sides always see the same bytes.

The five workloads mirror the shapes of a DeepSeek-style sparse-attention
indexer as the vLLM-fork page ``candidate_blocks.py`` describes it (packed
column space, per-row ``[start, end)`` windows, decode rows sharing bounds in
groups of ``row_repeat``): a tiny checkable case, a decode batch, a packed
prefill chunk, a long-context decode batch and a large packed prefill.
Every draw uses ``numpy.random.Generator(PCG64(seed))`` with seed =
workload index - 1, in the order written below.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np


@dataclass
class Workload:
    name: str
    logits: np.ndarray            # float32 [rows, width], row-major
    row_ks: np.ndarray | None     # int32 [groups] request starts, or None (all 0)
    row_ke: np.ndarray            # int32 [groups] request ends
    block_size: int
    topk_blocks: int
    row_repeat: int

    @property
    def rows(self) -> int:
        return int(self.logits.shape[0])

    @property
    def width(self) -> int:
        return int(self.logits.shape[1])

    def describe(self) -> dict:
        return {
            "workload": self.name, "rows": self.rows, "width": self.width,
            "block_size": self.block_size, "topk_blocks": self.topk_blocks,
            "row_repeat": self.row_repeat, "has_starts": self.row_ks is not None,
        }


NAMES = {
    1: "tiny-8x1000-b64-k4",
    2: "decode-64x32768-b64-k32-r2",
    3: "prefill-4096x16384-b64-k32",
    4: "longctx-decode-128x131072-b128-k16-r2",
    5: "large-prefill-8192x65536-b64-k64",
}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def tiny() -> Workload:
    """8 x 1000, N(0,1), 3 NaNs at distinct flat positions, ends in [0,1000], ends[0]=0."""
    rng = _rng(0)
    logits = rng.standard_normal((8, 1000), dtype=np.float32)
    flat = rng.choice(8 * 1000, size=3, replace=False)
    logits.reshape(-1)[flat] = np.float32(np.nan)
    ends = rng.integers(0, 1000, size=8, endpoint=True).astype(np.int32)
    ends[0] = 0
    return Workload(NAMES[1], logits, None, ends, 64, 4, 1)


def decode() -> Workload:
    """32 requests x row_repeat 2, width 32768, N(0, sd=2), ends in [1, 32768]."""
    rng = _rng(1)
    logits = rng.standard_normal((64, 32768), dtype=np.float32)
    logits *= np.float32(2.0)
    ends = rng.integers(1, 32768, size=32, endpoint=True).astype(np.int32)
    return Workload(NAMES[2], logits, None, ends, 64, 32, 2)


def prefill() -> Workload:
    """4 packed requests x 1024 queries, width 16384, causal ends start+3072+i+1."""
    rng = _rng(2)
    logits = rng.standard_normal((4096, 16384), dtype=np.float32)
    q = np.arange(4096) // 1024
    i = np.arange(4096) % 1024
    ks = (4096 * q).astype(np.int32)
    ke = (4096 * q + 3072 + i + 1).astype(np.int32)
    return Workload(NAMES[3], logits, ks, ke, 64, 32, 1)


def longctx_decode() -> Workload:
    """64 requests x row_repeat 2, width 131072, N(0,1) with 1% -inf then 1e-6 NaN."""
    rng = _rng(3)
    shape = (128, 131072)
    logits = rng.standard_normal(shape, dtype=np.float32)
    logits[rng.random(shape, dtype=np.float32) < np.float32(0.01)] = -np.inf
    logits[rng.random(shape, dtype=np.float32) < np.float32(1e-6)] = np.nan
    ends = rng.integers(65536, 131072, size=64, endpoint=True).astype(np.int32)
    return Workload(NAMES[4], logits, None, ends, 128, 16, 2)


def large_prefill(rows: int = 8192) -> Workload:
    """2 packed requests x 4096 queries, width 65536, uniform(-8,8) rounded to 1/16.

    Drawn in chunks of 512 rows: u ~ U[0,1) (float32), x = 16u - 8, then
    rint(16x)/16 (round half to even; small negatives become -0.0).
    ``rows`` < 8192 draws only the first ``rows`` rows (same bytes).
    """
    rng = _rng(4)
    width = 65536
    logits = np.empty((rows, width), dtype=np.float32)
    for r0 in range(0, rows, 512):
        r1 = min(r0 + 512, rows)
        x = rng.random((r1 - r0, width), dtype=np.float32)
        x *= np.float32(16.0)
        x -= np.float32(8.0)
        x *= np.float32(16.0)
        np.rint(x, out=x)
        x /= np.float32(16.0)
        logits[r0:r1] = x
    r = np.arange(8192)
    ks = np.where(r < 4096, 0, 32768).astype(np.int32)
    ke = (ks + 28672 + (r % 4096) + 1).astype(np.int32)
    return Workload(NAMES[5], logits, ks[:rows].copy(), ke[:rows].copy(), 64, 64, 1)


def dcp_local_logits(rows: int = 8192, world: int = 8) -> Workload:
    """Rank 0's share of the large prefill under decode-context parallelism
    over ``world`` ranks: tokens are dealt t mod world, so the rank holds
    width 65536 / world local columns and scores blocks of 64 / world of
    them (pin off; the reduce across ranks and the pin come after).  Values
    are a fresh draw of the large prefill's distribution at the local shape
    (uniform(-8, 8) rounded to 1/16, in 512-row chunks, seed 400); the bounds
    are the large prefill's, mapped to rank 0's columns: start ceil(s / world),
    end ceil(e / world)."""
    rng = _rng(400)
    width, B = 65536 // world, 64 // world
    logits = np.empty((rows, width), dtype=np.float32)
    for r0 in range(0, rows, 512):
        r1 = min(r0 + 512, rows)
        x = rng.random((r1 - r0, width), dtype=np.float32)
        x *= np.float32(16.0)
        x -= np.float32(8.0)
        x *= np.float32(16.0)
        np.rint(x, out=x)
        x /= np.float32(16.0)
        logits[r0:r1] = x
    r = np.arange(rows)
    gs = np.where(r < rows // 2, 0, 32768).astype(np.int64)
    ge = gs + 28672 + (r % max(rows // 2, 1)) + 1
    ks = (-(-gs // world)).astype(np.int32)
    ke = (-(-ge // world)).astype(np.int32)
    return Workload(f"dcp-local-logits-{rows}x{width}-b{B}", logits, ks, ke, B, 0, 1)


def config(i: int) -> Workload:
    return {1: tiny, 2: decode, 3: prefill, 4: longctx_decode, 5: large_prefill}[i]()


# Values drawn for tiny random cases: they force ties, +-0, +-inf and NaN.
SPECIAL_VALUES = np.array([-1.0, -0.0, 0.0, 1.0, 2.0, np.inf, -np.inf, np.nan],
                          dtype=np.float32)


def random_case(seed: int, max_rows: int = 6, max_width: int = 40, max_block: int = 9,
                max_k: int = 12, special: bool = True, ld_pad: int = 0) -> Workload:
    """A small random case: odd widths, unaligned/empty/overlong windows, row_repeat 1-3.

    Bounds include starts >= ends, ends = 0, negative starts, ends past width
    and starts past width, so every reading of the definition is exercised.
    """
    rng = _rng(1_000_000 + seed)
    rows = int(rng.integers(1, max_rows, endpoint=True))
    width = int(rng.integers(1, max_width, endpoint=True))
    B = int(rng.integers(1, max_block, endpoint=True))
    R = int(rng.integers(1, 3, endpoint=True))
    k = int(rng.integers(0, max_k, endpoint=True))
    if special:
        vals = SPECIAL_VALUES[rng.integers(0, len(SPECIAL_VALUES), size=(rows, width))]
    else:
        vals = rng.standard_normal((rows, width), dtype=np.float32)
    logits = np.zeros((rows, width + ld_pad), dtype=np.float32)
    logits[:, :width] = vals
    logits = logits[:, :width]
    groups = -(-rows // R)
    has_starts = bool(rng.integers(0, 2))
    ks = rng.integers(-3, width + 2, size=groups, endpoint=True).astype(np.int32)
    ke = rng.integers(0, width + 4, size=groups, endpoint=True).astype(np.int32)
    return Workload(f"random-{seed}", logits, ks if has_starts else None, ke, B, k, R)


def many_rows_case(seed: int, rows: int, width: int, block_size: int, row_repeat: int = 1,
                   topk: int = 8) -> Workload:
    """Many rows of one width: N(0,1) values with -inf at 1 % and NaN at 0.01 %
    of the positions; starts uniform in [-B, width / 2], ends uniform in
    [start - 8, width + B], so windows are empty, ragged, clipped or whole."""
    rng = _rng(2_000_000 + seed)
    logits = rng.standard_normal((rows, width), dtype=np.float32)
    u = rng.random((rows, width), dtype=np.float32)
    logits[u < 0.01] = -np.inf
    logits[u < 1e-4] = np.nan
    groups = -(-rows // row_repeat)
    ks = rng.integers(-block_size, width // 2, size=groups, endpoint=True)
    ke = ks + rng.integers(-8, width + block_size, size=groups, endpoint=True)
    ke = np.clip(ke, 0, width + block_size)
    return Workload(f"many-rows-{seed}-{rows}x{width}-b{block_size}-r{row_repeat}", logits,
                    ks.astype(np.int32), ke.astype(np.int32), block_size, topk, row_repeat)


def sha256(*arrays) -> str:
    h = hashlib.sha256()
    for a in arrays:
        if a is not None:
            h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


# ---------------------------------------------------------------------------
# Inputs of the steps after selection (seeds 100+).  Shapes follow the pages:
# the decode-context-parallel branch of candidate_blocks.py reduces a
# [rows, max_global_blocks] score matrix; the LSE correction of page 3 works
# on out [B, H, D] and lses [N, B, H].  The model dimensions used for the LSE
# workload (H = 128 heads, D = 512 latent columns, N = 8 ranks) are those of a
# DeepSeek-style MLA decode with the latent output per head; the pages state
# no shape for it, so this is the choice made here.


@dataclass
class ScoresWorkload:
    name: str
    scores: np.ndarray            # float32 [rows, nscore]: reduced block scores
    global_row_ke: np.ndarray     # int32 [groups]
    global_block_size: int
    max_global_blocks: int
    topk_blocks: int
    row_repeat: int


def dcp_prefill_scores(rows: int = 8192) -> ScoresWorkload:
    """DCP share of the large prefill: block scores of 8192 rows over 1024
    global blocks of 64 tokens, values drawn as the block maxima of the large
    prefill would fall (uniform(-8, 8) rounded to 1/16: heavy ties), a few
    NaN and -inf blocks; the global end of query i of either packed request
    is its context length 28672 + i + 1 (request-local, as the DCP pin
    reads it), so the pin lands inside the 1024 blocks."""
    g = _rng(100)
    x = np.rint(g.uniform(-8.0, 8.0, size=(rows, 1024)).astype(np.float32) * 16.0) / 16.0
    x = x.astype(np.float32)
    x[g.random((rows, 1024)) < 1e-4] = np.nan
    x[g.random((rows, 1024)) < 1e-2] = -np.inf
    half = rows // 2
    i = np.arange(rows, dtype=np.int64) % max(half, 1)
    ends = (28672 + i + 1).astype(np.int32)
    return ScoresWorkload(f"dcp-prefill-scores-{rows}x1024-g64-k64", x, ends, 64, 1024, 64, 1)


def random_scores_case(seed: int, max_rows: int = 40, max_nscore: int = 3000) -> ScoresWorkload:
    g = _rng(200 + seed)
    rows = int(g.integers(1, max_rows + 1))
    R = int(g.integers(1, 4))
    nscore = int(g.integers(0, max_nscore + 1))
    mgb = int(g.integers(0, 2 * max(nscore, 1) + 2))
    G = int(g.integers(1, 200))
    k = int(g.integers(0, 300))
    vals = np.array([-2.0, -0.5, 0.25, 1.0, 3.0, np.inf, -np.inf, np.nan], np.float32)
    x = g.standard_normal((rows, nscore)).astype(np.float32)
    pick = g.random((rows, nscore)) < 0.3
    x[pick] = vals[g.integers(0, len(vals), size=int(pick.sum()))]
    ends = g.integers(-5, mgb * G + 3 * G + 2, size=-(-rows // R)).astype(np.int32)
    return ScoresWorkload(f"scores-case-{seed}", x, ends, G, mgb, k, R)


@dataclass
class LseWorkload:
    name: str
    out: np.ndarray     # float32 [B, H, D]
    lses: np.ndarray    # float32 [N, B, H] (base-2)
    cp_rank: int


def lse_merge(B: int = 256, H: int = 128, D: int = 512, N: int = 8, seed: int = 300) -> LseWorkload:
    """Partial MLA attention outputs ~ N(0, 1) and base-2 LSEs ~ 12 + 4 N(0, 1),
    with 1% of (rank, b, h) entries -inf (a rank that held no context)."""
    g = _rng(seed)
    out = g.standard_normal((B, H, D)).astype(np.float32)
    lses = (12.0 + 4.0 * g.standard_normal((N, B, H))).astype(np.float32)
    lses[g.random((N, B, H)) < 0.01] = -np.inf
    return LseWorkload(f"lse-merge-{B}x{H}x{D}-n{N}", out, lses, 3 % N)
