"""Independent brute-force statement of candidate-block selection (pure Python).

Used only on tiny inputs to pin the C oracle.  It is written from the
equivalent statement of the method, not from the oracle's code: list every
block whose score is not -inf in ranking order (NaN first, then value
descending with -0 == +0, then block id ascending), keep the first k, pad
with -1.  Block scores come from Python's ``max`` with an explicit key that
makes +0 beat -0; NaN anywhere in a block makes the block NaN.

Follows the vLLM-fork candidate_blocks.py diff page: ``_max_with_nan``
(NaN-propagating max), ``_block_scores_kernel`` (masked load with -inf,
newest-block pin) and ``_select_candidate_blocks_impl`` (early-outs, top-k,
-1 padded output, bounds shared by ``row_repeat`` rows).
"""
from __future__ import annotations

import math

NAN = float("nan")
INF = float("inf")


def _score(values):
    if not values:
        return -INF
    if any(math.isnan(v) for v in values):
        return NAN
    return max(values, key=lambda v: (v, math.copysign(1.0, v)))


def row_scores(row, width, s, e, B, pin=True):
    nblocks = -(-width // B)
    cols = [c for c in range(max(s, 0), min(e, width))]   # in-window columns
    groups = {}
    for c in cols:
        groups.setdefault((c - s) // B, []).append(float(row[c]))
    scores = [_score(groups.get(b, [])) for b in range(nblocks)]
    if pin and e > s and (e - s - 1) // B < nblocks:
        scores[(e - s - 1) // B] = INF
    return scores


def select_row(scores, k):
    valid = [b for b, v in enumerate(scores) if not (v == -INF)]
    ranked = sorted(valid, key=lambda b: (0 if math.isnan(scores[b]) else 1,
                                          0.0 if math.isnan(scores[b]) else -scores[b] + 0.0,
                                          b))
    ranked = ranked[:min(k, len(scores))]
    return ranked + [-1] * (k - len(ranked))


def select(logits, row_ks, row_ke, k, B, R):
    rows, width = len(logits), (len(logits[0]) if len(logits) else 0)
    if rows == 0:
        return []
    if width == 0:
        return [[-1] * k for _ in range(rows)]
    out = []
    for r in range(rows):
        g = r // R
        s = int(row_ks[g]) if row_ks is not None else 0
        e = int(row_ke[g])
        out.append(select_row(row_scores(logits[r], width, s, e, B), k))
    return out


def scores(logits, row_ks, row_ke, B, R, pin=True):
    rows = len(logits)
    width = len(logits[0]) if rows else 0
    res = []
    for r in range(rows):
        g = r // R
        s = int(row_ks[g]) if row_ks is not None else 0
        e = int(row_ke[g])
        res.append(row_scores(logits[r], width, s, e, B, pin))
    return res
