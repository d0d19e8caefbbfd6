"""CPU oracle for DSA candidate-block selection (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its
binding) never touches it, and the two share no code.

The arithmetic lives in ``oracle.c`` (plain loops, one qsort per row); this
module compiles it with gcc and marshals numpy arrays through ctypes.  The
definition it implements is stated at the top of ``oracle.c`` and follows
the vLLM-fork page ``candidate_blocks.py`` (functions ``_max_with_nan``,
``_block_scores_kernel``, ``_block_scores``, ``_select_candidate_blocks_impl``
with its DCP branch, and the masking function after it) and page 3
(``_correct_attn_cp_out_kernel`` / ``correct_attn_out``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (plain -O2, no intrinsics)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-Wall", "-Wextra", "-fPIC",
             "-shared", "-pthread", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def _open(path):
    lib = ctypes.CDLL(path)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
    lib.oracle_block_scores.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, i32, vp,
                                        i64, ctypes.c_int]
    lib.oracle_block_scores.restype = ctypes.c_int
    lib.oracle_select_candidate_blocks.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32,
                                                   i32, vp, i64, vp, i64, ctypes.c_int]
    lib.oracle_select_candidate_blocks.restype = ctypes.c_int
    lib.oracle_select_from_scores.argtypes = [vp, i64, i64, i64, i64, vp, i32, i32, i32, vp, i64]
    lib.oracle_select_from_scores.restype = ctypes.c_int
    lib.oracle_score_key.argtypes = [ctypes.c_float]
    lib.oracle_score_key.restype = ctypes.c_uint32
    lib.oracle_key_score.argtypes = [ctypes.c_uint32]
    lib.oracle_key_score.restype = ctypes.c_float
    lib.oracle_score_keys.argtypes = [vp, i64, i64, i64, vp, i64]
    lib.oracle_score_keys.restype = ctypes.c_int
    lib.oracle_select_from_keys.argtypes = [vp, i64, i64, i64, i64, vp, i32, i32, i32, vp, i64]
    lib.oracle_select_from_keys.restype = ctypes.c_int
    lib.oracle_mask_candidates.argtypes = [vp, i64, i64, i64, vp, vp, vp, i64, i32, i32, i32]
    lib.oracle_mask_candidates.restype = ctypes.c_int
    lib.oracle_correct_attn_out.argtypes = ([vp] + [i64] * 6 + [vp] + [i64] * 5 + [vp] + [i64] * 3
                                            + [vp, i64, i64])
    lib.oracle_correct_attn_out.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _override is not None:
        return _override
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = _open(_LIB)
    return _lib


_override = None


class use_library:
    """Context manager: route this module's calls to another build of the
    oracle (the mutation tests load deliberately broken copies this way)."""

    def __init__(self, path):
        self.lib = _open(path)

    def __enter__(self):
        global _override
        self._prev, _override = _override, self.lib
        return self

    def __exit__(self, *exc):
        global _override
        _override = self._prev
        return False


def _ptr(a):
    return None if a is None else a.ctypes.data


def _ld(a):
    """Row stride in elements (an empty or one-row array may report any stride)."""
    if a.shape[0] <= 1 or a.shape[1] == 0:
        return max(int(a.shape[1]), 1)
    # a one-column array may report any column stride
    assert (a.shape[1] == 1 or a.strides[1] == a.itemsize) and a.strides[0] % a.itemsize == 0
    return a.strides[0] // a.itemsize


def _check_inputs(logits, row_ks, row_ke, row_repeat):
    assert logits.dtype == np.float32 and logits.ndim == 2
    _ld(logits)
    rows = logits.shape[0]
    groups = -(-rows // row_repeat) if rows else 0
    row_ke = np.ascontiguousarray(row_ke, dtype=np.int32).reshape(-1)
    assert row_ke.size >= groups
    if row_ks is not None:
        row_ks = np.ascontiguousarray(row_ks, dtype=np.int32).reshape(-1)
        assert row_ks.size >= groups
    return row_ks, row_ke


def block_scores(logits: np.ndarray, row_ks, row_ke, block_size: int, row_repeat: int = 1,
                 pin_newest: bool = True, nthreads: int = 1) -> np.ndarray:
    """fp32 block scores [rows, ceil(width/block_size)] (pinned if asked)."""
    row_ks, row_ke = _check_inputs(logits, row_ks, row_ke, row_repeat)
    rows, width = logits.shape
    nblocks = -(-width // block_size)
    scores = np.empty((rows, nblocks), dtype=np.float32)
    if rows and width:
        rc = _load().oracle_block_scores(
            _ptr(logits), rows, width, _ld(logits), _ptr(row_ks), _ptr(row_ke),
            block_size, row_repeat, int(bool(pin_newest)), _ptr(scores), nblocks, nthreads)
        assert rc == 0
    return scores


def select_candidate_blocks(logits: np.ndarray, row_ks, row_ke, topk_blocks: int,
                            block_size: int, out: np.ndarray, row_repeat: int = 1,
                            scores_out: np.ndarray | None = None, nthreads: int = 1) -> None:
    """Fill int32 ``out[rows, >=topk_blocks]`` in place; -1 padded."""
    row_ks, row_ke = _check_inputs(logits, row_ks, row_ke, row_repeat)
    rows, width = logits.shape
    assert out.dtype == np.int32 and out.ndim == 2
    assert out.shape[0] == rows and out.shape[1] >= topk_blocks
    ld_scores = 0
    if scores_out is not None:
        assert scores_out.dtype == np.float32 and scores_out.shape[0] == rows
        ld_scores = _ld(scores_out)
    rc = _load().oracle_select_candidate_blocks(
        _ptr(logits), rows, width, _ld(logits), _ptr(row_ks), _ptr(row_ke),
        topk_blocks, block_size, row_repeat, _ptr(out), _ld(out),
        _ptr(scores_out), ld_scores, nthreads)
    assert rc == 0


def select_from_scores(scores: np.ndarray, global_row_ke, topk_blocks: int,
                       global_block_size: int, max_global_blocks: int, out: np.ndarray,
                       row_repeat: int = 1) -> None:
    """DCP branch after the reduce: pin from the global ends (clamped), rows with
    end <= 0 select nothing, then the ordered -1 padded top-k.  ``scores`` is
    fp32 [rows, nscore]; columns past ``max_global_blocks`` are dropped and
    missing ones are -inf."""
    assert scores.dtype == np.float32 and scores.ndim == 2
    rows, nscore = scores.shape
    ends = np.ascontiguousarray(global_row_ke, dtype=np.int32).reshape(-1)
    assert ends.size >= (-(-rows // row_repeat) if rows else 0)
    assert out.dtype == np.int32 and out.shape[0] == rows and out.shape[1] >= topk_blocks
    ld = _ld(scores) if nscore else 1
    rc = _load().oracle_select_from_scores(_ptr(scores), rows, nscore, ld, max_global_blocks,
                                           _ptr(ends), row_repeat, global_block_size,
                                           topk_blocks, _ptr(out), _ld(out))
    assert rc == 0


def score_key(x: float) -> int:
    """Order-preserving uint32 code of one fp32 score (see oracle.c)."""
    return int(_load().oracle_score_key(float(x)))


def key_score(k: int) -> float:
    """The score a code stands for (the canonical NaN for the NaN code)."""
    return float(_load().oracle_key_score(int(k)))


def score_keys(scores: np.ndarray) -> np.ndarray:
    """uint32 codes of an fp32 [rows, n] matrix, element by element."""
    assert scores.dtype == np.float32 and scores.ndim == 2
    rows, n = scores.shape
    keys = np.empty((rows, n), dtype=np.uint32)
    if rows and n:
        rc = _load().oracle_score_keys(_ptr(scores), rows, n, _ld(scores), _ptr(keys), n)
        assert rc == 0
    return keys


def block_score_keys(logits: np.ndarray, row_ks, row_ke, block_size: int, row_repeat: int = 1,
                     pin_newest: bool = True, nthreads: int = 1) -> np.ndarray:
    """uint32 codes of the block scores [rows, ceil(width/block_size)]."""
    return score_keys(block_scores(logits, row_ks, row_ke, block_size, row_repeat, pin_newest,
                                   nthreads))


def select_from_keys(keys: np.ndarray, global_row_ke, topk_blocks: int, global_block_size: int,
                     max_global_blocks: int, out: np.ndarray, row_repeat: int = 1) -> None:
    """select_from_scores on a uint32 [rows, nkeys] matrix of score codes."""
    assert keys.dtype == np.uint32 and keys.ndim == 2
    rows, nkeys = keys.shape
    ends = np.ascontiguousarray(global_row_ke, dtype=np.int32).reshape(-1)
    assert ends.size >= (-(-rows // row_repeat) if rows else 0)
    assert out.dtype == np.int32 and out.shape[0] == rows and out.shape[1] >= topk_blocks
    ld = _ld(keys) if nkeys else 1
    rc = _load().oracle_select_from_keys(_ptr(keys), rows, nkeys, ld, max_global_blocks,
                                         _ptr(ends), row_repeat, global_block_size, topk_blocks,
                                         _ptr(out), _ld(out))
    assert rc == 0


def mask_candidates(logits: np.ndarray, row_ks, row_ke, candidates: np.ndarray,
                    topk_blocks: int, block_size: int, row_repeat: int = 1) -> None:
    """In place: every column outside [s, e) or whose request-local block is
    not among ``candidates[r, :topk_blocks]`` becomes -inf."""
    row_ks, row_ke = _check_inputs(logits, row_ks, row_ke, row_repeat)
    rows, width = logits.shape
    assert candidates.dtype == np.int32 and candidates.shape[0] == rows
    assert candidates.shape[1] >= topk_blocks
    if rows and width:
        rc = _load().oracle_mask_candidates(_ptr(logits), rows, width, _ld(logits),
                                            _ptr(row_ks), _ptr(row_ke), _ptr(candidates),
                                            _ld(candidates), topk_blocks, block_size,
                                            row_repeat)
        assert rc == 0


def correct_attn_out(out: np.ndarray, lses: np.ndarray, cp_rank: int):
    """Base-2 LSE correction: returns (new_out [H, B, D], lse [B, H]) in float64
    for fp32 ``out [B, H, D]`` and ``lses [N, B, H]`` (any strides)."""
    assert out.dtype == np.float32 and out.ndim == 3
    assert lses.dtype == np.float32 and lses.ndim == 3
    B, H, D = out.shape
    N = lses.shape[0]
    assert lses.shape[1:] == (B, H) and 0 <= cp_rank < N
    new = np.empty((H, B, D), dtype=np.float64)
    lse = np.empty((B, H), dtype=np.float64)
    isz = out.itemsize
    o = [st // isz for st in out.strides]
    l = [st // lses.itemsize for st in lses.strides]
    n = [st // 8 for st in new.strides]
    v = [st // 8 for st in lse.strides]
    rc = _load().oracle_correct_attn_out(_ptr(out), B, H, D, o[0], o[1], o[2], _ptr(lses), N,
                                         l[0], l[1], l[2], cp_rank, _ptr(new), n[0], n[1],
                                         n[2], _ptr(lse), v[0], v[1])
    assert rc == 0
    return new, lse
