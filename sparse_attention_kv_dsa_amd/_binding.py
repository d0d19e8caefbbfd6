"""ctypes binding of libdsa.so (include/dsa.h).

Argument marshalling only: every step of the selection runs in the HIP
library.  PyTorch supplies device memory and the current HIP stream.  If
the library has not been built, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from . import build as _build

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)

_lib = None
_lock = threading.Lock()


class DsaError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        name = status_string(code)
        super().__init__(f"{what}: {name} ({code})")


def lib() -> ctypes.CDLL:
    """The loaded libdsa.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                path = _build.lib_path("libdsa.so")
                if not os.path.exists(path):
                    raise RuntimeError(
                        f"{path} is missing: build it with `python -m sparse_attention_kv_dsa_amd.build`"
                        " (there is no fallback implementation)")
                L = ctypes.CDLL(path)
                i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
                L.dsa_block_scores.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, i32, vp, i64, vp]
                L.dsa_block_scores.restype = ctypes.c_int
                L.dsa_select_workspace_bytes.argtypes = [i64, i64, i32, i32]
                L.dsa_select_workspace_bytes.restype = sz
                L.dsa_select_candidate_blocks.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, i32,
                                                          vp, i64, vp, i64, vp, sz, vp]
                L.dsa_select_candidate_blocks.restype = ctypes.c_int
                L.dsa_select_candidate_blocks_plan.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32,
                                                               i32, vp, i64, vp, i64, vp, sz, i32,
                                                               i32, vp]
                L.dsa_select_candidate_blocks_plan.restype = ctypes.c_int
                L.dsa_select_candidate_blocks_noalloc.argtypes = [vp, i64, i64, i64, vp, vp, i32,
                                                                  i32, i32, vp, i64, vp, i64, vp]
                L.dsa_select_candidate_blocks_noalloc.restype = ctypes.c_int
                L.dsa_select_plan.argtypes = [i64, i64, i32, i32, ctypes.POINTER(i32),
                                              ctypes.POINTER(i32)]
                L.dsa_select_plan.restype = ctypes.c_int
                L.dsa_status_string.argtypes = [ctypes.c_int]
                L.dsa_status_string.restype = ctypes.c_char_p
                L.dsa_select_from_scores.argtypes = [vp, i64, i64, i64, i64, vp, i32, i32, i32,
                                                     vp, i64, vp]
                L.dsa_select_from_scores.restype = ctypes.c_int
                L.dsa_block_score_keys.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, i32, vp,
                                                   i64, vp]
                L.dsa_block_score_keys.restype = ctypes.c_int
                L.dsa_select_from_keys.argtypes = [vp, i64, i64, i64, i64, vp, i32, i32, i32,
                                                   vp, i64, vp]
                L.dsa_select_from_keys.restype = ctypes.c_int
                L.dsa_mask_candidates.argtypes = [vp, i64, i64, i64, vp, vp, vp, i64, i32, i32,
                                                  i32, vp]
                L.dsa_mask_candidates.restype = ctypes.c_int
                L.dsa_correct_attn_out.argtypes = ([vp] + [i64] * 6 + [vp] + [i64] * 5 + [vp]
                                                   + [i64] * 3 + [vp, i64, i64, vp])
                L.dsa_correct_attn_out.restype = ctypes.c_int
                _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().dsa_status_string(code).decode()


def _raise(code: int, what: str):
    if code != DSA_OK:
        raise DsaError(code, what)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ld(t: torch.Tensor) -> int:
    if t.dim() != 2:
        raise ValueError("expected a 2-D tensor")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("rows must be contiguous (stride(1) == 1)")
    return t.stride(0) if t.shape[0] > 1 else max(int(t.shape[1]), 1)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _bounds(t, name, groups, device):
    if t is None:
        return None
    if t.dtype != torch.int32 or t.device != device:
        raise ValueError(f"{name} must be int32 on {device}")
    t = t.reshape(-1)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < groups:
        raise ValueError(f"{name} needs at least {groups} entries")
    return t


def _check_logits(logits):
    if logits.dtype != torch.float32 or logits.device.type != "cuda":
        raise ValueError("logits must be float32 on a HIP device")
    return _ld(logits)


def select_workspace_bytes(rows: int, width: int, block_size: int, topk_blocks: int) -> int:
    return int(lib().dsa_select_workspace_bytes(rows, width, block_size, topk_blocks))


def select_plan(rows: int, width: int, block_size: int, topk_blocks: int) -> tuple[int, int]:
    plan, cb = ctypes.c_int32(), ctypes.c_int32()
    _raise(lib().dsa_select_plan(rows, width, block_size, topk_blocks, ctypes.byref(plan),
                                 ctypes.byref(cb)), "dsa_select_plan")
    return plan.value, cb.value


def _capturing(device) -> bool:
    return torch.cuda.is_current_stream_capturing()


class Workspace:
    """Device scratch for the split and pair plans of
    dsa_select_candidate_blocks: allocated zeroed (the pair plan's arrival
    counters must start at zero; every call leaves them zero), one per stream
    that may run concurrently.  Calls whose plan is another one get no
    default workspace.

    Graph capture: a captured call keeps the address of the buffer it was
    captured with, so a workspace never frees a buffer it replaces (a graph
    captured earlier may still replay into it), and it refuses to allocate
    or grow while the current stream is capturing: size it before capture
    (select_workspace_bytes gives the size)."""

    def __init__(self, device, nbytes: int = 0):
        self.device = torch.device(device)
        if _capturing(self.device):
            raise RuntimeError("dsa.Workspace: cannot allocate while a HIP graph is being "
                               "captured; create it (sized with select_workspace_bytes) before "
                               "capture")
        self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        self._replaced: list = []

    def ensure(self, nbytes: int) -> "Workspace":
        if nbytes > self.buf.numel():
            if _capturing(self.device):
                raise RuntimeError(
                    f"dsa.Workspace: {nbytes} bytes needed but {self.buf.numel()} held, and a "
                    "HIP graph is being captured; size the workspace before capture "
                    "(select_workspace_bytes)")
            self._replaced.append(self.buf)   # an earlier graph may still use it
            self.buf = torch.zeros(nbytes, dtype=torch.uint8, device=self.device)
        return self


_workspaces: dict = {}


def _default_workspace(device, stream: int, nbytes: int) -> Workspace:
    key = (device.index, stream)
    ws = _workspaces.get(key)
    if ws is None:
        ws = _workspaces[key] = Workspace(device, nbytes)
    return ws.ensure(nbytes)


def block_scores(logits: torch.Tensor, row_ks: torch.Tensor | None, row_ke: torch.Tensor,
                 block_size: int, row_repeat: int = 1, pin_newest: bool = True,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 block scores [rows, ceil(width / block_size)] (dsa_block_scores)."""
    ld = _check_logits(logits)
    rows, width = logits.shape
    nblocks = -(-width // block_size) if block_size > 0 else 0
    if out is None:
        out = torch.empty((rows, nblocks), dtype=torch.float32, device=logits.device)
    groups = -(-rows // row_repeat) if row_repeat > 0 else 0
    ks = _bounds(row_ks, "row_ks", groups, logits.device)
    ke = _bounds(row_ke, "row_ke", groups, logits.device)
    code = lib().dsa_block_scores(_ptr(logits), rows, width, ld, _ptr(ks), _ptr(ke), block_size,
                                  row_repeat, int(bool(pin_newest)), _ptr(out), _ld(out),
                                  _stream(logits.device))
    _raise(code, "dsa_block_scores")
    return out


def block_score_keys(logits: torch.Tensor, row_ks: torch.Tensor | None, row_ke: torch.Tensor,
                     block_size: int, row_repeat: int = 1, pin_newest: bool = True,
                     out: torch.Tensor | None = None) -> torch.Tensor:
    """Block scores as order-preserving uint32 codes [rows, ceil(width / block_size)]
    (dsa_block_score_keys): an integer maximum over codes is the scores' own
    maximum, NaN and +-0 included.  ``out`` may be uint32 or int32 (bit
    patterns).  torch has no uint32 maximum: to reduce with torch, view the
    codes as int32 and flip the sign bit (``c ^ -2**31``), whose signed order
    is the codes' unsigned order."""
    ld = _check_logits(logits)
    rows, width = logits.shape
    nblocks = -(-width // block_size) if block_size > 0 else 0
    if out is None:
        out = torch.empty((rows, nblocks), dtype=torch.uint32, device=logits.device)
    if out.dtype not in (torch.uint32, torch.int32) or out.device != logits.device:
        raise ValueError("out must be uint32 or int32 on the logits' device")
    groups = -(-rows // row_repeat) if row_repeat > 0 else 0
    ks = _bounds(row_ks, "row_ks", groups, logits.device)
    ke = _bounds(row_ke, "row_ke", groups, logits.device)
    code = lib().dsa_block_score_keys(_ptr(logits), rows, width, ld, _ptr(ks), _ptr(ke),
                                      block_size, row_repeat, int(bool(pin_newest)), _ptr(out),
                                      _ld(out), _stream(logits.device))
    _raise(code, "dsa_block_score_keys")
    return out


def select_candidate_blocks(logits: torch.Tensor, row_ks: torch.Tensor | None,
                            row_ke: torch.Tensor, topk_blocks: int, block_size: int,
                            out: torch.Tensor, row_repeat: int = 1, *,
                            scores_out: torch.Tensor | None = None,
                            workspace: Workspace | None = None,
                            plan: int = 0, plan_arg: int = 0) -> None:
    """Fill int32 ``out[rows, >=topk_blocks]`` with the selected block ids, -1 padded.

    Mirrors ``select_candidate_blocks(logits, row_ks, row_ke, topk_blocks,
    block_size, out, row_repeat)`` of the vLLM-fork candidate_blocks.py page
    (non-DCP branch).  ``plan``/``plan_arg`` pick a launch plan (0 =
    automatic, see dsa_select_candidate_blocks_plan); every plan gives
    identical results.
    """
    ld = _check_logits(logits)
    rows, width = logits.shape
    if out.dtype != torch.int32 or out.device != logits.device:
        raise ValueError("out must be int32 on the logits' device")
    if out.shape[0] != rows:
        raise ValueError("out must have one row per logits row")
    groups = -(-rows // row_repeat) if row_repeat > 0 else 0
    ks = _bounds(row_ks, "row_ks", groups, logits.device)
    ke = _bounds(row_ke, "row_ke", groups, logits.device)
    ld_scores = 0
    if scores_out is not None:
        if scores_out.dtype != torch.float32 or scores_out.device != logits.device:
            raise ValueError("scores_out must be float32 on the logits' device")
        ld_scores = _ld(scores_out)
    stream = _stream(logits.device)
    # Only the split and pair plans touch the workspace: no default one for the others.
    chosen = plan
    if plan == 0 and rows >= 0 and width >= 0 and block_size > 0 and topk_blocks >= 0:
        chosen = select_plan(rows, width, block_size, topk_blocks)[0]
    ws_ptr, ws_bytes = None, 0
    if chosen in (2, 4) or workspace is not None:
        need = select_workspace_bytes(rows, width, block_size, topk_blocks) if block_size > 0 else 0
        if workspace is None:
            workspace = _default_workspace(logits.device, stream, need)
        else:
            workspace.ensure(need)
        ws_ptr, ws_bytes = workspace.buf.data_ptr(), workspace.buf.numel()
    code = lib().dsa_select_candidate_blocks_plan(
        _ptr(logits), rows, width, ld, _ptr(ks), _ptr(ke), topk_blocks, block_size, row_repeat,
        _ptr(out), _ld(out), _ptr(scores_out), ld_scores, ws_ptr, ws_bytes, plan, plan_arg,
        stream)
    _raise(code, "dsa_select_candidate_blocks")


def select_candidate_blocks_noalloc(logits: torch.Tensor, row_ks: torch.Tensor | None,
                                    row_ke: torch.Tensor, topk_blocks: int, block_size: int,
                                    out: torch.Tensor, row_repeat: int = 1, *,
                                    scores_out: torch.Tensor | None = None) -> None:
    """select_candidate_blocks with no workspace and no allocation
    (dsa_select_candidate_blocks_noalloc): plans that need scratch use the
    library's static per-GPU array, so calls on one GPU must not overlap."""
    ld = _check_logits(logits)
    rows, width = logits.shape
    if out.dtype != torch.int32 or out.device != logits.device or out.shape[0] != rows:
        raise ValueError("out must be int32 [rows, >= topk_blocks] on the logits' device")
    groups = -(-rows // row_repeat) if row_repeat > 0 else 0
    ks = _bounds(row_ks, "row_ks", groups, logits.device)
    ke = _bounds(row_ke, "row_ke", groups, logits.device)
    ld_scores = 0
    if scores_out is not None:
        if scores_out.dtype != torch.float32 or scores_out.device != logits.device:
            raise ValueError("scores_out must be float32 on the logits' device")
        ld_scores = _ld(scores_out)
    code = lib().dsa_select_candidate_blocks_noalloc(
        _ptr(logits), rows, width, ld, _ptr(ks), _ptr(ke), topk_blocks, block_size, row_repeat,
        _ptr(out), _ld(out), _ptr(scores_out), ld_scores, _stream(logits.device))
    _raise(code, "dsa_select_candidate_blocks_noalloc")


def select_from_scores(scores: torch.Tensor, global_row_ke: torch.Tensor, topk_blocks: int,
                       global_block_size: int, max_global_blocks: int, out: torch.Tensor,
                       row_repeat: int = 1) -> None:
    """DCP selection after the reduce (dsa_select_from_scores): ``scores``
    fp32 [rows, nscore] (the element-wise maximum of every rank's unpinned
    local block scores), pin from the global ends, -1 padded ids in ``out``."""
    if scores.dtype != torch.float32 or scores.device.type != "cuda":
        raise ValueError("scores must be float32 on a HIP device")
    rows, nscore = scores.shape
    ld = _ld(scores) if nscore else 1
    if out.dtype != torch.int32 or out.device != scores.device or out.shape[0] != rows:
        raise ValueError("out must be int32 [rows, >= topk_blocks] on the scores' device")
    groups = -(-rows // row_repeat) if row_repeat > 0 else 0
    ke = _bounds(global_row_ke, "global_row_ke", groups, scores.device)
    code = lib().dsa_select_from_scores(_ptr(scores) if nscore else None, rows, nscore, ld,
                                        max_global_blocks, _ptr(ke), row_repeat,
                                        global_block_size, topk_blocks, _ptr(out), _ld(out),
                                        _stream(scores.device))
    _raise(code, "dsa_select_from_scores")


def select_from_keys(keys: torch.Tensor, global_row_ke: torch.Tensor, topk_blocks: int,
                     global_block_size: int, max_global_blocks: int, out: torch.Tensor,
                     row_repeat: int = 1) -> None:
    """DCP selection after an integer-maximum reduce of uint32 score codes
    (dsa_select_from_keys): ``keys`` uint32 or int32 (bit patterns)
    [rows, nkeys]; otherwise as select_from_scores."""
    if keys.dtype not in (torch.uint32, torch.int32) or keys.device.type != "cuda":
        raise ValueError("keys must be uint32 or int32 on a HIP device")
    rows, nkeys = keys.shape
    ld = _ld(keys) if nkeys else 1
    if out.dtype != torch.int32 or out.device != keys.device or out.shape[0] != rows:
        raise ValueError("out must be int32 [rows, >= topk_blocks] on the keys' device")
    groups = -(-rows // row_repeat) if row_repeat > 0 else 0
    ke = _bounds(global_row_ke, "global_row_ke", groups, keys.device)
    code = lib().dsa_select_from_keys(_ptr(keys) if nkeys else None, rows, nkeys, ld,
                                      max_global_blocks, _ptr(ke), row_repeat, global_block_size,
                                      topk_blocks, _ptr(out), _ld(out), _stream(keys.device))
    _raise(code, "dsa_select_from_keys")


def mask_candidates(logits: torch.Tensor, row_ks: torch.Tensor | None, row_ke: torch.Tensor,
                    candidates: torch.Tensor, topk_blocks: int, block_size: int,
                    row_repeat: int = 1) -> None:
    """In place: columns outside [s, e) or outside the row's first
    ``topk_blocks`` candidate blocks become -inf (dsa_mask_candidates)."""
    ld = _check_logits(logits)
    rows, width = logits.shape
    if candidates.dtype != torch.int32 or candidates.device != logits.device:
        raise ValueError("candidates must be int32 on the logits' device")
    if candidates.shape[0] != rows:
        raise ValueError("candidates must have one row per logits row")
    groups = -(-rows // row_repeat) if row_repeat > 0 else 0
    ks = _bounds(row_ks, "row_ks", groups, logits.device)
    ke = _bounds(row_ke, "row_ke", groups, logits.device)
    code = lib().dsa_mask_candidates(_ptr(logits), rows, width, ld, _ptr(ks), _ptr(ke),
                                     _ptr(candidates), _ld(candidates), topk_blocks, block_size,
                                     row_repeat, _stream(logits.device))
    _raise(code, "dsa_mask_candidates")


def correct_attn_out(out: torch.Tensor, lses: torch.Tensor, cp_rank: int,
                     new_output: torch.Tensor | None = None,
                     lse: torch.Tensor | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Base-2 LSE correction of one rank's partial attention output
    (dsa_correct_attn_out; page 3, correct_attn_out): fp32 ``out [B, H, D]``
    (or [B, 1, H, D]) and ``lses [N, B, H]`` (or with a size-1 extra dim) give
    ``(new_output [H, B, D], lse [B, H])``."""
    if out.dim() == 4 and out.shape[1] == 1:
        out = out.squeeze(1)
    if lses.dim() == 4 and lses.shape[-1] == 1:
        lses = lses.squeeze(-1)
    if lses.dim() == 4 and lses.shape[1] == 1:
        lses = lses.squeeze(1)
    if out.dim() != 3 or lses.dim() != 3:
        raise ValueError("expected out [B, H, D] and lses [N, B, H]")
    for t, name in ((out, "out"), (lses, "lses")):
        if t.dtype != torch.float32 or t.device.type != "cuda":
            raise ValueError(f"{name} must be float32 on a HIP device")
    B, H, D = out.shape
    N = lses.shape[0]
    if tuple(lses.shape[1:]) != (B, H):
        raise ValueError("lses must be [N, B, H] for out [B, H, D]")
    if new_output is None:
        new_output = torch.empty((H, B, D), dtype=torch.float32, device=out.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=out.device)
    if new_output.shape != (H, B, D) or lse.shape != (B, H):
        raise ValueError("new_output must be [H, B, D] and lse [B, H]")
    code = lib().dsa_correct_attn_out(
        _ptr(out), B, H, D, *out.stride(), _ptr(lses), N, *lses.stride(), cp_rank,
        _ptr(new_output), *new_output.stride(), _ptr(lse), *lse.stride(), _stream(out.device))
    _raise(code, "dsa_correct_attn_out")
    return new_output, lse
