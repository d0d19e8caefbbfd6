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
                L.dsa_select_plan.argtypes = [i64, i64, i32, i32, ctypes.POINTER(i32),
                                              ctypes.POINTER(i32)]
                L.dsa_select_plan.restype = ctypes.c_int
                L.dsa_status_string.argtypes = [ctypes.c_int]
                L.dsa_status_string.restype = ctypes.c_char_p
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


class Workspace:
    """Device scratch for the split plan of dsa_select_candidate_blocks
    (no initialisation needed; one per stream that may run concurrently)."""

    def __init__(self, device, nbytes: int = 0):
        self.device = torch.device(device)
        self.buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=self.device)

    def ensure(self, nbytes: int) -> "Workspace":
        if nbytes > self.buf.numel():
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
    need = select_workspace_bytes(rows, width, block_size, topk_blocks) if block_size > 0 else 0
    if workspace is None:
        workspace = _default_workspace(logits.device, stream, need)
    else:
        workspace.ensure(need)
    code = lib().dsa_select_candidate_blocks_plan(
        _ptr(logits), rows, width, ld, _ptr(ks), _ptr(ke), topk_blocks, block_size, row_repeat,
        _ptr(out), _ld(out), _ptr(scores_out), ld_scores, workspace.buf.data_ptr(),
        workspace.buf.numel(), plan, plan_arg, stream)
    _raise(code, "dsa_select_candidate_blocks")
