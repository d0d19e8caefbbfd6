"""Host-side checks of the C ABI (no GPU needed, no compute launched).

- libdsa.so / libdsa_calib.so load and export every function include/*.h declares;
- every invalid argument is rejected on the host with its status code before
  anything is enqueued (fake device pointers are never dereferenced);
- the workspace size and the automatic plan are pure host arithmetic.
"""
import ctypes
import glob
import os
import re

import pytest
import torch

from sparse_attention_kv_dsa_amd import build as dsa_build
from sparse_attention_kv_dsa_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))
FAKE = 0x10000          # 4096-aligned, never dereferenced by a rejected call
FAKE2 = 0x20000


def _declared(path):
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(dsa_\w+)\s*\(", text, flags=re.M)))


def test_headers_exist():
    names = [os.path.basename(h) for h in HEADERS]
    assert "dsa.h" in names and "dsa_calib.h" in names


@pytest.mark.parametrize("header,lib", [("dsa.h", "libdsa.so"), ("dsa_calib.h", "libdsa_calib.so")])
def test_library_exports_every_declared_symbol(header, lib):
    path = dsa_build.lib_path(lib)
    assert os.path.exists(path), f"{lib} not built"
    L = ctypes.CDLL(path)
    decl = _declared(os.path.join(ROOT, "include", header))
    assert decl, header
    for name in decl:
        assert hasattr(L, name), f"{lib} does not export {name}"


def test_status_strings():
    assert [B.status_string(i) for i in range(5)] == [
        "DSA_OK", "DSA_ERR_INVALID_ARG", "DSA_ERR_UNSUPPORTED", "DSA_ERR_WORKSPACE", "DSA_ERR_HIP"]
    assert B.status_string(99) == "unknown"


def test_workspace_bytes():
    L = B.lib()
    # one uint32 key per row and block
    # 2 KiB of pair-plan arrival counters, then rows of keys padded to 32
    assert L.dsa_select_workspace_bytes(64, 32768, 64, 32) == 2048 + 64 * 512 * 4
    assert L.dsa_select_workspace_bytes(65, 100, 7, 3) == 2048 + 65 * 32 * 4
    assert L.dsa_select_workspace_bytes(3, 100000, 64, 3) == 2048 + 3 * 1568 * 4
    assert L.dsa_select_workspace_bytes(0, 100, 7, 3) == 0
    assert L.dsa_select_workspace_bytes(5, 0, 7, 3) == 0
    assert L.dsa_select_workspace_bytes(5, 100, 0, 3) == 0
    assert L.dsa_select_workspace_bytes(5, 100, 4, -1) == 0
    # rows past LDS (the split plan reads their keys from the workspace)
    assert L.dsa_select_workspace_bytes(2, 1 << 20, 16, 32) == 2048 + 2 * 65536 * 4
    assert L.dsa_select_workspace_bytes(2, 1 << 20, 1, 8200) == 0   # select state past LDS
    assert L.dsa_select_workspace_bytes(1 << 30, 1 << 40, 1, 4) == 0  # past any size_t


def test_auto_plan():
    assert B.select_plan(4096, 16384, 64, 32) == (3, 0)    # many short rows: a wave per row
    assert B.select_plan(8192, 65536, 64, 64) == (1, 4)    # many long rows: a workgroup per row
    assert B.select_plan(2048, 131072, 128, 32) == (1, 8)  # longer rows: eight waves each
    assert B.select_plan(8, 1000, 64, 4) == (3, 0)         # one chunk per row anyway
    # fewer rows of one chunk each: four waves per row (rows of <= 2K: a wave)
    assert B.select_plan(512, 8192, 64, 32) == (1, 4)
    assert B.select_plan(128, 2048, 64, 32) == (3, 0)
    # decode batches of up to 256 rows of >= 16K columns (<= 128K columns
    # beyond 128 rows): the pair plan, plan_arg = waves | parts << 8
    assert B.select_plan(64, 32768, 64, 32) == (4, 8 | 4 << 8)
    assert B.select_plan(64, 65536, 64, 32) == (4, 8 | 4 << 8)
    assert B.select_plan(64, 131072, 64, 32) == (4, 8 | 4 << 8)
    assert B.select_plan(32, 32768, 64, 32) == (4, 8 | 4 << 8)    # parts of >= 8K columns
    assert B.select_plan(32, 65536, 64, 32) == (4, 8 | 8 << 8)
    assert B.select_plan(128, 131072, 128, 16) == (4, 8 | 2 << 8)
    assert B.select_plan(96, 262144, 128, 16) == (4, 16 | 2 << 8)
    assert B.select_plan(16, 131072, 128, 16) == (4, 8 | 8 << 8)
    assert B.select_plan(1, 262144, 128, 16) == (4, 16 | 8 << 8)
    assert B.select_plan(8, 16384, 64, 32) == (4, 8 | 2 << 8)
    assert B.select_plan(128, 16384, 64, 32) == (4, 8 | 2 << 8)
    assert B.select_plan(192, 65536, 64, 32) == (4, 8 | 2 << 8)
    assert B.select_plan(256, 131072, 64, 32) == (4, 8 | 2 << 8)
    # one workgroup per row: more rows, or rows too long for the pair plan
    assert B.select_plan(512, 16384, 64, 32) == (1, 4)
    assert B.select_plan(300, 32768, 64, 32) == (1, 8)
    assert B.select_plan(256, 262144, 64, 32) == (1, 16)
    assert B.select_plan(600, 131072, 128, 16) == (1, 8)
    assert B.select_plan(512, 65536, 64, 32) == (1, 4)
    assert B.select_plan(320, 262144, 64, 32) == (1, 16)
    assert B.select_plan(224, 524288, 64, 32) == (1, 16)
    assert B.select_plan(600, 32768, 64, 32) == (1, 4)
    # more than 128 rows, too few for their length: split
    assert B.select_plan(192, 262144, 64, 32) == (2, 384)
    p, cb = B.select_plan(300, 1 << 20, 128, 16)
    assert p == 2 and cb % 2 == 0 and cb >= 1
    # rows past LDS, however few or many: split
    assert B.select_plan(4, 15312 * 4 + 4, 4, 3)[0] == 2
    assert B.select_plan(64, 1 << 20, 16, 32)[0] == 2
    assert B.select_plan(4096, 1 << 20, 8, 2048)[0] == 2


def _sel(**kw):
    a = dict(logits=FAKE, rows=4, width=64, ld=64, ks=None, ke=FAKE, k=4, B=8, R=1, out=FAKE2,
             ld_out=4, scores=None, ld_scores=0, ws=FAKE, ws_bytes=1 << 20, plan=0, cb=0)
    a.update(kw)
    return B.lib().dsa_select_candidate_blocks_plan(
        a["logits"], a["rows"], a["width"], a["ld"], a["ks"], a["ke"], a["k"], a["B"], a["R"],
        a["out"], a["ld_out"], a["scores"], a["ld_scores"], a["ws"], a["ws_bytes"], a["plan"],
        a["cb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), 1), (dict(width=-1), 1), (dict(B=0), 1), (dict(R=0), 1), (dict(k=-1), 1),
    (dict(ld=63), 1), (dict(ld_out=3), 1), (dict(plan=5), 1), (dict(plan=-1), 1), (dict(cb=-1), 1),
    (dict(plan=1, cb=17), 1), (dict(plan=3, cb=4), 1),
    (dict(scores=FAKE, ld_scores=7), 1),         # nblocks = 8
    (dict(out=None), 1), (dict(out=FAKE2 + 2), 1), (dict(logits=None), 1), (dict(ke=None), 1),
    (dict(logits=FAKE + 2), 1), (dict(scores=FAKE + 1, ld_scores=8), 1),
    (dict(ws=None, plan=2), 3), (dict(ws_bytes=100, plan=2), 3), (dict(ws=FAKE + 2, plan=2), 3),
    (dict(ws=None, plan=2, cb=3), 3), (dict(ws=FAKE + 64, plan=2), 3),
    (dict(plan=4, cb=17), 1), (dict(plan=4, cb=2 << 16), 1),
    (dict(plan=4, ws=None), 3),
    (dict(plan=4, ws_bytes=2047), 3), (dict(plan=4, ws=FAKE + 64), 3),
    (dict(plan=4, rows=257), 2),                                     # 256 arrival counters
    # keys past LDS: only the split plan, and only with its workspace (here
    # 2048 + 4 * 65536 * 4 bytes, more than the 1 MiB given)
    (dict(width=1 << 20, ld=1 << 20, B=16, k=4096, ld_out=4096), 3),
    (dict(width=1 << 20, ld=1 << 20, B=16, k=4096, ld_out=4096, plan=1), 2),
    (dict(width=1 << 20, ld=1 << 20, B=16, k=4096, ld_out=4096, plan=4), 2),
    (dict(width=15312 * 4 + 4, ld=1 << 16, B=4, k=3, ld_out=3, plan=3), 2),  # 15316 + 48 + 1024 > 16384
    (dict(width=15312 * 4 + 4, ld=1 << 16, B=4, k=3, ld_out=3, plan=2, ws=None), 3),
    (dict(width=15312 * 4, ld=1 << 16, B=4, k=3, ld_out=3, plan=2, ws=None), 3),  # 15312 + 48 + 1024 fits
    # the select state alone past LDS: 48 + 16400 words
    (dict(width=1 << 20, ld=1 << 20, B=1, k=8200, ld_out=8200, ws_bytes=1 << 30), 2),
    (dict(rows=0), 0), (dict(k=0), 0), (dict(rows=0, logits=None, ke=None, out=None), 0),
])
def test_select_rejects_on_host(kw, code):
    assert _sel(**kw) == code


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="reaches a kernel launch with placeholder pointers: host-only check")
def test_rows_past_lds_reach_the_launch():
    """Rows past LDS pass every host check under the automatic and the split
    plan when the workspace holds their keys (DSA_ERR_HIP = 4 here, with no
    GPU)."""
    shape = dict(width=15312 * 4 + 4, ld=1 << 16, B=4, k=3, ld_out=3)
    assert _sel(**shape) == 4 and _sel(**shape, plan=2) == 4 and _sel(**shape, plan=2, cb=7) == 4
    big = dict(width=1 << 20, ld=1 << 20, B=16, k=4096, ld_out=4096, ws_bytes=(1 << 20) + 2048)
    assert _sel(**big) == 4


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="reaches a kernel launch with placeholder pointers: host-only check")
def test_auto_plan_without_workspace_takes_the_group_plan():
    """A pair-plan shape with no (or a too small or misaligned) workspace is
    not rejected under the automatic plan: it passes every host check and
    reaches the launch (DSA_ERR_HIP = 4 here, with no GPU), while the
    explicit pair plan reports DSA_ERR_WORKSPACE."""
    shape = dict(rows=64, width=32768, ld=32768, B=64, k=32, ld_out=32)
    assert B.select_plan(64, 32768, 64, 32)[0] == 4
    for ws in (dict(ws=None), dict(ws_bytes=100), dict(ws=FAKE + 64)):
        assert _sel(**shape, **ws) == 4
        assert _sel(**shape, **ws, plan=4) == 3


def _bs(keys=False, **kw):
    a = dict(logits=FAKE, rows=4, width=64, ld=64, ks=None, ke=FAKE, B=8, R=1, pin=1,
             scores=FAKE2, ld_scores=8)
    a.update(kw)
    fn = B.lib().dsa_block_score_keys if keys else B.lib().dsa_block_scores
    return fn(a["logits"], a["rows"], a["width"], a["ld"], a["ks"], a["ke"], a["B"], a["R"],
              a["pin"], a["scores"], a["ld_scores"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=-1), 1), (dict(width=-1), 1), (dict(B=0), 1), (dict(R=0), 1), (dict(pin=2), 1),
    (dict(ld=10), 1), (dict(ld_scores=7), 1), (dict(logits=None), 1), (dict(ke=None), 1),
    (dict(scores=None), 1), (dict(logits=FAKE + 1), 1), (dict(scores=FAKE2 + 3), 1),
    (dict(rows=0), 0), (dict(width=0, ld_scores=0), 0),
])
def test_block_scores_rejects_on_host(kw, code):
    assert _bs(**kw) == code
    assert _bs(keys=True, **kw) == code   # the uint32-code variant checks alike


def test_calib_rejects_on_host():
    L = ctypes.CDLL(dsa_build.lib_path("libdsa_calib.so"))
    L.dsa_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.dsa_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
    assert L.dsa_calib_copy(FAKE, FAKE2, 17, None) == 1
    assert L.dsa_calib_copy(FAKE + 4, FAKE2, 16, None) == 1
    assert L.dsa_calib_copy(None, FAKE2, 16, None) == 1
    assert L.dsa_calib_copy(FAKE, FAKE2, 0, None) == 0
    assert L.dsa_calib_read(FAKE, 16, None, None) == 1
    assert L.dsa_calib_read_sink_words() >= 1
    L.dsa_calib_fill.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p]
    assert L.dsa_calib_fill(FAKE + 8, 16, 0, None) == 1
    assert L.dsa_calib_fill(FAKE, 24, 0, None) == 1
    assert L.dsa_calib_fill(None, 16, 0, None) == 1
    assert L.dsa_calib_fill(FAKE, 0, 0, None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 64)
    with pytest.raises(ValueError):
        B.select_candidate_blocks(x, None, torch.zeros(4, dtype=torch.int32), 4, 8,
                                  torch.zeros(4, 4, dtype=torch.int32))


# --- the entry points after selection: host-side argument checks (no launch)

def _sfs(keys=False, **kw):
    a = dict(scores=FAKE, rows=4, nscore=8, ld=8, mgb=8, ke=FAKE, R=1, G=4, k=4, out=FAKE2, ld_out=4)
    a.update(kw)
    fn = B.lib().dsa_select_from_keys if keys else B.lib().dsa_select_from_scores
    return fn(a["scores"], a["rows"], a["nscore"], a["ld"], a["mgb"], a["ke"], a["R"], a["G"],
              a["k"], a["out"], a["ld_out"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=0), 0), (dict(k=0), 0), (dict(rows=0, scores=None, ke=None, out=None), 0),
    (dict(rows=-1), 1), (dict(nscore=-1), 1), (dict(mgb=-1), 1), (dict(R=0), 1), (dict(G=0), 1),
    (dict(k=-1), 1), (dict(ld=7), 1), (dict(ld_out=3), 1), (dict(ke=None), 1), (dict(out=None), 1),
    (dict(out=FAKE2 + 2), 1), (dict(scores=None), 1), (dict(scores=FAKE + 1), 1),
    (dict(mgb=1 << 20, k=4), 2),                      # the scores do not fit in LDS
])
def test_select_from_scores_rejects_on_host(kw, code):
    assert _sfs(**kw) == code
    assert _sfs(keys=True, **kw) == code   # the uint32-code variant checks alike


def _mask(**kw):
    a = dict(logits=FAKE, rows=4, width=64, ld=64, ks=None, ke=FAKE, cand=FAKE2, ld_cand=4, k=4,
             B=8, R=1)
    a.update(kw)
    return B.lib().dsa_mask_candidates(a["logits"], a["rows"], a["width"], a["ld"], a["ks"],
                                       a["ke"], a["cand"], a["ld_cand"], a["k"], a["B"], a["R"],
                                       None)


@pytest.mark.parametrize("kw,code", [
    (dict(rows=0), 0), (dict(width=0), 0), (dict(rows=0, logits=None, ke=None, cand=None), 0),
    (dict(rows=-1), 1), (dict(width=-1), 1), (dict(B=0), 1), (dict(R=0), 1), (dict(k=-1), 1),
    (dict(ld=63), 1), (dict(ld_cand=3), 1), (dict(logits=None), 1), (dict(ke=None), 1),
    (dict(cand=None), 1), (dict(logits=FAKE + 2), 1), (dict(cand=FAKE2 + 1), 1),
])
def test_mask_rejects_on_host(kw, code):
    assert _mask(**kw) == code


def _lse(**kw):
    a = dict(out=FAKE, B=2, H=3, D=8, o=(24, 8, 1), lses=FAKE2, N=4, l=(6, 3, 1), rank=1,
             new=FAKE, n=(16, 8, 1), v=FAKE2, vs=(3, 1))
    a.update(kw)
    return B.lib().dsa_correct_attn_out(a["out"], a["B"], a["H"], a["D"], *a["o"], a["lses"],
                                        a["N"], *a["l"], a["rank"], a["new"], *a["n"], a["v"],
                                        *a["vs"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), 0), (dict(H=0), 0), (dict(B=0, out=None, lses=None, new=None, v=None), 0),
    (dict(B=-1), 1), (dict(D=-1), 1), (dict(N=0), 1), (dict(N=-1), 1), (dict(rank=4), 1),
    (dict(rank=-1), 1), (dict(lses=None), 1), (dict(v=None), 1), (dict(out=None), 1),
    (dict(new=None), 1), (dict(lses=FAKE2 + 2), 1), (dict(new=FAKE + 1), 1),
])
def test_correct_attn_out_rejects_on_host(kw, code):
    assert _lse(**kw) == code


def test_noalloc_host_checks():
    """dsa_select_candidate_blocks_noalloc rejects on the host, before any
    device call: invalid arguments, and a shape whose plan needs more than
    its static scratch (16 MiB).  With no GPU visible, a shape that passes
    fails at the device query (DSA_ERR_HIP) without touching memory."""
    import torch
    L = B.lib()

    def call(rows, width, B_, k, ld=None, ke=FAKE, out=FAKE2):
        return L.dsa_select_candidate_blocks_noalloc(FAKE, rows, width, ld or width, None, ke, k,
                                                     B_, 1, out, k, None, 0, None)

    assert B.select_plan(300, 600000, 40, 16)[0] == 2
    assert B.select_workspace_bytes(300, 600000, 40, 16) > 16 << 20
    assert call(300, 600000, 40, 16) == 3            # the split plan's keys exceed the scratch
    assert call(-1, 100, 8, 4) == 1 and call(4, 100, 0, 4) == 1 and call(4, 100, 8, -1) == 1
    assert call(4, 100, 8, 4, ld=99) == 1 and call(4, 100, 8, 4, ke=None) == 1
    assert call(0, 100, 8, 4) == 0 and call(4, 100, 8, 0) == 0   # nothing to do
    if torch.cuda.device_count() == 0:
        assert call(64, 32768, 64, 32) == 4           # pair plan: no device to hold the scratch
