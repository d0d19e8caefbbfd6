"""dsa_select_candidate_blocks_noalloc, the entry point for callers that
cannot allocate (it uses the library's static per-GPU scratch instead of a
workspace), against dsa_select_candidate_blocks with a caller workspace,
both called through the C ABI: ids and fp32 scores bit-exact, on two calls
in a row, the second with a smaller input, for the pair plan (decode
batches) and the split plan; and a shape whose plan needs more scratch than
the array holds is rejected with DSA_ERR_WORKSPACE, writing nothing.
Expected values of the first pair also come from the oracle."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_kv_dsa_amd as dsa
from sparse_attention_kv_dsa_amd import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
SCRATCH_BYTES = 16 << 20   # DSA_NOALLOC_SCRATCH_BYTES


def _i32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def _both(w):
    """(noalloc ids, noalloc scores, workspace ids, workspace scores)."""
    L = dsa.lib()
    x = torch.from_numpy(w.logits).to(DEV)
    ks, ke = _i32(w.row_ks), _i32(w.row_ke)
    nb = -(-w.width // w.block_size)
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    res = []
    for variant in ("noalloc", "workspace"):
        out = torch.full((w.rows, w.topk_blocks), 12345, dtype=torch.int32, device=DEV)
        sc = torch.full((w.rows, nb), 777.0, dtype=torch.float32, device=DEV)
        args = (x.data_ptr(), w.rows, w.width, w.width, None if ks is None else ks.data_ptr(),
                ke.data_ptr(), w.topk_blocks, w.block_size, w.row_repeat, out.data_ptr(),
                w.topk_blocks, sc.data_ptr(), nb)
        if variant == "noalloc":
            code = L.dsa_select_candidate_blocks_noalloc(*args, stream)
        else:
            need = dsa.select_workspace_bytes(w.rows, w.width, w.block_size, w.topk_blocks)
            ws = torch.zeros(need + 128, dtype=torch.uint8, device=DEV)
            base = (ws.data_ptr() + 127) // 128 * 128
            code = L.dsa_select_candidate_blocks(*args, base, need, stream)
        assert code == 0, (variant, dsa.status_string(code))
        torch.cuda.synchronize()
        res += [out.cpu().numpy(), sc.cpu().numpy()]
    return res


def _check(w):
    plan = dsa.select_plan(w.rows, w.width, w.block_size, w.topk_blocks)[0]
    assert plan in (2, 4), plan   # a plan that uses the scratch
    assert dsa.select_workspace_bytes(w.rows, w.width, w.block_size, w.topk_blocks) <= SCRATCH_BYTES
    ids, sc, ids_ws, sc_ws = _both(w)
    assert np.array_equal(ids, ids_ws), w.name
    assert np.array_equal(sc.view(np.uint32), sc_ws.view(np.uint32)), w.name
    return ids, sc


def test_noalloc_pair_plan_twice_smaller_second():
    for cfg in (4, 2):   # long-context decode, then the smaller decode batch
        w = workloads.config(cfg)
        ids, sc = _check(w)
        exp = np.empty_like(ids)
        exp_sc = np.empty_like(sc)
        oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks, w.block_size,
                                       exp, w.row_repeat, scores_out=exp_sc, nthreads=8)
        assert np.array_equal(ids, exp) and np.array_equal(sc.view(np.uint32), exp_sc.view(np.uint32))


def test_noalloc_split_plan_twice_smaller_second():
    for rows, width in ((190, 262144), (150, 200000)):
        w = workloads.many_rows_case(77 + rows, rows, width, 64, 1, 32)
        _check(w)


def test_noalloc_rejects_more_than_its_scratch():
    rows, width, B, k = 300, 600000, 40, 16   # the split plan, 300 x 15008 keys > 16 MiB
    assert dsa.select_plan(rows, width, B, k)[0] == 2
    assert dsa.select_workspace_bytes(rows, width, B, k) > SCRATCH_BYTES
    x = torch.zeros((rows, width), dtype=torch.float32, device=DEV)
    ke = torch.full((rows,), width, dtype=torch.int32, device=DEV)
    out = torch.full((rows, k), 7, dtype=torch.int32, device=DEV)
    code = dsa.lib().dsa_select_candidate_blocks_noalloc(
        x.data_ptr(), rows, width, width, None, ke.data_ptr(), k, B, 1, out.data_ptr(), k, None, 0,
        ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert code == 3   # DSA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7).all())


def test_noalloc_binding_and_plans_without_scratch():
    """The binding function, and a shape whose plan needs no scratch (the
    prefill chunk, one wave per row)."""
    w = workloads.config(3)
    x = torch.from_numpy(w.logits).to(DEV)
    out = torch.empty((w.rows, w.topk_blocks), dtype=torch.int32, device=DEV)
    dsa.select_candidate_blocks_noalloc(x, _i32(w.row_ks), _i32(w.row_ke), w.topk_blocks,
                                        w.block_size, out, w.row_repeat)
    ref = torch.empty_like(out)
    dsa.select_candidate_blocks(x, _i32(w.row_ks), _i32(w.row_ke), w.topk_blocks, w.block_size,
                                ref, w.row_repeat)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
