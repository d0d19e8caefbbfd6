"""Every entry point captured in a HIP graph and replayed three times, with
the program's own eager work and a synchronisation between replays: each
replay reproduces the eager result bit for bit.  Outputs are overwritten
with junk before every replay, so each replay must rewrite them."""
import numpy as np
import pytest
import torch

import sparse_attention_kv_dsa_amd as dsa
from sparse_attention_kv_dsa_amd import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _check_replays(run, outputs, clear):
    run()
    torch.cuda.synchronize()
    ref = [_bits(o).clone() for o in outputs]
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run()
    busy = torch.zeros(1 << 20, device=DEV)
    for rep in range(3):
        clear()
        busy.add_(1.0)  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outputs, ref):
            assert torch.equal(_bits(o), r), f"replay {rep} differs from the eager call"


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


@pytest.mark.parametrize("cfg,plan", [(2, 0), (2, 2), (4, 0), (3, 0), (1, 3), (4, 4), (2, 4)])
def test_select_in_graph(cfg, plan):
    w = workloads.config(cfg)
    x = torch.from_numpy(w.logits).to(DEV)
    ks = None if w.row_ks is None else _i32(w.row_ks)
    ke = _i32(w.row_ke)
    nb = -(-w.width // w.block_size)
    out = torch.empty((w.rows, w.topk_blocks), dtype=torch.int32, device=DEV)
    sc = torch.empty((w.rows, nb), dtype=torch.float32, device=DEV)
    ws = dsa.Workspace(DEV, dsa.select_workspace_bytes(w.rows, w.width, w.block_size,
                                                       w.topk_blocks))

    def run():
        dsa.select_candidate_blocks(x, ks, ke, w.topk_blocks, w.block_size, out, w.row_repeat,
                                    scores_out=sc, workspace=ws, plan=plan)

    def clear():
        out.fill_(12345)
        sc.fill_(777.0)

    _check_replays(run, [out, sc], clear)


def test_block_scores_and_dcp_select_in_graph():
    w = workloads.config(2)
    x = torch.from_numpy(w.logits).to(DEV)
    ke = _i32(w.row_ke)
    nb = -(-w.width // w.block_size)
    sc = torch.empty((w.rows, nb), dtype=torch.float32, device=DEV)
    ends = _i32(w.row_ke)
    out = torch.empty((w.rows, w.topk_blocks), dtype=torch.int32, device=DEV)

    def run():
        dsa.block_scores(x, None, ke, w.block_size, w.row_repeat, pin_newest=False, out=sc)
        dsa.select_from_scores(sc, ends, w.topk_blocks, w.block_size, nb, out, w.row_repeat)

    def clear():
        sc.fill_(777.0)
        out.fill_(12345)

    _check_replays(run, [sc, out], clear)


def test_mask_and_lse_in_graph():
    w = workloads.config(3)
    rows = 512
    logits = np.ascontiguousarray(w.logits[:rows])
    pristine = torch.from_numpy(logits).to(DEV)
    x = pristine.clone()
    ks, ke = _i32(w.row_ks[:rows]), _i32(w.row_ke[:rows])
    cand = torch.empty((rows, w.topk_blocks), dtype=torch.int32, device=DEV)
    dsa.select_candidate_blocks(x, ks, ke, w.topk_blocks, w.block_size, cand)
    lw = workloads.lse_merge(B=16, H=8, D=128, N=4, seed=9)
    o = torch.from_numpy(lw.out).to(DEV)
    lses = torch.from_numpy(lw.lses).to(DEV)
    new = torch.empty((8, 16, 128), dtype=torch.float32, device=DEV)
    lse = torch.empty((16, 8), dtype=torch.float32, device=DEV)

    def run():
        dsa.mask_candidates(x, ks, ke, cand, w.topk_blocks, w.block_size)
        dsa.correct_attn_out(o, lses, 1, new_output=new, lse=lse)

    def clear():
        x.copy_(pristine)  # the mask works in place
        new.fill_(777.0)
        lse.fill_(777.0)

    _check_replays(run, [x, new, lse], clear)


def test_block_score_keys_and_select_from_keys_in_graph():
    w = workloads.config(2)
    x = torch.from_numpy(w.logits).to(DEV)
    ke = _i32(w.row_ke)
    nb = -(-w.width // w.block_size)
    codes = torch.empty((w.rows, nb), dtype=torch.int32, device=DEV)
    out = torch.empty((w.rows, w.topk_blocks), dtype=torch.int32, device=DEV)

    def run():
        dsa.block_score_keys(x, None, ke, w.block_size, w.row_repeat, pin_newest=False, out=codes)
        dsa.select_from_keys(codes, ke, w.topk_blocks, w.block_size, nb, out, w.row_repeat)

    def clear():
        codes.fill_(12345)
        out.fill_(12345)

    _check_replays(run, [codes, out], clear)


def test_workspace_is_not_allocated_under_capture():
    """A call whose plan needs a workspace, captured on a stream that has
    none yet, raises instead of allocating inside the capture."""
    w = workloads.config(2)
    x = torch.from_numpy(w.logits).to(DEV)
    ke = _i32(w.row_ke)
    out = torch.empty((w.rows, w.topk_blocks), dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream(DEV)
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="captured"):
        with torch.cuda.graph(graph, stream=side):
            dsa.select_candidate_blocks(x, None, ke, w.topk_blocks, w.block_size, out,
                                        w.row_repeat, plan=4)
    torch.cuda.synchronize()


def test_graph_keeps_its_workspace_after_growth():
    """A graph captured with a workspace keeps replaying correctly after an
    eager call has grown that workspace: the replaced buffer stays alive."""
    small, big = workloads.config(2), workloads.config(4)
    xs, xb = torch.from_numpy(small.logits).to(DEV), torch.from_numpy(big.logits).to(DEV)
    ke_s, ke_b = _i32(small.row_ke), _i32(big.row_ke)
    ws = dsa.Workspace(DEV, dsa.select_workspace_bytes(small.rows, small.width, small.block_size,
                                                       small.topk_blocks))
    out = torch.empty((small.rows, small.topk_blocks), dtype=torch.int32, device=DEV)
    out_b = torch.empty((big.rows, big.topk_blocks), dtype=torch.int32, device=DEV)

    def run():
        dsa.select_candidate_blocks(xs, None, ke_s, small.topk_blocks, small.block_size, out,
                                    small.row_repeat, workspace=ws, plan=4)

    run()
    torch.cuda.synchronize()
    ref = out.clone()
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        run()
    old = ws.buf.data_ptr()
    dsa.select_candidate_blocks(xb, None, ke_b, big.topk_blocks, big.block_size, out_b,
                                big.row_repeat, workspace=ws, plan=4)   # grows the workspace
    torch.cuda.synchronize()
    assert ws.buf.data_ptr() != old
    big_ref = out_b.clone()
    for _ in range(3):
        out.fill_(12345)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        dsa.select_candidate_blocks(xb, None, ke_b, big.topk_blocks, big.block_size, out_b,
                                    big.row_repeat, workspace=ws, plan=4)
        torch.cuda.synchronize()
        assert torch.equal(out_b, big_ref)
