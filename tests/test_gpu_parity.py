"""GPU parity: the HIP library against the CPU oracle, element by element.

Block ids (values and order) must match exactly; block scores must match bit
for bit (the max is exact, NaN is the canonical 0x7FC00000).  Inputs come from
the seeded generators in sparse_attention_kv_dsa_amd.workloads; expected
values come only from oracle/.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import sparse_attention_kv_dsa_amd as dsa
from sparse_attention_kv_dsa_amd import workloads
from bound_rows import bound_rows, counted_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _say(*a):
    print(*a, flush=True)


def dev_logits(x: np.ndarray, ld_pad: int = 0, offset: int = 0, pad_value=np.nan):
    """Copy [rows, width] to the GPU with row stride width+ld_pad, starting
    `offset` floats into the allocation; the padding holds `pad_value`, so a
    read outside a row's first `width` columns would show up in the results."""
    rows, width = x.shape
    ld = width + ld_pad
    flat = torch.full((offset + rows * ld,), float(pad_value), dtype=torch.float32, device=DEV)
    view = flat[offset:offset + rows * ld].view(rows, ld) if rows else flat[:0].view(0, ld)
    if rows and width:
        view[:, :width].copy_(torch.from_numpy(np.ascontiguousarray(x)))
    return view[:, :width]


def dev_i32(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def pair_arg(cb: int) -> int:
    """An assorted pair-plan argument: waves | parts << 8 | spread << 16."""
    waves = (0, 1, 4, 16)[cb % 4]
    parts = (0, 2, 3, 8, 1, 32)[cb % 6]
    return waves | parts << 8 | ((cb // 3) % 2) << 16


def gpu_select(w, plan=0, cb=0, ld_pad=0, offset=0, with_scores=True, ld_out_pad=0):
    """cb: the plan argument (plan 1: waves per workgroup, plan 2: blocks per
    chunk; plans 3 and 4 map it onto their own arguments)."""
    if plan == 1 and cb:
        cb = 1 + (cb - 1) % 16
    if plan == 3:
        cb = 16 if cb % 2 else 8
    if plan == 4:
        cb = pair_arg(cb)
    x = dev_logits(w.logits, ld_pad, offset)
    nb = -(-w.width // w.block_size)
    out_full = torch.full((w.rows, w.topk_blocks + ld_out_pad), 12345, dtype=torch.int32, device=DEV)
    out = out_full[:, :w.topk_blocks]
    sc = None
    if with_scores:
        sc = torch.full((w.rows, max(nb, 1)), 777.0, dtype=torch.float32, device=DEV)[:, :nb]
    dsa.select_candidate_blocks(x, dev_i32(w.row_ks), dev_i32(w.row_ke), w.topk_blocks,
                                w.block_size, out, w.row_repeat, scores_out=sc, plan=plan,
                                plan_arg=cb)
    torch.cuda.synchronize()
    if ld_out_pad:
        assert (out_full[:, w.topk_blocks:] == 12345).all(), "wrote past topk_blocks"
    return out.cpu().numpy(), (None if sc is None else sc.cpu().numpy())


HOST_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_select(w):
    nb = -(-w.width // w.block_size)
    out = np.empty((w.rows, w.topk_blocks), dtype=np.int32)
    sc = np.empty((w.rows, nb), dtype=np.float32)
    oracle.select_candidate_blocks(w.logits, w.row_ks, w.row_ke, w.topk_blocks, w.block_size,
                                   out, w.row_repeat, scores_out=sc if nb else None,
                                   nthreads=HOST_THREADS)
    return out, sc


def assert_same(got_out, got_sc, exp_out, exp_sc, ctx=""):
    if got_out.ndim == 2 and got_out.shape[1] == 0 and got_sc is not None:
        # topk_blocks == 0 writes nothing at all, not even the optional scores
        assert (got_sc == 777.0).all(), ctx
        return
    if not np.array_equal(got_out, exp_out):
        bad = np.argwhere(got_out != exp_out)
        r = bad[0][0]
        raise AssertionError(f"{ctx}: ids differ in {len(np.unique(bad[:, 0]))} rows; first row {r}:"
                             f"\n gpu    {got_out[r].tolist()}\n oracle {exp_out[r].tolist()}")
    if got_sc is not None and exp_sc is not None and exp_sc.size:
        gb, eb = got_sc.view(np.uint32), exp_sc.view(np.uint32)
        if not np.array_equal(gb, eb):
            bad = np.argwhere(gb != eb)
            r, b = bad[0]
            raise AssertionError(f"{ctx}: scores differ at {len(bad)} places; first [{r},{b}]: "
                                 f"gpu {gb[r, b]:#010x} oracle {eb[r, b]:#010x}")


# ------------------------------------------------------------------ small ---

GOLDEN_CASES = None


def _golden():
    import json
    import os
    global GOLDEN_CASES
    if GOLDEN_CASES is None:
        with open(os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")) as fh:
            GOLDEN_CASES = json.load(fh)["cases"]
    return GOLDEN_CASES


def _golden_workload(c):
    conv = {"nan": np.nan, "inf": np.inf, "-inf": -np.inf, "-0": -0.0}
    width = len(c["logits"][0])
    x = np.array([[conv[v] if isinstance(v, str) else float(v) for v in r] for r in c["logits"]],
                 dtype=np.float32).reshape(len(c["logits"]), width)
    ks = None if c["row_ks"] is None else np.array(c["row_ks"], np.int32)
    return workloads.Workload(c["id"], x, ks, np.array(c["row_ke"], np.int32), c["block_size"],
                              c["topk"], c["row_repeat"])


@pytest.mark.parametrize("plan,cb", [(1, 0), (1, 1), (1, 16), (2, 1), (2, 2), (3, 0), (3, 1),
                                     (4, 0), (4, 1), (4, 3), (4, 5), (4, 7)])
def test_hand_worked_rows(plan, cb):
    for c in _golden():
        w = _golden_workload(c)
        got, sc = gpu_select(w, plan, cb)
        assert got.tolist() == c["out"], c["id"]
        exp_out, exp_sc = oracle_select(w)
        assert_same(got, sc, exp_out, exp_sc, c["id"])


@pytest.mark.parametrize("plan", [1, 2, 3, 4])
def test_random_tiny_cases(plan):
    """400 tiny cases: NaN, +-0, +-inf, ties, odd widths and block sizes,
    negative/overlong/empty windows, row_repeat 1-3, k 0-12."""
    for seed in range(400):
        w = workloads.random_case(seed, ld_pad=seed % 5)
        cb = 1 + seed % 3
        got, sc = gpu_select(w, plan, cb, ld_pad=seed % 5, offset=seed % 4)
        exp_out, exp_sc = oracle_select(w)
        assert_same(got, sc, exp_out, exp_sc, f"seed {seed} plan {plan} cb {cb} {w.describe()}")


MEDIUM_B = [1, 3, 4, 5, 8, 12, 16, 32, 64, 100, 128, 256, 512]


@pytest.mark.parametrize("plan", [1, 2, 3, 4])
def test_random_medium_cases(plan):
    """Several tiles per row and ragged tails, aligned (vector) and unaligned
    (scalar) rows, both launch plans with assorted chunk sizes."""
    rng = np.random.default_rng(7 + plan)
    for i in range(60):
        rows = int(rng.integers(1, 41))
        width = int(rng.integers(1, 6001))
        if i % 3 == 0:
            width = (width // 4) * 4 + 4
        B = int(MEDIUM_B[i % len(MEDIUM_B)])
        R = int(rng.integers(1, 4))
        k = int(rng.integers(0, 101))
        g = -(-rows // R)
        vals = rng.standard_normal((rows, width)).astype(np.float32)
        if i % 2:
            vals = np.round(vals * 2) / 2        # ties
            vals[rng.random((rows, width)) < 0.01] = np.nan
            vals[rng.random((rows, width)) < 0.02] = -np.inf
        ks = None
        if i % 4 == 1:
            ks = (rng.integers(0, width // 4 + 1, size=g) * 4).astype(np.int32)
        elif i % 4 == 3:
            ks = rng.integers(-5, width + 5, size=g).astype(np.int32)
        base = ks if ks is not None else np.zeros(g, np.int32)
        ke = np.clip(base + rng.integers(-10, width + 10, size=g), -3, width + 9).astype(np.int32)
        w = workloads.Workload(f"medium-{i}", vals, ks, ke, B, k, R)
        ld_pad = [0, 0, 4, 1, 3][i % 5]
        offset = [0, 0, 0, 4, 1][i % 5]
        cb = int(rng.integers(1, 40))
        got, sc = gpu_select(w, plan, cb, ld_pad=ld_pad, offset=offset, ld_out_pad=3)
        exp_out, exp_sc = oracle_select(w)
        assert_same(got, sc, exp_out, exp_sc, f"case {i} plan {plan} cb {cb} {w.describe()}")


@pytest.mark.parametrize("pin", [True, False])
def test_block_scores(pin):
    rng = np.random.default_rng(21)
    for i in range(80):
        w = workloads.random_case(500 + i, max_rows=9, max_width=3000, max_block=300,
                                  special=i % 2 == 0, ld_pad=i % 3)
        x = dev_logits(w.logits, i % 3, offset=(i % 2) * 4)
        got = dsa.block_scores(x, dev_i32(w.row_ks), dev_i32(w.row_ke), w.block_size,
                               w.row_repeat, pin_newest=pin)
        torch.cuda.synchronize()
        exp = oracle.block_scores(w.logits, w.row_ks, w.row_ke, w.block_size, w.row_repeat,
                                  pin_newest=pin)
        assert_same(np.zeros(1), got.cpu().numpy(), np.zeros(1), exp, f"block_scores {i}")
    del rng


def test_block_scores_configs():
    for i in (1, 2, 3, 4):
        w = workloads.config(i)
        _say("block scores", w.name)
        x = dev_logits(w.logits)
        for pin in (True, False):
            got = dsa.block_scores(x, dev_i32(w.row_ks), dev_i32(w.row_ke), w.block_size,
                                   w.row_repeat, pin_newest=pin).cpu().numpy()
            exp = oracle.block_scores(w.logits, w.row_ks, w.row_ke, w.block_size, w.row_repeat,
                                      pin_newest=pin, nthreads=8)
            assert_same(np.zeros(1), got, np.zeros(1), exp, f"{w.name} pin={pin}")


@pytest.mark.parametrize("seed,rows,width,B,R", [
    (1, 1100, 33000, 64, 1),   # >= 1024 rows, >= 32K columns: whole rows, four waves
    (2, 2048, 32768, 128, 2),
    (3, 1030, 5003, 7, 1),     # two-wave whole rows on the any-alignment path
    (4, 1024, 16384, 8, 3),    # two-wave whole rows, vector path
    (5, 1023, 40000, 16, 1),   # just under 1024 rows: chunks
])
def test_block_scores_many_rows(seed, rows, width, B, R):
    w = workloads.many_rows_case(seed, rows, width, B, R)
    _say("block scores", w.name)
    x = dev_logits(w.logits)
    for pin in (True, False):
        got = dsa.block_scores(x, dev_i32(w.row_ks), dev_i32(w.row_ke), w.block_size,
                               w.row_repeat, pin_newest=pin).cpu().numpy()
        exp = oracle.block_scores(w.logits, w.row_ks, w.row_ke, w.block_size, w.row_repeat,
                                  pin_newest=pin, nthreads=8)
        assert_same(np.zeros(1), got, np.zeros(1), exp, f"{w.name} pin={pin}")


@pytest.mark.parametrize("B", [4, 8, 16])
def test_block_scores_small_blocks_in_chunks(B):
    """Small blocks, where a chunk's scores are staged in LDS and stored
    after its streaming: few long rows (many chunks per row, chunk offsets
    past 0), and many rows of one whole-row chunk; windows empty, ragged,
    clipped or whole; scores and codes as the oracle's."""
    for rows, width, seed in ((5, 300001, 31), (1100, 8200, 32)):
        w = workloads.many_rows_case(seed + B, rows, width, B, 1)
        _say("block scores", w.name)
        x = dev_logits(w.logits, 1, offset=4)
        for pin in (True, False):
            got = dsa.block_scores(x, dev_i32(w.row_ks), dev_i32(w.row_ke), B, 1,
                                   pin_newest=pin).cpu().numpy()
            exp = oracle.block_scores(w.logits, w.row_ks, w.row_ke, B, 1, pin_newest=pin,
                                      nthreads=HOST_THREADS)
            assert_same(np.zeros(1), got, np.zeros(1), exp, f"{w.name} pin={pin}")
            codes = dsa.block_score_keys(x, dev_i32(w.row_ks), dev_i32(w.row_ke), B, 1,
                                         pin_newest=pin)
            torch.cuda.synchronize()
            expk = oracle.block_score_keys(w.logits, w.row_ks, w.row_ke, B, 1, pin_newest=pin,
                                           nthreads=HOST_THREADS)
            assert np.array_equal(codes.view(torch.int32).cpu().numpy().view(np.uint32), expk), (
                w.name, pin)


def test_random_many_rows():
    """Random shapes around the block scores' plan thresholds (1024 rows,
    32K columns): scores and ids of every row bit-exact, B from 1 to 300,
    row_repeat 1-3, k up to 100, windows empty, ragged, clipped or whole."""
    rng = np.random.default_rng(777)
    for case in range(40):
        rows = int(rng.choice([int(rng.integers(1, 200)), int(rng.integers(1000, 1100))]))
        width = int(rng.integers(1, 40000))
        B = int(rng.choice([1, 3, 4, 7, 8, 16, 32, 64, 128, 300]))
        if -(-width // B) > 4096:
            B = 64
        R = int(rng.integers(1, 4))
        k = int(rng.choice([1, 8, 16, 32, 33, 64, 65, 100]))
        w = workloads.many_rows_case(10_000 + case, rows, width, B, R, k)
        got, sc = gpu_select(w)
        exp_out, exp_sc = oracle_select(w)
        assert_same(got, sc, exp_out, exp_sc, f"case {case} {w.name} k={k}")
        pin = bool(case % 2)
        x = dev_logits(w.logits)
        gs = dsa.block_scores(x, dev_i32(w.row_ks), dev_i32(w.row_ke), B, R,
                              pin_newest=pin).cpu().numpy()
        es = oracle.block_scores(w.logits, w.row_ks, w.row_ke, B, R, pin_newest=pin, nthreads=8)
        assert_same(np.zeros(1), gs, np.zeros(1), es, f"block scores case {case} {w.name}")


def test_split_plan_long_rows():
    """The split plan on rows of 20K-300K columns, where its key-streaming
    kernel meets whole tiles inside the window and rolls its loads across
    rounds: ids and scores bit-exact for assorted chunk sizes."""
    rng = np.random.default_rng(4242)
    for case in range(12):
        rows = int(rng.integers(1, 300))
        width = int(rng.integers(20000, 300000))
        B = int(rng.choice([7, 16, 64, 128]))
        if -(-width // B) > 4096:
            B = 128 if -(-width // 128) <= 4096 else 256
        R = int(rng.integers(1, 4))
        k = int(rng.choice([1, 16, 32, 64, 65]))
        w = workloads.many_rows_case(300_000 + case, rows, width, B, R, k)
        cb = int(rng.choice([0, 32, 64, 256, 1000]))
        got, sc = gpu_select(w, plan=2, cb=cb)
        exp_out, exp_sc = oracle_select(w)
        assert_same(got, sc, exp_out, exp_sc, f"case {case} {w.name} cb={cb}")


# ---------------------------------------------------------------- configs ---

@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_config_full(cfg):
    w = workloads.config(cfg)
    _say("config", cfg, w.name, "plan", dsa.select_plan(w.rows, w.width, w.block_size,
                                                          w.topk_blocks))
    exp_out, exp_sc = oracle_select(w)
    got, sc = gpu_select(w)
    assert_same(got, sc, exp_out, exp_sc, w.name)
    # the other plans give the same bits
    auto = dsa.select_plan(w.rows, w.width, w.block_size, w.topk_blocks)[0]
    for plan in sorted({1, 2, 3} - {auto}):
        got2, sc2 = gpu_select(w, plan=plan)
        assert_same(got2, sc2, exp_out, exp_sc, f"{w.name} plan {plan}")
    if w.rows <= 256:
        for cb in range(6):   # pair plan: parts on one XCD and spread over XCDs
            got2, sc2 = gpu_select(w, plan=4, cb=cb)
            assert_same(got2, sc2, exp_out, exp_sc, f"{w.name} plan 4 arg {pair_arg(cb):#x}")


def _check_properties(out, nblocks):
    for r in range(out.shape[0]):
        row = out[r]
        ids = row[row >= 0]
        n = len(ids)
        assert (row[n:] == -1).all(), r
        assert len(np.unique(ids)) == n and (ids < nblocks).all(), r


def test_config5_full():
    """Large prefill at full size (2 GiB of logits, heavy ties) in the launch
    plan the benchmark times: ids and fp32 scores of all 8192 rows bit-exact
    against the oracle (run on every host core)."""
    w = workloads.config(5)
    _say("config 5 generated", w.name, "plan", dsa.select_plan(w.rows, w.width, w.block_size,
                                                                 w.topk_blocks))
    got, sc = gpu_select(w)
    exp_out, exp_sc = oracle_select(w)
    assert_same(got, sc, exp_out, exp_sc, "config 5, all rows")
    nb = -(-w.width // w.block_size)
    _check_properties(got, nb)
    # heavy ties: most rows end their selection in a run of equal scores,
    # broken by ascending block id
    s_sel = np.take_along_axis(exp_sc, np.maximum(exp_out, 0), axis=1)
    assert (s_sel[:, -1] == s_sel[:, -2]).mean() > 0.5
    # and the other plans that hold this shape give the same bits
    for plan, cb in ((3, 0), (2, 0)):
        got2, sc2 = gpu_select(w, plan=plan, cb=cb)
        assert_same(got2, sc2, exp_out, exp_sc, f"config 5 plan {plan}")


def _abi_select(w, workspace, ws_bytes, scores=False):
    """dsa_select_candidate_blocks (the automatic-plan entry point) called
    through ctypes with a caller-owned workspace, on the current stream."""
    import ctypes
    x = dev_logits(w.logits)
    ks, ke = dev_i32(w.row_ks), dev_i32(w.row_ke)
    nb = -(-w.width // w.block_size)
    out = torch.full((w.rows, w.topk_blocks), 12345, dtype=torch.int32, device=DEV)
    sc = torch.full((w.rows, nb), 777.0, dtype=torch.float32, device=DEV) if scores else None
    code = dsa.lib().dsa_select_candidate_blocks(
        x.data_ptr(), w.rows, w.width, x.stride(0), None if ks is None else ks.data_ptr(),
        ke.data_ptr(), w.topk_blocks, w.block_size, w.row_repeat, out.data_ptr(), w.topk_blocks,
        None if sc is None else sc.data_ptr(), nb if scores else 0, workspace, ws_bytes,
        ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))
    assert code == 0, dsa.status_string(code)
    torch.cuda.synchronize()
    return out.cpu().numpy(), None if sc is None else sc.cpu().numpy()


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_exported_entry_point(cfg):
    """The exported dsa_select_candidate_blocks itself (page:
    select_candidate_blocks, non-DCP branch), not the plan variant: with a
    zeroed caller workspace (configs 2 and 4 run the pair plan, which uses
    it, over several calls), and with none (the automatic plan then falls
    back to one that needs none)."""
    w = workloads.config(cfg)
    exp_out, exp_sc = oracle_select(w)
    need = dsa.select_workspace_bytes(w.rows, w.width, w.block_size, w.topk_blocks)
    ws = torch.zeros(need + 256, dtype=torch.uint8, device=DEV)
    base = (ws.data_ptr() + 127) // 128 * 128
    for i in range(3):
        got, sc = _abi_select(w, base, need, scores=(i == 0))
        assert_same(got, sc, exp_out, exp_sc if i == 0 else None, f"{w.name} call {i}")
    assert int(ws[base - ws.data_ptr():base - ws.data_ptr() + 2048].count_nonzero()) == 0
    got, sc = _abi_select(w, None, 0, scores=True)
    assert_same(got, sc, exp_out, exp_sc, f"{w.name} without workspace")


# ------------------------------------------------------------ behaviour ----

def test_degenerate_shapes():
    out = torch.full((3, 4), 7, dtype=torch.int32, device=DEV)
    ke = torch.zeros(3, dtype=torch.int32, device=DEV)
    dsa.select_candidate_blocks(torch.empty((3, 0), device=DEV), None, ke, 4, 8, out)
    torch.cuda.synchronize()
    assert (out == -1).all()                       # width == 0 -> -1
    out.fill_(7)
    dsa.select_candidate_blocks(torch.empty((0, 10), device=DEV), None, ke, 4, 8, out[:0])
    dsa.select_candidate_blocks(torch.ones((3, 10), device=DEV), None, ke + 10, 0, 8, out[:, :0])
    torch.cuda.synchronize()
    assert (out == 7).all()                        # rows == 0 / topk == 0 write nothing


def test_errors_write_nothing():
    x = torch.ones((4, 64), device=DEV)
    ke = torch.full((4,), 64, dtype=torch.int32, device=DEV)
    out = torch.full((4, 4), 7, dtype=torch.int32, device=DEV)
    for kwargs in (dict(block_size=0), dict(row_repeat=0)):
        args = dict(block_size=8, row_repeat=1)
        args.update(kwargs)
        with pytest.raises(dsa.DsaError) as e:
            dsa.select_candidate_blocks(x, None, ke, 4, args["block_size"], out, args["row_repeat"])
        assert e.value.code == 1
    with pytest.raises(dsa.DsaError) as e:
        dsa.select_candidate_blocks(x, None, ke, 5, 8, out)   # ld_out < topk
    assert e.value.code == 1
    big = torch.ones((1, 1 << 16), device=DEV)
    outb = torch.full((1, 8200), 7, dtype=torch.int32, device=DEV)
    with pytest.raises(dsa.DsaError) as e:  # 16384 keys past LDS: only the split plan holds them
        dsa.select_candidate_blocks(big, None, ke[:1], 4, 4, outb, plan=1)
    assert e.value.code == 2
    with pytest.raises(dsa.DsaError) as e:  # k = 8200: the select state alone exceeds LDS
        dsa.select_candidate_blocks(big, None, ke[:1], 8200, 4, outb)
    assert e.value.code == 2
    ws = dsa.Workspace(DEV, 64)
    lib = dsa.lib()
    code = lib.dsa_select_candidate_blocks_plan(x.data_ptr(), 4, 64, 64, None, ke.data_ptr(), 4, 8,
                                                1, out.data_ptr(), 4, None, 0, ws.buf.data_ptr(),
                                                64, 2, 0, torch.cuda.current_stream().cuda_stream)
    assert code == 3   # the split plan needs 4 * 8 keys * 4 bytes
    torch.cuda.synchronize()
    assert (out == 7).all() and (outb == 7).all()


def test_repeat_calls_bit_identical():
    w = workloads.config(2)
    x = dev_logits(w.logits)
    ks, ke = dev_i32(w.row_ks), dev_i32(w.row_ke)
    ws = dsa.Workspace(DEV)
    first = None
    for plan, cb in ((2, 0), (2, 4), (1, 0), (1, 16), (3, 0), (3, 16), (4, 0), (4, 8 | 4 << 8),
                     (4, 1 << 16)):
        for _ in range(50):
            out = torch.empty((w.rows, w.topk_blocks), dtype=torch.int32, device=DEV)
            dsa.select_candidate_blocks(x, ks, ke, w.topk_blocks, w.block_size, out, w.row_repeat,
                                        workspace=ws, plan=plan, plan_arg=cb)
            o = out.cpu().numpy()
            if first is None:
                first = o
            assert np.array_equal(o, first)
    exp_out, _ = oracle_select(w)
    assert np.array_equal(first, exp_out)


def test_pair_plan_leaves_counters_zero():
    """The pair plan's per-row arrival counters (the workspace's first 2048
    bytes) are zero after every completed call, whatever the part count,
    the XCD dealing (spread) or the row lengths, so the next call starts
    clean; results stay identical over repeated calls."""
    rng = np.random.default_rng(11)
    for rows, width, B, k in ((64, 32768, 64, 32), (128, 40000, 128, 16), (256, 5000, 8, 40),
                              (5, 70000, 64, 3)):
        x = rng.standard_normal((rows, width)).astype(np.float32)
        ke = rng.integers(-3, width + 3, size=rows).astype(np.int32)
        w = workloads.Workload(f"pair-{rows}x{width}", x, None, ke, B, k, 1)
        exp_out, _ = oracle_select(w)
        xd, ked = dev_logits(x), dev_i32(ke)
        ws = dsa.Workspace(DEV, dsa.select_workspace_bytes(rows, width, B, k))
        for arg in (0, 8 | 2 << 8, 4 | 8 << 8, 16 | 3 << 8 | 1 << 16, 1 | 32 << 8):
            for _ in range(3):
                out = torch.full((rows, k), 7, dtype=torch.int32, device=DEV)
                dsa.select_candidate_blocks(xd, None, ked, k, B, out, 1, workspace=ws, plan=4,
                                            plan_arg=arg)
                torch.cuda.synchronize()
                assert np.array_equal(out.cpu().numpy(), exp_out), (w.name, hex(arg))
                assert int(ws.buf[:2048].count_nonzero()) == 0, (w.name, hex(arg))


@pytest.mark.parametrize("rows,width,B,k,R,starts", [
    (8, 16384, 64, 32, 1, False), (200, 20000, 64, 32, 1, True), (256, 16384, 64, 64, 2, False),
    (160, 131072, 128, 16, 2, True)])
def test_auto_plan_pair_shapes(rows, width, B, k, R, starts):
    """Shapes the automatic plan gives the pair plan (up to 256 rows of 16K
    columns or more): run through the default plan with a workspace, every
    row's ids and scores as the oracle's."""
    assert dsa.select_plan(rows, width, B, k)[0] == 4
    rng = np.random.default_rng(rows + width)
    x = rng.standard_normal((rows, width)).astype(np.float32)
    x[rng.random((rows, width)) < 1e-3] = -np.inf
    groups = -(-rows // R)
    ks = rng.integers(-B, width // 3, size=groups).astype(np.int32) if starts else None
    ke = ((ks if starts else 0) + rng.integers(-5, width + B, size=groups)).astype(np.int32)
    w = workloads.Workload(f"auto-pair-{rows}x{width}", x, ks, ke, B, k, R)
    exp_out, exp_sc = oracle_select(w)
    xd = dev_logits(x)
    ws = dsa.Workspace(DEV, dsa.select_workspace_bytes(rows, width, B, k))
    out = torch.full((rows, k), 7, dtype=torch.int32, device=DEV)
    nb = -(-width // B)
    sc = torch.full((rows, nb), 777.0, dtype=torch.float32, device=DEV)
    dsa.select_candidate_blocks(xd, dev_i32(ks), dev_i32(ke), k, B, out, R, scores_out=sc,
                                workspace=ws)
    torch.cuda.synchronize()
    assert_same(out.cpu().numpy(), sc.cpu().numpy(), exp_out, exp_sc, w.name)


def test_two_streams_two_workspaces():
    wa, wb = workloads.config(2), workloads.config(4)
    exp_a, _ = oracle_select(wa)
    exp_b, _ = oracle_select(wb)
    xa, xb = dev_logits(wa.logits), dev_logits(wb.logits)
    sa, sb = torch.cuda.Stream(DEV), torch.cuda.Stream(DEV)
    wsa, wsb = dsa.Workspace(DEV), dsa.Workspace(DEV)
    outs_a, outs_b = [], []
    torch.cuda.synchronize()
    for _ in range(20):
        oa = torch.empty((wa.rows, wa.topk_blocks), dtype=torch.int32, device=DEV)
        ob = torch.empty((wb.rows, wb.topk_blocks), dtype=torch.int32, device=DEV)
        with torch.cuda.stream(sa):
            dsa.select_candidate_blocks(xa, None, dev_i32(wa.row_ke), wa.topk_blocks,
                                        wa.block_size, oa, wa.row_repeat, workspace=wsa)
        with torch.cuda.stream(sb):
            dsa.select_candidate_blocks(xb, None, dev_i32(wb.row_ke), wb.topk_blocks,
                                        wb.block_size, ob, wb.row_repeat, workspace=wsb)
        outs_a.append(oa)
        outs_b.append(ob)
    torch.cuda.synchronize()
    for oa, ob in zip(outs_a, outs_b):
        assert np.array_equal(oa.cpu().numpy(), exp_a)
        assert np.array_equal(ob.cpu().numpy(), exp_b)


def test_large_k_and_full_sort():
    rng = np.random.default_rng(3)
    for k, width, B in ((4096, 40000, 8), (300, 20000, 64), (2000, 2000, 1)):
        x = np.round(rng.standard_normal((6, width)).astype(np.float32) * 4) / 4
        ke = rng.integers(0, width + 1, size=6).astype(np.int32)
        w = workloads.Workload(f"k{k}", x, None, ke, B, k, 1)
        for plan in (1, 2, 3, 4):
            got, sc = gpu_select(w, plan, 7)
            exp_out, exp_sc = oracle_select(w)
            assert_same(got, sc, exp_out, exp_sc, f"k={k} plan {plan}")


def test_bounds_by_wave_count_and_k():
    """The candidate bound of the workgroup select for every wave-count
    parity: 64 group maxima (k <= 32), 128 (32 < k <= 64; one maxima row per
    wave for even counts, two for odd counts up to 8) and the radix passes
    (k > 64, and odd counts above 8 with 32 < k <= 64)."""
    rng = np.random.default_rng(17)
    x = np.round(rng.standard_normal((6, 40000)).astype(np.float32) * 8) / 8
    x[0] = np.abs(x[0]) + 2.0          # same sign and exponent range: clustered keys
    x[1, ::5] = -np.inf
    ke = np.array([40000, 39000, 30000, 20000, 9000, 4500], np.int32)
    for k in (31, 33, 64, 65, 100):
        w = workloads.Workload(f"bounds-k{k}", x, None, ke, 32, k, 1)
        exp_out, exp_sc = oracle_select(w)
        for waves in (1, 2, 3, 5, 7, 8, 9, 12, 15, 16):
            got, sc = gpu_select(w, 1, waves)
            assert_same(got, sc, exp_out, exp_sc, f"k={k} waves={waves}")


def test_all_equal_scores_take_lowest_ids():
    x = np.full((3, 4096), 1.5, np.float32)
    ke = np.array([4096, 100, 4095], np.int32)
    w = workloads.Workload("flat", x, None, ke, 64, 10, 1)
    got, _ = gpu_select(w, 1)
    assert got[0].tolist() == [63] + list(range(9))
    assert got[1].tolist() == [1, 0] + [-1] * 8
    exp_out, _ = oracle_select(w)
    assert np.array_equal(got, exp_out)


@pytest.mark.parametrize("plan", [1, 2, 3, 4])
def test_select_size_boundaries(plan):
    """Rows on each side of the select's size boundaries: the direct rank
    (up to 64 blocks), one to several waves' worth of keys and candidates
    (64, 128, 256, 512, 1024), and, with the heavy ties here, more than 256
    candidates at the bound (the exact fallback); NaN and -inf rows too."""
    rng = np.random.default_rng(99)
    B = 4
    for n in (1, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025, 2000):
        width = n * B
        rows = 6
        x = (rng.integers(0, 6, size=(rows, width)) / 2).astype(np.float32)
        x[1, ::7] = np.nan
        x[2] = -np.inf
        x[3, : width // 2] = -np.inf
        ke = np.full(rows, width, np.int32)
        ke[4] = width - 3
        for k in (1, 16, 64, min(n, 300)):
            w = workloads.Workload(f"n{n}-k{k}", x, None, ke, B, k, 1)
            got, sc = gpu_select(w, plan, 3)
            exp_out, exp_sc = oracle_select(w)
            assert_same(got, sc, exp_out, exp_sc, f"n={n} k={k} plan {plan}")


@pytest.mark.parametrize("plan", [1, 2, 3, 4])
def test_select_bound_paths(plan):
    """Block maxima built around the candidate bound (tests/bound_rows.py:
    maxima packed within 2^16 codes, a band that overflows a 16-bit bound
    into the exact fallback, ties, N(0, 1)) for k with 128 groups (48, 64)
    and with 64 (16, 32), under every plan and an odd and an even wave
    count: ids and scores as the oracle's."""
    B = 4
    for rows, nb in ((8, 1024), (8, 1000), (6, 1500)):
        s = bound_rows(rows, nb, 7 + nb)
        x = (np.repeat(s, B, axis=1)
             - np.tile(np.arange(B, dtype=np.float32), nb)).astype(np.float32)   # block max = s
        ke = np.full(rows, nb * B, np.int32)
        ke[1] = nb * B - 5
        for k in (64, 48, 32, 16):   # 128 groups, then 64
            w = workloads.Workload(f"bound-{rows}x{nb}-k{k}", x, None, ke, B, k, 1)
            exp_out, exp_sc = oracle_select(w)
            for cb in (3, 4):
                got, sc = gpu_select(w, plan, cb)
                assert_same(got, sc, exp_out, exp_sc, f"nb={nb} k={k} plan {plan} arg {cb}")


@pytest.mark.parametrize("plan", [1, 2, 3, 4])
def test_candidate_counts_around_one_wave(plan):
    """Rows whose candidate count at the 64-group bound (k <= 32) is set
    exactly (tests/bound_rows.py: counted_rows): 17 to 133 candidates,
    straddling the 64 that one wave ranks per pass (up to 64 candidates the
    workgroup selects of up to 8 waves split the rank over their waves),
    with tied scores among them; every plan, 2-9 waves for the group plan,
    assorted waves and parts for the pair plan."""
    B, nb = 4, 512
    for k, extras in ((32, (0, 1, 30, 31, 32, 33, 60, 100)),
                      (16, (0, 1, 40, 46, 47, 48, 49, 64)),
                      (24, (0, 30, 31, 32, 33, 39, 40))):
        s = counted_rows(nb, k, extras, 40 + k)
        x = (np.repeat(s, B, axis=1)
             - np.tile(np.arange(B, dtype=np.float32), nb)).astype(np.float32)   # block max = s
        ke = np.full(len(extras), nb * B, np.int32)
        w = workloads.Workload(f"counted-k{k}", x, None, ke, B, k, 1)
        exp_out, exp_sc = oracle_select(w)
        for cb in {1: (2, 3, 4, 8, 9), 4: (0, 1, 2, 4, 6, 8)}.get(plan, (0, 3)):
            got, sc = gpu_select(w, plan, cb)
            assert_same(got, sc, exp_out, exp_sc, f"k={k} plan {plan} arg {cb}")


@pytest.mark.parametrize("plan", [1, 2, 3, 4])
def test_select_at_lds_limit(plan):
    """The largest row the LDS holds: 15312 blocks (15312 keys + 48 control
    words + 1024 words of select area = 16384 words = 64 KiB); one block more
    takes the split plan's select from the workspace (test_rows_past_lds)."""
    rng = np.random.default_rng(plan)
    nb, B, rows = 15312, 4, 3
    width = nb * B
    x = (np.rint(rng.standard_normal((rows, width)) * 8) / 8).astype(np.float32)
    x[0, ::1000] = np.nan
    ke = np.array([width, width // 3, 17], np.int32)
    for k in (3, 200):
        w = workloads.Workload(f"lds-limit-k{k}", x, None, ke, B, k, 1)
        got, sc = gpu_select(w, plan, {2: 1000, 4: 3}.get(plan, 0))
        exp_out, exp_sc = oracle_select(w)
        assert_same(got, sc, exp_out, exp_sc, f"lds limit k={k} plan {plan}")


@pytest.mark.parametrize("plan", [0, 2])
def test_rows_past_lds(plan):
    """Rows whose keys exceed LDS (the split plan, its select reading the
    keys from the workspace): one block past the limit, 65536 blocks, and
    token-level blocks (B = 1, 131072 columns, k = 2048); bounds by group
    maxima, by radix and the exact fallback (k > 256, all-equal rows), ties,
    NaN, windows with and without starts; ids and scores against the
    oracle.  Then the allocation-free entry point on the same rows."""
    rng = np.random.default_rng(60 + plan)
    cases = [(6, 15313 * 4, 4, (3, 64, 200, 300)), (4, 1 << 20, 16, (32, 64)),
             (2, 131072, 1, (2048,))]
    for rows, width, B, ks_k in cases:
        x = (np.rint(rng.standard_normal((rows, width)) * 8) / 8).astype(np.float32)
        x[0, ::997] = np.nan
        x[rows - 1] = np.float32(0.5)  # all equal: the bound admits every block
        R = 2
        g = rows // R
        starts = [None, rng.integers(0, width // 8, size=g).astype(np.int32)]
        for j, ks in enumerate(starts):
            base = np.zeros(g, np.int64) if ks is None else ks.astype(np.int64)
            ke = np.minimum(base + rng.integers(width // 2, width + 1, size=g),
                            width + 3).astype(np.int32)
            for k in ks_k:
                w = workloads.Workload(f"past-lds-{width}-{B}-k{k}", x, ks, ke, B, k, R)
                _say(f"rows past LDS: {rows} x {width}, B {B}, k {k}, starts {j}, plan {plan}")
                got, sc = gpu_select(w, plan, 0 if plan == 0 else 1 + j * 999)
                exp_out, exp_sc = oracle_select(w)
                assert_same(got, sc, exp_out, exp_sc, f"past LDS {w.describe()} plan {plan}")
        if plan == 0:
            w = workloads.Workload(f"past-lds-noalloc-{width}", x, None, ke, B, ks_k[0], R)
            o = torch.full((rows, ks_k[0]), 12345, dtype=torch.int32, device=DEV)
            dsa.select_candidate_blocks_noalloc(torch.from_numpy(x).to(DEV), None, dev_i32(ke),
                                                ks_k[0], B, o, R)
            torch.cuda.synchronize()
            assert np.array_equal(o.cpu().numpy(), oracle_select(w)[0])


def test_random_shapes_past_lds():
    """48 random shapes whose rows exceed LDS: B 1-16, up to 200,000 columns,
    k from 0 to 2048 (both sides of the 256-word candidate store), ties,
    all-equal rows, NaN, -inf, windows with starts, unaligned rows, the
    automatic plan and the split plan with assorted chunks."""
    for seed in range(48):
        rng = np.random.default_rng(9000 + seed)
        B = int(rng.choice([1, 2, 3, 4, 8, 16]))
        width = int(rng.integers(15313 * B, max(15313 * B + 1, 200000)))
        rows = int(rng.integers(1, 12))
        k = int(rng.choice([0, 1, 5, 32, 33, 64, 65, 200, 256, 257, 300, 1000, 2048]))
        R = int(rng.integers(1, 4))
        g = -(-rows // R)
        x = rng.standard_normal((rows, width), dtype=np.float32)
        if seed % 4 == 1:
            x = np.rint(x * 4) / 4
        elif seed % 4 == 2:
            x = np.rint(x * 64) / 64
        elif seed % 4 == 3:
            x[:] = np.float32(0.25)
        if seed % 5 == 0:
            x[rng.random((rows, width)) < 1e-4] = np.nan
        if seed % 7 == 0:
            x[rng.random((rows, width)) < 0.3] = -np.inf
        x = x.astype(np.float32)
        ks = None if seed % 2 else rng.integers(-3, width // 8, size=g).astype(np.int32)
        base = np.zeros(g, np.int64) if ks is None else ks.astype(np.int64)
        ke = np.clip(base + rng.integers(-5, width + 20, size=g), -3, width + 9).astype(np.int32)
        plan = (0, 0, 2)[seed % 3]
        w = workloads.Workload(f"past-lds-random-{seed}", x, ks, ke, B, k, R)
        got, sc = gpu_select(w, plan, (0, 1, 64, 5000)[seed % 4] if plan == 2 else 0,
                             ld_pad=(0, 4, 1)[seed % 3], offset=(0, 0, 1, 4)[seed % 4],
                             ld_out_pad=2)
        exp_out, exp_sc = oracle_select(w)
        assert_same(got, sc, exp_out, exp_sc, f"seed {seed} plan {plan} {w.describe()}")


def test_rows_past_4_gib():
    """Row offsets past 2^32 bytes: 72 rows 64 MB apart (4.6 GB of logits,
    NaN after each row's first 6000 columns), so the last rows start beyond
    4 GiB.  Every plan on an aligned base (16-byte loads) and an unaligned
    one (scalar loads), against the oracle on every row; then the block
    scores, the selection from scores and from codes (the rows' first 1000
    columns) and the mask on the same rows, the mask leaving the NaN gaps
    between the rows untouched."""
    rng = np.random.default_rng(44)
    rows, width, B, k, R = 72, 6000, 64, 24, 2
    ld = 16_000_000
    assert (rows - 3) * ld * 4 > 2 ** 32
    groups = rows // R
    x = (np.rint(rng.standard_normal((rows, width)) * 4) / 4).astype(np.float32)
    x[rng.random((rows, width)) < 1e-3] = np.nan
    ks = np.where(np.arange(groups) % 3 == 0, 0,
                  rng.integers(-5, width // 2, size=groups)).astype(np.int32)
    ke = np.clip(ks + rng.integers(-10, width + 40, size=groups), -3, width + 9).astype(np.int32)
    w = workloads.Workload("past-4gib", x, ks, ke, B, k, R)
    exp_out, exp_sc = oracle_select(w)
    for offset in (0, 1):
        for plan in (1, 2, 3, 4):
            _say(f"rows past 4 GiB: base offset {offset}, plan {plan}")
            got, sc = gpu_select(w, plan, 0, ld_pad=ld - width, offset=offset)
            assert_same(got, sc, exp_out, exp_sc, f"past 4 GiB offset {offset} plan {plan}")
    _say("rows past 4 GiB: block scores")
    xd = dev_logits(x, ld - width)
    got = dsa.block_scores(xd, dev_i32(ks), dev_i32(ke), B, R, pin_newest=True)
    exp = oracle.block_scores(x, ks, ke, B, R, pin_newest=True, nthreads=HOST_THREADS)
    assert np.array_equal(got.cpu().numpy().view(np.uint32), exp.view(np.uint32))
    _say("rows past 4 GiB: select from scores, from keys")
    nscore, gB = 1000, 64  # the rows' first 1000 columns as reduced scores / raw codes
    gke = (ke.astype(np.int64) * 10).astype(np.int32)
    for keys in (False, True):
        o = torch.full((rows, k), 12345, dtype=torch.int32, device=DEV)
        e = np.empty((rows, k), np.int32)
        if keys:
            dsa.select_from_keys(xd[:, :nscore].view(torch.int32), dev_i32(gke), k, gB, nscore,
                                 o, R)
            oracle.select_from_keys(np.ascontiguousarray(x[:, :nscore]).view(np.uint32), gke, k,
                                    gB, nscore, e, R)
        else:
            dsa.select_from_scores(xd[:, :nscore], dev_i32(gke), k, gB, nscore, o, R)
            oracle.select_from_scores(np.ascontiguousarray(x[:, :nscore]), gke, k, gB, nscore,
                                      e, R)
        torch.cuda.synchronize()
        assert np.array_equal(o.cpu().numpy(), e), f"select from {'keys' if keys else 'scores'}"
    _say("rows past 4 GiB: mask")
    dsa.mask_candidates(xd, dev_i32(ks), dev_i32(ke), torch.from_numpy(exp_out).to(DEV),
                        k, B, R)
    torch.cuda.synchronize()
    exp_m = x.copy()
    oracle.mask_candidates(exp_m, ks, ke, exp_out, k, B, R)
    assert np.array_equal(xd.cpu().numpy().view(np.uint32), exp_m.view(np.uint32))
    gaps = xd.as_strided((rows, ld - width), (ld, 1), xd.storage_offset() + width)
    assert bool(torch.isnan(gaps).all())


def test_more_rows_than_one_grid():
    """More work items than one launch's grid (2^20 workgroups): the kernels
    stride over the rest.  1.1M short rows, grouped 3 to a bound."""
    rng = np.random.default_rng(5)
    rows, width, B, k, R = 1_100_000, 16, 4, 2, 3
    x = rng.integers(-8, 8, size=(rows, width)).astype(np.float32)
    groups = -(-rows // R)
    ke = rng.integers(0, width + 1, size=groups).astype(np.int32)
    w = workloads.Workload("many-rows", x, None, ke, B, k, R)
    exp_out, exp_sc = oracle_select(w)
    for plan in (1, 3):
        got, sc = gpu_select(w, plan)
        assert_same(got, sc, exp_out, exp_sc, f"many rows plan {plan}")
