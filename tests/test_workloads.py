"""The seeded synthetic inputs follow their stated recipes and are reproducible."""
import numpy as np

from sparse_attention_kv_dsa_amd import workloads


def test_tiny_recipe():
    w = workloads.tiny()
    assert w.logits.shape == (8, 1000) and w.logits.dtype == np.float32
    assert np.isnan(w.logits).sum() == 3
    assert w.row_ks is None and w.row_ke[0] == 0
    assert ((w.row_ke >= 0) & (w.row_ke <= 1000)).all()
    assert (w.block_size, w.topk_blocks, w.row_repeat) == (64, 4, 1)
    assert workloads.sha256(w.logits, w.row_ke) == workloads.sha256(workloads.tiny().logits,
                                                                    workloads.tiny().row_ke)


def test_decode_recipe():
    w = workloads.decode()
    assert w.logits.shape == (64, 32768) and w.row_ke.shape == (32,)
    assert ((w.row_ke >= 1) & (w.row_ke <= 32768)).all()
    assert 1.9 < float(w.logits[:4].std()) < 2.1
    assert (w.block_size, w.topk_blocks, w.row_repeat) == (64, 32, 2)


def test_prefill_bounds():
    # bounds are deterministic; check them without drawing the 256 MiB matrix
    q, i = np.arange(4096) // 1024, np.arange(4096) % 1024
    ks, ke = 4096 * q, 4096 * q + 3072 + i + 1
    assert ks[1024] == 4096 and ke[0] == 3073 and ke[4095] == 12288 + 4096


def test_large_prefill_prefix_rows_are_reproducible():
    a = workloads.large_prefill(rows=8)
    b = workloads.large_prefill(rows=8)
    assert (a.logits.view(np.uint32) == b.logits.view(np.uint32)).all()
    x = a.logits
    assert (np.abs(x) <= 8).all() and (np.rint(x * 16) == x * 16).all()
    assert (np.signbit(x) & (x == 0)).any()          # -0.0 occurs
    assert a.row_ks.tolist() == [0] * 8 and a.row_ke[0] == 28673


def test_random_cases_cover_edge_bounds():
    seen = set()
    for seed in range(300):
        w = workloads.random_case(seed)
        ks = w.row_ks if w.row_ks is not None else np.zeros_like(w.row_ke)
        for s, e in zip(ks, w.row_ke):
            seen.add("empty" if e <= s else "ok")
            if e > w.width:
                seen.add("end_past_width")
            if s < 0:
                seen.add("negative_start")
            if s > w.width:
                seen.add("start_past_width")
    assert {"empty", "ok", "end_past_width", "negative_start", "start_past_width"} <= seen
