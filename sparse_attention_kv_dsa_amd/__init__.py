"""MI355X (gfx950) candidate-block selection for a DeepSeek-style sparse-attention indexer.

The work runs in ``libdsa.so`` (hand-written HIP kernels behind the C ABI of
include/dsa.h); this package is its Python binding.  Build the library with
``python -m sparse_attention_kv_dsa_amd.build``.

    select_candidate_blocks(logits, row_ks, row_ke, topk_blocks, block_size, out, row_repeat=1)
    block_scores(logits, row_ks, row_ke, block_size, row_repeat=1, pin_newest=True)
"""
from ._binding import (  # noqa: F401
    DsaError,
    Workspace,
    block_scores,
    lib,
    select_candidate_blocks,
    select_plan,
    select_workspace_bytes,
    status_string,
)
