"""MI355X (gfx950) candidate-block selection for a DeepSeek-style sparse-attention indexer.

The work runs in ``libdsa.so`` (hand-written HIP kernels behind the C ABI of
include/dsa.h); this package is its Python binding.  Build the library with
``python -m sparse_attention_kv_dsa_amd.build``.

    select_candidate_blocks(logits, row_ks, row_ke, topk_blocks, block_size, out, row_repeat=1)
    select_candidate_blocks_noalloc(...)    # the same with no workspace and no allocation
    block_scores(logits, row_ks, row_ke, block_size, row_repeat=1, pin_newest=True)
    block_score_keys(...)                   # the same scores as order-preserving uint32 codes
    select_from_scores(scores, global_row_ke, topk_blocks, global_block_size,
                       max_global_blocks, out, row_repeat=1)      # DCP, after the reduce
    select_from_keys(keys, ...)             # the same, after an integer-maximum reduce of codes
    mask_candidates(logits, row_ks, row_ke, candidates, topk_blocks, block_size, row_repeat=1)
    correct_attn_out(out, lses, cp_rank) -> (new_output, lse)    # base-2 LSE merge
"""
from ._binding import (  # noqa: F401
    DsaError,
    Workspace,
    block_score_keys,
    block_scores,
    correct_attn_out,
    lib,
    mask_candidates,
    select_candidate_blocks,
    select_candidate_blocks_noalloc,
    select_from_keys,
    select_from_scores,
    select_plan,
    select_workspace_bytes,
    status_string,
)
