/*
 * dsa.h - C ABI of the MI355X (gfx950) candidate-block selector for a
 * DeepSeek-style sparse-attention (DSA) indexer.
 *
 * Source of the operation: the vLLM-fork page
 * "launcher/dcp2/diffs/02-model_executor_kernels_attention_dsa_candidate_blocks.py.diff"
 * (candidate_blocks.py): _max_with_nan, _block_scores_kernel, _block_scores,
 * select_candidate_blocks / _select_candidate_blocks_impl (non-DCP branch).
 *
 * Notation used below.
 *   logits   fp32 [rows, ld_logits] row-major; the first `width` columns of a
 *            row are the packed indexer logits of that row.
 *   R        row_repeat: rows r share the bounds of group g = r / R
 *            (decode rows of one request).
 *   s, e     s = row_ks ? row_ks[g] : 0, e = row_ke[g]: the row's window
 *            [s, e) in packed column space.  row_ks / row_ke are int32
 *            device arrays with at least ceil(rows / R) entries.
 *   B        block_size.  nblocks = ceil(width / B) for every row.
 *   block b  request-local: columns [s + b*B, s + (b+1)*B).  Its elements are
 *            the columns of that range that also lie in [s, e) and [0, width).
 *   score[b] the IEEE-754-2019 maximum of its elements (NaN propagates and
 *            is returned as the canonical quiet NaN 0x7FC00000; -0 < +0);
 *            -inf when the block has no element.
 *   pin      when e > s, block p = (e - s - 1) / B, if p < nblocks, scores
 *            +inf (this overrides NaN).
 *   ranking  NaN first, then larger value first (-0 == +0), then smaller
 *            block id first.
 *   out      out[j] for j < topk_blocks: the j-th ranked block id, or -1 when
 *            j >= min(topk_blocks, nblocks) or that block scores -inf.
 *
 * Bounds are device data and are not validated; the kernels never read
 * outside [row, row + min(e, width)) whatever their values, and compute the
 * definition above for any int32 values (the expected use is 0 <= s <= e <=
 * width).
 *
 * Conventions for every entry point:
 *   - The caller owns every buffer.  The library allocates nothing, keeps no
 *     global state and never synchronises: work is enqueued on `stream`.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     error the call returns the code and writes nothing.
 *   - `logits` must be 4-byte aligned; a row whose (logits + r*ld_logits + s)
 *     is 16-byte aligned takes the vectorised path, any other row a scalar
 *     path with identical results.
 *   - DSA_ERR_HIP: the launch failed (hipGetLastError after the launch).
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dsa_status_t {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* a size, stride, pointer or alignment is invalid */
  DSA_ERR_UNSUPPORTED = 2, /* valid but beyond what the kernels hold (LDS/grid) */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing, misaligned or too small */
  DSA_ERR_HIP = 4          /* the HIP runtime reported an error */
} dsa_status_t;

/*
 * Block scores, with or without the newest-block pin
 * (page: _block_scores / _block_scores_kernel with PIN_NEWEST).
 *
 *   scores   fp32 [rows, ld_scores], ld_scores >= nblocks; every b < nblocks
 *            of every row is written.
 *   pin_newest  0 or 1.
 *
 * rows == 0 or width == 0: DSA_OK, nothing written.
 * Invalid: rows < 0, width < 0, block_size < 1, row_repeat < 1,
 *   ld_logits < width, ld_scores < nblocks, null logits/row_ke/scores when
 *   there is work, logits or scores not 4-byte aligned, pin_newest not 0/1.
 */
dsa_status_t dsa_block_scores(const float* logits, int64_t rows, int64_t width,
                              int64_t ld_logits, const int32_t* row_ks,
                              const int32_t* row_ke, int32_t block_size,
                              int32_t row_repeat, int32_t pin_newest, float* scores,
                              int64_t ld_scores, hipStream_t stream);

/*
 * Bytes of device workspace the split plan of dsa_select_candidate_blocks
 * needs for this shape (one uint32 score key per row and block); enough for
 * every plan.  Pure host arithmetic; returns 0 for invalid or empty shapes.
 */
size_t dsa_select_workspace_bytes(int64_t rows, int64_t width, int32_t block_size,
                                  int32_t topk_blocks);

/*
 * Candidate-block selection: one HBM pass over the in-window logits, block
 * scores kept as order-preserving keys (in LDS; in the workspace under the
 * split plan), pin, top-k, ordered -1 padded store (page:
 * select_candidate_blocks, non-DCP branch; the tie order, score descending
 * then block id ascending, is this library's rule).
 *
 *   out         int32 [rows, ld_out], ld_out >= topk_blocks; columns
 *               [0, topk_blocks) of every row are written.
 *   scores_out  nullable fp32 [rows, ld_scores], ld_scores >= nblocks: the
 *               pinned block scores, for checking; ld_scores is ignored when
 *               scores_out is NULL.
 *   workspace   device scratch for the split plan (few long rows): at least
 *               dsa_select_workspace_bytes(...) bytes, 4-byte aligned,
 *               no initialisation needed.  Other plans do not touch it and
 *               it may then be NULL (dsa_select_plan tells the plan).  Calls
 *               that may run concurrently need separate workspaces.
 *
 * rows == 0 or topk_blocks == 0: DSA_OK, nothing written.
 * width == 0: out[r][j] = -1 for j < topk_blocks (page: the early exit of
 *   _select_candidate_blocks_impl for an empty width); logits/row_ke may
 *   then be NULL.
 * Invalid: negative sizes, block_size < 1, row_repeat < 1, topk_blocks < 0,
 *   ld_logits < width, ld_out < topk_blocks, ld_scores < nblocks when
 *   scores_out is given, null logits/row_ke/out when there is work,
 *   misaligned pointers.
 * Unsupported: 4 * (roundup4(nblocks) + 16 + roundup4(max(512, 2*kcap))) > 65536
 *   with kcap = max(1, min(topk_blocks, nblocks)) (a row's block scores and
 *   select scratch must fit in LDS), or more than 2^31 - 1 rows.
 */
dsa_status_t dsa_select_candidate_blocks(const float* logits, int64_t rows, int64_t width,
                                         int64_t ld_logits, const int32_t* row_ks,
                                         const int32_t* row_ke, int32_t topk_blocks,
                                         int32_t block_size, int32_t row_repeat,
                                         int32_t* out, int64_t ld_out, float* scores_out,
                                         int64_t ld_scores, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * dsa_select_candidate_blocks with an explicit launch plan, for tests and
 * tuning.  Results are identical for every plan.
 *   plan          0: automatic (what dsa_select_candidate_blocks uses);
 *                 1: one workgroup per row (its waves stream the row, one
 *                    wave selects);
 *                 2: split: a first kernel streams chunks of `plan_arg`
 *                    blocks of every row on many CUs into the workspace, a
 *                    second kernel selects, one wave per row;
 *                 3: one wave per row (stream and select), several rows per
 *                    workgroup.
 *   plan_arg      plan 1: waves per workgroup, 1..16 (0: 4);
 *                 plan 2: blocks per chunk, >= 1 (0: automatic);
 *                 plan 3: float4 loads in flight per lane, 8 or 16 (0: 8).
 */
dsa_status_t dsa_select_candidate_blocks_plan(
    const float* logits, int64_t rows, int64_t width, int64_t ld_logits,
    const int32_t* row_ks, const int32_t* row_ke, int32_t topk_blocks, int32_t block_size,
    int32_t row_repeat, int32_t* out, int64_t ld_out, float* scores_out, int64_t ld_scores,
    void* workspace, size_t workspace_bytes, int32_t plan, int32_t plan_arg,
    hipStream_t stream);

/* The automatic plan for a shape: *plan = 1, 2 or 3 and its *plan_arg. */
dsa_status_t dsa_select_plan(int64_t rows, int64_t width, int32_t block_size,
                             int32_t topk_blocks, int32_t* plan, int32_t* plan_arg);

/* Static string naming a status code ("DSA_OK", ...); "unknown" otherwise. */
const char* dsa_status_string(dsa_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
