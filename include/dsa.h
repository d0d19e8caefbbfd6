/*
 * dsa.h - C ABI of the MI355X (gfx950) candidate-block selector for a
 * DeepSeek-style sparse-attention (DSA) indexer.
 *
 * Source of the operation: the vLLM-fork page
 * "launcher/dcp2/diffs/02-model_executor_kernels_attention_dsa_candidate_blocks.py.diff"
 * (candidate_blocks.py): _max_with_nan, _block_scores_kernel, _block_scores,
 * select_candidate_blocks / _select_candidate_blocks_impl (non-DCP branch;
 * the DCP branch's selection after its reduce; the candidate masking after
 * it), and page 3 (sglang dcp kernels.py) for the log-sum-exp correction.
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
 * Bounds are device data and are not validated; whatever their values, the
 * selection and block-score kernels read logits only inside the row's window
 * [row + max(s, 0), row + min(e, width)), and compute the definition above
 * for any int32 values (the expected use is 0 <= s <= e <= width).
 *
 * Conventions for every entry point:
 *   - The caller owns every buffer.  The library allocates nothing, keeps no
 *     global state and never synchronises: work is enqueued on `stream`.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     error the call returns the code and writes nothing.
 *   - `logits` must be 4-byte aligned; a row whose (logits + r*ld_logits + s)
 *     is 16-byte aligned, with s >= 0 and at least 4 columns in its window,
 *     takes the vectorised path (16-byte loads of whole in-window groups of
 *     4 columns, scalar loads for the last 1-3), any other row a scalar path
 *     with identical results.
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
 * dsa_block_scores with every score written as its order-preserving uint32
 * code instead of fp32: the form in which the local block scores of the
 * page's decode-context-parallel branch (_select_candidate_blocks_impl, DCP
 * branch: unpinned local scores, then an all-reduce MAX over the ranks)
 * reduce exactly by an integer maximum, whatever a collective does with
 * floats.  The code of a score x:
 *   x NaN (any sign or payload)   -> 0xFFC00000 (the code of 0x7FC00000);
 *   sign bit of x clear (+0, ...)  -> bits(x) | 0x80000000;
 *   sign bit of x set (-0, ...)    -> ~bits(x).
 * Unsigned order of codes is the order of the IEEE-754-2019 maximum the
 * scores use (NaN above +inf, +0 above -0), so max(code(a), code(b)) ==
 * code(maximum(a, b)).  -inf (a block with no element) is 0x007FFFFF, a
 * pinned block 0xFF800000.
 *
 *   keys     uint32 [rows, ld_keys], ld_keys >= nblocks; every b < nblocks of
 *            every row is written.
 * Arguments, early exits and errors as dsa_block_scores.
 */
dsa_status_t dsa_block_score_keys(const float* logits, int64_t rows, int64_t width,
                                  int64_t ld_logits, const int32_t* row_ks,
                                  const int32_t* row_ke, int32_t block_size,
                                  int32_t row_repeat, int32_t pin_newest, uint32_t* keys,
                                  int64_t ld_keys, hipStream_t stream);

/*
 * Bytes of device workspace the split and pair plans of
 * dsa_select_candidate_blocks need for this shape: 2048 bytes of per-row
 * arrival counters (pair plan, up to 256 rows), then one uint32 score key
 * per row and block, rows padded to 32 keys.  Enough for every plan.  Pure
 * host arithmetic; returns 0 for invalid or empty shapes and for shapes no
 * plan holds (see Unsupported under dsa_select_candidate_blocks).
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
 *   workspace   device scratch for the split and pair plans (long rows):
 *               at least dsa_select_workspace_bytes(...) bytes, 128-byte
 *               aligned.  Its first 2048 bytes (the pair plan's arrival
 *               counters) must be zero before the first call that uses it,
 *               e.g. one hipMemset after allocation; every call that
 *               completes leaves them zero again, and no other plan writes
 *               them.  The rest needs no initialisation.  Other plans do
 *               not touch the workspace.  When the automatic plan (what
 *               dsa_select_plan names) needs one and none is given (NULL,
 *               too small or misaligned), the call runs the group plan
 *               instead.  Calls that may run concurrently need separate
 *               workspaces.
 *
 * rows == 0 or topk_blocks == 0: DSA_OK, nothing written.
 * width == 0: out[r][j] = -1 for j < topk_blocks (page: the early exit of
 *   _select_candidate_blocks_impl for an empty width); logits/row_ke may
 *   then be NULL.
 * Invalid: negative sizes, block_size < 1, row_repeat < 1, topk_blocks < 0,
 *   ld_logits < width, ld_out < topk_blocks, ld_scores < nblocks when
 *   scores_out is given, null logits/row_ke/out when there is work,
 *   misaligned pointers.
 * Rows past LDS: when 4 * (roundup4(nblocks) + 48 + roundup4(max(1024,
 *   2*kcap))) > 65536, with kcap = max(1, min(topk_blocks, nblocks)) (a
 *   row's keys and select state exceed one workgroup's 64 KiB of LDS), only
 *   the split plan holds the rows: its select reads the keys from the
 *   workspace instead of LDS (every pass over the keys reads HBM or L2, so
 *   these rows select slower than rows held in LDS).  The automatic plan
 *   takes it, and returns DSA_ERR_WORKSPACE when the workspace is missing
 *   or too small.
 * Unsupported: 4 * (48 + roundup4(max(1024, 2*kcap))) > 65536 (the select
 *   state alone exceeds LDS, topk_blocks above 8168), rows past LDS under a
 *   plan other than the split plan, more than 2^31 - 1 rows or
 *   2^31 - 8193 blocks, or a workspace size past size_t.
 */
dsa_status_t dsa_select_candidate_blocks(const float* logits, int64_t rows, int64_t width,
                                         int64_t ld_logits, const int32_t* row_ks,
                                         const int32_t* row_ke, int32_t topk_blocks,
                                         int32_t block_size, int32_t row_repeat,
                                         int32_t* out, int64_t ld_out, float* scores_out,
                                         int64_t ld_scores, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/* Bytes of the static device scratch of dsa_select_candidate_blocks_noalloc
 * (per GPU, held until the process ends). */
#define DSA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * dsa_select_candidate_blocks for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no workspace argument.  The split and pair plans use instead a
 * static device array of DSA_NOALLOC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends; this call allocates nothing
 * (no hipMalloc, no allocating library routine).  Its first call on a device
 * takes the array's address there (hipGetSymbolAddress) and enqueues a small
 * kernel on `stream` that clears the pair plan's arrival counters; calls
 * that complete leave them zero.
 *
 * Results are those of dsa_select_candidate_blocks (the same automatic plan).
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (other streams, other threads) race and must not be issued
 * concurrently; calls on different GPUs are independent.
 *
 * DSA_ERR_WORKSPACE: the automatic plan of this shape needs more scratch
 *   than DSA_NOALLOC_SCRATCH_BYTES (dsa_select_workspace_bytes(...) bytes);
 *   nothing is written.  Shapes whose plan needs no scratch always run.
 * DSA_ERR_HIP: also when the device or the array's address cannot be
 *   obtained.  Other arguments, early exits and errors as
 *   dsa_select_candidate_blocks.
 */
dsa_status_t dsa_select_candidate_blocks_noalloc(const float* logits, int64_t rows,
                                                 int64_t width, int64_t ld_logits,
                                                 const int32_t* row_ks, const int32_t* row_ke,
                                                 int32_t topk_blocks, int32_t block_size,
                                                 int32_t row_repeat, int32_t* out, int64_t ld_out,
                                                 float* scores_out, int64_t ld_scores,
                                                 hipStream_t stream);

/*
 * dsa_select_candidate_blocks with an explicit launch plan, for tests and
 * tuning.  Results are identical for every plan.
 *   plan          0: automatic (what dsa_select_candidate_blocks uses);
 *                 1: one workgroup per row (its waves stream the row, then
 *                    select it together);
 *                 2: split: a first kernel streams chunks of `plan_arg`
 *                    blocks of every row on many CUs into the workspace as
 *                    keys, a second kernel selects, one workgroup per row
 *                    (reading the keys into LDS, or, for rows past LDS,
 *                    straight from the workspace);
 *                 3: one wave per row (stream and select), several rows per
 *                    workgroup;
 *                 4: pair: several workgroups share a row, each streaming a
 *                    range of its blocks and publishing its keys in the
 *                    workspace; the last to arrive (per-row atomic counter)
 *                    gathers the rest and selects.  The ranges have a fixed
 *                    size, ceil(nblocks / parts) rounded up to 32 blocks, so
 *                    a shorter row uses fewer of its workgroups.  A row's
 *                    workgroups are dealt to one XCD so that the keys pass
 *                    through its L2; a part that ran on another XCD is
 *                    streamed again by the selecting workgroup.  At most
 *                    256 rows.
 *   plan_arg      plan 1: waves per workgroup, 1..16 (0: 4);
 *                 plan 2: blocks per chunk, >= 1 (0: automatic);
 *                 plan 3: float4 loads in flight per lane, 8 or 16 (0: 8);
 *                 plan 4: waves | parts << 8 | spread << 16: waves per
 *                    workgroup 0..16 and workgroups per row 0..255 (0:
 *                    automatic; 1 selects each row in one workgroup);
 *                    spread 1 deals a row's workgroups to different XCDs
 *                    (for tests of the fallback).
 */
dsa_status_t dsa_select_candidate_blocks_plan(
    const float* logits, int64_t rows, int64_t width, int64_t ld_logits,
    const int32_t* row_ks, const int32_t* row_ke, int32_t topk_blocks, int32_t block_size,
    int32_t row_repeat, int32_t* out, int64_t ld_out, float* scores_out, int64_t ld_scores,
    void* workspace, size_t workspace_bytes, int32_t plan, int32_t plan_arg,
    hipStream_t stream);

/* The automatic plan for a shape: *plan = 1, 2, 3 or 4 and its *plan_arg. */
dsa_status_t dsa_select_plan(int64_t rows, int64_t width, int32_t block_size,
                             int32_t topk_blocks, int32_t* plan, int32_t* plan_arg);

/* Static string naming a status code ("DSA_OK", ...); "unknown" for any
 * other int value. */
const char* dsa_status_string(int status);

/*
 * Selection from a reduced block-score matrix: the part of the page's
 * decode-context-parallel (DCP) branch of _select_candidate_blocks_impl that
 * follows its all-reduce.  There each rank scores its share of the columns
 * (token t on rank t mod W) at the local block size B/W with the pin off
 * (dsa_block_scores with pin_newest = 0), the element-wise maximum over the
 * ranks gives the global block scores, and every rank then calls this with
 * the global bounds so that all ranks pin and select alike.
 *
 *   scores      fp32 [rows, ld_scores]: the first nscore columns are block
 *               scores; nblocks = max(max_global_blocks, 1); columns
 *               >= min(nscore, nblocks) count as -inf, columns >= nblocks are
 *               ignored.  May be NULL when nscore == 0.
 *   global_row_ke  int32 device array, e = global_row_ke[r / row_repeat]:
 *               the row's global context length.
 *   pin         block min(floor((e - 1) / global_block_size), nblocks - 1)
 *               scores +inf; rows with e <= 0 select nothing (all -1).
 *   out         int32 [rows, ld_out]: the ranking and -1 padding of
 *               dsa_select_candidate_blocks, k' = min(topk_blocks, nblocks).
 *
 * rows == 0 or topk_blocks == 0: DSA_OK, nothing written.
 * Invalid: negative sizes, row_repeat < 1, global_block_size < 1,
 *   ld_scores < nscore (nscore > 0), ld_out < topk_blocks, null or
 *   misaligned pointers when there is work.
 * Unsupported: 4 * (roundup4(nblocks) + 48 + roundup4(max(1024, 2*kcap))) > 65536,
 *   kcap = max(1, min(topk_blocks, nblocks)): a row's scores and select state
 *   must fit in one workgroup's LDS (there is no workspace to hold them).
 */
dsa_status_t dsa_select_from_scores(const float* scores, int64_t rows, int64_t nscore,
                                    int64_t ld_scores, int64_t max_global_blocks,
                                    const int32_t* global_row_ke, int32_t row_repeat,
                                    int32_t global_block_size, int32_t topk_blocks, int32_t* out,
                                    int64_t ld_out, hipStream_t stream);

/*
 * dsa_select_from_scores on a matrix of the uint32 codes that
 * dsa_block_score_keys writes (after the ranks' codes are reduced with an
 * integer maximum): the same pin, e <= 0 rule, ranking and -1 padded output,
 * for the scores the codes stand for.  A code that dsa_block_score_keys
 * never writes (above 0xFF800000 or below 0x007FFFFF: the codes of NaNs with
 * other payloads or signs) stands for NaN, as every NaN does in
 * dsa_select_from_scores.
 *
 *   keys   uint32 [rows, ld_keys], nkeys columns; may be NULL when
 *          nkeys == 0.
 * Arguments, early exits and errors as dsa_select_from_scores (nkeys and
 * ld_keys in the places of nscore and ld_scores).
 */
dsa_status_t dsa_select_from_keys(const uint32_t* keys, int64_t rows, int64_t nkeys,
                                  int64_t ld_keys, int64_t max_global_blocks,
                                  const int32_t* global_row_ke, int32_t row_repeat,
                                  int32_t global_block_size, int32_t topk_blocks, int32_t* out,
                                  int64_t ld_out, hipStream_t stream);

/*
 * Candidate masking of packed logits, in place (page: the masking function
 * after _select_candidate_blocks_impl, documented as masking packed logits
 * outside the causal bounds and outside the request-local candidates; its
 * body is not shown, so this is the plain reading): column c < width of row
 * r keeps its value when s <= c < e and its request-local block (c - s) / B
 * is one of candidates[r][0 .. topk_blocks) (negative entries match
 * nothing); every other column becomes -inf.  Kept columns are not written.
 * Under DCP pass the local block size: local block b is this rank's share of
 * global block b, so the candidate ids apply unchanged.
 *
 *   candidates  int32 [rows, ld_cand], ld_cand >= topk_blocks (the `out` of
 *               a selection); may be NULL when topk_blocks == 0.
 *
 * rows == 0 or width == 0: DSA_OK, nothing written.
 * Invalid: negative sizes, block_size < 1, row_repeat < 1, ld_logits <
 *   width, ld_cand < topk_blocks, null or misaligned pointers when there is
 *   work.  Rows with 16-byte aligned starts and ld_logits % 4 == 0 are
 *   written with 16-byte stores.
 */
dsa_status_t dsa_mask_candidates(float* logits, int64_t rows, int64_t width, int64_t ld_logits,
                                 const int32_t* row_ks, const int32_t* row_ke,
                                 const int32_t* candidates, int64_t ld_cand,
                                 int32_t topk_blocks, int32_t block_size, int32_t row_repeat,
                                 hipStream_t stream);

/*
 * Base-2 log-sum-exp correction of one context-parallel rank's partial
 * attention output (page 3, sglang dcp kernels.py: _correct_attn_cp_out_kernel
 * / correct_attn_out).  For every b < B, h < H, with l_n = lses[n][b][h]:
 *   l_n counts as -inf when it is NaN or +inf; m = max_n l_n (0 if -inf);
 *   final = log2(sum_n 2^(l_n - m)) + m;
 *   d = lses[cp_rank][b][h] - final (raw value), -inf if NaN or +inf;
 *   lse_out[b][h] = final;  new_out[h][b][x] = out[b][h][x] * 2^d, x < D.
 * All tensors fp32, strides in elements (any sign), caller-owned; fp32
 * arithmetic (exp2/log2 of the hardware, see the parity tolerance).
 *
 *   out      [B, H, D] at out + b*out_sb + h*out_sh + x*out_sd
 *   lses     [N, B, H] at lses + n*lse_sn + b*lse_sb + h*lse_sh
 *   new_out  [H, B, D] at new_out + h*new_sh + b*new_sb + x*new_sd
 *   lse_out  [B, H]    at lse_out + b*lse_out_sb + h*lse_out_sh
 *
 * B == 0 or H == 0: DSA_OK, nothing written.
 * Invalid: negative sizes, N < 1, cp_rank outside [0, N), null or
 *   misaligned pointers when there is work (out and new_out may be NULL
 *   when D == 0).  Unit D strides, D % 4 == 0, 16-byte aligned bases and
 *   B/H strides that are multiples of 4 take 16-byte loads and stores.
 */
dsa_status_t dsa_correct_attn_out(const float* out, int64_t B, int64_t H, int64_t D,
                                  int64_t out_sb, int64_t out_sh, int64_t out_sd,
                                  const float* lses, int64_t N, int64_t lse_sn, int64_t lse_sb,
                                  int64_t lse_sh, int64_t cp_rank, float* new_out,
                                  int64_t new_sh, int64_t new_sb, int64_t new_sd, float* lse_out,
                                  int64_t lse_out_sb, int64_t lse_out_sh, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
