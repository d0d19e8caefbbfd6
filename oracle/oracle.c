/*
 * CPU oracle for DSA candidate-block selection.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * Source: the vLLM-fork page "dcp2/diffs/02-model_executor_kernels_attention_
 * dsa_candidate_blocks.py.diff" (candidate_blocks.py), functions
 * _max_with_nan, _block_scores_kernel, _block_scores and
 * _select_candidate_blocks_impl (non-DCP branch), and its docstring.
 *
 * Definition (with the readings this project takes where the page is
 * silent; every reading is listed in the design notes):
 *   rows r, packed columns c < width, block size B, row_repeat R.
 *   g = r div R; s = starts ? starts[g] : 0; e = ends[g].
 *   nblocks = ceil(width / B) for every row.
 *   Block b is request-local: columns [s + bB, s + (b+1)B).  Its element set
 *   is C_b = those columns that also lie in [s, e) and in [0, width).
 *   score[b] = IEEE-754-2019 maximum over C_b: -inf when C_b is empty, the
 *   canonical quiet NaN (bits 0x7FC00000) when any element is NaN, else the
 *   largest element where -0 < +0.
 *   Pin: if pin is on and e > s, p = (e - s - 1) div B; if p < nblocks then
 *   score[p] = +inf (this overrides a NaN).
 *   Ranking: NaN first, then by value descending (-0 == +0), ties by block id
 *   ascending.  k' = min(k, nblocks).  out[j] = the j-th ranked block when
 *   j < k' and its score is not -inf, else -1, for j < k.
 *
 * Precision: the method only compares fp32 values and returns one of them,
 * so no rounding occurs anywhere; the oracle compares the fp32 values as
 * they are.
 *
 * Also defined below, each with its source: the selection from a reduced
 * block-score matrix under decode context parallelism (oracle_select_from_
 * scores), the order-preserving uint32 codes of block scores that make that
 * reduce exact on integers (oracle_score_key, oracle_select_from_keys), the
 * candidate masking of packed logits (oracle_mask_candidates) and the
 * base-2 log-sum-exp correction of partial attention outputs
 * (oracle_correct_attn_out, page 3).
 *
 * Parity status: block scores, pin and the ordered select are pinned by the
 * hand-worked rows, the brute-force full sort, the B=1, torch.topk and
 * column-interleave decompositions in tests/.  The NaN placement in the
 * ranking and the -0/+0 tie are fixed by the stated rule only (no page prints
 * an output to compare against).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* 0x7FC00000 as a float, built without type punning tricks. */
static float canonical_nan(void) {
  uint32_t bits = 0x7FC00000u;
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

/* Bounds of row r: g = r div R (rows of a decode group share bounds). */
static void row_bounds(int64_t r, const int32_t* starts, const int32_t* ends,
                       int32_t row_repeat, int64_t* s, int64_t* e) {
  int64_t g = r / row_repeat;
  *s = starts ? (int64_t)starts[g] : 0;
  *e = (int64_t)ends[g];
}

/* Score of block b of one row: the NaN-propagating maximum over C_b. */
static float block_score(const float* row, int64_t width, int64_t s, int64_t e,
                         int64_t block_size, int64_t b) {
  int64_t lo = s + b * block_size;
  int64_t hi = lo + block_size;
  if (lo < s) lo = s;
  if (lo < 0) lo = 0;
  if (hi > e) hi = e;
  if (hi > width) hi = width;
  int have = 0, saw_nan = 0;
  float best = 0.0f;
  for (int64_t c = lo; c < hi; ++c) {
    float x = row[c];
    if (isnan(x)) {
      saw_nan = 1;
    } else if (!have) {
      best = x;
      have = 1;
    } else if (x > best) {
      best = x;
    } else if (x == best && signbit(best) && !signbit(x)) {
      best = x; /* +0 is larger than -0 */
    }
  }
  if (saw_nan) return canonical_nan();
  if (!have) return -INFINITY;
  return best;
}

/* All nblocks scores of row r, with the optional pin of the newest block. */
static void row_scores(const float* logits, int64_t width, int64_t ld,
                       const int32_t* starts, const int32_t* ends,
                       int32_t block_size, int32_t row_repeat, int pin,
                       int64_t r, int64_t nblocks, float* scores) {
  int64_t s, e;
  row_bounds(r, starts, ends, row_repeat, &s, &e);
  const float* row = logits + r * ld;
  for (int64_t b = 0; b < nblocks; ++b)
    scores[b] = block_score(row, width, s, e, block_size, b);
  if (pin && e > s) {
    int64_t p = (e - s - 1) / block_size;
    if (p < nblocks) scores[p] = INFINITY;
  }
}

typedef struct {
  float score;
  int32_t id;
} ranked_t;

/* Ranking order: NaN first; then larger value first (-0 == +0 because the
 * comparison is numeric); then smaller block id first. */
static int rank_cmp(const void* pa, const void* pb) {
  const ranked_t* a = (const ranked_t*)pa;
  const ranked_t* b = (const ranked_t*)pb;
  int na = isnan(a->score) != 0, nb = isnan(b->score) != 0;
  if (na != nb) return na ? -1 : 1;
  if (!na) {
    if (a->score > b->score) return -1;
    if (a->score < b->score) return 1;
  }
  return (a->id > b->id) - (a->id < b->id);
}

typedef struct {
  const float* logits;
  int64_t rows, width, ld;
  const int32_t* starts;
  const int32_t* ends;
  int32_t topk, block_size, row_repeat, pin;
  int32_t* out;
  int64_t ld_out;
  float* scores_out;
  int64_t ld_scores;
  int64_t r0, r1;
  int status;
} job_t;

static void* select_rows(void* arg) {
  job_t* j = (job_t*)arg;
  int64_t nblocks = (j->width + j->block_size - 1) / j->block_size;
  float* scores = (float*)malloc(sizeof(float) * (size_t)(nblocks ? nblocks : 1));
  ranked_t* order = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)(nblocks ? nblocks : 1));
  if (!scores || !order) {
    free(scores);
    free(order);
    j->status = 1;
    return NULL;
  }
  int64_t kk = j->topk < nblocks ? j->topk : nblocks; /* k' = min(k, nblocks) */
  for (int64_t r = j->r0; r < j->r1; ++r) {
    row_scores(j->logits, j->width, j->ld, j->starts, j->ends, j->block_size,
               j->row_repeat, j->pin, r, nblocks, scores);
    if (j->scores_out)
      memcpy(j->scores_out + r * j->ld_scores, scores, sizeof(float) * (size_t)nblocks);
    if (!j->out) continue;
    for (int64_t b = 0; b < nblocks; ++b) {
      order[b].score = scores[b];
      order[b].id = (int32_t)b;
    }
    qsort(order, (size_t)nblocks, sizeof(ranked_t), rank_cmp);
    int32_t* o = j->out + r * j->ld_out;
    for (int64_t q = 0; q < j->topk; ++q) {
      int keep = q < kk && !(isinf(order[q].score) && order[q].score < 0);
      o[q] = keep ? order[q].id : -1;
    }
  }
  free(scores);
  free(order);
  return NULL;
}

static int run_rows(job_t proto, int nthreads) {
  if (nthreads < 1) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  if (nthreads > proto.rows) nthreads = (int)(proto.rows ? proto.rows : 1);
  job_t jobs[256];
  pthread_t tids[256];
  int started[256];
  int64_t per = (proto.rows + nthreads - 1) / nthreads;
  int status = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = proto;
    jobs[t].r0 = t * per < proto.rows ? t * per : proto.rows;
    jobs[t].r1 = (t + 1) * per < proto.rows ? (t + 1) * per : proto.rows;
    jobs[t].status = 0;
    started[t] = nthreads > 1 && pthread_create(&tids[t], NULL, select_rows, &jobs[t]) == 0;
    if (!started[t]) select_rows(&jobs[t]);
  }
  for (int t = 0; t < nthreads; ++t) {
    if (started[t]) pthread_join(tids[t], NULL);
    status |= jobs[t].status;
  }
  return status;
}

/*
 * Block scores of every row: scores[r * ld_scores + b] for b < nblocks.
 * `starts` may be NULL (all starts are 0).  Returns 0, or 1 on allocation
 * failure.
 */
int oracle_block_scores(const float* logits, int64_t rows, int64_t width, int64_t ld,
                        const int32_t* starts, const int32_t* ends, int32_t block_size,
                        int32_t row_repeat, int32_t pin, float* scores,
                        int64_t ld_scores, int nthreads) {
  if (rows <= 0 || width <= 0) return 0;
  job_t j;
  memset(&j, 0, sizeof j);
  j.logits = logits;
  j.rows = rows;
  j.width = width;
  j.ld = ld;
  j.starts = starts;
  j.ends = ends;
  j.block_size = block_size;
  j.row_repeat = row_repeat;
  j.pin = pin;
  j.scores_out = scores;
  j.ld_scores = ld_scores;
  return run_rows(j, nthreads);
}

/*
 * Candidate-block selection: out[r * ld_out + j] for j < topk.
 * rows == 0 leaves `out` untouched; width == 0 fills it with -1.
 * `scores_out` (nullable) receives the pinned block scores.
 */
int oracle_select_candidate_blocks(const float* logits, int64_t rows, int64_t width,
                                   int64_t ld, const int32_t* starts,
                                   const int32_t* ends, int32_t topk, int32_t block_size,
                                   int32_t row_repeat, int32_t* out, int64_t ld_out,
                                   float* scores_out, int64_t ld_scores, int nthreads) {
  if (rows <= 0) return 0;
  if (width <= 0) {
    for (int64_t r = 0; r < rows; ++r)
      for (int64_t q = 0; q < topk; ++q) out[r * ld_out + q] = -1;
    return 0;
  }
  job_t j;
  memset(&j, 0, sizeof j);
  j.logits = logits;
  j.rows = rows;
  j.width = width;
  j.ld = ld;
  j.starts = starts;
  j.ends = ends;
  j.topk = topk;
  j.block_size = block_size;
  j.row_repeat = row_repeat;
  j.pin = 1;
  j.out = out;
  j.ld_out = ld_out;
  j.scores_out = scores_out;
  j.ld_scores = ld_scores;
  return run_rows(j, nthreads);
}

/* ------------------------------------------------------------------------
 * Selection from a block-score matrix under decode context parallelism.
 *
 * Source: the same page, _select_candidate_blocks_impl, DCP branch.  Each
 * rank scores its interleaved share of the columns at the local block size
 * with the pin off; the element-wise maximum over ranks gives the global
 * block scores (one all-reduce); every rank then pins and selects from the
 * global bounds.  This function is the part after the reduce:
 *   nblocks = max(max_global_blocks, 1);
 *   full[b] = scores[r][b] for b < min(nscore, nblocks), else -inf;
 *   e = global_ends[r div R];
 *   p = clamp(floor((e - 1) / G), 0, nblocks - 1); full[p] = +inf;
 *   if e <= 0 every full[b] = -inf (rows without context select nothing);
 *   then the ranking and the -1 padded output of the non-DCP branch, with
 *   k' = min(k, nblocks).
 * The clamp (rather than skipping a pin past the last block) and the pin
 * from the global end alone (no start) are the page's.
 */
static int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
  return q;
}

int oracle_select_from_scores(const float* scores, int64_t rows, int64_t nscore,
                              int64_t ld_scores, int64_t max_global_blocks,
                              const int32_t* global_ends, int32_t row_repeat,
                              int32_t global_block_size, int32_t topk, int32_t* out,
                              int64_t ld_out) {
  if (rows <= 0) return 0;
  int64_t nblocks = max_global_blocks > 1 ? max_global_blocks : 1;
  int64_t kk = topk < nblocks ? topk : nblocks;
  float* full = (float*)malloc(sizeof(float) * (size_t)nblocks);
  ranked_t* order = (ranked_t*)malloc(sizeof(ranked_t) * (size_t)nblocks);
  if (!full || !order) {
    free(full);
    free(order);
    return 1;
  }
  int64_t ncopy = nscore < nblocks ? nscore : nblocks;
  for (int64_t r = 0; r < rows; ++r) {
    int64_t e = (int64_t)global_ends[r / row_repeat];
    for (int64_t b = 0; b < nblocks; ++b)
      full[b] = b < ncopy ? scores[r * ld_scores + b] : -INFINITY;
    int64_t p = floor_div(e - 1, global_block_size);
    if (p < 0) p = 0;
    if (p > nblocks - 1) p = nblocks - 1;
    full[p] = INFINITY;
    if (e <= 0)
      for (int64_t b = 0; b < nblocks; ++b) full[b] = -INFINITY;
    for (int64_t b = 0; b < nblocks; ++b) {
      order[b].score = full[b];
      order[b].id = (int32_t)b;
    }
    qsort(order, (size_t)nblocks, sizeof(ranked_t), rank_cmp);
    int32_t* o = out + r * ld_out;
    for (int64_t q = 0; q < topk; ++q) {
      /* slots past k' = min(k, nblocks) are -1; order[] holds nblocks entries */
      const int in_k = q < kk;
      o[q] = (in_k && !(isinf(order[q].score) && order[q].score < 0)) ? order[q].id : -1;
    }
  }
  free(full);
  free(order);
  return 0;
}

/* ------------------------------------------------------------------------
 * Block scores as order-preserving uint32 codes, for an exact integer reduce.
 *
 * Source: the same page, DCP branch of _select_candidate_blocks_impl: the
 * ranks' unpinned local block scores are combined by an all-reduce MAX, which
 * must keep the scores' own maximum (NaN propagates, +0 beats -0).  Carried
 * as integers, that reduce is exact whatever a collective does with floats,
 * provided each score is first mapped to a code whose unsigned order is the
 * order of that maximum.  The code used here (this project's choice; the
 * page reduces floats):
 *   NaN (any sign or payload)        -> 0xFFC00000, the code of 0x7FC00000;
 *   x with the sign bit clear (+0..) -> bits(x) + 0x80000000;
 *   x with the sign bit set (-0..)   -> 0xFFFFFFFF - bits(x).
 * Negatives then fall below every non-negative, larger magnitudes of
 * negatives lower; -0 sits just below +0; +inf below the NaN code.
 */
uint32_t oracle_score_key(float x) {
  uint32_t u;
  if (isnan(x)) return 0xFFC00000u;
  memcpy(&u, &x, sizeof u);
  if (signbit(x)) return 0xFFFFFFFFu - u;
  return u + 0x80000000u;
}

/* The inverse of oracle_score_key (a NaN code gives the canonical NaN). */
float oracle_key_score(uint32_t k) {
  uint32_t u = k >= 0x80000000u ? k - 0x80000000u : 0xFFFFFFFFu - k;
  float x;
  memcpy(&x, &u, sizeof x);
  return x;
}

/* codes[i] = oracle_score_key(scores[i]) for a [rows, n] matrix. */
int oracle_score_keys(const float* scores, int64_t rows, int64_t n, int64_t ld_scores,
                      uint32_t* keys, int64_t ld_keys) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < n; ++b)
      keys[r * ld_keys + b] = oracle_score_key(scores[r * ld_scores + b]);
  return 0;
}

/* oracle_select_from_scores on a matrix of codes: every code is turned back
 * into its score, then the selection runs unchanged. */
int oracle_select_from_keys(const uint32_t* keys, int64_t rows, int64_t nkeys, int64_t ld_keys,
                            int64_t max_global_blocks, const int32_t* global_ends,
                            int32_t row_repeat, int32_t global_block_size, int32_t topk,
                            int32_t* out, int64_t ld_out) {
  if (rows <= 0) return 0;
  int64_t n = nkeys > 0 ? nkeys : 0;
  float* scores = (float*)malloc(sizeof(float) * (size_t)(rows * n > 0 ? rows * n : 1));
  if (!scores) return 1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < n; ++b) scores[r * n + b] = oracle_key_score(keys[r * ld_keys + b]);
  int rc = oracle_select_from_scores(scores, rows, n, n > 0 ? n : 1, max_global_blocks, global_ends,
                                     row_repeat, global_block_size, topk, out, ld_out);
  free(scores);
  return rc;
}

/* ------------------------------------------------------------------------
 * Candidate masking of packed logits (the step after selection).
 *
 * Source: the same page, the masking function whose docstring says it masks
 * packed logits outside the causal bounds and outside the request-local
 * candidates (its name and body are not shown).  Reading taken: for row r
 * with bounds s, e (g = r div R), column c < width keeps its value when
 * s <= c < e and its request-local block (c - s) div B is one of
 * cand[r][0 .. topk) (entries < 0 match nothing); every other column becomes
 * -inf.  In place.
 */
int oracle_mask_candidates(float* logits, int64_t rows, int64_t width, int64_t ld,
                           const int32_t* starts, const int32_t* ends, const int32_t* cand,
                           int64_t ld_cand, int32_t topk, int32_t block_size,
                           int32_t row_repeat) {
  for (int64_t r = 0; r < rows; ++r) {
    int64_t s, e;
    row_bounds(r, starts, ends, row_repeat, &s, &e);
    const int32_t* cr = cand + r * ld_cand;
    float* row = logits + r * ld;
    for (int64_t c = 0; c < width; ++c) {
      int keep = 0;
      if (c >= s && c < e) {
        int64_t b = (c - s) / block_size;
        for (int32_t j = 0; j < topk && !keep; ++j) keep = cr[j] >= 0 && (int64_t)cr[j] == b;
      }
      if (!keep) row[c] = -INFINITY;
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------
 * Base-2 log-sum-exp correction of one rank's partial attention output.
 *
 * Source: page 3 (sglang dcp kernels.py), _correct_attn_cp_out_kernel and
 * correct_attn_out.  For every (b, h), with l_n = lses[n][b][h], n < N:
 *   l_n is replaced by -inf when it is NaN or +inf;
 *   m = max_n l_n, or 0 when that maximum is -inf;
 *   final = log2(sum_n 2^(l_n - m)) + m;
 *   d = lses[rank][b][h] - final (the raw value), replaced by -inf when it
 *   is NaN or +inf; factor = 2^d;
 *   vlse[b][h] = final; new_out[h][b][:] = out[b][h][:] * factor.
 * fp32 inputs, arithmetic in double here; all strides in elements.
 */
int oracle_correct_attn_out(const float* out, int64_t B, int64_t H, int64_t D, int64_t o_sb,
                            int64_t o_sh, int64_t o_sd, const float* lses, int64_t N,
                            int64_t l_sn, int64_t l_sb, int64_t l_sh, int64_t rank,
                            double* new_out, int64_t n_sh, int64_t n_sb, int64_t n_sd,
                            double* vlse, int64_t v_sb, int64_t v_sh) {
  for (int64_t b = 0; b < B; ++b) {
    for (int64_t h = 0; h < H; ++h) {
      double m = -INFINITY;
      for (int64_t n = 0; n < N; ++n) {
        double l = (double)lses[n * l_sn + b * l_sb + h * l_sh];
        if (isnan(l) || (isinf(l) && l > 0)) l = -INFINITY;
        if (l > m) m = l;
      }
      if (isinf(m) && m < 0) m = 0.0;
      double acc = 0.0;
      for (int64_t n = 0; n < N; ++n) {
        double l = (double)lses[n * l_sn + b * l_sb + h * l_sh];
        if (isnan(l) || (isinf(l) && l > 0)) l = -INFINITY;
        acc += exp2(l - m);
      }
      double final_lse = log2(acc) + m;
      double d = (double)lses[rank * l_sn + b * l_sb + h * l_sh] - final_lse;
      if (isnan(d) || (isinf(d) && d > 0)) d = -INFINITY;
      double factor = exp2(d);
      vlse[b * v_sb + h * v_sh] = final_lse;
      for (int64_t x = 0; x < D; ++x)
        new_out[h * n_sh + b * n_sb + x * n_sd] = (double)out[b * o_sb + h * o_sh + x * o_sd] * factor;
    }
  }
  return 0;
}
