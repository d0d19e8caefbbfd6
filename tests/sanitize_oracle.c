/*
 * oracle/oracle.c under AddressSanitizer and UndefinedBehaviorSanitizer.
 *
 * tests/test_sanitize_cpu.py builds this driver together with oracle.c,
 * both instrumented, and feeds it a text file of cases (the hand-worked
 * rows and seeded random cases); the driver runs the oracle's functions on
 * each and prints their results, which the test compares with the regular
 * build of the oracle.  A sanitizer report aborts the run.
 *
 * Input, whitespace separated, one record per case:
 *   S rows width ld B R k has_starts threads   then starts (if any), ends, logits (hex bits)
 *   F rows n ld mgb R G k                       then ends, scores (hex bits)
 *   M rows width ld B R k has_starts ld_cand    then starts, ends, candidates, logits
 *   L B H D N rank                              then out (B*H*D), lses (N*B*H), hex bits
 * Output: one line per case with its results (ints, or hex bits of floats).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_select_candidate_blocks(const float*, int64_t, int64_t, int64_t, const int32_t*,
                                   const int32_t*, int32_t, int32_t, int32_t, int32_t*, int64_t,
                                   float*, int64_t, int);
int oracle_block_scores(const float*, int64_t, int64_t, int64_t, const int32_t*, const int32_t*,
                        int32_t, int32_t, int32_t, float*, int64_t, int);
int oracle_select_from_scores(const float*, int64_t, int64_t, int64_t, int64_t, const int32_t*,
                              int32_t, int32_t, int32_t, int32_t*, int64_t);
int oracle_score_keys(const float*, int64_t, int64_t, int64_t, uint32_t*, int64_t);
int oracle_select_from_keys(const uint32_t*, int64_t, int64_t, int64_t, int64_t, const int32_t*,
                            int32_t, int32_t, int32_t, int32_t*, int64_t);
int oracle_mask_candidates(float*, int64_t, int64_t, int64_t, const int32_t*, const int32_t*,
                           const int32_t*, int64_t, int32_t, int32_t, int32_t);
int oracle_correct_attn_out(const float*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t,
                            const float*, int64_t, int64_t, int64_t, int64_t, int64_t, double*,
                            int64_t, int64_t, int64_t, double*, int64_t, int64_t);

static FILE* in;

static long long rd_i(void) {
  long long v;
  if (fscanf(in, "%lld", &v) != 1) exit(3);
  return v;
}

/* exact-size allocations: every array holds exactly what its case needs */
static int32_t* rd_i32(int64_t n) {
  int32_t* a = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) a[i] = (int32_t)rd_i();
  return a;
}

static float* rd_f32(int64_t n) {
  float* a = (float*)malloc(sizeof(float) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) {
    unsigned int b;
    if (fscanf(in, "%x", &b) != 1) exit(3);
    uint32_t u = b;
    memcpy(&a[i], &u, 4);
  }
  return a;
}

static void pr_f32(const float* a, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    uint32_t u;
    memcpy(&u, &a[i], 4);
    printf(" %08x", u);
  }
}

int main(int argc, char** argv) {
  if (argc < 2 || !(in = fopen(argv[1], "r"))) return 2;
  char tag[4];
  int cases = 0;
  while (fscanf(in, "%3s", tag) == 1) {
    ++cases;
    if (tag[0] == 'S') {
      int64_t rows = rd_i(), width = rd_i(), ld = rd_i(), B = rd_i(), R = rd_i(), k = rd_i();
      int has_starts = (int)rd_i(), threads = (int)rd_i();
      int64_t groups = rows ? (rows + R - 1) / R : 0;
      int32_t* starts = has_starts ? rd_i32(groups) : NULL;
      int32_t* ends = rd_i32(groups);
      /* the last row holds only its first `width` columns (no slack after it) */
      int64_t n = rows ? (rows - 1) * ld + width : 0;
      float* x = rd_f32(n);
      int64_t nb = (width + B - 1) / B;
      int32_t* out = (int32_t*)malloc(sizeof(int32_t) * (size_t)(rows * k > 0 ? rows * k : 1));
      float* sc = (float*)malloc(sizeof(float) * (size_t)(rows * nb > 0 ? rows * nb : 1));
      int rc = oracle_select_candidate_blocks(x, rows, width, ld, starts, ends, (int32_t)k,
                                              (int32_t)B, (int32_t)R, out, k, nb ? sc : NULL,
                                              nb, threads);
      printf("S %d", rc);
      for (int64_t i = 0; i < rows * k; ++i) printf(" %d", out[i]);
      pr_f32(sc, rows * nb);
      rc = oracle_block_scores(x, rows, width, ld, starts, ends, (int32_t)B, (int32_t)R, 0, sc, nb,
                               threads);
      printf(" | %d", rc);
      if (rows && width) pr_f32(sc, rows * nb);
      printf("\n");
      free(starts);
      free(ends);
      free(x);
      free(out);
      free(sc);
    } else if (tag[0] == 'F') {
      int64_t rows = rd_i(), n = rd_i(), ld = rd_i(), mgb = rd_i(), R = rd_i(), G = rd_i(),
              k = rd_i();
      int64_t groups = rows ? (rows + R - 1) / R : 0;
      int32_t* ends = rd_i32(groups);
      int64_t cnt = rows && n ? (rows - 1) * ld + n : 0;
      float* s = rd_f32(cnt);
      int32_t* out = (int32_t*)malloc(sizeof(int32_t) * (size_t)(rows * k > 0 ? rows * k : 1));
      int rc = oracle_select_from_scores(n ? s : NULL, rows, n, ld, mgb, ends, (int32_t)R,
                                         (int32_t)G, (int32_t)k, out, k);
      printf("F %d", rc);
      for (int64_t i = 0; i < rows * k; ++i) printf(" %d", out[i]);
      uint32_t* keys = (uint32_t*)malloc(sizeof(uint32_t) * (size_t)(rows * n > 0 ? rows * n : 1));
      oracle_score_keys(s, rows, n, ld, keys, n);
      rc = oracle_select_from_keys(n ? keys : NULL, rows, n, n ? n : 1, mgb, ends, (int32_t)R,
                                   (int32_t)G, (int32_t)k, out, k);
      printf(" | %d", rc);
      for (int64_t i = 0; i < rows * k; ++i) printf(" %d", out[i]);
      printf("\n");
      free(ends);
      free(s);
      free(out);
      free(keys);
    } else if (tag[0] == 'M') {
      int64_t rows = rd_i(), width = rd_i(), ld = rd_i(), B = rd_i(), R = rd_i(), k = rd_i();
      int has_starts = (int)rd_i();
      int64_t ld_cand = rd_i();
      int64_t groups = rows ? (rows + R - 1) / R : 0;
      int32_t* starts = has_starts ? rd_i32(groups) : NULL;
      int32_t* ends = rd_i32(groups);
      int32_t* cand = rd_i32(rows ? (rows - 1) * ld_cand + k : 0);
      int64_t n = rows ? (rows - 1) * ld + width : 0;
      float* x = rd_f32(n);
      int rc = oracle_mask_candidates(x, rows, width, ld, starts, ends, cand, ld_cand, (int32_t)k,
                                      (int32_t)B, (int32_t)R);
      printf("M %d", rc);
      pr_f32(x, n);
      printf("\n");
      free(starts);
      free(ends);
      free(cand);
      free(x);
    } else if (tag[0] == 'L') {
      int64_t B = rd_i(), H = rd_i(), D = rd_i(), N = rd_i(), rank = rd_i();
      float* o = rd_f32(B * H * D);
      float* l = rd_f32(N * B * H);
      double* nw = (double*)malloc(sizeof(double) * (size_t)(B * H * D > 0 ? B * H * D : 1));
      double* v = (double*)malloc(sizeof(double) * (size_t)(B * H > 0 ? B * H : 1));
      int rc = oracle_correct_attn_out(o, B, H, D, H * D, D, 1, l, N, B * H, H, 1, rank, nw, B * D,
                                       D, 1, v, H, 1);
      printf("L %d", rc);
      for (int64_t i = 0; i < B * H; ++i) printf(" %.17g", v[i]);
      for (int64_t i = 0; i < B * H * D; ++i) printf(" %.17g", nw[i]);
      printf("\n");
      free(o);
      free(l);
      free(nw);
      free(v);
    } else {
      return 4;
    }
  }
  fclose(in);
  fprintf(stderr, "cases %d\n", cases);
  return 0;
}
