// Host replay of the streaming loads' index arithmetic (stream_geom.h, the
// same header the HIP kernels include).  For random rows it checks that
//   (1) every column a load touches, vector or scalar path, lies in the
//       row's window [max(s, 0), min(e, width)), for any tile index a
//       rolled load may use;
//   (2) the columns whose values enter block b's maximum are exactly the
//       window columns of block b, [s + bB, s + (b+1)B) ∩ [max(s,0), min(e,width)),
//       each counted once, for every chunk [b0, b1) a launch plan may ask for.
// Prints "ok <cases>" or the first failing case; exit status 0 on success.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "stream_geom.h"

using namespace dsa_geom;

static int fail(const char* what, long long a, long long b, long long c, long long d) {
  printf("FAIL %s: %lld %lld %lld %lld\n", what, a, b, c, d);
  return 1;
}

int main(int argc, char** argv) {
  const long cases = argc > 1 ? atol(argv[1]) : 20000;
  std::mt19937_64 rng(12345);
  auto uni = [&](int64_t lo, int64_t hi) {  // inclusive
    return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1));
  };
  long vec_cases = 0, scalar_cases = 0, tail_cases = 0;
  for (long it = 0; it < cases; ++it) {
    const int G = 1 << uni(0, 6);
    const int32_t B_vec = 4 * G;
    const int32_t B_any = (int32_t)uni(1, 300);
    const int64_t width = uni(1, it % 3 == 0 ? 40000 : 3000);
    const int64_t s = uni(-70, width + 10);
    const int64_t e = uni(s - 10, width + 300);
    const int64_t base_mis = uni(0, 3) * 4;  // row base address mod 16 (bytes)
    const int64_t lo = s > 0 ? s : 0;
    const int64_t hi = e < width ? e : width;
    if (hi <= lo) continue;
    const int nw = 1 << uni(0, 4);
    const int U = uni(0, 1) ? 8 : 16;

    // ---- vector path
    const uintptr_t row_s = (uintptr_t)(0x100000 + base_mis + 4 * s);
    if (vec_path_ok(row_s, s, hi - s)) {
      ++vec_cases;
      const int32_t span = (int32_t)(hi - s);
      const int64_t nblocks = (width + B_vec - 1) / B_vec;
      int64_t nvb = (hi - s + B_vec - 1) / B_vec;
      if (nvb > nblocks) nvb = nblocks;
      // a chunk, as the split and pair plans cut rows, or the whole row
      int32_t b0 = 0, b1 = (int32_t)nvb;
      if (uni(0, 1)) {
        b0 = (int32_t)uni(0, nvb - 1);
        b1 = (int32_t)uni(b0 + 1, nvb);
      }
      const VecChunk c = vec_chunk(span, b0, b1, G);
      std::vector<int> seen((size_t)(b1 - b0) * B_vec, 0);  // chunk columns entering a max
      for (int wv = 0; wv < nw; ++wv) {
        if (wv >= c.ntiles) continue;
        const int32_t tmax = c.ntiles + nw * U;  // past every rolled load
        for (int32_t t = 0; t <= tmax; ++t) {
          for (int lane = 0; lane < 64; ++lane) {
            const int32_t u = vec_load_unit(c, t, lane);
            const int64_t c0 = s + 4 * (int64_t)u;
            if (u < 0 || c0 < lo || c0 + 4 > hi) return fail("vec load outside window", s, e, width, u);
            const int32_t uu = c.ub + (t << 6) + lane;  // the unit this slot stands for
            if (t % nw != wv || t >= c.ntiles) continue;
            const int32_t cols = vec_unit_cols(c, span, uu);
            if (cols == 4) {
              if (u != uu) return fail("whole unit not loaded itself", s, e, uu, u);
              for (int q = 0; q < 4; ++q) {
                const int64_t col = 4 * (int64_t)uu + q - 4 * (int64_t)c.ub;
                if (col < 0 || col >= (int64_t)seen.size()) return fail("unit outside chunk", s, e, uu, q);
                seen[(size_t)col]++;
              }
            } else if (cols > 0) {
              ++tail_cases;
              if (uu != c.nfull || c.tail_tile != t || c.tail_lane != lane || cols != c.tail_cols)
                return fail("partial unit not the tail", s, e, uu, c.nfull);
              for (int q = 0; q < 3; ++q) {
                const int64_t col = s + vec_tail_col(c, q);
                if (col < lo || col >= hi) return fail("tail load outside window", s, e, width, q);
              }
              for (int q = 0; q < cols; ++q) {
                const int64_t col = 4 * (int64_t)uu + q - 4 * (int64_t)c.ub;
                seen[(size_t)col]++;
              }
            }
          }
        }
      }
      // exactly the chunk's window columns, once each
      for (size_t i = 0; i < seen.size(); ++i) {
        const int64_t col = s + 4 * (int64_t)c.ub + (int64_t)i;
        const int want = (col >= lo && col < hi) ? 1 : 0;
        if (seen[i] != want) return fail("vec coverage", s, e, col, seen[i]);
      }
    }

    // ---- scalar path (any block size, any alignment, any start)
    {
      ++scalar_cases;
      const int32_t B = B_any;
      const int64_t nblocks = (width + B - 1) / B;
      int64_t nvb = (hi - s + B - 1) / B;
      if (nvb > nblocks) nvb = nblocks;
      if (nvb <= 0) continue;
      const int64_t b0 = uni(0, nvb - 1);
      const int64_t b1 = uni(b0 + 1, nvb);
      int gl = 1;
      while (gl * 2 <= B && gl < 64) gl *= 2;
      for (int64_t b = b0; b < b1 + 64; ++b) {  // lanes past b1 in the last group too
        const ScalarBlock r = scalar_block(s, lo, hi, b, B, b1);
        int64_t want_lo = std::max<int64_t>(s + b * B, lo), want_hi = std::min<int64_t>(s + (b + 1) * B, hi);
        if (b >= b1 || want_hi < want_lo) want_lo = want_hi = 0;
        if (b < b1 && want_hi > want_lo && (r.lo != want_lo || r.hi != want_hi))
          return fail("scalar block range", s, e, b, r.lo);
        if (b >= b1 && r.hi > r.lo) return fail("scalar block past b1", s, e, b, r.hi);
        for (int sub = 0; sub < gl; ++sub)
          for (int64_t cc = r.lo + sub; cc < r.hi; cc += 4 * gl)
            for (int q = 0; q < 4; ++q) {
              const int64_t col = scalar_load_col(r, cc + (int64_t)q * gl);
              if (col < lo || col >= hi) return fail("scalar load outside window", s, e, b, col);
            }
      }
    }
  }
  if (vec_cases < cases / 10 || tail_cases == 0) return fail("too few vector cases", vec_cases, tail_cases, 0, 0);
  printf("ok %ld vector %ld scalar %ld tail %ld\n", cases, vec_cases, scalar_cases, tail_cases);
  return 0;
}
