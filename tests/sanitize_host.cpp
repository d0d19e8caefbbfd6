// Host code of libdsa under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// tests/test_sanitize_cpu.py builds this driver together with csrc/dsa.hip,
// the host side instrumented (-Xarch_host -fsanitize=...), the kernels not.
// It calls every entry point with argument values at the edges of their
// types, on fake pointers: pure host arithmetic (plan and workspace sizing,
// status strings), calls the host checks reject before anything is enqueued,
// and calls that pass them, whose launch then fails (DSA_ERR_HIP) before any
// memory is touched because no GPU is visible.  It refuses to run where a GPU
// is visible (those launches would dereference the fake pointers there).  A
// sanitizer report aborts the run; the driver prints "ok <calls>" at the end.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "dsa.h"

namespace {

long calls = 0;
int failures = 0;

void expect(bool ok, const char* what, long long a, long long b) {
  ++calls;
  if (!ok) {
    ++failures;
    printf("FAIL %s: %lld %lld\n", what, a, b);
  }
}

const float* const kLogits = reinterpret_cast<const float*>(0x10000);
float* const kScores = reinterpret_cast<float*>(0x20000);
int32_t* const kOut = reinterpret_cast<int32_t*>(0x30000);
const int32_t* const kEnds = reinterpret_cast<const int32_t*>(0x40000);
void* const kWs = reinterpret_cast<void*>(0x80000);

}  // namespace

int main() {
  int ndev = 0;
  const bool no_gpu = hipGetDeviceCount(&ndev) != hipSuccess || ndev == 0;
  (void)hipGetLastError();
  if (!no_gpu) {
    printf("skip: a GPU is visible\n");
    return 0;
  }

  const std::vector<int64_t> sizes = {-1, 0, 1, 7, 8, 63, 64, 65, 128, 129, 1023, 1024, 4095,
                                      16384, 32768, 65536, 1 << 20, INT32_MAX,
                                      (int64_t)INT32_MAX + 1, (int64_t)1 << 40, (int64_t)1 << 62,
                                      INT64_MAX};
  const std::vector<int32_t> small = {-1, 0, 1, 3, 4, 8, 16, 32, 33, 64, 65, 128, 255, 256,
                                      4096, INT32_MAX};

  // plan and workspace sizing: pure host arithmetic for every combination
  for (int64_t rows : sizes)
    for (int64_t width : sizes)
      for (int32_t B : small)
        for (int32_t k : {-1, 0, 1, 32, 64, 300, INT32_MAX}) {
          int32_t plan = -7, arg = -7;
          const dsa_status_t st = dsa_select_plan(rows, width, B, k, &plan, &arg);
          const bool bad = rows < 0 || width < 0 || B < 1 || k < 0;
          expect(bad ? st == DSA_ERR_INVALID_ARG : (st == DSA_OK && plan >= 1 && plan <= 4),
                 "dsa_select_plan", rows, width);
          const size_t ws = dsa_select_workspace_bytes(rows, width, B, k);
          expect(!(bad || rows == 0 || width == 0) || ws == 0, "workspace of an invalid shape",
                 rows, width);
        }
  expect(dsa_select_plan(1, 1, 1, 1, nullptr, nullptr) == DSA_ERR_INVALID_ARG, "plan null", 0, 0);

  for (int c : {INT32_MIN, -3, -1, 0, 1, 2, 3, 4, 5, 8, INT32_MAX})
    expect(dsa_status_string(c) != nullptr, "status", c, 0);

  // selection: every argument at the edges; rejected calls enqueue nothing
  for (int64_t rows : sizes)
    for (int64_t width : sizes)
      for (int32_t B : {-1, 0, 1, 4, 64, INT32_MAX})
        for (int32_t k : {-1, 0, 1, 64, 4096, INT32_MAX})
          for (int32_t plan : {-1, 0, 1, 2, 3, 4, 5}) {
            const int64_t ld = width;
            dsa_status_t st = dsa_select_candidate_blocks_plan(
                kLogits, rows, width, ld, nullptr, kEnds, k, B, 1, kOut, k, nullptr, 0, nullptr,
                0, plan, 0, nullptr);
            if (st == DSA_OK && rows > 0 && k > 0)
              expect(false, "selection accepted without a GPU call", rows, width);
            // a too-small leading dimension is always rejected
            if (width > 0) {
              st = dsa_select_candidate_blocks_plan(kLogits, rows, width, width - 1, nullptr,
                                                    kEnds, k, B, 1, kOut, k, nullptr, 0, kWs,
                                                    1 << 20, plan, 0, nullptr);
              expect(st == DSA_ERR_INVALID_ARG || (rows == 0 && st == DSA_ERR_INVALID_ARG),
                     "ld < width accepted", rows, width);
            }
            (void)st;
          }

  // calls that pass every check: their launch fails with no GPU
  for (int32_t plan : {0, 1, 2, 3, 4}) {
    const dsa_status_t st = dsa_select_candidate_blocks_plan(
        kLogits, 64, 32768, 32768, nullptr, kEnds, 32, 64, 2, kOut, 32, kScores, 512, kWs,
        1 << 20, plan, 0, nullptr);
    expect(st == DSA_ERR_HIP, "launch without a GPU", plan, st);
  }
  expect(dsa_select_candidate_blocks(kLogits, 3, 0, 0, nullptr, nullptr, 4, 8, 1, kOut, 4,
                                     nullptr, 0, nullptr, 0, nullptr) == DSA_ERR_HIP,
         "fill without a GPU", 0, 0);

  // block scores and their uint32 codes
  for (int64_t rows : sizes)
    for (int64_t width : sizes)
      for (int32_t B : {-1, 0, 1, 8, INT32_MAX})
        for (int pin : {-1, 0, 1, 2}) {
          const int64_t nb = (B > 0 && width >= 0) ? width / B + (width % B != 0) : 0;
          for (int keys = 0; keys < 2; ++keys) {
            const dsa_status_t st =
                keys ? dsa_block_score_keys(kLogits, rows, width, width, nullptr, kEnds, B, 1,
                                            pin, reinterpret_cast<uint32_t*>(kScores), nb - 1,
                                            nullptr)
                     : dsa_block_scores(kLogits, rows, width, width, nullptr, kEnds, B, 1, pin,
                                        kScores, nb - 1, nullptr);
            // ld_scores = nblocks - 1 is too small whenever there are blocks
            expect(st != DSA_OK || rows == 0 || width == 0 || nb == 0, "block scores accepted",
                   rows, width);
          }
        }

  // selection from scores or codes
  for (int64_t rows : sizes)
    for (int64_t n : sizes)
      for (int64_t mgb : sizes)
        for (int32_t k : {-1, 0, 1, 64, INT32_MAX}) {
          for (int keys = 0; keys < 2; ++keys) {
            const dsa_status_t st =
                keys ? dsa_select_from_keys(reinterpret_cast<const uint32_t*>(kLogits), rows, n,
                                            n - 1, mgb, kEnds, 1, 64, k, kOut, k, nullptr)
                     : dsa_select_from_scores(kLogits, rows, n, n - 1, mgb, kEnds, 1, 64, k,
                                              kOut, k, nullptr);
            expect(st != DSA_OK || rows == 0 || k == 0, "select_from accepted", rows, n);
          }
        }

  // masking
  for (int64_t rows : sizes)
    for (int64_t width : sizes)
      for (int32_t k : {-1, 0, 1, INT32_MAX}) {
        const dsa_status_t st = dsa_mask_candidates(const_cast<float*>(kLogits), rows, width,
                                                    width - 1, nullptr, kEnds, kOut, k, k, 64, 1,
                                                    nullptr);
        expect(st != DSA_OK || rows == 0 || width == 0, "mask accepted", rows, width);
        const dsa_status_t st2 = dsa_mask_candidates(const_cast<float*>(kLogits), rows, width,
                                                     width, nullptr, kEnds, kOut, k, k, 64, 1,
                                                     nullptr);
        expect(st2 != DSA_OK || rows <= 0 || width <= 0, "mask launched without a GPU", rows,
               width);
      }

  // LSE correction
  for (int64_t b : sizes)
    for (int64_t h : sizes)
      for (int64_t n : {-1, 0, 1, 8, 70})
        for (int64_t rank : {-1, 0, 7, 70}) {
          // fake strides (never dereferenced): constants, not products of the
          // extreme sizes
          const dsa_status_t st = dsa_correct_attn_out(
              kLogits, b, h, 512, 1 << 20, 512, 1, kScores, n, 1 << 20, 1024, 1, rank, kScores,
              1 << 20, 512, 1, kScores, 1024, 1, nullptr);
          const bool valid_sizes = b > 0 && h > 0 && n >= 1 && rank >= 0 && rank < n;
          expect(!(valid_sizes && st == DSA_OK), "lse accepted without a GPU call", b, h);
        }

  if (failures) {
    printf("%d failures\n", failures);
    return 1;
  }
  printf("ok %ld calls\n", calls);
  return 0;
}
