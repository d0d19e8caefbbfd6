// stream_geom.h - which logits columns the streaming loads of dsa.hip touch.
//
// The candidate-block selection reads, per row, only the columns of its
// window [max(s, 0), min(e, width)) (the masked window load of
// _block_scores_kernel on the vLLM-fork page
// "02-model_executor_kernels_attention_dsa_candidate_blocks.py.diff": columns
// outside the window count as -inf and need not be read).  The integer
// arithmetic that keeps every load inside that range lives here, as plain
// functions that also compile for the host, so that a CPU test can replay it
// for any bounds, alignment and block size (tests/test_stream_geom_cpu.py).
//
// Vector path (B = 4*G, G a power of two <= 64): a row's window, counted
// from the request start s, holds `span` columns.  Unit u is the float4 of
// columns [s + 4u, s + 4u + 4).  The first nfull = span / 4 units lie wholly
// inside the window and are the only float4s ever loaded; the partial unit
// nfull (span % 4 columns, when span % 4 != 0) is read with scalar loads by
// the one lane that owns it.  A chunk of blocks [b0, b1) covers units
// [b0*G, min(b1*G, ceil(span/4))), dealt in 64-unit tiles to the waves of a
// workgroup; a lane's load for any tile index t >= 0 is clamped into the
// chunk's last whole unit (or, for a chunk holding only the partial unit,
// the unit before it), so even the rolled loads past the chunk's last tile
// stay inside the window.
//
// Scalar path (any B, any alignment): lanes stride over one block's window
// columns; a masked slot re-reads the block's first window column.
#ifndef DSA_STREAM_GEOM_H
#define DSA_STREAM_GEOM_H

#include <stdint.h>

#if defined(__HIP__)
#define DSA_HD __host__ __device__ __forceinline__
#else
#define DSA_HD static inline
#endif

namespace dsa_geom {

// The vector path applies when the request start is a non-negative column,
// (row + s) is 16-byte aligned, at least one whole unit is in the window,
// and byte offsets of units from (row + s) fit in 32 bits.
DSA_HD bool vec_path_ok(uintptr_t row_s_addr, int64_t s, int64_t span) {
  return s >= 0 && (row_s_addr & 15u) == 0 && span >= 4 && span < ((int64_t)1 << 30);
}

struct VecChunk {
  int32_t ub;         // first unit of the chunk
  int32_t ue;         // one past its last unit holding a window column
  int32_t ntiles;     // 64-unit tiles of the chunk
  int32_t nfull;      // units of the row wholly inside the window
  int32_t full_end;   // units [ub, full_end) of the chunk are whole
  int32_t ulast;      // the unit a clamped load reads
  int32_t tail_cols;  // columns of the partial unit nfull (0: none)
  int32_t tail_tile;  // tile of the chunk holding the partial unit, or -1
  int32_t tail_lane;  // lane of that tile holding it
};

// span >= 4 (vec_path_ok); 0 <= b0 <= b1; G in {1, 2, ..., 64}.
DSA_HD VecChunk vec_chunk(int32_t span, int32_t b0, int32_t b1, int32_t G) {
  VecChunk c;
  const int32_t nu_row = (span + 3) >> 2;  // units holding a window column
  c.nfull = span >> 2;
  c.tail_cols = span & 3;
  c.ub = b0 * G;
  c.ue = b1 * G < nu_row ? b1 * G : nu_row;
  c.ntiles = c.ue > c.ub ? (c.ue - c.ub + 63) >> 6 : 0;
  c.full_end = c.ue < c.nfull ? c.ue : c.nfull;
  c.ulast = c.full_end > 0 ? c.full_end - 1 : 0;
  const bool tail_here = c.tail_cols != 0 && c.nfull >= c.ub && c.nfull < c.ue;
  c.tail_tile = tail_here ? (c.nfull - c.ub) >> 6 : -1;
  c.tail_lane = tail_here ? (c.nfull - c.ub) & 63 : 0;
  return c;
}

// The unit lane `lane` loads for tile t (any t >= 0): its own unit while
// that is whole, else the clamp unit.
DSA_HD int32_t vec_load_unit(const VecChunk& c, int32_t t, int32_t lane) {
  const int32_t u = c.ub + (t << 6) + lane;
  return u < c.full_end ? u : c.ulast;
}

// Window columns of unit u that count: 4 for a whole unit of the chunk,
// 1..3 for the partial unit (its values come from the scalar tail loads),
// 0 past the chunk.
DSA_HD int32_t vec_unit_cols(const VecChunk& c, int32_t span, int32_t u) {
  if (u >= c.ue) return 0;
  const int32_t lim = span - 4 * u;
  return lim > 4 ? 4 : lim;
}

// Column (relative to s) of the partial unit's q-th scalar load, q < 3:
// element q while it is in the window, else element 0 again (a duplicate
// changes no maximum).
DSA_HD int32_t vec_tail_col(const VecChunk& c, int32_t q) {
  return 4 * c.nfull + (q < c.tail_cols ? q : 0);
}

// Scalar path: the columns [lo, hi) of block b that lie in the window
// [win_lo, win_hi) (win_lo = max(s, 0), win_hi = min(e, width)); an empty
// range for blocks at or past b1.
struct ScalarBlock {
  int64_t lo, hi;
};

DSA_HD ScalarBlock scalar_block(int64_t s, int64_t win_lo, int64_t win_hi, int64_t b, int32_t B,
                                int64_t b1) {
  ScalarBlock r;
  const int64_t cs = s + b * B;  // first column of block b
  r.lo = b < b1 ? (cs > win_lo ? cs : win_lo) : 0;
  r.hi = b < b1 ? (cs + B < win_hi ? cs + B : win_hi) : 0;
  return r;
}

// The column a scalar load slot reads: c itself inside [lo, hi), else lo.
DSA_HD int64_t scalar_load_col(const ScalarBlock& r, int64_t c) { return c < r.hi ? c : r.lo; }

}  // namespace dsa_geom

#endif  // DSA_STREAM_GEOM_H
