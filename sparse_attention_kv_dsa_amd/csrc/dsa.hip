// dsa.hip - gfx950 kernels and C ABI for DSA candidate-block selection.
//
// What is computed follows the vLLM-fork page
// "launcher/dcp2/diffs/02-model_executor_kernels_attention_dsa_candidate_blocks.py.diff":
// _max_with_nan (NaN-propagating max), _block_scores_kernel (masked window
// load with -inf fill, newest-block pin), _block_scores, the non-DCP branch
// of _select_candidate_blocks_impl (early-outs, top-k, -1 padding), the DCP
// branch's selection after its reduce, and the candidate masking after it;
// and page 3 (sglang dcp kernels.py) for the log-sum-exp correction.  The
// full contract is stated in include/dsa.h.
//
// How it is computed here (MI355X / CDNA4, wave64):
//   * One HBM pass over the in-window logits.  A block of B = 4*G columns is
//     G lanes of one float4 each; a wave instruction reads 1 KiB contiguous,
//     every lane keeps kUnroll independent 16-byte loads in flight.  The
//     loads are nontemporal (each logit is read once) and, where the block
//     maxima go to LDS, roll: a tile's next load is issued as soon as the
//     tile has been reduced.
//   * The per-lane max of a float4 and the G-lane reduction use the IEEE-754-
//     2019 maximum (v_maximum3_f32 on gfx950: NaN-propagating, -0 < +0);
//     the lanes of a block are combined with DPP quad/row permutes inside a
//     16-lane row and DPP row broadcasts across rows; where the block maxima
//     become keys, the reduction runs on the keys (integer maximum).
//   * Scores are kept as order-preserving uint32 keys (unsigned order ==
//     float order, canonical NaN on top), in LDS for the select.
//   * Top-k prunes, then ranks: a lower bound on the k-th largest key (the
//     k-th largest of 64 group maxima for k <= 32, of 128 for k <= 64, radix
//     passes over 8-bit digits above), then the keys at or above it (the
//     candidates) are
//     compacted into LDS as distinct 64-bit words (key, inverted block id),
//     and a candidate's output slot is the number of larger words.  Every
//     wave of a row's workgroup takes part; rows with more candidates than
//     the LDS holds fall back to an exact one-wave radix select.
//   * Launch plans: short rows take one wave per row (four rows per
//     workgroup, no barrier at all); long rows, and decode batches with
//     enough rows to keep HBM busy, take a workgroup per row whose waves
//     stream the row into LDS and then select it together; decode batches
//     of up to 128 long rows share each row among 2-8 workgroups of one XCD,
//     which hand their keys to the last of them through that XCD's L2 (a
//     per-row arrival counter, no waiting); more rows, too few for their
//     length, are split in chunks over many CUs by a streaming kernel that
//     writes the block keys, and a second kernel selects, one workgroup per
//     row.  A hand-off through memory instead (agent-scope fences, or
//     device-scope stores and loads) measured slower than the kernel
//     boundary.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "dsa.h"
#include "stream_geom.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;
// The pair plan (one workgroup per CU, latency-bound) streams its parts with
// 4 loads in flight per lane: decode batch 6.89 -> 6.34 us, long-context
// decode 13.76 -> 13.45 against 8 (2, 3 and 6 were slower, 12 and 16 far
// slower); the wave, group and block-score kernels lost 1-3 % at 4.
constexpr int kPairUnroll = 4;

constexpr size_t kLdsLimit = 65536;
constexpr size_t kGroupLdsThree = 160 * 1024 / 4 + 256;  // > 1/4 of a CU's LDS: three per CU
constexpr int64_t kMaxGrid = 1 << 20;

// Order-preserving keys: for non-NaN floats a < b  <=>  key(a) < key(b) as
// unsigned, with key(-0) < key(+0).  Every NaN maps to the key of the
// canonical NaN 0x7FC00000, which is above key(+inf).
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;
constexpr uint32_t kKeyPosInf = 0xFF800000u;
constexpr uint32_t kKeyNaN = 0xFFC00000u;
constexpr uint32_t kKeyNegZero = 0x7FFFFFFFu;
constexpr uint32_t kKeyPosZero = 0x80000000u;

__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (v != v) return kKeyNaN;
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// Ranking key: -inf (and below) -> 0, "not a candidate"; -0 ranks as +0.
__device__ __forceinline__ uint32_t rank_key(uint32_t k) {
  return k <= kKeyNegInf ? 0u : (k == kKeyNegZero ? kKeyPosZero : k);
}

__device__ __forceinline__ float fmaximum(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ float canonical(float v) {
  return v != v ? __uint_as_float(0x7FC00000u) : v;
}

template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Maximum over aligned groups of G lanes; every lane of a group ends with the
// group's value.  All 64 lanes must be active.
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 2) v = fmaximum(v, dpp_move<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v = fmaximum(v, dpp_move<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v = fmaximum(v, dpp_move<0x141>(v));   // row_half_mirror
  if constexpr (G >= 16) v = fmaximum(v, dpp_move<0x140>(v));  // row_mirror
  if constexpr (G >= 32)                                       // lane ^ 16
    v = fmaximum(v, __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(
                                                   __builtin_bit_cast(int, v), 0x401F)));
  if constexpr (G >= 64) v = fmaximum(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum over aligned groups of G lanes (G a power of two <= 64); every lane
// of a group ends with the group's value.  All 64 lanes must be active.
template <int G>
__device__ __forceinline__ uint32_t group_umax(uint32_t v) {
  if constexpr (G >= 2) v = umax(v, dpp_u32<0xB1>(v));    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v = umax(v, dpp_u32<0x4E>(v));    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v = umax(v, dpp_u32<0x141>(v));   // row_half_mirror
  if constexpr (G >= 16) v = umax(v, dpp_u32<0x140>(v));  // row_mirror
  if constexpr (G >= 32) v = umax(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  if constexpr (G >= 64) v = umax(v, (uint32_t)__shfl_xor((int)v, 32));
  return v;
}

// The vector path's reductions over G lanes: the same as group_max /
// group_umax up to G = 16; beyond, the steps across rows go through DPP row
// broadcasts (lane 15 of a row into the next row, lane 31 into rows 2 and 3)
// instead of a swizzle and a bpermute, so the group's value is only whole in
// its lane kTailLane<G> (the first lane of its last row).
template <int G>
constexpr int kTailLane = G >= 64 ? 48 : (G >= 32 ? 16 : 0);

template <int G>
__device__ __forceinline__ float group_max_tail(float v) {
  if constexpr (G <= 16) {
    return group_max<G>(v);
  } else {
    v = group_max<16>(v);
    v = fmaximum(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                  __builtin_bit_cast(int, v),
                                                  __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false)));
    if constexpr (G >= 64)
      v = fmaximum(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                                    __builtin_bit_cast(int, v),
                                                    __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false)));
    return v;
  }
}

template <int G>
__device__ __forceinline__ uint32_t group_umax_tail(uint32_t v) {
  if constexpr (G <= 16) {
    return group_umax<G>(v);
  } else {
    v = group_umax<16>(v);
    v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
    if constexpr (G >= 64)
      v = umax(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
    return v;
  }
}

// Streaming loads: each logit is read once, so the loads are nontemporal
// (measured 1-12 % faster per workload on this chip than cached loads).
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const void* p) {
  const f32x4 r = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ float load_stream(const float* p) {
  return __builtin_nontemporal_load(p);
}

__device__ __forceinline__ float group_max_dyn(float v, int gl) {
  for (int off = gl >> 1; off >= 1; off >>= 1) v = fmaximum(v, __shfl_xor(v, off));
  return v;
}

struct Params {
  const float* logits;
  int64_t rows, width, ld;
  const int32_t* ks;
  const int32_t* ke;
  int32_t B, R, pin, k;
  int32_t nblocks, chunk_blocks, nchunks;
  int32_t kcap;        // max(1, min(k, nblocks)): selected-set capacity
  int32_t keys_words;  // LDS words for one row's keys (nblocks rounded up to 4)
  int32_t wave_words;  // LDS words of one row's select state (keys, control, area)
  int32_t* out;
  int64_t ld_out;
  float* scores;  // block-scores output, or the optional write-back
  int64_t ld_scores;
  uint32_t* ws_keys;  // split and pair plans: [rows, ws_ld] score keys
  int64_t ws_ld;      // row stride of ws_keys, a multiple of 32 (128-byte lines)
  uint64_t* ws_count; // pair plan: per-row arrival counters, zero between calls
  int32_t parts;      // pair plan: workgroups per row
  int32_t spread;     // pair plan: a row's parts on consecutive workgroups (other XCDs)
  int32_t r_shift;    // log2(R) when R is a power of two, else -1
  int32_t h_shift;    // pair plan: log2(parts) when a power of two, else -1
  int64_t items;      // work items of the launch
};

// Per-row geometry derived from the bounds (all in 64-bit: bounds are
// arbitrary int32 device data).
struct RowGeom {
  const float* row;
  int64_t s;      // request start (block 0 begins here)
  int64_t lo;     // first column that may be read: max(s, 0)
  int64_t hi;     // one past the last: min(e, width)
  int32_t nvb;    // blocks [0, nvb) may hold elements
  int32_t pin;    // pinned block, or -1
  int32_t nsel;   // blocks [0, nsel) can be candidates
};

// n / d for 0 <= n < 2^33 and 1 <= d < 2^31: the 32-bit divide when n fits.
__device__ __forceinline__ int64_t div_bound(int64_t n, int32_t d) {
  if ((n >> 32) == 0) return (int64_t)((uint32_t)n / (uint32_t)d);
  return n / d;
}

// Row group (the bounds index) of row r < 2^31: a shift for a power-of-two
// row_repeat, else a 32-bit divide.
__device__ __forceinline__ int64_t row_group(const Params& p, int64_t r) {
  if (p.r_shift >= 0) return r >> p.r_shift;
  return (int64_t)((uint32_t)r / (uint32_t)p.R);
}

// Called by every lane of a wave (uniform control flow).  G > 0: the
// block size is 4*G, a power of two, and the divides by it are shifts.
template <int G = 0>
__device__ __forceinline__ RowGeom row_geom(const Params& p, int64_t r, bool pin) {
  // n >= 0
  auto div_b = [&](int64_t n) -> int64_t {
    if constexpr (G > 0) return n >> __builtin_ctz(4 * G);
    else return div_bound(n, p.B);
  };
  RowGeom g;
  const int64_t grp = row_group(p, r);
  // one load brings both bounds (lane 0: the start, the others: the end),
  // one memory round trip instead of two; every lane of the wave is active
  const int32_t* bp = ((threadIdx.x & 63) == 0 && p.ks) ? p.ks + grp : p.ke + grp;
  const int32_t bv = *bp;
  g.s = p.ks ? (int64_t)__builtin_amdgcn_readlane(bv, 0) : 0;
  const int64_t e = (int64_t)__builtin_amdgcn_readlane(bv, 1);
  g.row = p.logits + r * p.ld;
  g.lo = g.s > 0 ? g.s : 0;
  g.hi = e < p.width ? e : p.width;
  int64_t nvb = 0;
  if (g.hi > g.lo) nvb = div_b(g.hi - g.s + p.B - 1);
  if (nvb > p.nblocks) nvb = p.nblocks;
  g.nvb = (int32_t)nvb;
  g.pin = -1;
  if (pin && e > g.s) {
    const int64_t q = div_b(e - g.s - 1);
    if (q < p.nblocks) g.pin = (int32_t)q;
  }
  g.nsel = g.nvb > g.pin + 1 ? g.nvb : g.pin + 1;
  return g;
}

// Orders this wave's LDS accesses (a wave's LDS operations complete in
// issue order; this keeps the compiler from moving them across).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// This wave's index in the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_index() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Streams blocks [b0, b1) (b1 <= nvb) of a row on the vector path
// (dsa_geom::vec_path_ok): B = 4*G, and every float4 loaded is a whole unit
// of the window (stream_geom.h); the window's partial last unit, if any, is
// read with up to three scalar loads by the lane that owns it.  The chunk's
// 1 KiB tiles are dealt to `nw` waves; this is wave `wv`, which takes tiles
// wv, wv + nw, ... in rounds of U.  Calls emit(b, max) once per block, from
// one lane of the block.
//
// The loads are branch-free: a lane past the chunk's last whole unit
// re-reads that unit and is masked.  ROLL: tile j's load for the next round
// is issued as soon as tile j has been reduced, so U loads stay in flight
// across rounds instead of draining at each round's end.  Emits into HBM
// then sit in the same in-order memory counter as the loads; whether
// rolling still pays is measured per caller.  FULL: a tile wholly inside the
// window (a wave-uniform test) skips the per-unit masks.
template <int G, int U, bool ROLL, bool FULL, class Emit>
__device__ __forceinline__ void stream_vec(const RowGeom& g, int32_t b0, int32_t b1, int wv,
                                           int nw, const Emit& emit) {
  const int lane = threadIdx.x & 63;
  const int32_t span = (int32_t)(g.hi - g.s);  // window columns from s
  const dsa_geom::VecChunk c = dsa_geom::vec_chunk(span, b0, b1, G);
  if (wv >= c.ntiles) return;
  const float ninf = -__builtin_inff();
  const char* cbase = reinterpret_cast<const char*>(g.row + g.s);
  // The partial unit: its owner lane reads its 1-3 columns before the
  // float4 loads are issued.  Loads return in order, so once the first
  // tile's float4 has arrived the tail has too; it is then moved to a
  // scalar register (readlane), which keeps it out of the vector registers
  // of the streaming loop.
  float tail_v = ninf;
  if (c.tail_tile >= 0 && c.tail_tile % nw == wv && lane == c.tail_lane) {
    const float* tp = g.row + g.s;
    const float t0 = load_stream(tp + dsa_geom::vec_tail_col(c, 0));
    const float t1 = load_stream(tp + dsa_geom::vec_tail_col(c, 1));
    const float t2 = load_stream(tp + dsa_geom::vec_tail_col(c, 2));
    tail_v = fmaximum(t0, fmaximum(t1, t2));
  }
  float tail = ninf;  // wave-uniform: set once the first round is in flight
  // uniform base + 32-bit byte offset: the scalar-base form of the load
  auto load = [&](int32_t t) -> float4 {
    const uint32_t off = (uint32_t)dsa_geom::vec_load_unit(c, t, lane) << 4;
    return load_stream(static_cast<const void*>(cbase + off));
  };
  auto reduce = [&](int32_t t, const float4& x4) {
    const int32_t u = c.ub + (t << 6) + lane;
    float m;
    if (FULL && c.ub + (t << 6) + 64 <= c.full_end) {  // wave-uniform: all whole units
      m = fmaximum(fmaximum(x4.x, x4.y), fmaximum(x4.z, x4.w));
    } else {
      const int32_t cols = dsa_geom::vec_unit_cols(c, span, u);
      const float m4 = fmaximum(fmaximum(x4.x, x4.y), fmaximum(x4.z, x4.w));
      m = cols == 4 ? m4 : (cols > 0 ? tail : ninf);
    }
    if constexpr (Emit::kKey) {
      // emitters of keys: the group maximum taken on the keys, whose DPP
      // moves fold into the integer maximum (one instruction per step
      // instead of a move and a float maximum): large prefill 151.66 ->
      // 151.36 us, prefill chunk 13.48 -> 13.36, decode batch 6.94 -> 6.88;
      // with the row broadcasts of group_umax_tail at G = 32, long-context
      // decode 14.20 -> 13.80 (14.10 with them on floats)
      const uint32_t k = group_umax_tail<G>(order_key(m));
      if (t < c.ntiles) {
        const int32_t b = b0 + (((t << 6) + lane) / G);
        if ((lane % G) == kTailLane<G> && b < b1) emit.key(b, k);
      }
    } else {
      m = group_max_tail<G>(m);
      if (t < c.ntiles) {
        const int32_t b = b0 + (((t << 6) + lane) / G);
        if ((lane % G) == kTailLane<G> && b < b1) emit(b, m);
      }
    }
  };
  const int32_t step = nw * U;
  float4 v[U];
  if constexpr (ROLL) {
    const int32_t rounds = (c.ntiles - wv + step - 1) / step;  // wave-uniform, >= 1
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = load(wv + j * nw);
    tail = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tail_v), c.tail_lane));
    int32_t t0 = wv;
    for (int32_t r = 1; r < rounds; ++r, t0 += step) {
#pragma unroll
      for (int j = 0; j < U; ++j) {
        reduce(t0 + j * nw, v[j]);
        v[j] = load(t0 + step + j * nw);
      }
    }
#pragma unroll
    for (int j = 0; j < U; ++j) reduce(t0 + j * nw, v[j]);
  } else {
    tail = __builtin_bit_cast(
        float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, tail_v), c.tail_lane));
    for (int32_t t0 = wv; t0 < c.ntiles; t0 += step) {
#pragma unroll
      for (int j = 0; j < U; ++j) v[j] = load(t0 + j * nw);
#pragma unroll
      for (int j = 0; j < U; ++j) reduce(t0 + j * nw, v[j]);
    }
  }
}

// Any block size and alignment: gl = largest power of two <= min(B, 64)
// lanes share a block, each striding over the block's window columns with
// scalar loads, four in flight; a masked slot re-reads the block's first
// window column (stream_geom.h).  Blocks are dealt to `nw` waves; this is
// wave `wv`.
template <class Emit>
__device__ __forceinline__ void stream_scalar(const RowGeom& g, int32_t B, int32_t b0,
                                              int32_t b1, int wv, int nw, const Emit& emit) {
  const int lane = threadIdx.x & 63;
  int gl = 1;
  while (gl * 2 <= B && gl < 64) gl *= 2;
  const int per_wave = 64 / gl;
  const int sub = lane & (gl - 1);
  const float ninf = -__builtin_inff();
  for (int64_t bb = (int64_t)b0 + (int64_t)wv * per_wave; bb < b1;
       bb += (int64_t)nw * per_wave) {
    const int64_t b = bb + lane / gl;
    const dsa_geom::ScalarBlock blk = dsa_geom::scalar_block(g.s, g.lo, g.hi, b, B, b1);
    float m = ninf;
    for (int64_t c = blk.lo + sub; c < blk.hi; c += 4 * gl) {
      float x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        x[q] = load_stream(g.row + dsa_geom::scalar_load_col(blk, c + (int64_t)q * gl));
#pragma unroll
      for (int q = 0; q < 4; ++q) m = fmaximum(m, c + (int64_t)q * gl < blk.hi ? x[q] : ninf);
    }
    m = group_max_dyn(m, gl);
    if (sub == 0 && b < b1) emit((int32_t)b, m);
  }
}

template <int G, int U, bool ROLL, bool FULL = false, class Emit>
__device__ __forceinline__ void stream_blocks(const Params& p, const RowGeom& g, int32_t b0,
                                              int32_t b1, int wv, int nw, const Emit& emit) {
  if (b1 <= b0) return;
  if constexpr (G > 0) {
    if (dsa_geom::vec_path_ok(reinterpret_cast<uintptr_t>(g.row + g.s), g.s, g.hi - g.s)) {
      stream_vec<G, U, ROLL, FULL>(g, b0, b1, wv, nw, emit);
      return;
    }
  }
  stream_scalar(g, p.B, b0, b1, wv, nw, emit);
}

// Emitters take a block's maximum as a float (operator()) and, where kKey,
// as its order-preserving key (key()), the form the vector path reduces in.
struct EmitKey {  // LDS or HBM key array of one row
  static constexpr bool kKey = true;
  uint32_t* keys;
  __device__ void operator()(int32_t b, float m) const { keys[b] = order_key(m); }
  __device__ void key(int32_t b, uint32_t k) const { keys[b] = k; }
};

struct EmitScore {
  static constexpr bool kKey = false;
  float* row;
  int32_t pin;
  __device__ void operator()(int32_t b, float m) const {
    row[b] = b == pin ? __builtin_inff() : canonical(m);
  }
};

template <bool KEYS>
struct EmitStaged {  // scores or codes of one row chunk, staged in LDS
  static constexpr bool kKey = KEYS;
  uint32_t* lds;
  int32_t b0, pin;
  __device__ void operator()(int32_t b, float m) const {
    lds[b - b0] = KEYS ? (b == pin ? kKeyPosInf : order_key(m))
                       : __float_as_uint(b == pin ? __builtin_inff() : canonical(m));
  }
  __device__ void key(int32_t b, uint32_t k) const { lds[b - b0] = b == pin ? kKeyPosInf : k; }
};

struct EmitScoreKey {  // the same scores as order-preserving uint32 codes
  static constexpr bool kKey = true;
  uint32_t* row;
  int32_t pin;
  __device__ void operator()(int32_t b, float m) const {
    row[b] = b == pin ? kKeyPosInf : order_key(m);
  }
  __device__ void key(int32_t b, uint32_t k) const { row[b] = b == pin ? kKeyPosInf : k; }
};

// ---------------------------------------------------------------- select --
//
// Top-k of one row's block keys, in four steps with no sort of the whole row:
//  (A) every key becomes a rank key (-inf -> 0 "no candidate", -0 -> +0);
//      group l of the 64 groups holds the keys i with i mod 64 == l, and
//      each group takes its maximum;
//  (C) T0 = the keff-th largest group maximum, keff = min(k, #nonzero keys).
//      keff groups each hold a key >= T0, so T0 is a lower bound on the
//      keff-th largest key: every selected key is >= T0.  For 32 < k <= 64
//      the same holds with 128 groups; for larger k the bound comes from
//      radix passes instead (bound_radix);
//  (E) the keys >= T0 (the candidates, few for any spread of values) are
//      compacted into LDS as 64-bit words (rank key << 32 | ~block id), which
//      are distinct and order exactly as the selection order (key descending,
//      then id ascending);
//  (G) each candidate's rank is the count of larger words; ranks < keff give
//      the output slots directly.
// More than kCandCap candidates (heavy ties at T0, or k in the hundreds)
// fall back to an exact one-wave radix select over the LDS keys.

constexpr int kCtlWords = 48;       // per-row control words in LDS
constexpr int kCtlValid = 0;        // #nonzero rank keys
constexpr int kCtlCand = 1;         // #candidates (atomic add)
constexpr int kCtlT0 = 2;           // candidate threshold
constexpr int kCtlArrival = 8;      // pair plan: the row counter before this arrival (2 words)
constexpr int kCtlSlotCount = 16;   // 16 per-wave slots: nonzero keys
constexpr int kCtlSlotBound = 32;   // 16 per-wave slots: bound candidates
constexpr int kCandCap = 256;   // candidates held in LDS (64-bit words)
constexpr int kAreaMinWords = 1024;  // candidates, or one row of 64 maxima per wave
// the rank reads whole runs of 8 candidates; up to 8 maxima rows of 64 words
// may precede the candidate store in the area
static_assert(kCandCap % 8 == 0 && kAreaMinWords >= 8 * 64 + 2 * kCandCap, "select area layout");

__device__ __forceinline__ uint32_t group_umax_dyn(uint32_t v, int gl) {
  switch (gl) {
    case 1: return v;
    case 2: return group_umax<2>(v);
    case 4: return group_umax<4>(v);
    case 8: return group_umax<8>(v);
    case 16: return group_umax<16>(v);
    case 32: return group_umax<32>(v);
    default: return group_umax<64>(v);
  }
}

template <bool WG>
__device__ __forceinline__ void row_barrier() {
  if constexpr (WG) __syncthreads();
  else wave_sync();
}

// Score key of block i < nsel of a row whose blocks [0, nvb) sit in keys[].
__device__ __forceinline__ uint32_t block_key(const uint32_t* keys, const RowGeom& g, int32_t i) {
  const uint32_t raw = keys[i < g.nvb ? i : 0];  // keys[0] is in bounds; masked below
  return i == g.pin ? kKeyPosInf : (i < g.nvb ? raw : kKeyNegInf);
}

// Candidate word: rank key above, inverted id below; 0 for a non-candidate.
__device__ __forceinline__ uint64_t cand_word(uint32_t rk, uint32_t i) {
  return rk ? (((uint64_t)rk << 32) | (uint64_t)(~i)) : 0ull;
}

// Ranks cand[0, ncand) (distinct words, 0 = empty): slot r < keff of the
// output takes the id of the word with r larger words.  Wave `wave` of `nw`
// takes every nw-th group of 64 candidates.  WIDE: runs of 16 words (eight
// reads in flight, two independent sums) ahead of the runs of 8, a shorter
// chain for kernels that can spare the registers.
template <bool WIDE = false>
__device__ __forceinline__ void rank_candidates(const uint64_t* cand, int32_t ncand, int32_t keff,
                                                int32_t* out_row, int wave, int nw) {
  const int lane = threadIdx.x & 63;
  const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(cand);
  for (int32_t base = wave * 64; base < ncand; base += nw * 64) {
    const int32_t idx = base + lane;
    const uint64_t ci = idx < ncand ? cand[idx] : 0ull;
    uint32_t r = 0;
    int32_t j = 0;
    if constexpr (WIDE) {
      uint32_t r1 = 0;
      for (; j + 16 <= ncand; j += 16) {
        const ulonglong2 a = c2[(j >> 1) + 0], b = c2[(j >> 1) + 1];
        const ulonglong2 c = c2[(j >> 1) + 2], d = c2[(j >> 1) + 3];
        const ulonglong2 e = c2[(j >> 1) + 4], f = c2[(j >> 1) + 5];
        const ulonglong2 g = c2[(j >> 1) + 6], h = c2[(j >> 1) + 7];
        r += (uint32_t)(a.x > ci) + (uint32_t)(a.y > ci) + (uint32_t)(b.x > ci) +
             (uint32_t)(b.y > ci) + (uint32_t)(c.x > ci) + (uint32_t)(c.y > ci) +
             (uint32_t)(d.x > ci) + (uint32_t)(d.y > ci);
        r1 += (uint32_t)(e.x > ci) + (uint32_t)(e.y > ci) + (uint32_t)(f.x > ci) +
              (uint32_t)(f.y > ci) + (uint32_t)(g.x > ci) + (uint32_t)(g.y > ci) +
              (uint32_t)(h.x > ci) + (uint32_t)(h.y > ci);
      }
      r += r1;
    }
    for (; j + 8 <= ncand; j += 8) {  // broadcast reads, four in flight
      const ulonglong2 a = c2[(j >> 1) + 0], b = c2[(j >> 1) + 1];
      const ulonglong2 c = c2[(j >> 1) + 2], d = c2[(j >> 1) + 3];
      r += (uint32_t)(a.x > ci) + (uint32_t)(a.y > ci) + (uint32_t)(b.x > ci) + (uint32_t)(b.y > ci) +
           (uint32_t)(c.x > ci) + (uint32_t)(c.y > ci) + (uint32_t)(d.x > ci) + (uint32_t)(d.y > ci);
    }
    if (j < ncand) {  // the last 1-7 words: one round of loads, the words past ncand
      // masked (the store holds kCandCap words, a multiple of 8, and ncand <=
      // kCandCap); one load and wait per word measured 7.64 -> 7.56 us on the
      // decode batch
      const ulonglong2 a = c2[(j >> 1) + 0], b = c2[(j >> 1) + 1];
      const ulonglong2 c = c2[(j >> 1) + 2], d = c2[(j >> 1) + 3];
      const int32_t m = ncand - j;  // wave-uniform, 1..7
      r += (uint32_t)(a.x > ci) + (uint32_t)(m > 1 && a.y > ci) + (uint32_t)(m > 2 && b.x > ci) +
           (uint32_t)(m > 3 && b.y > ci) + (uint32_t)(m > 4 && c.x > ci) +
           (uint32_t)(m > 5 && c.y > ci) + (uint32_t)(m > 6 && d.x > ci);
    }
    if (idx < ncand && ci != 0ull && r < (uint32_t)keff) out_row[r] = (int32_t)(~(uint32_t)ci);
  }
}

// ncand <= 64 candidates on nw = 2-8 waves: every wave ranks all of them
// against its own share of the list (one to four rounds of broadcast reads
// instead of ncand / 8 dependent rounds in one wave); the partial counts
// meet in `part` (nw rows of 64 words) and wave 0 adds them up and stores.
// Holds a workgroup barrier.  Decode batch 7.53 -> 7.22 us, long-context
// decode 14.59 -> 14.43, against rank_candidates in wave 0 alone.
__device__ __forceinline__ void rank_candidates_split(const uint64_t* cand, int32_t ncand,
                                                      int32_t keff, int32_t* out_row,
                                                      uint32_t* part, int wave, int nw) {
  const int lane = threadIdx.x & 63;
  const ulonglong2* c2 = reinterpret_cast<const ulonglong2*>(cand);
  const uint64_t ci = lane < ncand ? cand[lane] : 0ull;
  const int32_t per = (((ncand + nw - 1) / nw) + 7) & ~7;  // a multiple of 8
  const int32_t j0 = wave * per;
  const int32_t j1 = j0 + per < ncand ? j0 + per : ncand;
  uint32_t r = 0;
  for (int32_t j = j0; j < j1; j += 8) {  // words past j1 (below 64) are masked
    const ulonglong2 a = c2[(j >> 1) + 0], b = c2[(j >> 1) + 1];
    const ulonglong2 c = c2[(j >> 1) + 2], d = c2[(j >> 1) + 3];
    const int32_t m = j1 - j;  // wave-uniform, >= 1
    r += (uint32_t)(a.x > ci) + (uint32_t)(m > 1 && a.y > ci) + (uint32_t)(m > 2 && b.x > ci) +
         (uint32_t)(m > 3 && b.y > ci) + (uint32_t)(m > 4 && c.x > ci) +
         (uint32_t)(m > 5 && c.y > ci) + (uint32_t)(m > 6 && d.x > ci) +
         (uint32_t)(m > 7 && d.y > ci);
  }
  part[wave * 64 + lane] = r;
  __syncthreads();
  if (wave == 0) {
    uint32_t t = 0;
    for (int w = 0; w < nw; ++w) t += part[w * 64 + lane];
    if (lane < ncand && t < (uint32_t)keff) out_row[t] = (int32_t)(~(uint32_t)ci);
  }
}

// Radix select (8-bit digits from the top) over the LDS rank keys of one
// wave's slot array (slot j of lane l is key j*64 + l): the selection is every
// key >= tg, then the first need_eq keys equal to T in id order.
__device__ void threshold_radix_lds(const uint32_t* keys, int32_t nsel, uint32_t keff,
                                    uint32_t* hist, uint32_t& tg, uint32_t& T, int32_t& need_eq) {
  const int lane = threadIdx.x & 63;
  const int32_t nj = (nsel + 63) >> 6;
  uint32_t prefix = 0u, remaining = keff;
  for (int shift = 24; shift >= 0; shift -= 8) {
    reinterpret_cast<uint4*>(hist)[lane] = make_uint4(0u, 0u, 0u, 0u);
    wave_sync();
    const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
    for (int32_t j = 0; j < nj; ++j) {
      const int32_t i = j * 64 + lane;
      const uint32_t kj = i < nsel ? rank_key(keys[i]) : 0u;
      if (kj != 0u && (kj & hmask) == prefix) atomicAdd(&hist[(kj >> shift) & 255u], 1u);
    }
    wave_sync();
    // lane l holds bins 255-4l (q = 0) down to 252-4l (q = 3); `a0` counts the
    // matching keys in higher bins (the lanes before this one)
    const uint4 h = reinterpret_cast<const uint4*>(hist)[63 - lane];
    const uint32_t tot = h.x + h.y + h.z + h.w;
    uint32_t inc = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_up(inc, off);
      if (lane >= off) inc += y;
    }
    const uint32_t a0 = inc - tot, a1 = a0 + h.w, a2 = a1 + h.z, a3 = a2 + h.y;
    const bool h0 = a0 < remaining && remaining <= a1;
    const bool h1 = a1 < remaining && remaining <= a2;
    const bool h2 = a2 < remaining && remaining <= a3;
    const bool h3 = a3 < remaining && remaining <= a3 + h.x;
    const uint64_t hit = __ballot(h0 || h1 || h2 || h3);
    const int src = (int)__builtin_ctzll(hit);  // exactly one lane holds the bucket
    const uint32_t q = h0 ? 0u : (h1 ? 1u : (h2 ? 2u : 3u));
    const uint32_t aq = h0 ? a0 : (h1 ? a1 : (h2 ? a2 : a3));
    const uint32_t cq = h0 ? h.w : (h1 ? h.z : (h2 ? h.y : h.x));
    const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)(255u - 4u * lane - q), src);
    const uint32_t rem = (uint32_t)__builtin_amdgcn_readlane((int)(remaining - aq), src);
    const uint32_t cb = (uint32_t)__builtin_amdgcn_readlane((int)cq, src);
    prefix |= d << shift;
    wave_sync();
    if (rem == cb) {  // the whole bucket is taken: every key >= prefix
      tg = prefix;
      T = 0u;
      need_eq = 0;
      return;
    }
    remaining = rem;
  }
  T = prefix;
  tg = prefix + 1u;
  need_eq = (int32_t)remaining;
}

// Exact top-k by one wave over LDS keys[0, nsel) (pin and -inf fill already
// in place), for rows the candidate bound cannot shrink to kCandCap.
// `scratch`: 16-byte aligned, max(512, 2*kcap) words.
__device__ void select_wave_exact(const uint32_t* keys, int32_t nsel, int32_t k, int32_t kcap,
                                  int32_t* out_row, uint32_t* scratch) {
  const int lane = threadIdx.x & 63;
  const int32_t nj = (nsel + 63) >> 6;
  uint32_t nvalid = 0;
  for (int32_t j = 0; j < nj; ++j) {
    const int32_t i = j * 64 + lane;
    nvalid += (uint32_t)__popcll(__ballot(i < nsel && rank_key(keys[i]) != 0u));
  }
  const int32_t keff = (uint32_t)k < nvalid ? k : (int32_t)nvalid;
  if (keff > 0) {
    uint32_t tg = 1u, T = 0u;
    int32_t need_eq = 0;
    if ((uint32_t)keff < nvalid) threshold_radix_lds(keys, nsel, (uint32_t)keff, scratch, tg, T, need_eq);
    // keys >= tg go to sel_* in id order; the first need_eq keys equal to T
    // fill the last slots directly
    uint32_t* sel_key = scratch;
    uint32_t* sel_id = scratch + kcap;
    const int32_t c_gt = keff - need_eq;
    uint32_t pos_gt = 0, pos_eq = 0;
    for (int32_t j = 0; j < nj; ++j) {
      const int32_t i = j * 64 + lane;
      const uint32_t kj = i < nsel ? rank_key(keys[i]) : 0u;
      const bool is_gt = kj >= tg && kj != 0u;
      const bool is_eq = need_eq > 0 && kj == T && kj != 0u;
      const uint64_t m_gt = __ballot(is_gt);
      const uint64_t m_eq = __ballot(is_eq);
      if (is_gt) {
        const uint32_t r = pos_gt + lanes_below(m_gt);
        sel_key[r] = kj;
        sel_id[r] = (uint32_t)i;
      }
      if (is_eq) {
        const uint32_t r = pos_eq + lanes_below(m_eq);
        if (r < (uint32_t)need_eq) out_row[c_gt + (int32_t)r] = i;
      }
      pos_gt += (uint32_t)__popcll(m_gt);
      pos_eq += (uint32_t)__popcll(m_eq);
    }
    wave_sync();
    // order the outright selection: rank = #larger + #equal earlier in id order
    for (int32_t i = lane; i < c_gt; i += 64) {
      const uint32_t ki = sel_key[i];
      int32_t r = 0;
      for (int32_t j = 0; j < c_gt; ++j) {
        const uint32_t kj = sel_key[j];
        r += (kj > ki) || (kj == ki && j < i);
      }
      out_row[r] = (int32_t)sel_id[i];
    }
    wave_sync();
  }
  for (int32_t j = keff + lane; j < k; j += 64) out_row[j] = -1;
}

// Rank key of block i for the select; 0 for i >= nsel.  The LDS read is
// unconditional (clamped to a valid index) so the code stays branch-free.
__device__ __forceinline__ uint32_t select_rank_key(const uint32_t* keys, const RowGeom& g,
                                                    int32_t i) {
  const uint32_t raw = keys[i < g.nvb ? i : 0];
  uint32_t key = i < g.nvb ? raw : kKeyNegInf;
  key = i == g.pin ? kKeyPosInf : key;
  return i < g.nsel ? rank_key(key) : 0u;
}

// Clears the LDS state select_row expects zeroed: the first 256 words of
// `area` (the radix histogram) and the control counters below the per-wave
// slots.  Thread t clears area[t] (and area[t + nt]): with nt = 128 each wave
// clears its own maxima row.  Call before the barrier that precedes
// select_row (the streaming never touches these words).
__device__ __forceinline__ void select_row_prepare(uint32_t* ctl, uint32_t* area, int tid, int nt) {
  for (int t = tid; t < 256; t += nt) area[t] = 0u;
  if (tid < kCtlSlotCount) ctl[tid] = 0u;  // per-wave slots are written before they are read
}

// A lane's rank keys of one row, read from LDS once when the row has at most
// kKeyRegs keys per lane, so the passes over the keys (counts, histograms,
// compaction) work from registers instead of one dependent LDS read per key.
// Iteration j of wave `wave` covers key i = wave*64 + j*nt + lane.  Only the
// narrow workgroups of many-row selects (several keys per lane) gain: with
// one key per lane the cache costs registers and occupancy, so kernels
// choose it at compile time (KC).
constexpr int kKeyRegs = 8;
struct LaneKeys {
  uint32_t v[kKeyRegs];
  int32_t nj;   // iterations per lane (wave-uniform)
  bool cached;  // nj <= kKeyRegs: v[0, nj) hold the keys
};

template <bool KC>
__device__ __forceinline__ LaneKeys lane_keys(const uint32_t* keys, const RowGeom& g, int wave,
                                              int nt) {
  const int lane = threadIdx.x & 63;
  const int32_t first = wave * 64;
  LaneKeys lk;
  lk.nj = g.nsel > first ? (g.nsel - first + nt - 1) / nt : 0;
  lk.cached = KC && lk.nj <= kKeyRegs;
#pragma unroll
  for (int j = 0; j < kKeyRegs; ++j)  // all reads in flight at once
    lk.v[j] = (lk.cached && j < lk.nj) ? select_rank_key(keys, g, first + j * nt + lane) : 0u;
  return lk;
}

// Calls f(i, rank key of i) for this lane's keys, in iteration order (the
// same order for every lane, so f may hold ballots).
// HK (keys in HBM): eight keys loaded per step before f sees them.
template <bool HK = false, class F>
__device__ __forceinline__ void for_lane_keys(const LaneKeys& lk, const uint32_t* keys,
                                              const RowGeom& g, int wave, int nt, F&& f) {
  const int lane = threadIdx.x & 63;
  if (lk.cached) {
#pragma unroll
    for (int j = 0; j < kKeyRegs; ++j)
      if (j < lk.nj) f(wave * 64 + j * nt + lane, lk.v[j]);  // wave-uniform
  } else if constexpr (HK) {
    for (int32_t base = wave * 64; base < g.nsel; base += 8 * nt) {  // wave-uniform
      uint32_t kv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) kv[q] = select_rank_key(keys, g, base + q * nt + lane);
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (base + q * nt < g.nsel) f(base + q * nt + lane, kv[q]);  // wave-uniform
    }
  } else {
    for (int32_t base = wave * 64; base < g.nsel; base += nt)  // wave-uniform
      f(base + lane, select_rank_key(keys, g, base + lane));
  }
}

// Candidate bound by radix passes, for larger k: 8-bit digits of the rank
// keys from the top, one workgroup histogram per pass (LDS atomic adds, which
// stay cheap under conflicts), wave 0 finds the digit bucket that holds the
// keff-th largest key; it stops as soon as the keys at or above the bucket's
// lowest value fit the candidate store (or all 32 bits are fixed).  Leaves
// T0 in ctl[kCtlT0] and the nonzero count in ctl[kCtlValid].  `hist` is 256
// zeroed words.
constexpr int kCtlPrefix = 3;   // radix: digits fixed so far
constexpr int kCtlRemain = 4;   // radix: keys still needed below the prefix's higher part
constexpr int kCtlAbove = 5;    // radix: keys above the current bucket
constexpr int kCtlDone = 6;     // radix: bound final

// EXACT: no early stop, every digit fixed: T0 is then the keff-th largest
// key, kCtlAbove the count of keys above it and kCtlRemain the keys equal to
// it that complete the keff.
template <bool WG, bool HK = false, bool EXACT = false>
__device__ __forceinline__ void bound_radix(const RowGeom& g, int32_t k, const uint32_t* keys,
                                            const LaneKeys& lk, uint32_t* ctl, uint32_t* hist,
                                            int wave, int nw) {
  const int lane = threadIdx.x & 63;
  const int nt = nw * 64;
  uint32_t prefix = 0u, hmask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    uint32_t nv = 0u;
    for_lane_keys<HK>(lk, keys, g, wave, nt, [&](int32_t, uint32_t rk) {
      if (rk != 0u && (rk & hmask) == prefix) atomicAdd(&hist[(rk >> shift) & 255u], 1u);
      if (shift == 24) nv += (uint32_t)__popcll(__ballot(rk != 0u));
    });
    if (shift == 24 && lane == 0 && nv != 0u) atomicAdd(&ctl[kCtlValid], nv);
    row_barrier<WG>();
    if (wave == 0) {
      uint32_t remaining, above;
      if (shift == 24) {
        const uint32_t nvalid = ctl[kCtlValid];
        remaining = (uint32_t)k < nvalid ? (uint32_t)k : nvalid;
        above = 0u;
      } else {
        remaining = ctl[kCtlRemain];
        above = ctl[kCtlAbove];
      }
      // lane l holds bins 255-4l (q = 0) down to 252-4l (q = 3); a0 counts
      // the matching keys in higher bins (the lanes before this one)
      uint4* h4 = reinterpret_cast<uint4*>(hist);
      const uint4 h = h4[63 - lane];
      h4[63 - lane] = make_uint4(0u, 0u, 0u, 0u);  // zeroed for the next pass
      const uint32_t tot = h.x + h.y + h.z + h.w;
      uint32_t inc = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(inc, off);
        if (lane >= off) inc += y;
      }
      const uint32_t a0 = inc - tot, a1 = a0 + h.w, a2 = a1 + h.z, a3 = a2 + h.y;
      const bool h0 = a0 < remaining && remaining <= a1;
      const bool h1 = a1 < remaining && remaining <= a2;
      const bool h2 = a2 < remaining && remaining <= a3;
      const bool h3 = a3 < remaining && remaining <= a3 + h.x;
      const uint64_t hit = __ballot(h0 || h1 || h2 || h3);
      if (lane == 0) {
        if (hit == 0ull) {  // keff == 0: nothing to select
          ctl[kCtlT0] = 0xFFFFFFFFu;
          ctl[kCtlDone] = 1u;
        }
      }
      if (hit != 0ull) {
        const int src = (int)__builtin_ctzll(hit);
        const uint32_t qd = h0 ? 0u : (h1 ? 1u : (h2 ? 2u : 3u));
        const uint32_t aq = h0 ? a0 : (h1 ? a1 : (h2 ? a2 : a3));
        const uint32_t cq = h0 ? h.w : (h1 ? h.z : (h2 ? h.y : h.x));
        const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)(255u - 4u * lane - qd), src);
        const uint32_t above_d = (uint32_t)__builtin_amdgcn_readlane((int)aq, src);
        const uint32_t cnt_d = (uint32_t)__builtin_amdgcn_readlane((int)cq, src);
        if (lane == 0) {
          const uint32_t np = prefix | (d << shift);
          const uint32_t na = above + above_d;
          ctl[kCtlPrefix] = np;
          ctl[kCtlRemain] = remaining - above_d;
          ctl[kCtlAbove] = na;
          if ((!EXACT && na + cnt_d <= (uint32_t)kCandCap) || shift == 0) {
            ctl[kCtlT0] = np;  // keys >= np: the na above plus the bucket's cnt_d
            ctl[kCtlDone] = 1u;
          }
        }
      }
    }
    row_barrier<WG>();
    if (ctl[kCtlDone] != 0u) return;  // workgroup-uniform
    prefix = ctl[kCtlPrefix];
    hmask |= 255u << shift;
  }
}

// Sum over aligned groups of 16 lanes (a DPP row); every lane of the row ends
// with the row's sum.  All 64 lanes must be active.
__device__ __forceinline__ uint32_t row_sum16(uint32_t v) {
  v += dpp_u32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_u32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_u32<0x141>(v);  // row_half_mirror
  v += dpp_u32<0x140>(v);  // row_mirror
  return v;
}

// Candidate bounds of select_row_general.
constexpr int kBoundGroups64 = 0;   // k <= 32
constexpr int kBoundRadix = 1;      // k > 64
constexpr int kBoundGroups128 = 2;  // 32 < k <= 64

// The bound select_row uses for k on nw waves (also chosen on the host for
// kernels compiled for one bound).
__host__ __device__ inline int select_bound(int32_t k, int nw) {
  if (k <= 32) return kBoundGroups64;
  if (k <= 64 && ((nw & 1) == 0 || nw <= 8)) return kBoundGroups128;
  return kBoundRadix;
}

// T0 from group maxima held one (N = 1: 64 groups) or two (N = 2: 128
// groups) per lane of one wave: the largest value with at least kq maxima at
// or above it (the kq-th largest maximum), bit by bit from the top, each
// step a ballot per maximum register.  Any t with at least kq maxima >= t
// bounds the keff-th key from below; the exact kq-th maximum only trims
// candidates.  So the search stops after the top 16 bits unless more than
// kq + kq/4 maxima lie at or above t (maxima packed within 2^16 codes of
// each other, where the lower bits still separate them).  Each step is a
// dependent chain of ballots and scalar arithmetic.
template <int N>
__device__ __forceinline__ uint32_t maxima_bound(uint32_t g0, uint32_t g1, uint32_t kq) {
  uint32_t t = 0u, ct = 64u * N;  // ct: maxima >= t (all of them for t = 0)
#pragma unroll
  for (int bit = 31; bit >= 16; --bit) {
    const uint32_t c = t | (1u << bit);
    uint32_t cnt = (uint32_t)__popcll(__ballot(g0 >= c));
    if constexpr (N == 2) cnt += (uint32_t)__popcll(__ballot(g1 >= c));
    if (cnt >= kq) {
      t = c;
      ct = cnt;
    }
  }
  if (ct > kq + (kq >> 2)) {  // wave-uniform
    // Fewer than kq maxima lie above the 2^16-code bucket [t, t + 2^16),
    // so the kq-th largest lies in it: when every maximum in the bucket has
    // one value (ties), that value is the exact bound and the 16 low steps
    // are skipped.
    const bool in0 = g0 >= t && g0 - t < 65536u;
    uint32_t hi = in0 ? g0 : 0u, nlo = in0 ? ~g0 : 0u;
    if constexpr (N == 2) {
      const bool in1 = g1 >= t && g1 - t < 65536u;
      hi = umax(hi, in1 ? g1 : 0u);
      nlo = umax(nlo, in1 ? ~g1 : 0u);
    }
    hi = (uint32_t)__builtin_amdgcn_readlane((int)group_umax_tail<64>(hi), 63);
    nlo = (uint32_t)__builtin_amdgcn_readlane((int)group_umax_tail<64>(nlo), 63);
    if (hi == ~nlo) {  // wave-uniform
      t = hi;
    } else {
      for (int bit = 15; bit >= 0; --bit) {
        const uint32_t c = t | (1u << bit);
        uint32_t cnt = (uint32_t)__popcll(__ballot(g0 >= c));
        if constexpr (N == 2) cnt += (uint32_t)__popcll(__ballot(g1 >= c));
        if (cnt >= kq) t = c;
      }
    }
  }
  return t;
}

// The exact select of a row whose keys sit in HBM (select_keys_hbm_kernel),
// for rows the candidate bound cannot shrink to kCandCap (k above it, or
// ties at the bound), by the whole workgroup: radix passes fix the keff-th
// largest key T, the keys above T (fewer than keff, so they fit the area)
// are ranked by count, and the keys equal to T fill the remaining slots in
// id order, 8 x nt ids per step until enough are placed.  Called by every
// wave after the compaction's barrier.
template <bool WG>
__device__ void exact_select_hbm(const RowGeom& g, int32_t k, const uint32_t* keys,
                                 const LaneKeys& lk, uint32_t* ctl, uint32_t* area,
                                 int32_t* out_row, int wave, int nw) {
  const int lane = threadIdx.x & 63;
  const int tid = wave * 64 + lane;
  const int nt = nw * 64;
  row_barrier<WG>();  // every wave has read the candidate count
  for (int t = tid; t < 256; t += nt) area[t] = 0u;  // the radix histogram
  if (tid == 0) {
    ctl[kCtlValid] = 0u;
    ctl[kCtlCand] = 0u;
    ctl[kCtlDone] = 0u;
  }
  row_barrier<WG>();
  bound_radix<WG, true, true>(g, k, keys, lk, ctl, area, wave, nw);
  const uint32_t nvalid = ctl[kCtlValid];
  const int32_t keff = (uint32_t)k < nvalid ? k : (int32_t)nvalid;
  if (keff > 0) {  // workgroup-uniform
    const uint32_t T = ctl[kCtlT0];
    const uint32_t above = ctl[kCtlAbove];  // keys > T: fewer than keff
    const uint32_t need_eq = (uint32_t)keff - above;
    uint64_t* cand = reinterpret_cast<uint64_t*>(area);
    for_lane_keys<true>(lk, keys, g, wave, nt, [&](int32_t i, uint32_t rk) {
      const bool c = rk > T;
      const uint64_t m = __ballot(c);
      if (m != 0ull) {
        uint32_t b0 = 0u;
        if (lane == 0) b0 = atomicAdd(&ctl[kCtlCand], (uint32_t)__popcll(m));
        b0 = (uint32_t)__builtin_amdgcn_readlane((int)b0, 0);
        if (c) cand[b0 + lanes_below(m)] = cand_word(rk, (uint32_t)i);
      }
    });
    row_barrier<WG>();
    rank_candidates(cand, (int32_t)above, (int32_t)above, out_row, wave, nw);
    row_barrier<WG>();  // the rank has read the candidates: the area takes the tie counts
    uint32_t* wcnt = area;  // [8][16]: the ties of each slice and wave of a step
    uint32_t run = 0u;      // ties placed by the earlier steps
    for (int32_t base = 0; base < g.nsel && run < need_eq; base += 8 * nt) {  // workgroup-uniform
      // slice q of the step holds ids base + q*nt + [0, nt), wave w its w-th 64
      uint32_t kv[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) kv[q] = select_rank_key(keys, g, base + q * nt + wave * 64 + lane);
      uint64_t m[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        m[q] = __ballot(kv[q] == T);  // 0 past nsel, and T > 0
        if (lane == 0) wcnt[q * 16 + wave] = (uint32_t)__popcll(m[q]);
      }
      row_barrier<WG>();
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        uint32_t before = 0u, total = 0u;
        for (int w = 0; w < nw; ++w) {
          const uint32_t c = wcnt[q * 16 + w];
          before += w < wave ? c : 0u;
          total += c;
        }
        const uint32_t pos = run + before + lanes_below(m[q]);
        if (kv[q] == T && pos < need_eq) out_row[above + pos] = base + q * nt + wave * 64 + lane;
        run += total;
      }
      row_barrier<WG>();  // the counts are rewritten by the next step
    }
  }
  for (int32_t j = keff + tid; j < k; j += nt) out_row[j] = -1;
}

// The general path of select_row (nsel > 64).  The candidate bound T0 comes
// from NG group maxima (NG = 64 or 128), group l holding the keys i with
// i mod NG == l: T0 = the keff-th largest group maximum (keff <= NG), or
// from bound_radix for larger k.  Same-address LDS max serialises per lane
// on this chip, so the maxima and the bound go through per-wave LDS rows
// and slots, not atomics.
template <bool WG, int BOUND, bool KC, bool PRE = false, bool HK = false>
__device__ __forceinline__ void select_row_general(const Params& p, const RowGeom& g,
                                                   uint32_t* keys, uint32_t* ctl, uint32_t* area,
                                                   int32_t* out_row, int wave, int nw,
                                                   const LaneKeys& pre) {
  const int lane = threadIdx.x & 63;
  const int tid = wave * 64 + lane;
  const int nt = nw * 64;
  const int32_t nsel = g.nsel, k = p.k;
  // with 64 groups on up to 8 waves, the candidates go past the waves' maxima
  // rows (area holds at least 1024 words): no barrier between the bound and
  // the compaction
  const bool past = BOUND == kBoundGroups64 && WG && nw <= 8;
  uint64_t* cand = reinterpret_cast<uint64_t*>(area + (past ? nw * 64 : 0));
  uint32_t t0, nvalid;
  const LaneKeys lk = PRE ? pre : lane_keys<KC>(keys, g, wave, nt);
  if constexpr (HK) {
    if (k > kCandCap) {  // no bound leaves k or more keys within the store: exact at once
      exact_select_hbm<WG>(g, k, keys, lk, ctl, area, out_row, wave, nw);
      return;
    }
  }

  if constexpr (BOUND == kBoundRadix) {
    bound_radix<WG, HK>(g, k, keys, lk, ctl, area, wave, nw);
    t0 = ctl[kCtlT0];
    nvalid = ctl[kCtlValid];
  } else if constexpr (BOUND == kBoundGroups128) {
    // (A) key i belongs to group (i & 63) + 64 * ((i >> 6) & 1).  A lane's
    // keys i = wave*64 + j*nt + lane fall in half (wave + j*nw) & 1: with an
    // even wave count always the wave's parity (one maxima row per wave),
    // with an odd one (nw <= 8) alternately (two rows per wave).
    uint32_t m0 = 0u, m1 = 0u, nv = 0u;
    const bool two_rows = (nw & 1) != 0;
    for_lane_keys<HK>(lk, keys, g, wave, nt, [&](int32_t i, uint32_t rk) {
      if (two_rows && ((i >> 6) & 1)) m1 = umax(m1, rk);
      else m0 = umax(m0, rk);  // one half per wave for an even wave count
      nv += (uint32_t)__popcll(__ballot(rk != 0u));
    });
    if (two_rows) {
      area[(2 * wave) * 64 + lane] = m0;
      area[(2 * wave + 1) * 64 + lane] = m1;
    } else {
      area[wave * 64 + lane] = umax(m0, m1);
    }
    if (lane == 0) ctl[kCtlSlotCount + wave] = nv;
    row_barrier<WG>();
    // (C) wave 0: the 128 group maxima (g0: groups 0-63, g1: 64-127), then
    // T0 bit by bit from the top: the largest value with at least keff
    // maxima at or above it is the keff-th largest maximum.  One wave does
    // it (the others wait at the barrier anyway): where many rows share a
    // CU, its compares are VALU time the other waves would also spend.
    nvalid = (uint32_t)__builtin_amdgcn_readlane(
        (int)row_sum16(lane < nw ? ctl[kCtlSlotCount + lane] : 0u), 0);
    if (wave == 0) {
      uint32_t g0 = 0u, g1 = 0u;
      for (int w = 0; w < nw; ++w) {
        if (two_rows) {
          g0 = umax(g0, area[(2 * w) * 64 + lane]);
          g1 = umax(g1, area[(2 * w + 1) * 64 + lane]);
        } else if (w & 1) {
          g1 = umax(g1, area[w * 64 + lane]);
        } else {
          g0 = umax(g0, area[w * 64 + lane]);
        }
      }
      const uint32_t kq = (uint32_t)k < nvalid ? (uint32_t)k : nvalid;
      const uint32_t t = maxima_bound<2>(g0, g1, kq);
      if (lane == 0) ctl[kCtlT0] = t;
    }
    row_barrier<WG>();  // T0 is out, and the maxima rows are read before candidates overwrite them
    t0 = ctl[kCtlT0];
  } else {
    // (A) per lane: maximum of its keys (all in group `lane`), into this
    // wave's row of `area`; per wave: its count of nonzero keys.
    uint32_t tmax = 0u, nv = 0u;
    for_lane_keys<HK>(lk, keys, g, wave, nt, [&](int32_t, uint32_t rk) {
      tmax = umax(tmax, rk);
      nv += (uint32_t)__popcll(__ballot(rk != 0u));
    });
    if constexpr (!WG) {
      // one wave holds all 64 maxima: a bit search of at least 16 ballots
      // instead of testing each maximum against all of them (64 ballots)
      nvalid = nv;
      t0 = maxima_bound<1>(tmax, 0u, (uint32_t)k < nvalid ? (uint32_t)k : nvalid);
    } else {
      area[wave * 64 + lane] = tmax;
      if (lane == 0) ctl[kCtlSlotCount + wave] = nv;
      row_barrier<WG>();
      if (past) {
        // (C) every wave: the 64 group maxima (maximum over the waves' rows),
        // keff and the bit search, the same in every wave: no slots and no
        // second barrier (decode batch 7.71 -> 7.56 us, long-context decode
        // 14.68 -> 14.53, against the slice test below)
        uint32_t gmx = 0u;
        for (int w = 0; w < nw; ++w) gmx = umax(gmx, area[w * 64 + lane]);
        nvalid = (uint32_t)__builtin_amdgcn_readlane(
            (int)row_sum16(lane < nw ? ctl[kCtlSlotCount + lane] : 0u), 0);
        const uint32_t kq = (uint32_t)k < nvalid ? (uint32_t)k : nvalid;
        t0 = maxima_bound<1>(gmx, 0u, kq);
      } else {
        // (C) every wave: the 64 group maxima (maximum over the waves' rows) and
        // keff; then a slice of the maxima tested against all of them: v
        // qualifies when #(maxima >= v) >= keff.  The wave's largest qualifying
        // v goes to its slot.
        uint32_t gmx = 0u;
        for (int w = 0; w < nw; ++w) gmx = umax(gmx, area[w * 64 + lane]);
        nvalid = (uint32_t)__builtin_amdgcn_readlane(
            (int)row_sum16(lane < nw ? ctl[kCtlSlotCount + lane] : 0u), 0);
        const uint32_t kq = (uint32_t)k < nvalid ? (uint32_t)k : nvalid;
        const int32_t len = (64 + nw - 1) / nw;
        const int32_t l0 = wave * len;
        const int32_t l1 = l0 + len < 64 ? l0 + len : 64;
        uint32_t best = 0u;
        for (int32_t l = l0; l < l1; ++l) {  // wave-uniform
          const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)gmx, l);
          const uint32_t c = (uint32_t)__popcll(__ballot(gmx >= v));
          best = (c >= kq && v > best) ? v : best;
        }
        if (lane == 0) ctl[kCtlSlotBound + wave] = best;
        row_barrier<WG>();
        t0 = (uint32_t)__builtin_amdgcn_readlane(
            (int)group_umax<16>(lane < nw ? ctl[kCtlSlotBound + lane] : 0u), 0);
      }
    }
  }
  const int32_t keff = (uint32_t)k < nvalid ? k : (int32_t)nvalid;

  // (E) compact the candidates (keys >= T0) into LDS.
  {
    const uint32_t tt = t0 > 1u ? t0 : 1u;
    if (KC && lk.cached) {
      // every ballot first, then one atomic reserves all of this wave's
      // slots.  Keys past the lane's count are 0, below tt >= 1.
      uint32_t tot = 0u;
#pragma unroll
      for (int j = 0; j < kKeyRegs; ++j) tot += (uint32_t)__popcll(__ballot(lk.v[j] >= tt));
      if (tot != 0u) {  // wave-uniform
        uint32_t b0 = 0u;
        if (lane == 0) b0 = atomicAdd(&ctl[kCtlCand], tot);
        uint32_t pos = (uint32_t)__builtin_amdgcn_readlane((int)b0, 0);
        const bool fits = pos + tot <= (uint32_t)kCandCap;  // else only the in-range slots
        uint32_t id0 = ~(uint32_t)(wave * 64 + lane);
        asm volatile("" : "+v"(id0));  // not hoisted out of the row loop (8 live VGPRs)
#pragma unroll
        for (int j = 0; j < kKeyRegs; ++j) {
          const bool c = lk.v[j] >= tt;
          const uint64_t m = __ballot(c);
          const uint32_t at = pos + lanes_below(m);
          if (c && (fits || at < (uint32_t)kCandCap))
            cand[at] = ((uint64_t)lk.v[j] << 32) | (uint64_t)(id0 - (uint32_t)(j * nt));
          pos += (uint32_t)__popcll(m);
        }
      }
    } else if constexpr (HK) {
      for_lane_keys<true>(lk, keys, g, wave, nt, [&](int32_t i, uint32_t rk) {
        const bool c = rk >= tt;
        const uint64_t m = __ballot(c);
        if (m != 0ull) {
          uint32_t b0 = 0u;
          if (lane == 0) b0 = atomicAdd(&ctl[kCtlCand], (uint32_t)__popcll(m));
          b0 = (uint32_t)__builtin_amdgcn_readlane((int)b0, 0);
          const uint32_t pos = b0 + lanes_below(m);
          if (c && pos < (uint32_t)kCandCap) cand[pos] = cand_word(rk, (uint32_t)i);
        }
      });
    } else {
      for (int32_t base = wave * 64; base < nsel; base += nt) {  // wave-uniform
        const int32_t i = base + lane;
        const uint32_t rk = select_rank_key(keys, g, i);
        const bool c = rk >= tt;
        const uint64_t m = __ballot(c);
        if (m != 0ull) {
          uint32_t b0 = 0u;
          if (lane == 0) b0 = atomicAdd(&ctl[kCtlCand], (uint32_t)__popcll(m));
          b0 = (uint32_t)__builtin_amdgcn_readlane((int)b0, 0);
          const uint32_t pos = b0 + lanes_below(m);
          if (c && pos < (uint32_t)kCandCap) cand[pos] = cand_word(rk, (uint32_t)i);
        }
      }
    }
  }
  row_barrier<WG>();

  // (G) rank the candidates, or fall back to the exact one-wave select.
  const int32_t ncand = (int32_t)ctl[kCtlCand];
  if (past && nw >= 2 && ncand <= 64) {  // workgroup-uniform
    // the maxima rows are dead past the compaction's barrier
    rank_candidates_split(cand, ncand, keff, out_row, area, wave, nw);
    for (int32_t j = keff + tid; j < k; j += nt) out_row[j] = -1;
  } else if (ncand <= kCandCap) {
    rank_candidates<!PRE>(cand, ncand, keff, out_row, wave, nw);
    for (int32_t j = keff + tid; j < k; j += nt) out_row[j] = -1;
  } else if constexpr (HK) {
    exact_select_hbm<WG>(g, k, keys, lk, ctl, area, out_row, wave, nw);
  } else {
    if constexpr (PRE) {  // the exact select reads the keys from LDS
#pragma unroll
      for (int j = 0; j < kKeyRegs; ++j) {
        const int32_t i = wave * 64 + j * nt + lane;
        if (j < lk.nj && i < nsel) keys[i] = lk.v[j];
      }
      row_barrier<WG>();
    }
    if (wave != 0) return;
    for (int32_t b = g.nvb + lane; b < nsel; b += 64) keys[b] = kKeyNegInf;
    wave_sync();
    if (g.pin >= 0 && lane == 0) keys[g.pin] = kKeyPosInf;
    wave_sync();
    select_wave_exact(keys, nsel, k, p.kcap, out_row, area);
  }
}

// Selects row r whose block keys [0, g.nvb) sit in LDS `keys`.  WG: all nw
// waves of the workgroup call this together (it holds workgroup barriers);
// otherwise one wave calls it with nw == 1.  `ctl` (kCtlWords) and `area`
// (16-byte aligned, max(kAreaMinWords, 2*kcap) words) are this row's LDS
// scratch, cleared by select_row_prepare before the caller's last barrier.
// Also writes the optional fp32 score row.
template <bool WG, bool KC = false, int FB = -1, bool PRE = false, bool HK = false>
__device__ __forceinline__ void select_row(const Params& p, int64_t r, const RowGeom& g,
                                           uint32_t* keys, uint32_t* ctl, uint32_t* area,
                                           int wave, int nw, const LaneKeys& pre = LaneKeys{}) {
  const int lane = threadIdx.x & 63;
  const int tid = wave * 64 + lane;
  const int nt = nw * 64;
  const int32_t nsel = g.nsel, k = p.k;
  int32_t* out_row = p.out + r * p.ld_out;

  if (!PRE && p.scores) {
    float* srow = p.scores + r * p.ld_scores;
    for (int32_t b = tid; b < p.nblocks; b += nt)
      srow[b] = b < nsel ? key_value(block_key(keys, g, b)) : -__builtin_inff();
  }

  if (nsel <= 64) {
    // One candidate per lane of wave 0: rank them all directly.
    if (wave == 0) {
      uint64_t* cand = reinterpret_cast<uint64_t*>(area);
      const uint32_t rk = PRE ? pre.v[0] : select_rank_key(keys, g, lane);
      const int32_t nvalid = (int32_t)__popcll(__ballot(rk != 0u));
      const int32_t keff = k < nvalid ? k : nvalid;
      cand[lane] = cand_word(rk, (uint32_t)lane);
      wave_sync();
      rank_candidates(cand, 64, keff, out_row, 0, 1);
      for (int32_t j = keff + lane; j < k; j += 64) out_row[j] = -1;
    }
    return;
  }
  if constexpr (FB >= 0) {
    select_row_general<WG, FB, KC, PRE, HK>(p, g, keys, ctl, area, out_row, wave, nw, pre);
  } else {
    const int bound = select_bound(k, nw);
    if (bound == kBoundGroups64)
      select_row_general<WG, kBoundGroups64, KC, PRE, HK>(p, g, keys, ctl, area, out_row, wave, nw,
                                                          pre);
    else if (bound == kBoundGroups128)
      select_row_general<WG, kBoundGroups128, KC, PRE, HK>(p, g, keys, ctl, area, out_row, wave,
                                                           nw, pre);
    else
      select_row_general<WG, kBoundRadix, KC, PRE, HK>(p, g, keys, ctl, area, out_row, wave, nw,
                                                       pre);
  }
}

// Plan "wave": one wave per row, blockDim/64 rows per workgroup, no barrier.
// U: float4 loads in flight per lane.  Per-wave LDS: keys, ctl, area.
template <int G, int U>
__global__ void __launch_bounds__(kThreads) select_wave_rows_kernel(Params p) {
  extern __shared__ uint32_t smem[];
  const int wave = wave_index();
  const int nw = blockDim.x >> 6;
  uint32_t* keys = smem + wave * p.wave_words;
  uint32_t* ctl = keys + p.keys_words;
  uint32_t* area = ctl + kCtlWords;
  for (int64_t r = (int64_t)blockIdx.x * nw + wave; r < p.items; r += (int64_t)gridDim.x * nw) {
    const RowGeom g = row_geom<G>(p, r, true);
    select_row_prepare(ctl, area, threadIdx.x & 63, 64);
    stream_blocks<G, U, true, true>(p, g, 0, g.nvb, 0, 1, EmitKey{keys});
    wave_sync();
    select_row<false>(p, r, g, keys, ctl, area, 0, 1);
    wave_sync();
  }
}

// Plan "group": all waves of a workgroup stream one row into LDS, then select
// it together.  NW (wave count) and FB (bound) fixed at compile time, or 0 and
// -1 for the launch's and k's: the fixed instances for the usual shapes hold
// fewer registers (4 waves, block size 64: 112 -> 85 VGPRs; from 6144 rows
// the host holds a CU to three such workgroups through their LDS request).
template <int G, int NW = 0, int FB = -1>
__global__ void __launch_bounds__(NW ? NW * 64 : 1024) select_group_rows_kernel(Params p) {
  extern __shared__ uint32_t smem[];
  const int wave = wave_index();
  const int nw = NW ? NW : (int)(blockDim.x >> 6);
  uint32_t* ctl = smem + p.keys_words;
  uint32_t* area = ctl + kCtlWords;
  for (int64_t r = blockIdx.x; r < p.items; r += gridDim.x) {
    // the divides by the block size kept here: the shifts of row_geom<G>
    // measured 151.5 -> 152.3 us on the large prefill (they took 1-2.5 %
    // off the wave and pair plans)
    const RowGeom g = row_geom(p, r, true);
    select_row_prepare(ctl, area, threadIdx.x, blockDim.x);
    stream_blocks<G, kUnroll, true, true>(p, g, 0, g.nvb, wave, nw, EmitKey{smem});
    __syncthreads();
    select_row<true, false, FB>(p, r, g, smem, ctl, area, wave, nw);
    if (r + gridDim.x < p.items) __syncthreads();  // LDS is reused by the next row
  }
}

// Plan "split", first kernel: item = r * nchunks + c streams blocks
// [c*chunk_blocks, (c+1)*chunk_blocks) of row r (in-window part only) into
// the HBM key matrix ws_keys[r, b].  Rolling loads and the full-tile path:
// 200x262144 40.8 -> 37.5 us, 160x524288 54.6 -> 52.3, 300x524288 100.8 ->
// 99.1 (whole split steps) against whole rounds with per-unit masks.
template <int G>
__global__ void __launch_bounds__(kThreads) stream_keys_kernel(Params p) {
  const int wave = wave_index();
  const int nw = blockDim.x >> 6;
  for (int64_t item = blockIdx.x; item < p.items; item += gridDim.x) {
    // items < 2^31 (checked on the host): a 32-bit divide
    const int64_t r = (int64_t)((uint32_t)item / (uint32_t)p.nchunks);
    const int32_t c = (int32_t)(item - r * p.nchunks);
    const RowGeom g = row_geom<G>(p, r, true);
    const int32_t b0 = c * p.chunk_blocks;
    if (b0 >= g.nvb) continue;
    const int32_t b1 = b0 + p.chunk_blocks < g.nvb ? b0 + p.chunk_blocks : g.nvb;
    stream_blocks<G, kUnroll, true, true>(p, g, b0, b1, wave, nw, EmitKey{p.ws_keys + r * p.ws_ld});
  }
}

// Plan "split", second kernel: one workgroup per row reads the row's keys
// back into LDS and selects.
__global__ void __launch_bounds__(1024) select_keys_kernel(Params p) {
  extern __shared__ uint32_t smem[];
  const int wave = wave_index();
  const int nw = blockDim.x >> 6;
  uint32_t* ctl = smem + p.keys_words;
  uint32_t* area = ctl + kCtlWords;
  for (int64_t r = blockIdx.x; r < p.items; r += gridDim.x) {
    const RowGeom g = row_geom(p, r, true);
    select_row_prepare(ctl, area, threadIdx.x, blockDim.x);
    const uint32_t* src = p.ws_keys + r * p.ws_ld;
    const int32_t nt = (int32_t)blockDim.x;
    for (int32_t b0 = 0; b0 < g.nvb; b0 += 4 * nt) {  // four loads in flight per lane
      uint32_t v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int32_t b = b0 + j * nt + (int32_t)threadIdx.x;
        v[j] = src[b < g.nvb ? b : g.nvb - 1];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int32_t b = b0 + j * nt + (int32_t)threadIdx.x;
        if (b < g.nvb) smem[b] = v[j];
      }
    }
    __syncthreads();
    select_row<true>(p, r, g, smem, ctl, area, wave, nw);
    if (r + gridDim.x < p.items) __syncthreads();
  }
}

// Plan "split", second kernel for rows whose keys exceed one workgroup's
// LDS: the select reads the keys where the first kernel left them (the row
// of the workspace, [0, nvb); the pin and the blocks past the window are
// applied as the keys are read) and keeps only its control words and
// candidate area in LDS.  Every pass over the keys reads HBM or L2 instead
// of LDS, eight loads in flight per lane, and the exact select runs on the
// whole workgroup (exact_select_hbm).
__global__ void __launch_bounds__(1024) select_keys_hbm_kernel(Params p) {
  extern __shared__ uint32_t smem[];
  const int wave = wave_index();
  const int nw = blockDim.x >> 6;
  uint32_t* ctl = smem;
  uint32_t* area = ctl + kCtlWords;
  for (int64_t r = blockIdx.x; r < p.items; r += gridDim.x) {
    const RowGeom g = row_geom(p, r, true);
    uint32_t* keys = p.ws_keys + r * p.ws_ld;  // only read
    select_row_prepare(ctl, area, threadIdx.x, blockDim.x);
    __syncthreads();
    select_row<true, false, -1, false, true>(p, r, g, keys, ctl, area, wave, nw);
    if (r + gridDim.x < p.items) __syncthreads();
  }
}

// Plan "pair": up to `parts` workgroups share a row.  Each streams one range
// of the row's blocks (a fixed number of 32-block key lines) into LDS,
// publishes its keys in the workspace and counts itself in on the row's
// counter; the last to arrive gathers the other ranges and selects the row.  Nobody waits, so
// any residency works.  The gather reads the other workgroups' keys through
// the L2 of its XCD: the hardware deals workgroups to the 8 XCDs round-robin,
// so workgroup i runs on XCD i mod 8 and the grid puts a row's parts on one
// XCD.  The counter records the XCD of every arrival (one 8-bit count per XCC
// id); if a part ran elsewhere, its keys may sit in another XCD's L2, and the
// last workgroup streams the other ranges again itself instead.  The last arrival
// resets the counter to zero for the next call.  `spread` deals a row's parts
// to consecutive workgroups instead, on different XCDs, which exercises that
// fallback.
__device__ __forceinline__ uint32_t xcc_id() {
  // hwreg(HW_REG_XCC_ID, 0, 16): the XCC (XCD) this wave runs on
  return (uint32_t)__builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11)) & 7u;
}

// FULL (chosen on the host): parts of 8 tiles or more per wave skip the
// masks on interior tiles; short parts measured faster without that test.
// NW and FB as in select_group_rows_kernel (8 waves, block size 64: 71 -> 61
// VGPRs; decode batch 7.92 -> 7.73 us, long-context decode 14.98 -> 14.76).
template <int G, bool FULL, int NW = 0, int FB = -1>
__global__ void __launch_bounds__(NW ? NW * 64 : 1024) select_pair_rows_kernel(Params p) {
  extern __shared__ uint32_t smem[];
  const int wave = wave_index();
  const int nw = NW ? NW : (int)(blockDim.x >> 6);
  const int tid = threadIdx.x;
  const int nt = nw * 64;
  const int H = p.parts;
  const uint32_t j = p.spread ? blockIdx.x : blockIdx.x >> 3;
  const uint32_t jh = p.h_shift >= 0 ? j >> p.h_shift : j / (uint32_t)H;
  const int64_t r = p.spread ? (int64_t)jh : (int64_t)jh * 8 + (blockIdx.x & 7);
  const int part = (int)(j - jh * (uint32_t)H);
  if (r >= p.rows) return;
  uint32_t* ctl = smem + p.keys_words;
  uint32_t* area = ctl + kCtlWords;
  uint64_t* s_old = reinterpret_cast<uint64_t*>(ctl + kCtlArrival);
  const RowGeom g = row_geom<G>(p, r, true);
  // parts of a fixed size (the widest row's share, whole 32-key lines, set
  // on the host), so that every busy workgroup streams about the same bytes;
  // a shorter row uses fewer of its parts and the others leave at once
  const int32_t cb = p.chunk_blocks;
  if (part > 0 && (int64_t)part * cb >= g.nvb) return;  // no divide before the loads
  select_row_prepare(ctl, area, tid, nt);
  const int32_t b0 = part * cb < g.nvb ? part * cb : g.nvb;
  const int32_t b1 = b0 + cb < g.nvb ? b0 + cb : g.nvb;
  stream_blocks<G, kPairUnroll, true, FULL>(p, g, b0, b1, wave, nw, EmitKey{smem});
  const int HP = g.nvb > 0 ? (g.nvb + cb - 1) / cb : 1;  // parts the row uses
  if (HP > 1) {  // workgroup-uniform; a row of one part needs no hand-off
    __syncthreads();
    uint32_t* wrow = p.ws_keys + r * p.ws_ld;
    for (int32_t b = b0 + tid; b < b1; b += nt) wrow[b] = smem[b];
    // every key store acknowledged by L2 before the arrival is counted
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const uint32_t xcc = xcc_id();
    if (tid == 0) *s_old = atomicAdd(reinterpret_cast<unsigned long long*>(p.ws_count + r),
                                    1ull << (8 * xcc));
    __syncthreads();
    const uint64_t old = *s_old;
    int arrived = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) arrived += (int)((old >> (8 * x)) & 255u);
    if (arrived != HP - 1) return;
    if (tid == 0) atomicExch(reinterpret_cast<unsigned long long*>(p.ws_count + r), 0ull);
    if ((int)((old >> (8 * xcc)) & 255u) == HP - 1) {
      // every other part published its keys in this XCD's L2; the loads are
      // agent-scope (they skip this CU's L1 and read the L2), which costs
      // nothing measurable against plain loads (decode batch 7.90 -> 7.91 us,
      // long-context decode 14.81 -> 14.82)
      for (int32_t c0 = 0; c0 < g.nvb; c0 += 4 * nt) {
        uint32_t v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int32_t b = c0 + q * nt + tid;
          v[q] = (b < g.nvb && (b < b0 || b >= b1))
                     ? __hip_atomic_load(wrow + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                     : 0u;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int32_t b = c0 + q * nt + tid;
          if (b < g.nvb && (b < b0 || b >= b1)) smem[b] = v[q];
        }
      }
    } else {
      stream_blocks<G, kPairUnroll, true, FULL>(p, g, 0, b0, wave, nw, EmitKey{smem});
      stream_blocks<G, kPairUnroll, true, FULL>(p, g, b1, g.nvb, wave, nw, EmitKey{smem});
    }
  }
  __syncthreads();
  select_row<true, false, FB>(p, r, g, smem, ctl, area, wave, nw);
}

// Block scores to HBM; item = r * nchunks + c covers blocks
// [c*chunk_blocks, (c+1)*chunk_blocks) of row r, in-window or not.  KEYS:
// the scores are written as their order-preserving uint32 codes (p.scores
// then points at uint32 storage), the form in which scores of several
// context-parallel ranks reduce exactly by an integer maximum.  The
// loads roll across rounds although the emits are HBM stores: measured on
// five shapes, the stores' place in the in-order memory counter costs less
// than the drained rounds did.
// Six waves per SIMD (at most 80 VGPRs, no spills) against the compiler's
// 95-97 VGPRs and four or five waves: 8192 one-wave rows of 8192 columns at
// B = 8 took 30.2 -> 28.1 us; other shapes were unchanged; seven waves spill
// and lost 10-20 % everywhere.
template <int G, bool KEYS, bool STAGE = false>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(6)))
block_scores_kernel(Params p) {
  const int wave = wave_index();
  const int nw = blockDim.x >> 6;
  for (int64_t item = blockIdx.x; item < p.items; item += gridDim.x) {
    // one chunk per row from 1024 rows on; else a 32-bit divide when it fits
    const int64_t r = p.nchunks == 1 ? item
                      : ((item >> 32) == 0 ? (int64_t)((uint32_t)item / (uint32_t)p.nchunks)
                                           : item / p.nchunks);
    const int32_t c = (int32_t)(item - r * p.nchunks);
    const RowGeom g = row_geom<G>(p, r, p.pin != 0);
    const int32_t b0 = c * p.chunk_blocks;
    const int32_t b1 = b0 + p.chunk_blocks < p.nblocks ? b0 + p.chunk_blocks : p.nblocks;
    const int32_t sb1 = b1 < g.nvb ? b1 : g.nvb;
    const int32_t f0 = b0 > g.nvb ? b0 : g.nvb;
    if constexpr (STAGE) {  // the chunk's scores staged in LDS, then stored in one pass
      extern __shared__ uint32_t sl[];
      stream_blocks<G, kUnroll, true, true>(p, g, b0, sb1, wave, nw, EmitStaged<KEYS>{sl, b0, g.pin});
      const uint32_t inf = KEYS ? kKeyPosInf : 0x7F800000u, ninf = KEYS ? kKeyNegInf : 0xFF800000u;
      for (int32_t b = f0 + (int32_t)threadIdx.x; b < b1; b += (int32_t)blockDim.x)
        sl[b - b0] = b == g.pin ? inf : ninf;
      __syncthreads();
      uint32_t* dst = reinterpret_cast<uint32_t*>(p.scores) + r * p.ld_scores + b0;
      for (int32_t i = (int32_t)threadIdx.x; i < b1 - b0; i += (int32_t)blockDim.x) dst[i] = sl[i];
      __syncthreads();
    } else if constexpr (KEYS) {
      uint32_t* krow = reinterpret_cast<uint32_t*>(p.scores) + r * p.ld_scores;
      stream_blocks<G, kUnroll, true, true>(p, g, b0, sb1, wave, nw, EmitScoreKey{krow, g.pin});
      for (int32_t b = f0 + (int32_t)threadIdx.x; b < b1; b += (int32_t)blockDim.x)
        krow[b] = b == g.pin ? kKeyPosInf : kKeyNegInf;
    } else {
      float* srow = p.scores + r * p.ld_scores;
      stream_blocks<G, kUnroll, true, true>(p, g, b0, sb1, wave, nw, EmitScore{srow, g.pin});
      for (int32_t b = f0 + (int32_t)threadIdx.x; b < b1; b += (int32_t)blockDim.x)
        srow[b] = b == g.pin ? __builtin_inff() : -__builtin_inff();
    }
  }
}

// Selection from a reduced block-score matrix (the decode-context-parallel
// branch after its all-reduce): one workgroup per row.  KEYS: the matrix
// holds order-preserving uint32 codes instead of fp32 scores (read through
// the same pointer).  Params reuse:
// logits = scores [rows, ld] holding `width` columns, ke = global ends,
// B = global block size, nblocks = max(max_global_blocks, 1).  Columns past
// min(width, nblocks) are -inf; the pin is floor((e-1)/B) clamped to the
// last block; rows with e <= 0 select nothing.
// FB: the candidate bound, fixed at compile time (the host knows k and the
// wave count), so each instance holds one bound's code.  PRE: every row has
// at most kKeyRegs keys per lane; the lanes load their keys straight into
// registers (all loads in flight at once) and the select works from there,
// with no LDS copy of the row unless it takes the exact fallback.  NW: the
// wave count when fixed at compile time (2, the many-rows case; 0: from the
// launch): 61 instead of 72 VGPRs, eight waves per SIMD, and about a sixth
// fewer VALU instructions on 8192 rows of 1024 scores (24.8 -> 21.8 us).
// Seven waves per SIMD (at most 72 VGPRs, no spills): rows' selects share
// each CU.  On 8192 rows of 1024 scores at k = 64 this took 36.3 -> 31.1 us
// against the compiler's own choice (83 VGPRs, five waves); six waves gave
// 32.4, eight spill to scratch and gave 32.0 (measured before FB and PRE;
// with them six and eight waves are still slower).
template <bool KEYS, int FB, bool PRE, int NW>
__global__ void __launch_bounds__(NW ? NW * 64 : 1024) __attribute__((amdgpu_waves_per_eu(7)))
select_scores_kernel(Params p) {
  extern __shared__ uint32_t smem[];
  const int wave = wave_index();
  const int lane = threadIdx.x & 63;
  const int nw = NW ? NW : (int)(blockDim.x >> 6);
  const int32_t nt = nw * 64;
  uint32_t* ctl = smem + p.keys_words;
  uint32_t* area = ctl + kCtlWords;
  const int32_t ncopy = p.width < p.nblocks ? (int32_t)p.width : p.nblocks;
  for (int64_t r = blockIdx.x; r < p.items; r += gridDim.x) {
    const int64_t e = (int64_t)p.ke[row_group(p, r)];
    RowGeom g;
    g.row = p.logits + r * p.ld;
    g.s = 0;
    g.lo = 0;
    g.hi = 0;
    g.nvb = 0;
    g.pin = -1;
    if (e > 0) {
      const int64_t q = (e - 1) / p.B;  // e - 1 >= 0: truncation is the floor
      g.nvb = ncopy;
      g.pin = (int32_t)(q < p.nblocks - 1 ? q : p.nblocks - 1);
    }
    g.nsel = g.nvb > g.pin + 1 ? g.nvb : g.pin + 1;
    if constexpr (PRE) {
      // key i = wave*64 + j*nt + lane, the order lane_keys uses
      const int32_t first = wave * 64;
      const int32_t nj = g.nsel > first ? (g.nsel - first + nt - 1) / nt : 0;  // wave-uniform
      uint32_t raw[kKeyRegs];
#pragma unroll
      for (int j = 0; j < kKeyRegs; ++j) {
        const int32_t i = first + j * nt + lane;
        // past the row's columns: -inf, whose rank key is 0 ("no candidate")
        raw[j] = (j < nj && i < g.nvb) ? reinterpret_cast<const uint32_t*>(g.row)[i]
                                       : (KEYS ? kKeyNegInf : 0xFF800000u);
      }
      select_row_prepare(ctl, area, threadIdx.x, blockDim.x);
      // two waves under a group-maxima bound: each wave zeroes only LDS words
      // it writes itself or that are written after the select's first
      // barrier, so no barrier is needed here (DCP select 21.22 -> 21.12 us);
      // the direct rank (<= 64 keys) and the radix bound read zeroed words
      // of the other wave first
      if (!(NW == 2 && (FB == kBoundGroups64 || FB == kBoundGroups128)) || g.nsel <= 64)
        __syncthreads();  // the loads stay in flight across it
      LaneKeys lk;
      lk.nj = nj;
      lk.cached = true;
#pragma unroll
      for (int j = 0; j < kKeyRegs; ++j) {  // the rank keys select_rank_key would give
        const int32_t i = first + j * nt + lane;
        uint32_t k;
        if constexpr (KEYS) {  // codes of any NaN stand for the canonical NaN's
          k = (raw[j] > kKeyPosInf || raw[j] < kKeyNegInf) ? kKeyNaN : raw[j];
        } else {
          k = order_key(__uint_as_float(raw[j]));
        }
        lk.v[j] = i == g.pin ? kKeyPosInf : rank_key(k);  // the pin lies below nsel
      }
      select_row<true, true, FB, true>(p, r, g, smem, ctl, area, wave, nw, lk);
    } else {
      select_row_prepare(ctl, area, threadIdx.x, blockDim.x);
      for (int32_t b0 = 0; b0 < g.nvb; b0 += 4 * nt) {  // four loads in flight per lane
        uint32_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int32_t b = b0 + j * nt + (int32_t)threadIdx.x;
          const int32_t bc = b < g.nvb ? b : g.nvb - 1;
          if constexpr (KEYS) {
            const uint32_t k = reinterpret_cast<const uint32_t*>(g.row)[bc];
            v[j] = (k > kKeyPosInf || k < kKeyNegInf) ? kKeyNaN : k;
          } else {
            v[j] = order_key(g.row[bc]);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int32_t b = b0 + j * nt + (int32_t)threadIdx.x;
          if (b < g.nvb) smem[b] = v[j];
        }
      }
      __syncthreads();
      select_row<true, true, FB>(p, r, g, smem, ctl, area, wave, nw);
    }
    if (r + gridDim.x < p.items) __syncthreads();  // LDS is reused by the next row
  }
}

// ------------------------------------------------------------- masking --

constexpr int kMaskChunk = 4096;                    // columns per work item (4K: measured best of 1K-32K)
constexpr int kMaskBitWords = kMaskChunk / 32 + 2;  // blocks of one chunk, as bits

struct MaskParams {
  float* logits;
  int64_t rows, width, ld;
  const int32_t* ks;
  const int32_t* ke;
  const int32_t* cand;
  int64_t ld_cand;
  int32_t k, B, R, b_shift;  // b_shift >= 0: B == 1 << b_shift
  int32_t vec_ok;            // row starts are 16-byte aligned
  int64_t nchunks, items;
};

// Item = r * nchunks + c covers columns [c*kMaskChunk, (c+1)*kMaskChunk) of
// row r.  A column keeps its value when it lies in [s, e) and its
// request-local block is one of the row's first k candidates; every other
// column becomes -inf.  Kept columns are neither read nor written: the
// kernel only writes.  The candidate ids load beside the bounds (one memory
// round trip before the first store), and a chunk with no in-window column
// builds no bitmap.
__global__ void __launch_bounds__(kThreads) mask_candidates_kernel(MaskParams m) {
  __shared__ uint32_t bits[kMaskBitWords];
  const int tid = threadIdx.x;
  const int nt = blockDim.x;
  const float ninf = -__builtin_inff();
  for (int64_t item = blockIdx.x; item < m.items; item += gridDim.x) {
    // 32-bit divides when they fit (they precede every load of the item)
    const int64_t r = ((item | m.nchunks) >> 32) == 0
                          ? (int64_t)((uint32_t)item / (uint32_t)m.nchunks)
                          : item / m.nchunks;
    const int64_t c0 = (item - r * m.nchunks) * kMaskChunk;
    const int64_t c1 = c0 + kMaskChunk < m.width ? c0 + kMaskChunk : m.width;
    const int64_t grp = m.R == 1 ? r : ((r >> 32) == 0 ? (int64_t)((uint32_t)r / (uint32_t)m.R)
                                                       : r / m.R);
    const int32_t* cr = m.k > 0 ? m.cand + r * m.ld_cand : m.cand;
    const int32_t cid = tid < m.k ? cr[tid] : -1;  // issued before the bounds are known
    // one load brings both bounds (lane 0 of each wave: the start, the
    // others: the end); every lane of the workgroup is active here
    const int32_t* bp = ((tid & 63) == 0 && m.ks) ? m.ks + grp : m.ke + grp;
    const int32_t bv = *bp;
    const int64_t s = m.ks ? (int64_t)__builtin_amdgcn_readlane(bv, 0) : 0;
    const int64_t e = (int64_t)__builtin_amdgcn_readlane(bv, 1);
    const int64_t lo = c0 > s ? c0 : s;  // in-window columns of this chunk: [lo, hi)
    const int64_t hi = c1 < e ? c1 : e;
    int64_t blo = 0, nb = 0;             // their blocks: [blo, blo + nb)
    uint64_t wmask = 0ull;               // small chunks: the kept blocks as one word per wave
    bool wave_mask = false;
    if (hi > lo) {  // workgroup-uniform
      blo = (lo - s) / m.B;
      nb = (hi - 1 - s) / m.B - blo + 1;
    }
    // at most 64 blocks and 64 candidates: every wave ORs the candidates'
    // bits into one 64-bit word itself, with no LDS bitmap and no barrier
    // (prefill chunk mask 40.64 -> 40.48 us)
    if (hi > lo && nb <= 64 && m.k <= 64) {  // workgroup-uniform
      wave_mask = true;
      const int lane = tid & 63;
      const int32_t cj = lane < m.k ? (lane == tid ? cid : cr[lane]) : -1;
      const int64_t id = (int64_t)cj - blo;
      uint64_t bit = (cj >= 0 && id >= 0 && id < nb) ? (1ull << id) : 0ull;
      uint32_t lo32 = (uint32_t)bit, hi32 = (uint32_t)(bit >> 32);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        lo32 |= (uint32_t)__shfl_xor((int)lo32, off);
        hi32 |= (uint32_t)__shfl_xor((int)hi32, off);
      }
      wmask = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)hi32) << 32) |
              (uint32_t)__builtin_amdgcn_readfirstlane((int)lo32);
    } else if (hi > lo) {  // workgroup-uniform
      const int32_t nw = (int32_t)((nb + 31) >> 5);
      for (int w = tid; w < nw; w += nt) bits[w] = 0u;
      __syncthreads();
      for (int32_t j = tid; j < m.k; j += nt) {
        const int32_t cj = j == tid ? cid : cr[j];
        const int64_t id = (int64_t)cj - blo;
        if (cj >= 0 && id >= 0 && id < nb) atomicOr(&bits[id >> 5], 1u << (id & 31));
      }
      __syncthreads();
    }
    float* row = m.logits + r * m.ld;
    // Columns [a, b) all become -inf: 16-byte stores where the row allows,
    // nontemporal (nothing reads them back here): 43.9 -> 40.2 us on the
    // prefill chunk's mask against cached stores.
    const f32x4 ninf4 = {ninf, ninf, ninf, ninf};
    auto fill = [&](int64_t a, int64_t b) {
      if (!m.vec_ok) {
        for (int64_t c = a + tid; c < b; c += nt) row[c] = ninf;
        return;
      }
      int64_t a4 = (a + 3) & ~(int64_t)3;  // [a4, b4): whole aligned float4s
      int64_t b4 = b & ~(int64_t)3;
      if (b4 < a4) a4 = b4 = a;            // fewer than one: all scalar (tail)
      for (int64_t c = a4 + 4 * (int64_t)tid; c < b4; c += 4 * (int64_t)nt)
        __builtin_nontemporal_store(ninf4, reinterpret_cast<f32x4*>(row + c));
      if (tid < a4 - a) row[a + tid] = ninf;   // at most 3 columns before
      if (tid < b - b4) row[b4 + tid] = ninf;  // at most 3 after (all, when short)
    };
    const int64_t wlo = hi > lo ? lo : c1;  // an empty window leaves nothing to test
    const int64_t whi = hi > lo ? hi : c1;
    fill(c0, wlo);
    fill(whi, c1);
    // In-window columns: -inf unless the column's block is a candidate.
    auto kept = [&](int64_t c) -> bool {
      const int64_t rel = c - s;
      const int64_t b = (m.b_shift >= 0 ? (rel >> m.b_shift) : rel / m.B) - blo;
      if (wave_mask) return (wmask >> b) & 1ull;
      return (bits[b >> 5] >> (b & 31)) & 1u;
    };
    if (m.vec_ok) {
      int64_t a4 = (wlo + 3) & ~(int64_t)3;
      int64_t b4 = whi & ~(int64_t)3;
      if (b4 < a4) a4 = b4 = wlo;
      // a float4 at c (a multiple of 4) lies in one block when B and s are
      // multiples of 4: one test for all four columns (workgroup-uniform;
      // 40.97 -> 40.64 us on the prefill chunk's mask)
      const bool one = (m.B & 3) == 0 && (s & 3) == 0;
      for (int64_t c = a4 + 4 * (int64_t)tid; c < b4; c += 4 * (int64_t)nt) {
        const bool k0 = kept(c);
        const bool k1 = one ? k0 : kept(c + 1), k2 = one ? k0 : kept(c + 2),
                   k3 = one ? k0 : kept(c + 3);
        if (!(k0 || k1 || k2 || k3)) {
          __builtin_nontemporal_store(ninf4, reinterpret_cast<f32x4*>(row + c));
        } else {
          if (!k0) row[c] = ninf;
          if (!k1) row[c + 1] = ninf;
          if (!k2) row[c + 2] = ninf;
          if (!k3) row[c + 3] = ninf;
        }
      }
      if (tid < a4 - wlo && !kept(wlo + tid)) row[wlo + tid] = ninf;
      if (tid < whi - b4 && !kept(b4 + tid)) row[b4 + tid] = ninf;
    } else {
      for (int64_t c = wlo + tid; c < whi; c += nt)
        if (!kept(c)) row[c] = ninf;
    }
    if (hi > lo && !wave_mask) __syncthreads();  // the bitmap is reused by the next item
  }
}

// ------------------------------------------------------ LSE correction --

struct LseParams {
  const float* out;
  int64_t B, H, D, o_sb, o_sh, o_sd;
  const float* lses;
  int64_t N, l_sn, l_sb, l_sh, rank;
  float* nout;
  int64_t n_sh, n_sb, n_sd;
  float* vlse;
  int64_t v_sb, v_sh;
  int32_t vec;  // unit D strides, D % 4 == 0, 16-byte aligned rows
};

// Sum over the wave, returned in every lane: the row sums by DPP, then row
// broadcasts (lane 15 into the next row, lane 31 into rows 2 and 3) leave
// the total in lane 63, read out as a uniform value (with the LSE maximum
// taken the same way: merge 27.22 -> 27.03 us against a swizzle and a
// bpermute).
__device__ __forceinline__ float wave_fsum(float v) {
  v += dpp_move<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_move<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_move<0x141>(v);  // row_half_mirror
  v += dpp_move<0x140>(v);  // row_mirror
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  v += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x143, 0xC, 0xF, false));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// NaN and +inf count as -inf for the merge.
__device__ __forceinline__ float lse_clean(float x) {
  return (x != x || x == __builtin_inff()) ? -__builtin_inff() : x;
}

// Base-2 log-sum-exp correction of one rank's partial attention output: one
// wave per (b, h).  Lanes hold the N ranks' LSEs (N > 64 in passes of 64);
// the wave reduces max and sum, forms final = log2(sum 2^(l - m)) + m and
// factor = 2^(l_rank - final), then scales the D-vector out[b][h] into
// new_out[h][b].
__global__ void __launch_bounds__(kThreads) correct_attn_out_kernel(LseParams q) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = blockDim.x >> 6;
  const int64_t pairs = q.B * q.H;
  const float ninf = -__builtin_inff();
  for (int64_t pr = (int64_t)blockIdx.x * nw + wave_index(); pr < pairs;
       pr += (int64_t)gridDim.x * nw) {
    const int64_t b = pr / q.H;
    const int64_t h = pr - b * q.H;
    const float* lrow = q.lses + b * q.l_sb + h * q.l_sh;
    float mx = ninf;
    for (int64_t n0 = 0; n0 < q.N; n0 += 64) {
      const int64_t n = n0 + lane;
      const float l = n < q.N ? lse_clean(lrow[n * q.l_sn]) : ninf;
      mx = fmaximum(mx, __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                            __builtin_bit_cast(int, group_max_tail<64>(l)), 63)));
    }
    const float m = mx == ninf ? 0.0f : mx;
    float acc = 0.0f;
    for (int64_t n0 = 0; n0 < q.N; n0 += 64) {
      const int64_t n = n0 + lane;
      const float l = n < q.N ? lse_clean(lrow[n * q.l_sn]) : ninf;
      acc += wave_fsum(exp2f(l - m));
    }
    const float final_lse = log2f(acc) + m;
    float d = lrow[q.rank * q.l_sn] - final_lse;
    d = (d != d || d == __builtin_inff()) ? ninf : d;
    const float factor = exp2f(d);
    if (lane == 0) q.vlse[b * q.v_sb + h * q.v_sh] = final_lse;
    const float* src = q.out + b * q.o_sb + h * q.o_sh;
    float* dst = q.nout + h * q.n_sh + b * q.n_sb;
    if (q.vec) {
      for (int64_t x = 4 * (int64_t)lane; x < q.D; x += 256) {
        const float4 v = *reinterpret_cast<const float4*>(src + x);
        *reinterpret_cast<float4*>(dst + x) =
            make_float4(v.x * factor, v.y * factor, v.z * factor, v.w * factor);
      }
    } else {
      for (int64_t x = lane; x < q.D; x += 64) dst[x * q.n_sd] = src[x * q.o_sd] * factor;
    }
  }
}

__global__ void __launch_bounds__(kThreads) clear_words_kernel(uint32_t* p, int32_t n) {
  for (int32_t i = (int32_t)(blockIdx.x * kThreads + threadIdx.x); i < n;
       i += (int32_t)(gridDim.x * kThreads))
    p[i] = 0u;
}

__global__ void __launch_bounds__(kThreads) fill_minus_one_kernel(int32_t* out, int64_t rows,
                                                                  int64_t ld, int32_t k) {
  const int64_t n = rows * k;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads) {
    const int64_t r = i / k;
    out[r * ld + (i - r * k)] = -1;
  }
}

// ------------------------------------------------------------------ host --

// log2(v) for a power of two v >= 1, else -1.
int32_t pow2_shift(int64_t v) {
  return v > 0 && (v & (v - 1)) == 0 ? (int32_t)__builtin_ctzll((unsigned long long)v) : -1;
}

// Lanes per block for the vector path: B = 4*G with G a power of two <= 64;
// 0 selects the scalar path for every row.
int lanes_per_block(int32_t B) {
  if (B % 4 != 0) return 0;
  const int g = B / 4;
  if (g > 64 || (g & (g - 1)) != 0) return 0;
  return g;
}

#define DSA_KERNEL_TABLE(KNAME)                                                       \
  void* KNAME##_ptr(int g) {                                                          \
    switch (g) {                                                                      \
      case 1: return reinterpret_cast<void*>(&KNAME<1>);                              \
      case 2: return reinterpret_cast<void*>(&KNAME<2>);                              \
      case 4: return reinterpret_cast<void*>(&KNAME<4>);                              \
      case 8: return reinterpret_cast<void*>(&KNAME<8>);                              \
      case 16: return reinterpret_cast<void*>(&KNAME<16>);                            \
      case 32: return reinterpret_cast<void*>(&KNAME<32>);                            \
      case 64: return reinterpret_cast<void*>(&KNAME<64>);                            \
      default: return reinterpret_cast<void*>(&KNAME<0>);                             \
    }                                                                                 \
  }

#define DSA_WAVE_TABLE(U)                                                             \
  void* select_wave_rows_u##U##_ptr(int g) {                                          \
    switch (g) {                                                                      \
      case 1: return reinterpret_cast<void*>(&select_wave_rows_kernel<1, U>);         \
      case 2: return reinterpret_cast<void*>(&select_wave_rows_kernel<2, U>);         \
      case 4: return reinterpret_cast<void*>(&select_wave_rows_kernel<4, U>);         \
      case 8: return reinterpret_cast<void*>(&select_wave_rows_kernel<8, U>);         \
      case 16: return reinterpret_cast<void*>(&select_wave_rows_kernel<16, U>);       \
      case 32: return reinterpret_cast<void*>(&select_wave_rows_kernel<32, U>);       \
      case 64: return reinterpret_cast<void*>(&select_wave_rows_kernel<64, U>);       \
      default: return reinterpret_cast<void*>(&select_wave_rows_kernel<0, U>);        \
    }                                                                                 \
  }

DSA_WAVE_TABLE(8)
DSA_WAVE_TABLE(16)
DSA_KERNEL_TABLE(select_group_rows_kernel)
DSA_KERNEL_TABLE(stream_keys_kernel)

#define DSA_PAIR_TABLE(NAME, FULL)                                                    \
  void* NAME(int g) {                                                                 \
    switch (g) {                                                                      \
      case 1: return reinterpret_cast<void*>(&select_pair_rows_kernel<1, FULL>);      \
      case 2: return reinterpret_cast<void*>(&select_pair_rows_kernel<2, FULL>);      \
      case 4: return reinterpret_cast<void*>(&select_pair_rows_kernel<4, FULL>);      \
      case 8: return reinterpret_cast<void*>(&select_pair_rows_kernel<8, FULL>);      \
      case 16: return reinterpret_cast<void*>(&select_pair_rows_kernel<16, FULL>);    \
      case 32: return reinterpret_cast<void*>(&select_pair_rows_kernel<32, FULL>);    \
      case 64: return reinterpret_cast<void*>(&select_pair_rows_kernel<64, FULL>);    \
      default: return reinterpret_cast<void*>(&select_pair_rows_kernel<0, FULL>);     \
    }                                                                                 \
  }
DSA_PAIR_TABLE(select_pair_rows_ptr, false)
DSA_PAIR_TABLE(select_pair_rows_full_ptr, true)

// Instances with the wave count and bound fixed, for block sizes 64 and 128
// (G = 16, 32) at the default wave counts; nullptr where none exists.
template <int G, int NW>
void* group_fixed(int fb) {
  if (fb == kBoundGroups64) return reinterpret_cast<void*>(&select_group_rows_kernel<G, NW, kBoundGroups64>);
  if (fb == kBoundGroups128) return reinterpret_cast<void*>(&select_group_rows_kernel<G, NW, kBoundGroups128>);
  return reinterpret_cast<void*>(&select_group_rows_kernel<G, NW, kBoundRadix>);
}
void* select_group_fixed_ptr(int g, int waves, int32_t k) {
  if (waves != kWaves) return nullptr;
  const int fb = select_bound(k, waves);
  if (g == 16) return group_fixed<16, kWaves>(fb);
  if (g == 32) return group_fixed<32, kWaves>(fb);
  return nullptr;
}
constexpr int kPairWaves = 8;
template <int G, bool FULL>
void* pair_fixed(int fb) {
  if (fb == kBoundGroups64)
    return reinterpret_cast<void*>(&select_pair_rows_kernel<G, FULL, kPairWaves, kBoundGroups64>);
  if (fb == kBoundGroups128)
    return reinterpret_cast<void*>(&select_pair_rows_kernel<G, FULL, kPairWaves, kBoundGroups128>);
  return reinterpret_cast<void*>(&select_pair_rows_kernel<G, FULL, kPairWaves, kBoundRadix>);
}
void* select_pair_fixed_ptr(int g, bool full, int waves, int32_t k) {
  if (waves != kPairWaves) return nullptr;
  const int fb = select_bound(k, waves);
  if (g == 16) return full ? pair_fixed<16, true>(fb) : pair_fixed<16, false>(fb);
  if (g == 32) return full ? pair_fixed<32, true>(fb) : pair_fixed<32, false>(fb);
  return nullptr;
}
#define DSA_SCORES_TABLE(NAME, KEYS)                                                  \
  void* NAME(int g) {                                                                 \
    switch (g) {                                                                      \
      case 1: return reinterpret_cast<void*>(&block_scores_kernel<1, KEYS>);          \
      case 2: return reinterpret_cast<void*>(&block_scores_kernel<2, KEYS>);          \
      case 4: return reinterpret_cast<void*>(&block_scores_kernel<4, KEYS>);          \
      case 8: return reinterpret_cast<void*>(&block_scores_kernel<8, KEYS>);          \
      case 16: return reinterpret_cast<void*>(&block_scores_kernel<16, KEYS>);        \
      case 32: return reinterpret_cast<void*>(&block_scores_kernel<32, KEYS>);        \
      case 64: return reinterpret_cast<void*>(&block_scores_kernel<64, KEYS>);        \
      default: return reinterpret_cast<void*>(&block_scores_kernel<0, KEYS>);         \
    }                                                                                 \
  }
DSA_SCORES_TABLE(block_scores_kernel_ptr, false)
DSA_SCORES_TABLE(block_keys_kernel_ptr, true)
// Instances that stage a chunk's scores in LDS, for block sizes 4, 8 and 16
// (one score per 16, 32 or 64 bytes read); nullptr for other block sizes.
template <int G>
void* block_staged(bool keys) {
  return keys ? reinterpret_cast<void*>(&block_scores_kernel<G, true, true>)
              : reinterpret_cast<void*>(&block_scores_kernel<G, false, true>);
}
void* block_staged_ptr(int g, bool keys) {
  if (g == 1) return block_staged<1>(keys);
  if (g == 2) return block_staged<2>(keys);
  if (g == 4) return block_staged<4>(keys);
  return nullptr;
}

// Launches `fn` over `items` work items with `threads` per workgroup and
// `per_group` items per workgroup.
dsa_status_t launch(void* fn, int64_t items, int threads, int per_group, size_t lds,
                    hipStream_t stream, Params& p) {
  p.items = items;
  int64_t grid = (items + per_group - 1) / per_group;
  if (grid > kMaxGrid) grid = kMaxGrid;
  void* args[] = {&p};
  hipError_t err = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(threads), args, lds, stream);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return DSA_ERR_HIP;
  }
  return DSA_OK;
}

bool misaligned(const void* ptr, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) != 0;
}

// ceil(a / b) for a >= 0, b >= 1, with no overflow for any such a.
int64_t cdiv(int64_t a, int64_t b) { return a / b + (a % b != 0 ? 1 : 0); }

int64_t select_kcap(int64_t nblocks, int32_t k) {
  const int64_t kc = k < nblocks ? k : nblocks;
  return kc > 0 ? kc : 1;
}

// LDS words of one row's select state: keys (nblocks rounded up to 4), the
// control words, then an area for the group maxima, the candidates
// (kCandCap 64-bit words) or, in the exact fallback, the radix histogram and
// the selected keys and ids (2 x kcap); a multiple of 4 words.
int64_t select_keys_words(int64_t nblocks) { return cdiv(nblocks, 4) * 4; }

// The select state without the keys: control words and area.
int64_t select_state_words(int64_t nblocks, int32_t k) {
  const int64_t sel = 2 * select_kcap(nblocks, k);
  return kCtlWords + cdiv(sel > kAreaMinWords ? sel : kAreaMinWords, 4) * 4;
}

int64_t select_wave_words(int64_t nblocks, int32_t k) {
  return select_keys_words(nblocks) + select_state_words(nblocks, k);
}

// Largest block count of a selection: the select's slot indices (up to
// 8 x 1024 past a row's nsel) stay within int32.
constexpr int64_t kMaxSelectBlocks = (int64_t)INT32_MAX - 8192;

// Rows whose keys and select state exceed one workgroup's LDS: only the
// split plan holds them, its select reading the keys from the workspace.
bool keys_past_lds(int64_t nblocks, int32_t k) {
  // the first test keeps the product below from overflowing for any nblocks
  return nblocks > (int64_t)kLdsLimit / 4 || select_wave_words(nblocks, k) * 4 > (int64_t)kLdsLimit;
}

// Plan ids (also the values of dsa_select_candidate_blocks_plan's `plan`).
enum { kPlanGroup = 1, kPlanSplit = 2, kPlanWave = 3, kPlanPair = 4 };

// Workspace layout: per-row arrival counters of the pair plan (zero between
// calls), then the score keys of the split and pair plans, rows 128-byte
// aligned.
constexpr int64_t kCountRows = 256;
constexpr size_t kCountBytes = kCountRows * 8;
constexpr uintptr_t kWsAlign = 128;
int64_t ws_row_words(int64_t nblocks) { return cdiv(nblocks, 32) * 32; }

// Chunk size for split rows: aim at ~2048 workgroups in total, 8K-32K columns
// each, and a multiple of the blocks one wave instruction covers.
int32_t auto_chunk_blocks(int64_t rows, int64_t width, int32_t B) {
  // rows * width / 2048 clamped to [8192, 32768], in 128-bit arithmetic
  // (the product of two int64 arguments may not fit in 64 bits)
  const __int128 want = rows > 0 ? ((__int128)rows * width) / 2048 : (__int128)width;
  const int64_t cols = want < 8192 ? 8192 : (want > 32768 ? 32768 : (int64_t)want);
  int64_t cb = cdiv(cols, B);
  const int g = lanes_per_block(B);
  if (g > 0) {
    const int per_tile = 64 / g;
    cb = cdiv(cb, per_tile) * per_tile;
  }
  if (cb < 1) cb = 1;
  if (cb > 0x3FFFFFFF) cb = 0x3FFFFFFF;
  return (int32_t)cb;
}

// Pair plan shape for `rows` rows of `width` columns: workgroups per row
// (fill the 256 CUs about once, at most 8, and parts of at least 8K
// columns) and waves per workgroup (16 for rows of 256K columns and more;
// measured on decode shapes of 8-128 rows and 32K-256K columns).
void pair_shape(int64_t rows, int64_t width, int* parts, int* waves) {
  const int64_t r8 = cdiv(rows, 8) * 8;
  int64_t n = r8 <= 32 ? 8 : (r8 <= 64 ? 4 : 2);
  const int64_t by_width = width / 8192 > 2 ? width / 8192 : 2;
  *parts = (int)(n < by_width ? n : by_width);
  *waves = width >= 262144 ? 16 : kPairWaves;
}

// ---------------------------------------------------- static scratch --
//
// dsa_select_candidate_blocks_noalloc's workspace: a file-scope device array
// that every GPU the library runs on holds once, until the process ends.
// Host code never uses the array's name as an address (on the host it is a
// stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// kept per device.  The first kCountBytes are the pair plan's arrival
// counters, cleared when the address is taken (and zero-initialised at
// load); every completed call leaves them zero.
static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The current device's scratch address, set up on its first use (the clear
// of the counters is enqueued on `stream`, ahead of the caller's work).
dsa_status_t device_scratch(hipStream_t stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return DSA_ERR_HIP;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return DSA_ERR_HIP;
    }
    clear_words_kernel<<<dim3(2), dim3(kThreads), 0, stream>>>(static_cast<uint32_t*>(ptr),
                                                                (int32_t)(kCountBytes / 4));
    if (hipGetLastError() != hipSuccess) return DSA_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

const char* dsa_status_string(int status) {
  switch (status) {  // any int: callers may pass codes this library never returns
    case DSA_OK: return "DSA_OK";
    case DSA_ERR_INVALID_ARG: return "DSA_ERR_INVALID_ARG";
    case DSA_ERR_UNSUPPORTED: return "DSA_ERR_UNSUPPORTED";
    case DSA_ERR_WORKSPACE: return "DSA_ERR_WORKSPACE";
    case DSA_ERR_HIP: return "DSA_ERR_HIP";
  }
  return "unknown";
}

size_t dsa_select_workspace_bytes(int64_t rows, int64_t width, int32_t block_size,
                                  int32_t topk_blocks) {
  if (rows <= 0 || width <= 0 || block_size < 1 || topk_blocks < 0) return 0;
  const int64_t nblocks = cdiv(width, block_size);
  // shapes no plan holds (a row's select state past LDS even with its keys in
  // the workspace): nothing to size
  if (rows > INT32_MAX || nblocks > kMaxSelectBlocks) return 0;
  if (select_state_words(nblocks, topk_blocks) * 4 > (int64_t)kLdsLimit) return 0;
  if ((uint64_t)ws_row_words(nblocks) > (UINT64_MAX / 8u) / (uint64_t)rows) return 0;  // no size_t
  return kCountBytes + (size_t)rows * (size_t)ws_row_words(nblocks) * 4u;
}

dsa_status_t dsa_select_plan(int64_t rows, int64_t width, int32_t block_size,
                             int32_t topk_blocks, int32_t* plan, int32_t* plan_arg) {
  if (rows < 0 || width < 0 || block_size < 1 || topk_blocks < 0 || !plan || !plan_arg)
    return DSA_ERR_INVALID_ARG;
  const int64_t nblocks = width > 0 ? cdiv(width, block_size) : 0;
  const int32_t cb = auto_chunk_blocks(rows, width, block_size);
  const int64_t nchunks = cdiv(nblocks, cb);
  *plan_arg = 0;
  if (keys_past_lds(nblocks, topk_blocks)) {
    *plan = kPlanSplit;  // the only plan for rows whose keys exceed LDS
  } else if (rows >= 1024 || nchunks <= 1) {
    // Enough rows to fill the GPU one row at a time: short rows one wave
    // each, long rows a whole workgroup each.  Fewer rows of one chunk each
    // (up to 8K-32K columns): four waves per row, except for rows of at most
    // 2K columns (512 x 8192: 6.69 us against 8.92 for a wave per row;
    // 128 x 2048: 5.15 against 4.98).
    // Many rows of 128K columns or more: eight waves per row (2048 x 131072
    // at B = 128: 88.6 us against 94.9 for four; 1024 x 262144: 101.4
    // against 102.4; sixteen were slower).
    *plan = width <= 16384 && (rows >= 1024 || width <= 2048) ? kPlanWave : kPlanGroup;
    if (*plan == kPlanGroup) *plan_arg = rows >= 1024 && width >= 131072 ? 8 : kWaves;
  } else if (rows <= kCountRows && width >= 16384 && (rows <= 128 || width <= 131072)) {
    // Decode batches of up to 256 rows of 16K columns or more (up to 128K
    // beyond 128 rows): 2-8 workgroups share each row (the pair plan), so
    // that every CU streams.  It beat the one-workgroup-per-row and split
    // plans on every such shape measured (8-256 rows, 16K-256K columns,
    // block sizes 64 and 128; e.g. 64 x 16384: 5.78 us against 6.54 for
    // four waves per row, 256 x 65536 at k = 64: 13.3 against 14.6); 192
    // rows of 256K columns took 34.6 us against 28.0 split.
    int parts, waves;
    pair_shape(rows, width, &parts, &waves);
    *plan = kPlanPair;
    *plan_arg = waves | parts << 8;
  } else if (rows >= cdiv(width, 1024) || width <= 32768 ||
             (width <= 524288 && rows >= 224)) {
    // Rows of up to 32K columns, or enough rows to keep HBM busy one CU per
    // row: 4-16 waves stream each row, the select fused behind them in the
    // same launch.  Against the split plan's two kernels the crossover sits
    // near 224 rows for rows of up to 512K columns (192 x 262144: 29.3 us
    // against 27.7 split; 210 x 400000: 44.7 against 41.2; 224 x 524288:
    // 55.0 against 58.7; 256 x 524288 at B = 128: 59.5 against 63.5) and
    // near rows = width / 1024 beyond (300 x 1048576: 137.1 against 134.2).
    // Waves per row by row length (the pair plan takes up to 256 rows of
    // 16K-128K columns): 4 up to 16K columns (512 x 16384: 8.59 us against 9.81 for
    // eight), 8 up to 32K below 512 rows, 4 at 64K (512 x 65536: 18.9
    // against 19.9), 8 at 128K (600 x 131072: 34.7 against 41.7 for four),
    // 16 beyond (320 x 262144: 43.6 against 51.2 for eight).
    *plan = kPlanGroup;
    *plan_arg = width <= 16384   ? kWaves
                : width <= 32768 ? (rows <= 512 ? 8 : kWaves)
                : width <= 65536 ? kWaves
                : width <= 131072 ? 8
                                  : 16;
  } else {
    // Few rows, or long rows: chunks of every row on all CUs, then a
    // selecting kernel (one CU streams only ~25-70 GB/s, so a row per CU
    // cannot keep HBM busy).
    *plan = kPlanSplit;
    *plan_arg = cb;
  }
  return DSA_OK;
}

}  // extern "C"

namespace {

// dsa_block_scores / dsa_block_score_keys: `scores` is fp32 or, with keys,
// uint32 storage.
dsa_status_t block_scores_impl(const float* logits, int64_t rows, int64_t width,
                               int64_t ld_logits, const int32_t* row_ks, const int32_t* row_ke,
                               int32_t block_size, int32_t row_repeat, int32_t pin_newest,
                               void* scores, int64_t ld_scores, bool keys, hipStream_t stream) {
  if (rows < 0 || width < 0 || block_size < 1 || row_repeat < 1) return DSA_ERR_INVALID_ARG;
  if (pin_newest != 0 && pin_newest != 1) return DSA_ERR_INVALID_ARG;
  if (ld_logits < width) return DSA_ERR_INVALID_ARG;
  const int64_t nblocks = cdiv(width, block_size);
  if (ld_scores < nblocks) return DSA_ERR_INVALID_ARG;
  if (rows == 0 || width == 0) return DSA_OK;
  if (!logits || !row_ke || !scores) return DSA_ERR_INVALID_ARG;
  if (misaligned(logits, 4) || misaligned(scores, 4)) return DSA_ERR_INVALID_ARG;
  if (rows > INT32_MAX || nblocks > INT32_MAX) return DSA_ERR_UNSUPPORTED;

  Params p = {};
  p.logits = logits;
  p.rows = rows;
  p.width = width;
  p.ld = ld_logits;
  p.ks = row_ks;
  p.ke = row_ke;
  p.B = block_size;
  p.R = row_repeat;
  p.r_shift = pow2_shift(row_repeat);
  p.pin = pin_newest;
  p.nblocks = (int32_t)nblocks;
  // Items are row chunks: 8K columns, doubled until at most 512 items
  // remain (few rows: chunks spread each row over many CUs), or whole rows
  // from 1024 rows on.  Whole rows take two waves below 32K columns (short
  // windows: more rows in flight per CU), else four.  Measured against fixed
  // 8K chunks of four waves: large prefill 8192x65536 300 -> 172 us, prefill
  // chunk 4096x16384 32 -> 13.5, 8192x8192 at B = 8 35 -> 30.5, 128x131072
  // 13.4 -> 11.7; 64x32768 unchanged at 4.5.  Two waves instead of one for
  // the short rows: 8192x4096 at B = 8 26.95 -> 25.5 us, 2048x16384 at
  // B = 16 25.4 -> 24.5, 8192x8192 at B = 8 50.1 -> 49.5 (full windows),
  // B = 64 unchanged; four waves were slower.
  const int g = lanes_per_block(block_size);
  int64_t ccols = 8192;
  while (ccols < width && cdiv(width, ccols) > 512 / rows) ccols *= 2;  // rows * chunks > 512
  int64_t cb = rows >= 1024 ? nblocks : cdiv(ccols, block_size);
  if (g > 0) cb = cdiv(cb, 64 / g) * (64 / g);
  if (cb > nblocks) cb = nblocks;
  const int threads = rows >= 1024 && width < 32768 ? 128 : kThreads;
  p.chunk_blocks = (int32_t)cb;
  p.nchunks = (int32_t)cdiv(nblocks, cb);
  p.scores = static_cast<float*>(scores);
  p.ld_scores = ld_scores;
  // small blocks: the chunk's scores go to LDS and out in one pass after the
  // streaming, so that no store sits among the loads in the memory counter
  // (8192 x 8192 at B = 8: 29.0 -> 28.3 us; at B >= 64, where a score comes
  // every 256 bytes or more, staging measured 1-2.5 % slower)
  void* st = cb * 4 <= 16384 ? block_staged_ptr(g, keys) : nullptr;
  if (st) return launch(st, rows * p.nchunks, threads, 1, (size_t)cb * 4, stream, p);
  return launch(keys ? block_keys_kernel_ptr(g) : block_scores_kernel_ptr(g), rows * p.nchunks,
                threads, 1, 0, stream, p);
}

}  // namespace

extern "C" {

dsa_status_t dsa_block_scores(const float* logits, int64_t rows, int64_t width,
                              int64_t ld_logits, const int32_t* row_ks,
                              const int32_t* row_ke, int32_t block_size,
                              int32_t row_repeat, int32_t pin_newest, float* scores,
                              int64_t ld_scores, hipStream_t stream) {
  return block_scores_impl(logits, rows, width, ld_logits, row_ks, row_ke, block_size,
                           row_repeat, pin_newest, scores, ld_scores, false, stream);
}

dsa_status_t dsa_block_score_keys(const float* logits, int64_t rows, int64_t width,
                                  int64_t ld_logits, const int32_t* row_ks,
                                  const int32_t* row_ke, int32_t block_size,
                                  int32_t row_repeat, int32_t pin_newest, uint32_t* keys,
                                  int64_t ld_keys, hipStream_t stream) {
  return block_scores_impl(logits, rows, width, ld_logits, row_ks, row_ke, block_size,
                           row_repeat, pin_newest, keys, ld_keys, true, stream);
}

dsa_status_t dsa_select_candidate_blocks_plan(
    const float* logits, int64_t rows, int64_t width, int64_t ld_logits,
    const int32_t* row_ks, const int32_t* row_ke, int32_t topk_blocks, int32_t block_size,
    int32_t row_repeat, int32_t* out, int64_t ld_out, float* scores_out, int64_t ld_scores,
    void* workspace, size_t workspace_bytes, int32_t plan, int32_t plan_arg,
    hipStream_t stream) {
  if (rows < 0 || width < 0 || block_size < 1 || row_repeat < 1 || topk_blocks < 0)
    return DSA_ERR_INVALID_ARG;
  if (plan < 0 || plan > 4 || plan_arg < 0) return DSA_ERR_INVALID_ARG;
  if (plan == kPlanGroup && plan_arg > 16) return DSA_ERR_INVALID_ARG;
  if (plan == kPlanPair && ((plan_arg & 255) > 16 || (plan_arg >> 16) > 1))
    return DSA_ERR_INVALID_ARG;
  if (plan == kPlanWave && plan_arg != 0 && plan_arg != 8 && plan_arg != 16)
    return DSA_ERR_INVALID_ARG;
  if (ld_logits < width || ld_out < topk_blocks) return DSA_ERR_INVALID_ARG;
  const int64_t nblocks = cdiv(width, block_size);
  if (scores_out && ld_scores < nblocks) return DSA_ERR_INVALID_ARG;
  if (rows == 0 || topk_blocks == 0) return DSA_OK;
  if (!out || misaligned(out, 4)) return DSA_ERR_INVALID_ARG;
  if (rows > INT32_MAX) return DSA_ERR_UNSUPPORTED;
  if (width == 0) {
    const int64_t n = rows * topk_blocks;
    int64_t grid = cdiv(n, kThreads);
    if (grid > kMaxGrid) grid = kMaxGrid;
    fill_minus_one_kernel<<<dim3((unsigned)grid), dim3(kThreads), 0, stream>>>(out, rows, ld_out,
                                                                              topk_blocks);
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_HIP;
  }
  if (!logits || !row_ke) return DSA_ERR_INVALID_ARG;
  if (misaligned(logits, 4) || (scores_out && misaligned(scores_out, 4)))
    return DSA_ERR_INVALID_ARG;
  if (nblocks > kMaxSelectBlocks) return DSA_ERR_UNSUPPORTED;
  const int64_t ww = select_wave_words(nblocks, topk_blocks);
  // keys past LDS: the split plan with its keys left in the workspace
  const bool hbm_keys = keys_past_lds(nblocks, topk_blocks);
  if (select_state_words(nblocks, topk_blocks) * 4 > (int64_t)kLdsLimit)
    return DSA_ERR_UNSUPPORTED;  // the select state alone exceeds LDS

  const size_t ws_need = dsa_select_workspace_bytes(rows, width, block_size, topk_blocks);
  if (ws_need == 0) return DSA_ERR_UNSUPPORTED;  // a workspace past any size_t
  const bool ws_ok = workspace && workspace_bytes >= ws_need && !misaligned(workspace, kWsAlign);
  if (plan == 0) {
    dsa_select_plan(rows, width, block_size, topk_blocks, &plan, &plan_arg);
    if ((plan == kPlanSplit || plan == kPlanPair) && !ws_ok) {
      if (hbm_keys) return DSA_ERR_WORKSPACE;  // no plan without one holds these rows
      // no usable workspace: the plan that needs none
      plan = kPlanGroup;
      plan_arg = width <= 32768 ? 8 : 16;
    }
  }
  if (hbm_keys && plan != kPlanSplit) return DSA_ERR_UNSUPPORTED;
  if (plan == kPlanSplit && plan_arg == 0) plan_arg = auto_chunk_blocks(rows, width, block_size);
  if (plan == kPlanPair && rows > kCountRows) return DSA_ERR_UNSUPPORTED;
  if ((plan == kPlanSplit || plan == kPlanPair) && !ws_ok) return DSA_ERR_WORKSPACE;

  Params p = {};
  p.logits = logits;
  p.rows = rows;
  p.width = width;
  p.ld = ld_logits;
  p.ks = row_ks;
  p.ke = row_ke;
  p.B = block_size;
  p.R = row_repeat;
  p.r_shift = pow2_shift(row_repeat);
  p.pin = 1;
  p.k = topk_blocks;
  p.nblocks = (int32_t)nblocks;
  p.kcap = (int32_t)select_kcap(nblocks, topk_blocks);
  p.keys_words = (int32_t)select_keys_words(nblocks);
  p.wave_words = (int32_t)ww;
  p.out = out;
  p.ld_out = ld_out;
  p.scores = scores_out;
  p.ld_scores = ld_scores;
  if (workspace) {
    p.ws_count = static_cast<uint64_t*>(workspace);
    p.ws_keys = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + kCountBytes);
    p.ws_ld = ws_row_words(nblocks);
  }
  const int g = lanes_per_block(block_size);
  // waves per workgroup for the one-wave-per-row kernel: one from 2048 rows
  // on (single-wave workgroups measured 1-7 % faster on prefill batches of
  // 2048-65536 rows, 2-10 % slower on 1024), else as many row states as fit
  // in LDS, up to four
  int64_t nw = (int64_t)kLdsLimit / (ww * 4);
  if (nw > kWaves) nw = kWaves;
  if (rows >= 2048) nw = 1;
  const size_t wave_lds = (size_t)(nw * ww * 4);
  if (plan == kPlanWave)
    return launch(plan_arg == 16 ? select_wave_rows_u16_ptr(g) : select_wave_rows_u8_ptr(g), rows,
                  64 * (int)nw, (int)nw, wave_lds, stream, p);
  if (plan == kPlanGroup) {
    const int waves = plan_arg > 0 ? plan_arg : kWaves;
    void* fn = select_group_fixed_ptr(g, waves, topk_blocks);
    if (!fn) fn = select_group_rows_kernel_ptr(g);
    // Many long rows (24 or more per CU): the LDS request holds a CU to three
    // rows at a time (gfx950: 160 KiB of LDS per CU).  Large prefill 150.45
    // -> 148.8 us against the five that registers allow (four: 149.9; two:
    // 171), 6144 x 65536 180.1 -> 176.5, 8192 x 32768 120.6 -> 119.9; with
    // fewer rows per CU the extra rounds of rows cost more (1024 x 65536
    // 39.4 -> 40.7, 4096 x 24576 50.7 -> 55.8), so they keep five.
    size_t lds = (size_t)ww * 4;
    if (rows >= 6144 && waves == kWaves && lds < kGroupLdsThree) lds = kGroupLdsThree;
    return launch(fn, rows, 64 * waves, 1, lds, stream, p);
  }
  if (plan == kPlanPair) {
    int parts, waves;
    pair_shape(rows, width, &parts, &waves);
    if ((plan_arg >> 8) & 255) parts = (plan_arg >> 8) & 255;
    if (plan_arg & 255) waves = plan_arg & 255;
    p.parts = parts;
    p.h_shift = pow2_shift(parts);
    p.spread = plan_arg >> 16;
    p.chunk_blocks = (int32_t)(((cdiv(nblocks, parts)) + 31) / 32 * 32);  // blocks per part
    // parts of 8 wave tiles or more per wave take the unmasked interior path
    const int64_t part_units = ((cdiv(nblocks, parts) + 31) / 32) * 32 * g;
    const bool full = part_units >= 64 * 8 * (int64_t)waves;
    void* fn = select_pair_fixed_ptr(g, full, waves, topk_blocks);
    if (!fn) fn = full ? select_pair_rows_full_ptr(g) : select_pair_rows_ptr(g);
    return launch(fn, 8 * parts * cdiv(rows, 8), 64 * waves, 1,
                  (size_t)ww * 4, stream, p);
  }
  p.chunk_blocks = plan_arg < p.nblocks ? plan_arg : p.nblocks;
  p.nchunks = (int32_t)cdiv(nblocks, p.chunk_blocks);
  if (rows * (int64_t)p.nchunks > (int64_t)INT32_MAX) return DSA_ERR_UNSUPPORTED;
  dsa_status_t st = launch(stream_keys_kernel_ptr(g), rows * p.nchunks, kThreads, 1, 0, stream, p);
  if (st != DSA_OK) return st;
  if (hbm_keys) {  // 16 waves per row; LDS holds the select state only
    p.keys_words = 0;
    return launch(reinterpret_cast<void*>(&select_keys_hbm_kernel), rows, 1024, 1,
                  (size_t)select_state_words(nblocks, topk_blocks) * 4, stream, p);
  }
  // one workgroup per row, one key per thread up to 1024 keys
  int64_t sel_waves = cdiv(nblocks, 64);
  if (sel_waves > 16) sel_waves = 16;
  return launch(reinterpret_cast<void*>(&select_keys_kernel), rows, 64 * (int)sel_waves, 1,
                (size_t)ww * 4, stream, p);
}

dsa_status_t dsa_select_candidate_blocks(const float* logits, int64_t rows, int64_t width,
                                         int64_t ld_logits, const int32_t* row_ks,
                                         const int32_t* row_ke, int32_t topk_blocks,
                                         int32_t block_size, int32_t row_repeat,
                                         int32_t* out, int64_t ld_out, float* scores_out,
                                         int64_t ld_scores, void* workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  return dsa_select_candidate_blocks_plan(logits, rows, width, ld_logits, row_ks, row_ke,
                                          topk_blocks, block_size, row_repeat, out, ld_out,
                                          scores_out, ld_scores, workspace, workspace_bytes, 0,
                                          0, stream);
}

dsa_status_t dsa_select_candidate_blocks_noalloc(const float* logits, int64_t rows,
                                                 int64_t width, int64_t ld_logits,
                                                 const int32_t* row_ks, const int32_t* row_ke,
                                                 int32_t topk_blocks, int32_t block_size,
                                                 int32_t row_repeat, int32_t* out, int64_t ld_out,
                                                 float* scores_out, int64_t ld_scores,
                                                 hipStream_t stream) {
  if (rows < 0 || width < 0 || block_size < 1 || row_repeat < 1 || topk_blocks < 0)
    return DSA_ERR_INVALID_ARG;
  int32_t plan = 0, plan_arg = 0;
  dsa_select_plan(rows, width, block_size, topk_blocks, &plan, &plan_arg);
  void* ws = nullptr;
  if (plan == kPlanSplit || plan == kPlanPair) {
    if (dsa_select_workspace_bytes(rows, width, block_size, topk_blocks) >
        (size_t)DSA_NOALLOC_SCRATCH_BYTES)
      return DSA_ERR_WORKSPACE;  // this shape's plan needs more than the static scratch
    if (rows > 0 && width > 0 && topk_blocks > 0) {
      const dsa_status_t st = device_scratch(stream, &ws);
      if (st != DSA_OK) return st;
    }
  }
  return dsa_select_candidate_blocks_plan(logits, rows, width, ld_logits, row_ks, row_ke,
                                          topk_blocks, block_size, row_repeat, out, ld_out,
                                          scores_out, ld_scores, ws,
                                          ws ? (size_t)DSA_NOALLOC_SCRATCH_BYTES : 0, plan,
                                          plan_arg, stream);
}

}  // extern "C"

namespace {

// dsa_select_from_scores / dsa_select_from_keys: `scores` holds fp32 scores
// or, with keys, their uint32 codes.
template <bool KEYS, int FB>
void* select_scores_fn(bool pre, bool two) {
  if (pre && two) return reinterpret_cast<void*>(&select_scores_kernel<KEYS, FB, true, 2>);
  return pre ? reinterpret_cast<void*>(&select_scores_kernel<KEYS, FB, true, 0>)
             : reinterpret_cast<void*>(&select_scores_kernel<KEYS, FB, false, 0>);
}

template <bool KEYS>
void* select_scores_fn(int fb, bool pre, bool two) {
  if (fb == kBoundGroups64) return select_scores_fn<KEYS, kBoundGroups64>(pre, two);
  if (fb == kBoundGroups128) return select_scores_fn<KEYS, kBoundGroups128>(pre, two);
  return select_scores_fn<KEYS, kBoundRadix>(pre, two);
}

dsa_status_t select_from_scores_impl(const void* scores, int64_t rows, int64_t nscore,
                                     int64_t ld_scores, int64_t max_global_blocks,
                                     const int32_t* global_row_ke, int32_t row_repeat,
                                     int32_t global_block_size, int32_t topk_blocks,
                                     int32_t* out, int64_t ld_out, bool keys,
                                     hipStream_t stream) {
  if (rows < 0 || nscore < 0 || max_global_blocks < 0 || row_repeat < 1 ||
      global_block_size < 1 || topk_blocks < 0)
    return DSA_ERR_INVALID_ARG;
  if ((nscore > 0 && ld_scores < nscore) || ld_out < topk_blocks) return DSA_ERR_INVALID_ARG;
  if (rows == 0 || topk_blocks == 0) return DSA_OK;
  if (!global_row_ke || !out || misaligned(out, 4)) return DSA_ERR_INVALID_ARG;
  if (nscore > 0 && (!scores || misaligned(scores, 4))) return DSA_ERR_INVALID_ARG;
  const int64_t nblocks = max_global_blocks > 1 ? max_global_blocks : 1;
  if (rows > INT32_MAX || nblocks > INT32_MAX) return DSA_ERR_UNSUPPORTED;
  const int64_t ww = select_wave_words(nblocks, topk_blocks);
  if (ww * 4 > (int64_t)kLdsLimit) return DSA_ERR_UNSUPPORTED;
  Params p = {};
  p.logits = static_cast<const float*>(scores);
  p.rows = rows;
  p.width = nscore;
  p.ld = nscore > 0 ? ld_scores : 1;
  p.ke = global_row_ke;
  p.B = global_block_size;
  p.R = row_repeat;
  p.r_shift = pow2_shift(row_repeat);
  p.pin = 1;
  p.k = topk_blocks;
  p.nblocks = (int32_t)nblocks;
  p.kcap = (int32_t)select_kcap(nblocks, topk_blocks);
  p.keys_words = (int32_t)select_keys_words(nblocks);
  p.wave_words = (int32_t)ww;
  p.out = out;
  p.ld_out = ld_out;
  // Few rows: a wider workgroup per row (latency); more rows: narrower
  // workgroups, so that several rows' selects share each CU (throughput).
  // Measured on 1024 scores with k = 64: 4 waves are best up to 512 rows,
  // 2 waves from 1024 rows on (8 and 16 waves were slower everywhere).
  int64_t waves = cdiv(nblocks, 64);
  const int64_t cap = rows <= 512 ? kWaves : 2;
  if (waves > cap) waves = cap;
  // the bound select_row would choose for this k and wave count
  const int fb = topk_blocks <= 32 ? kBoundGroups64
                 : ((topk_blocks <= 64 && ((waves & 1) == 0 || waves <= 8)) ? kBoundGroups128
                                                                           : kBoundRadix);
  const bool pre = cdiv(nblocks, 64 * waves) <= kKeyRegs;  // nsel <= nblocks on every row
  void* fn = keys ? select_scores_fn<true>(fb, pre, waves == 2)
                 : select_scores_fn<false>(fb, pre, waves == 2);
  return launch(fn, rows, 64 * (int)waves, 1, (size_t)ww * 4, stream, p);
}

}  // namespace

extern "C" {

dsa_status_t dsa_select_from_scores(const float* scores, int64_t rows, int64_t nscore,
                                    int64_t ld_scores, int64_t max_global_blocks,
                                    const int32_t* global_row_ke, int32_t row_repeat,
                                    int32_t global_block_size, int32_t topk_blocks, int32_t* out,
                                    int64_t ld_out, hipStream_t stream) {
  return select_from_scores_impl(scores, rows, nscore, ld_scores, max_global_blocks,
                                 global_row_ke, row_repeat, global_block_size, topk_blocks, out,
                                 ld_out, false, stream);
}

dsa_status_t dsa_select_from_keys(const uint32_t* keys, int64_t rows, int64_t nkeys,
                                  int64_t ld_keys, int64_t max_global_blocks,
                                  const int32_t* global_row_ke, int32_t row_repeat,
                                  int32_t global_block_size, int32_t topk_blocks, int32_t* out,
                                  int64_t ld_out, hipStream_t stream) {
  return select_from_scores_impl(keys, rows, nkeys, ld_keys, max_global_blocks, global_row_ke,
                                 row_repeat, global_block_size, topk_blocks, out, ld_out, true,
                                 stream);
}

dsa_status_t dsa_mask_candidates(float* logits, int64_t rows, int64_t width, int64_t ld_logits,
                                 const int32_t* row_ks, const int32_t* row_ke,
                                 const int32_t* candidates, int64_t ld_cand,
                                 int32_t topk_blocks, int32_t block_size, int32_t row_repeat,
                                 hipStream_t stream) {
  if (rows < 0 || width < 0 || block_size < 1 || row_repeat < 1 || topk_blocks < 0)
    return DSA_ERR_INVALID_ARG;
  if (ld_logits < width || ld_cand < topk_blocks) return DSA_ERR_INVALID_ARG;
  if (rows == 0 || width == 0) return DSA_OK;
  if (!logits || !row_ke || misaligned(logits, 4)) return DSA_ERR_INVALID_ARG;
  if (topk_blocks > 0 && (!candidates || misaligned(candidates, 4))) return DSA_ERR_INVALID_ARG;
  MaskParams m = {};
  m.logits = logits;
  m.rows = rows;
  m.width = width;
  m.ld = ld_logits;
  m.ks = row_ks;
  m.ke = row_ke;
  m.cand = candidates;
  m.ld_cand = ld_cand;
  m.k = topk_blocks;
  m.B = block_size;
  m.R = row_repeat;
  m.b_shift = (block_size & (block_size - 1)) == 0 ? __builtin_ctz((unsigned)block_size) : -1;
  m.vec_ok = !misaligned(logits, 16) && (ld_logits % 4) == 0;
  m.nchunks = cdiv(width, kMaskChunk);
  if (m.nchunks > INT64_MAX / rows) return DSA_ERR_UNSUPPORTED;  // rows * chunks must fit
  m.items = rows * m.nchunks;
  int64_t grid = m.items < kMaxGrid ? m.items : kMaxGrid;
  void* args[] = {&m};
  hipError_t err = hipLaunchKernel(reinterpret_cast<void*>(&mask_candidates_kernel),
                                   dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return DSA_ERR_HIP;
  }
  return DSA_OK;
}

dsa_status_t dsa_correct_attn_out(const float* out, int64_t B, int64_t H, int64_t D,
                                  int64_t out_sb, int64_t out_sh, int64_t out_sd,
                                  const float* lses, int64_t N, int64_t lse_sn, int64_t lse_sb,
                                  int64_t lse_sh, int64_t cp_rank, float* new_out,
                                  int64_t new_sh, int64_t new_sb, int64_t new_sd, float* lse_out,
                                  int64_t lse_out_sb, int64_t lse_out_sh, hipStream_t stream) {
  if (B < 0 || H < 0 || D < 0 || N < 0) return DSA_ERR_INVALID_ARG;
  if (B == 0 || H == 0) return DSA_OK;
  if (N < 1 || cp_rank < 0 || cp_rank >= N) return DSA_ERR_INVALID_ARG;
  if (B > INT32_MAX || H > INT32_MAX) return DSA_ERR_UNSUPPORTED;  // B * H must fit
  if (!lses || !lse_out || misaligned(lses, 4) || misaligned(lse_out, 4))
    return DSA_ERR_INVALID_ARG;
  if (D > 0 && (!out || !new_out || misaligned(out, 4) || misaligned(new_out, 4)))
    return DSA_ERR_INVALID_ARG;
  LseParams q = {};
  q.out = out;
  q.B = B;
  q.H = H;
  q.D = D;
  q.o_sb = out_sb;
  q.o_sh = out_sh;
  q.o_sd = out_sd;
  q.lses = lses;
  q.N = N;
  q.l_sn = lse_sn;
  q.l_sb = lse_sb;
  q.l_sh = lse_sh;
  q.rank = cp_rank;
  q.nout = new_out;
  q.n_sh = new_sh;
  q.n_sb = new_sb;
  q.n_sd = new_sd;
  q.vlse = lse_out;
  q.v_sb = lse_out_sb;
  q.v_sh = lse_out_sh;
  q.vec = out_sd == 1 && new_sd == 1 && D % 4 == 0 && !misaligned(out, 16) &&
          !misaligned(new_out, 16) && out_sb % 4 == 0 && out_sh % 4 == 0 && new_sh % 4 == 0 &&
          new_sb % 4 == 0;
  int64_t grid = cdiv(B * H, kWaves);
  if (grid > 8192) grid = 8192;
  void* args[] = {&q};
  hipError_t err = hipLaunchKernel(reinterpret_cast<void*>(&correct_attn_out_kernel),
                                   dim3((unsigned)grid), dim3(kThreads), args, 0, stream);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return DSA_ERR_HIP;
  }
  return DSA_OK;
}

}  // extern "C"

