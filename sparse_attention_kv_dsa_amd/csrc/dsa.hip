// dsa.hip - gfx950 kernels and C ABI for DSA candidate-block selection.
//
// What is computed follows the vLLM-fork page
// "launcher/dcp2/diffs/02-model_executor_kernels_attention_dsa_candidate_blocks.py.diff":
// _max_with_nan (NaN-propagating max), _block_scores_kernel (masked window
// load with -inf fill, newest-block pin), _block_scores, and the non-DCP
// branch of _select_candidate_blocks_impl (early-outs, top-k, -1 padding).
// The full contract is stated in include/dsa.h.
//
// How it is computed here (MI355X / CDNA4, wave64):
//   * One HBM pass over the in-window logits.  A block of B = 4*G columns is
//     G lanes of one float4 each; a wave instruction reads 1 KiB contiguous,
//     every lane keeps kUnroll independent 16-byte loads in flight.
//   * The per-lane max of a float4 and the G-lane reduction use the IEEE-754-
//     2019 maximum (v_maximum3_f32 on gfx950: NaN-propagating, -0 < +0);
//     the lanes of a block are combined with DPP quad/row permutes inside a
//     16-lane row, ds_swizzle across rows and a bpermute across halves.
//   * Scores are kept as order-preserving uint32 keys (unsigned order ==
//     float order, canonical NaN on top), in LDS for the select.
//   * Top-k: 8-bit-digit radix select in LDS finds the k-th largest rank key,
//     the candidates are compacted in block-id order (so ties resolve to the
//     lowest ids), and at most k-1 of them are ordered by counting rank.
//   * Few long rows (decode): rows are split into chunks that run on many
//     CUs; the last chunk of a row to finish (agent-scope counter) gathers
//     the row's keys and runs the select, so a call is still one launch.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kUnroll = 8;

// LDS words before the per-row key array: radix histogram, wave totals, misc.
constexpr int kHistWords = 256;
constexpr int kWaveWords = 8;
constexpr int kMiscWords = 16;
constexpr int kHeadWords = kHistWords + kWaveWords + kMiscWords;  // 280 words = 1120 B
constexpr size_t kLdsLimit = 65536;
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
  int32_t vec_ok;  // width % 4 == 0: float4 loads never cross the row's end
  int32_t* out;
  int64_t ld_out;
  float* scores;  // block-scores output, or the optional write-back
  int64_t ld_scores;
  uint32_t* ws_cnt;   // split select: one arrival counter per row
  uint32_t* ws_keys;  // split select: [rows, nblocks] score keys
  int64_t items;      // work items (rows * chunks)
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

__device__ __forceinline__ RowGeom row_geom(const Params& p, int64_t r, bool pin) {
  RowGeom g;
  int64_t grp = r / p.R;
  g.s = p.ks ? (int64_t)p.ks[grp] : 0;
  int64_t e = (int64_t)p.ke[grp];
  g.row = p.logits + r * p.ld;
  g.lo = g.s > 0 ? g.s : 0;
  g.hi = e < p.width ? e : p.width;
  int64_t nvb = 0;
  if (g.hi > g.lo) nvb = (g.hi - g.s + p.B - 1) / p.B;
  if (nvb > p.nblocks) nvb = p.nblocks;
  g.nvb = (int32_t)nvb;
  g.pin = -1;
  if (pin && e > g.s) {
    int64_t q = (e - g.s - 1) / p.B;
    if (q < p.nblocks) g.pin = (int32_t)q;
  }
  g.nsel = g.nvb > g.pin + 1 ? g.nvb : g.pin + 1;
  return g;
}

// Streams blocks [b0, b1) (b1 <= nvb) of a row on the vector path: s >= 0,
// (row + s) 16-byte aligned and width % 4 == 0, so every float4 that holds an
// in-window column lies inside the row.  B = 4*G.  Calls emit(b, max) once per
// block, from one lane of the block.
//
// The loads are branch-free: a lane past the chunk's last unit re-reads that
// unit (same cache line) and masks it, so all kUnroll loads of a lane issue
// back to back.
template <int G, class Emit>
__device__ __forceinline__ void stream_vec(const RowGeom& g, int32_t b0, int32_t b1,
                                           Emit& emit) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const float4* base = reinterpret_cast<const float4*>(g.row + g.s);
  const int32_t span = (int32_t)(g.hi - g.s);        // in-window columns from s
  const int32_t nu_row = (span + 3) >> 2;            // units holding one of them
  const int32_t ub = b0 * G;
  const int32_t ue = b1 * G < nu_row ? b1 * G : nu_row;
  const int32_t ntiles = (ue - ub + 63) >> 6;
  const float ninf = -__builtin_inff();
  for (int32_t t0 = wave; t0 < ntiles; t0 += kWaves * kUnroll) {
    float4 v[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int32_t u = ub + ((t0 + j * kWaves) << 6) + lane;
      v[j] = base[u < ue ? u : ue - 1];
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int32_t t = t0 + j * kWaves;
      const int32_t u = ub + (t << 6) + lane;
      const int32_t lim = u < ue ? span - 4 * u : 0;  // valid columns in this unit
      const float x = lim > 0 ? v[j].x : ninf;
      const float y = lim > 1 ? v[j].y : ninf;
      const float z = lim > 2 ? v[j].z : ninf;
      const float w = lim > 3 ? v[j].w : ninf;
      float m = fmaximum(fmaximum(x, y), fmaximum(z, w));
      m = group_max<G>(m);
      if (t < ntiles) {
        const int32_t b = b0 + (((t << 6) + lane) / G);
        if ((lane % G) == 0 && b < b1) emit(b, m);
      }
    }
  }
}

// Any block size and alignment: gl = largest power of two <= min(B, 64)
// lanes share a block, each striding over the block's in-window columns with
// scalar loads, four in flight; a masked slot re-reads the block's first
// in-window column.
template <class Emit>
__device__ __forceinline__ void stream_scalar(const RowGeom& g, int32_t B, int32_t b0,
                                              int32_t b1, Emit& emit) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int gl = 1;
  while (gl * 2 <= B && gl < 64) gl *= 2;
  const int per_wave = 64 / gl;
  const int sub = lane & (gl - 1);
  const float ninf = -__builtin_inff();
  for (int64_t bb = (int64_t)b0 + (int64_t)wave * per_wave; bb < b1;
       bb += (int64_t)kWaves * per_wave) {
    const int64_t b = bb + lane / gl;
    const int64_t cs = g.s + b * B;  // first column of block b
    const int64_t lo = b < b1 ? (cs > g.lo ? cs : g.lo) : 0;
    const int64_t hi = b < b1 ? (cs + B < g.hi ? cs + B : g.hi) : 0;
    float m = ninf;
    for (int64_t c = lo + sub; c < hi; c += 4 * gl) {
      float x[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t cq = c + (int64_t)q * gl;
        x[q] = g.row[cq < hi ? cq : lo];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) m = fmaximum(m, c + (int64_t)q * gl < hi ? x[q] : ninf);
    }
    m = group_max_dyn(m, gl);
    if (sub == 0 && b < b1) emit((int32_t)b, m);
  }
}

template <int G, class Emit>
__device__ __forceinline__ void stream_blocks(const Params& p, const RowGeom& g, int32_t b0,
                                              int32_t b1, Emit& emit) {
  if (b1 <= b0) return;
  if constexpr (G > 0) {
    if (p.vec_ok && g.s >= 0 && ((reinterpret_cast<uintptr_t>(g.row + g.s) & 15u) == 0)) {
      stream_vec<G>(g, b0, b1, emit);
      return;
    }
  }
  stream_scalar(g, p.B, b0, b1, emit);
}

struct EmitKeyLds {
  uint32_t* keys;
  __device__ void operator()(int32_t b, float m) const { keys[b] = order_key(m); }
};

struct EmitKeyGlobal {
  uint32_t* keys;
  __device__ void operator()(int32_t b, float m) const { keys[b] = order_key(m); }
};

struct EmitScore {
  float* row;
  int32_t pin;
  __device__ void operator()(int32_t b, float m) const {
    row[b] = b == pin ? __builtin_inff() : canonical(m);
  }
};

// ---------------------------------------------------------------- select --

__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  if (lane == 0) wave_tot[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += wave_tot[w];
  __syncthreads();
  return t;
}

// Exclusive prefix sum over threads in thread order.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wave_tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) before += (w < wave) ? wave_tot[w] : 0u;
  __syncthreads();
  return before + x - v;
}

// Top-k over the score keys keys[0, nsel) of one row (all threads of the
// workgroup call it).  Overwrites keys with rank keys.  Writes out_row[0, k).
__device__ void select_topk(uint32_t* smem, uint32_t* keys, int32_t nsel, int32_t k,
                            int32_t* out_row) {
  uint32_t* hist = smem;
  uint32_t* wave_tot = smem + kHistWords;
  uint32_t* misc = wave_tot + kWaveWords;
  uint32_t* sel_key = keys + nsel;
  const int tid = threadIdx.x;

  uint32_t cnt = 0;
  for (int32_t i = tid; i < nsel; i += kThreads) {
    const uint32_t rk = rank_key(keys[i]);
    keys[i] = rk;
    cnt += rk != 0u;
  }
  const uint32_t nvalid = block_sum(cnt, wave_tot);
  const int32_t keff = (uint32_t)k < nvalid ? k : (int32_t)nvalid;

  // Threshold: candidates are rank keys >= tgt, plus the first need_eq keys
  // equal to teq in block-id order.
  uint32_t tgt = 1u, teq = 0u;
  int32_t need_eq = 0;
  if (keff > 0 && (uint32_t)keff < nvalid) {
    uint32_t prefix = 0, remaining = (uint32_t)keff;
    bool whole_bucket = false;
    for (int shift = 24; shift >= 0; shift -= 8) {
      hist[tid] = 0u;  // kThreads == 256 bins
      __syncthreads();
      const uint32_t hmask = shift == 24 ? 0u : (0xFFFFFFFFu << (shift + 8));
      for (int32_t i = tid; i < nsel; i += kThreads) {
        const uint32_t rk = keys[i];
        if (rk != 0u && (rk & hmask) == prefix) atomicAdd(&hist[(rk >> shift) & 255u], 1u);
      }
      __syncthreads();
      // Thread t looks at digit 255 - t: the exclusive scan counts the keys
      // whose digit is larger.
      const uint32_t c = hist[255 - tid];
      const uint32_t above = block_exclusive_scan(c, wave_tot);
      if (above < remaining && above + c >= remaining) {
        misc[0] = 255u - tid;
        misc[1] = remaining - above;
        misc[2] = c;
      }
      __syncthreads();
      const uint32_t d = misc[0], rem = misc[1], cb = misc[2];
      __syncthreads();
      prefix |= d << shift;
      if (rem == cb) {  // the whole bucket is taken: every key >= prefix
        whole_bucket = true;
        break;
      }
      remaining = rem;
    }
    if (whole_bucket) {
      tgt = prefix;
    } else {
      tgt = prefix + 1u;
      teq = prefix;
      need_eq = (int32_t)remaining;
    }
  }
  const int32_t c_gt = keff - need_eq;

  // Compaction in block-id order: thread t owns ids [t*m, t*m + m).
  const int32_t m = (nsel + kThreads - 1) / kThreads;
  const int32_t i0 = tid * m;
  const int32_t i1 = i0 + m < nsel ? i0 + m : nsel;
  uint32_t ngt = 0, neq = 0;
  if (keff > 0) {
    for (int32_t i = i0; i < i1; ++i) {
      const uint32_t rk = keys[i];
      ngt += (rk >= tgt && rk != 0u);
      neq += (need_eq > 0 && rk == teq);
    }
  }
  const uint32_t packed = block_exclusive_scan((ngt << 16) | neq, wave_tot);
  uint32_t off_gt = packed >> 16, off_eq = packed & 0xFFFFu;
  if (keff > 0) {
    uint32_t* sel_id = sel_key + (keff > 0 ? keff : 1);
    for (int32_t i = i0; i < i1; ++i) {
      const uint32_t rk = keys[i];
      if (rk >= tgt && rk != 0u) {
        sel_key[off_gt] = rk;
        sel_id[off_gt] = (uint32_t)i;
        ++off_gt;
      } else if (need_eq > 0 && rk == teq) {
        if (off_eq < (uint32_t)need_eq) out_row[c_gt + (int32_t)off_eq] = i;
        ++off_eq;
      }
    }
    __syncthreads();
    // Order the keys above the threshold: rank = #larger + #equal with a
    // smaller id (sel_* is in id order).
    for (int32_t i = tid; i < c_gt; i += kThreads) {
      const uint32_t ki = sel_key[i];
      int32_t r = 0;
      for (int32_t j = 0; j < c_gt; ++j) {
        const uint32_t kj = sel_key[j];
        r += (kj > ki) || (kj == ki && j < i);
      }
      out_row[r] = (int32_t)sel_id[i];
    }
  }
  for (int32_t j = keff + tid; j < k; j += kThreads) out_row[j] = -1;
}

// Shared tail of both select kernels: keys[0, nvb) hold the streamed block
// keys; fill, pin, optional write-back, select.
__device__ void finish_row(const Params& p, int64_t r, const RowGeom& g, uint32_t* smem,
                           uint32_t* keys) {
  for (int32_t b = g.nvb + (int32_t)threadIdx.x; b < g.nsel; b += kThreads) keys[b] = kKeyNegInf;
  __syncthreads();
  if (g.pin >= 0 && threadIdx.x == 0) keys[g.pin] = kKeyPosInf;
  __syncthreads();
  if (p.scores) {
    float* srow = p.scores + r * p.ld_scores;
    for (int32_t b = threadIdx.x; b < p.nblocks; b += kThreads)
      srow[b] = b < g.nsel ? key_value(keys[b]) : -__builtin_inff();
  }
  select_topk(smem, keys, g.nsel, p.k, p.out + r * p.ld_out);
}

// One workgroup per row: stream the row into LDS keys, then select.
template <int G>
__global__ void __launch_bounds__(kThreads) select_rows_kernel(Params p) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem + kHeadWords;
  for (int64_t r = blockIdx.x; r < p.items; r += gridDim.x) {
    const RowGeom g = row_geom(p, r, true);
    EmitKeyLds emit{keys};
    stream_blocks<G>(p, g, 0, g.nvb, emit);
    __syncthreads();
    finish_row(p, r, g, smem, keys);
    __syncthreads();
  }
}

// Rows split in chunks of chunk_blocks blocks; item = r * nchunks + c.  Only
// the chunks that hold in-window blocks (at least chunk 0) take part; the last
// of them to arrive gathers the row's keys and selects.
template <int G>
__global__ void __launch_bounds__(kThreads) select_split_kernel(Params p) {
  extern __shared__ uint32_t smem[];
  uint32_t* keys = smem + kHeadWords;
  uint32_t* misc = smem + kHistWords + kWaveWords;
  for (int64_t item = blockIdx.x; item < p.items; item += gridDim.x) {
    const int64_t r = item / p.nchunks;
    const int32_t c = (int32_t)(item - r * p.nchunks);
    const RowGeom g = row_geom(p, r, true);
    const int32_t nact = g.nvb > 0 ? (g.nvb + p.chunk_blocks - 1) / p.chunk_blocks : 1;
    if (c >= nact) continue;  // uniform across the workgroup
    const int32_t b0 = c * p.chunk_blocks;
    const int32_t b1 = b0 + p.chunk_blocks < g.nvb ? b0 + p.chunk_blocks : g.nvb;
    uint32_t* wrow = p.ws_keys + r * p.nblocks;
    EmitKeyGlobal emit{wrow};
    stream_blocks<G>(p, g, b0, b1, emit);
    // Release this chunk's keys at agent scope (the chunks of a row run on
    // different XCDs, each with its own L2), then count the arrival.
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t old = atomicAdd(p.ws_cnt + r, 1u);
      const uint32_t last = old + 1u == (uint32_t)nact;
      if (last) __hip_atomic_store(p.ws_cnt + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __threadfence();
      misc[8] = last;
    }
    __syncthreads();
    const bool last = misc[8] != 0u;
    __syncthreads();
    if (!last) continue;
    __threadfence();  // acquire: the other chunks' keys
    for (int32_t b = threadIdx.x; b < g.nvb; b += kThreads)
      keys[b] = __hip_atomic_load(wrow + b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    finish_row(p, r, g, smem, keys);
    __syncthreads();
  }
}

// Block scores to HBM; item = r * nchunks + c covers blocks
// [c*chunk_blocks, (c+1)*chunk_blocks) of row r, in-window or not.
template <int G>
__global__ void __launch_bounds__(kThreads) block_scores_kernel(Params p) {
  for (int64_t item = blockIdx.x; item < p.items; item += gridDim.x) {
    const int64_t r = item / p.nchunks;
    const int32_t c = (int32_t)(item - r * p.nchunks);
    const RowGeom g = row_geom(p, r, p.pin != 0);
    const int32_t b0 = c * p.chunk_blocks;
    const int32_t b1 = b0 + p.chunk_blocks < p.nblocks ? b0 + p.chunk_blocks : p.nblocks;
    float* srow = p.scores + r * p.ld_scores;
    const int32_t sb1 = b1 < g.nvb ? b1 : g.nvb;
    EmitScore emit{srow, g.pin};
    stream_blocks<G>(p, g, b0, sb1, emit);
    const int32_t f0 = b0 > g.nvb ? b0 : g.nvb;
    for (int32_t b = f0 + (int32_t)threadIdx.x; b < b1; b += kThreads)
      srow[b] = b == g.pin ? __builtin_inff() : -__builtin_inff();
  }
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

DSA_KERNEL_TABLE(select_rows_kernel)
DSA_KERNEL_TABLE(select_split_kernel)
DSA_KERNEL_TABLE(block_scores_kernel)

dsa_status_t launch(void* fn, int64_t items, size_t lds, hipStream_t stream, Params& p) {
  p.items = items;
  const int64_t grid = items < kMaxGrid ? items : kMaxGrid;
  void* args[] = {&p};
  hipError_t err = hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), args, lds, stream);
  if (err != hipSuccess) {
    (void)hipGetLastError();
    return DSA_ERR_HIP;
  }
  return DSA_OK;
}

bool misaligned(const void* ptr, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(ptr) & (a - 1)) != 0;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

size_t counters_bytes(int64_t rows) { return (size_t)cdiv(rows * 4, 256) * 256; }

size_t select_lds_bytes(int64_t nblocks, int32_t k) {
  const int64_t kcap = k < nblocks ? k : nblocks;
  return (size_t)(kHeadWords + nblocks + 2 * (kcap > 0 ? kcap : 1)) * 4;
}

// Chunk size for split rows: aim at ~2048 workgroups in total, 2K-16K columns
// each, and a multiple of the blocks one wave instruction covers.
int32_t auto_chunk_blocks(int64_t rows, int64_t width, int32_t B) {
  int64_t cols = rows > 0 ? (rows * width) / 2048 : width;
  if (cols < 2048) cols = 2048;
  if (cols > 16384) cols = 16384;
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

}  // namespace

extern "C" {

const char* dsa_status_string(dsa_status_t status) {
  switch (status) {
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
  return counters_bytes(rows) + (size_t)rows * (size_t)nblocks * 4u;
}

dsa_status_t dsa_select_plan(int64_t rows, int64_t width, int32_t block_size,
                             int32_t topk_blocks, int32_t* plan, int32_t* chunk_blocks) {
  if (rows < 0 || width < 0 || block_size < 1 || topk_blocks < 0 || !plan || !chunk_blocks)
    return DSA_ERR_INVALID_ARG;
  const int64_t nblocks = width > 0 ? cdiv(width, block_size) : 0;
  const int32_t cb = auto_chunk_blocks(rows, width, block_size);
  const int64_t nchunks = cdiv(nblocks, cb);
  // Many rows fill the GPU one workgroup per row; few long rows are split.
  if (rows >= 1024 || nchunks <= 1) {
    *plan = 1;
    *chunk_blocks = 0;
  } else {
    *plan = 2;
    *chunk_blocks = cb;
  }
  return DSA_OK;
}

dsa_status_t dsa_block_scores(const float* logits, int64_t rows, int64_t width,
                              int64_t ld_logits, const int32_t* row_ks,
                              const int32_t* row_ke, int32_t block_size,
                              int32_t row_repeat, int32_t pin_newest, float* scores,
                              int64_t ld_scores, hipStream_t stream) {
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
  p.pin = pin_newest;
  p.nblocks = (int32_t)nblocks;
  p.vec_ok = (width % 4) == 0 && width < ((int64_t)1 << 30);
  // ~8K columns per workgroup, a whole number of wave tiles.
  int64_t cb = cdiv(8192, block_size);
  const int g = lanes_per_block(block_size);
  if (g > 0) cb = cdiv(cb, 64 / g) * (64 / g);
  if (cb > nblocks) cb = nblocks;
  p.chunk_blocks = (int32_t)cb;
  p.nchunks = (int32_t)cdiv(nblocks, cb);
  p.scores = scores;
  p.ld_scores = ld_scores;
  return launch(block_scores_kernel_ptr(g), rows * p.nchunks, 0, stream, p);
}

dsa_status_t dsa_select_candidate_blocks_plan(
    const float* logits, int64_t rows, int64_t width, int64_t ld_logits,
    const int32_t* row_ks, const int32_t* row_ke, int32_t topk_blocks, int32_t block_size,
    int32_t row_repeat, int32_t* out, int64_t ld_out, float* scores_out, int64_t ld_scores,
    void* workspace, size_t workspace_bytes, int32_t plan, int32_t chunk_blocks,
    hipStream_t stream) {
  if (rows < 0 || width < 0 || block_size < 1 || row_repeat < 1 || topk_blocks < 0)
    return DSA_ERR_INVALID_ARG;
  if (plan < 0 || plan > 2 || chunk_blocks < 0) return DSA_ERR_INVALID_ARG;
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
  const size_t lds = select_lds_bytes(nblocks, topk_blocks);
  if (lds > kLdsLimit) return DSA_ERR_UNSUPPORTED;
  const size_t need = dsa_select_workspace_bytes(rows, width, block_size, topk_blocks);
  if (!workspace || workspace_bytes < need || misaligned(workspace, 4)) return DSA_ERR_WORKSPACE;

  int32_t auto_plan = 1, auto_cb = 0;
  dsa_select_plan(rows, width, block_size, topk_blocks, &auto_plan, &auto_cb);
  if (plan == 0) {
    plan = auto_plan;
    chunk_blocks = auto_cb;
  }
  if (plan == 2 && chunk_blocks == 0) chunk_blocks = auto_chunk_blocks(rows, width, block_size);

  Params p = {};
  p.logits = logits;
  p.rows = rows;
  p.width = width;
  p.ld = ld_logits;
  p.ks = row_ks;
  p.ke = row_ke;
  p.B = block_size;
  p.R = row_repeat;
  p.pin = 1;
  p.k = topk_blocks;
  p.nblocks = (int32_t)nblocks;
  p.vec_ok = (width % 4) == 0 && width < ((int64_t)1 << 30);
  p.out = out;
  p.ld_out = ld_out;
  p.scores = scores_out;
  p.ld_scores = ld_scores;
  p.ws_cnt = static_cast<uint32_t*>(workspace);
  p.ws_keys = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + counters_bytes(rows));
  const int g = lanes_per_block(block_size);
  if (plan == 1) {
    p.chunk_blocks = p.nblocks;
    p.nchunks = 1;
    return launch(select_rows_kernel_ptr(g), rows, lds, stream, p);
  }
  p.chunk_blocks = chunk_blocks < p.nblocks ? chunk_blocks : p.nblocks;
  p.nchunks = (int32_t)cdiv(nblocks, p.chunk_blocks);
  if (rows * (int64_t)p.nchunks > (int64_t)INT32_MAX) return DSA_ERR_UNSUPPORTED;
  return launch(select_split_kernel_ptr(g), rows * p.nchunks, lds, stream, p);
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

}  // extern "C"
