// calib.hip - measurement helpers (copy, read stream, empty launch); see
// include/dsa_calib.h.  Not part of candidate-block selection.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa_calib.h"

namespace {

constexpr int kThreads = 256;
constexpr unsigned kGrid = 4096;

__global__ void __launch_bounds__(kThreads) copy_kernel(const uint4* __restrict__ src,
                                                        uint4* __restrict__ dst, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kThreads)
    dst[i] = src[i];
}

__global__ void __launch_bounds__(kThreads) read_kernel(const uint4* __restrict__ src, int64_t n,
                                                        uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  constexpr int U = 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  for (; i + (U - 1) * stride < n; i += U * stride) {
    uint4 v[U];
#pragma unroll
    for (int j = 0; j < U; ++j) v[j] = src[i + j * stride];
#pragma unroll
    for (int j = 0; j < U; ++j) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
  for (; i < n; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t w[kThreads / 64];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

__global__ void empty_kernel() {}

bool bad(const void* p, size_t bytes) {
  return !p || (reinterpret_cast<uintptr_t>(p) & 15u) != 0 || (bytes & 15u) != 0;
}

}  // namespace

extern "C" {

int dsa_calib_copy(const void* src, void* dst, size_t bytes, hipStream_t stream) {
  if (bad(src, bytes) || bad(dst, bytes)) return 1;
  if (bytes == 0) return 0;
  const int64_t n = (int64_t)(bytes / 16);
  copy_kernel<<<dim3(kGrid), dim3(kThreads), 0, stream>>>(static_cast<const uint4*>(src),
                                                          static_cast<uint4*>(dst), n);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

size_t dsa_calib_read_sink_words(void) { return kGrid; }

int dsa_calib_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bad(src, bytes) || !sink) return 1;
  if (bytes == 0) return 0;
  read_kernel<<<dim3(kGrid), dim3(kThreads), 0, stream>>>(static_cast<const uint4*>(src),
                                                          (int64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int dsa_calib_empty(hipStream_t stream) {
  empty_kernel<<<dim3(1), dim3(64), 0, stream>>>();
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"
