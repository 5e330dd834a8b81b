// Measurement helpers: a read-only bandwidth probe (16-byte lane loads, the
// decode kernels' load width) and a plain copy of known size used to
// calibrate the memory-traffic counters.  Neither is part of the method.

#include <hip/hip_runtime.h>

#include "internal.h"

namespace pkv {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

// Each workgroup reads whole tiles of kThreads x kUnroll x 16 bytes with
// non-temporal loads (the decode kernels' K/V loads are non-temporal too);
// the tail that does not fill a tile is read by workgroup 0.
__global__ __launch_bounds__(kThreads) void stream_read_kernel(const uint4* __restrict__ src, size_t n16,
                                                               float* __restrict__ sink) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u* s = (const v4u*)src;
  constexpr size_t tile = (size_t)kThreads * kUnroll;
  uint32_t acc = 0;
  for (size_t t = blockIdx.x; (t + 1) * tile <= n16; t += gridDim.x) {
    v4u v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(s + t * tile + u * kThreads + threadIdx.x);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (blockIdx.x == 0)
    for (size_t i = n16 / tile * tile + threadIdx.x; i < n16; i += kThreads) {
      const v4u v = s[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  for (int o = 32; o; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  __shared__ uint32_t sh[kThreads / 64];
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int w = 0; w < kThreads / 64; ++w) r ^= sh[w];
    sink[blockIdx.x] = __builtin_bit_cast(float, r & 0x007FFFFFu);  // a finite value that depends on the data
  }
}

__global__ __launch_bounds__(kThreads) void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                        size_t n16) {
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

}  // namespace

size_t stream_read_blocks(size_t bytes) {
  const size_t n16 = bytes / 16;
  size_t blocks = n16 / ((size_t)kThreads * kUnroll);
  if (blocks > 256 * 8) blocks = 256 * 8;
  return blocks ? blocks : 1;
}

hipError_t launch_stream_read(const void* src, size_t bytes, float* sink, hipStream_t s) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)stream_read_blocks(bytes)), dim3(kThreads), 0, s,
                     (const uint4*)src, bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  size_t n16 = bytes / 16;
  size_t blocks = (n16 + kThreads - 1) / kThreads;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, s, (uint4*)dst, (const uint4*)src,
                     n16);
  return hipGetLastError();
}

}  // namespace pkv
