// Copy-on-write block copy: physical block dst[i] of both pools becomes a copy
// of block src[i].
//
// "Paged Attention and KV Cache Fragmentation" (inferenceengineering.co),
// section "How PagedAttention maps an OS concept onto GPU memory": sequences
// that share a prefix or are beam-search branches point at the same physical
// blocks and diverge only where their content differs.  When one of them grows
// into a shared block that is only partly filled, the allocator gives it a
// fresh block and this kernel copies the shared tokens into it, before the new
// tokens are written.
//
// A block of one pool is contiguous in both pool layouts ([NB][H_kv][...]), so
// a pair is two flat copies of H_kv * D * bs * elem bytes.  One workgroup moves
// one tile of kCopyThreads x kCopyUnroll 16-byte units of one block of one
// pool; all loads of a thread are issued before its stores.

#include <hip/hip_runtime.h>

#include "internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyBlocksArgs a) {
  const long long per_pair = 2 * a.tiles;
  const int pair = (int)(blockIdx.x / per_pair);
  const long long r = blockIdx.x % per_pair;
  const int pool = (int)(r / a.tiles);
  const long long tile = r % a.tiles;
  const int src = a.src[pair], dst = a.dst[pair];
  // ids outside the pool are skipped (caller error); a self-copy is a no-op
  if ((unsigned)src >= (unsigned)a.NB || (unsigned)dst >= (unsigned)a.NB || src == dst) return;
  u32x4* base = (u32x4*)(pool == 0 ? a.k_pool : a.v_pool);
  const u32x4* from = base + (size_t)src * a.block_units;
  u32x4* to = base + (size_t)dst * a.block_units;
  const long long first = tile * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const long long i = first + (long long)u * kCopyThreads;
    if (i < a.block_units) v[u] = __builtin_nontemporal_load(from + i);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const long long i = first + (long long)u * kCopyThreads;
    if (i < a.block_units) to[i] = v[u];
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s) {
  const long long grid = (long long)a.n_pairs * 2 * a.tiles;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)grid), dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
