// Whole-block moves: copy-on-write copies between blocks of the pools, and the
// swap gather / scatter between blocks and a contiguous staging buffer.
//
// "Paged Attention and KV Cache Fragmentation" (inferenceengineering.co):
//   - section "How PagedAttention maps an OS concept onto GPU memory":
//     sequences that share a prefix or are beam-search branches point at the
//     same physical blocks and diverge only where their content differs.  When
//     one of them grows into a shared block that is only partly filled, the
//     allocator gives it a fresh block and the copy moves the shared tokens
//     into it, before the new tokens are written;
//   - section "Offloading paged KV blocks to CPU DRAM and NVMe": blocks move
//     between HBM and host memory, and the paged layout scatters them, which
//     turns the move into many small transfers.  The gather packs a set of
//     blocks into one contiguous buffer (device memory for one later DMA copy,
//     or mapped pinned host memory written directly); the scatter unpacks such
//     a buffer into the blocks swap-in hands out.
//
// A block of one pool is contiguous in both pool layouts ([NB][H_kv][...]), so
// every move is a flat copy of H_kv * D * bs * elem bytes; a staging record is
// the K block followed by the V block.  One workgroup moves one tile of
// kCopyThreads x kCopyUnroll 16-byte units of one block of one pool; all loads
// of a thread are issued before its stores.

#include <hip/hip_runtime.h>

#include "internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int MODE>
__global__ __launch_bounds__(kCopyThreads) void block_move_kernel(CopyBlocksArgs a) {
  const long long per_pair = 2 * a.tiles;
  const int i = (int)(blockIdx.x / per_pair);
  const long long r = blockIdx.x % per_pair;
  const int pool = (int)(r / a.tiles);
  const long long tile = r % a.tiles;
  u32x4* base = (u32x4*)(pool == 0 ? a.k_pool : a.v_pool);
  const size_t rec = (2 * (size_t)i + pool) * a.block_units;  // staging record of (i, pool)
  const u32x4* from;
  u32x4* to;
  if constexpr (MODE == kMovePairs) {
    const int src = a.src[i], dst = a.dst[i];
    // ids outside the pool are skipped (caller error); a self-copy is a no-op
    if ((unsigned)src >= (unsigned)a.NB || (unsigned)dst >= (unsigned)a.NB || src == dst) return;
    from = base + (size_t)src * a.block_units;
    to = base + (size_t)dst * a.block_units;
  } else if constexpr (MODE == kMoveGather) {
    const int src = a.src[i];
    if ((unsigned)src >= (unsigned)a.NB) return;
    from = base + (size_t)src * a.block_units;
    to = (u32x4*)a.staging + rec;
  } else {
    const int dst = a.dst[i];
    if ((unsigned)dst >= (unsigned)a.NB) return;
    from = (const u32x4*)a.staging + rec;
    to = base + (size_t)dst * a.block_units;
  }
  const long long first = tile * (kCopyThreads * kCopyUnroll) + threadIdx.x;
  u32x4 v[kCopyUnroll];
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const long long k = first + (long long)u * kCopyThreads;
    if (k < a.block_units) v[u] = __builtin_nontemporal_load(from + k);
  }
#pragma unroll
  for (int u = 0; u < kCopyUnroll; ++u) {
    const long long k = first + (long long)u * kCopyThreads;
    if (k < a.block_units) to[k] = v[u];
  }
}

}  // namespace

hipError_t launch_block_move(const CopyBlocksArgs& a, BlockMove mode, hipStream_t s) {
  const dim3 grid((unsigned)((long long)a.n_pairs * 2 * a.tiles));
  if (mode == kMovePairs)
    hipLaunchKernelGGL(block_move_kernel<kMovePairs>, grid, dim3(kCopyThreads), 0, s, a);
  else if (mode == kMoveGather)
    hipLaunchKernelGGL(block_move_kernel<kMoveGather>, grid, dim3(kCopyThreads), 0, s, a);
  else
    hipLaunchKernelGGL(block_move_kernel<kMoveScatter>, grid, dim3(kCopyThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
