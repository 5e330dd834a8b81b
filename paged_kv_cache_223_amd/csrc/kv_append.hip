// kv_append: scatter this step's K/V rows into their slots of the paged pools.
//
// "Paged Attention and KV Cache Fragmentation" (inferenceengineering.co),
// section "How PagedAttention maps an OS concept onto GPU memory": a token's
// keys and values go to the physical block that the sequence's table maps its
// logical position to; section "Quantization as a way to stretch paged memory
// further": an FP8 cache stores each value in one byte.
//
// One thread moves 8 consecutive head-dim elements of one (token, KV head):
// a 16-byte (bf16) / 8-byte (E4M3) / 2x16-byte (fp32) store into the K tile
// [D/X][bs][X] and 8 element stores into the V tile [D][bs].  Threads are
// ordered (token, head, 8-element group) so the K stores of one token are
// contiguous per 16-byte group.

#include <hip/hip_runtime.h>

#include "e4m3_encode.h"
#include "internal.h"

namespace pkv {
namespace {

template <int SRC, int DST>
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs p) {
  const int groups = p.D / 8;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long total = (long long)p.T * p.H_kv * groups;
  if (gid >= total) return;
  const int e = (int)(gid % groups);
  const int g = (int)((gid / groups) % p.H_kv);
  const int t = (int)(gid / ((long long)groups * p.H_kv));
  const long long slot = p.slots[t];
  if (slot < 0 || slot >= p.n_slots) return;
  const long long blk = slot / p.bs;
  const int off = (int)(slot % p.bs);
  const size_t src = ((size_t)t * p.H_kv + g) * p.D + 8 * e;
  const size_t tile = ((size_t)blk * p.H_kv + g) * (size_t)p.D * p.bs;  // element index of the (blk, g) tile
  const int d0 = 8 * e;
  for (int which = 0; which < 2; ++which) {
    const void* s = which ? p.v : p.k;
    void* pool = which ? p.v_pool : p.k_pool;
    if constexpr (DST == PKV_F32) {
      const float* sp = (const float*)s + src;
      const float4 lo = *(const float4*)sp, hi = *(const float4*)(sp + 4);
      float* pp = (float*)pool + tile;
      if (!which) {  // K: X = 4
        *(float4*)(pp + ((size_t)(d0 / 4) * p.bs + off) * 4) = lo;
        *(float4*)(pp + ((size_t)(d0 / 4 + 1) * p.bs + off) * 4) = hi;
      } else {
        const float v8[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) pp[(size_t)(d0 + j) * p.bs + off] = v8[j];
      }
    } else if constexpr (DST == PKV_BF16) {
      const uint4 x = *(const uint4*)((const uint16_t*)s + src);
      uint16_t* pp = (uint16_t*)pool + tile;
      if (!which) {  // K: X = 8, one 16-byte group
        *(uint4*)(pp + ((size_t)e * p.bs + off) * 8) = x;
      } else {
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int j = 0; j < 8; ++j)
          pp[(size_t)(d0 + j) * p.bs + off] = (uint16_t)(w[j / 2] >> (16 * (j % 2)));
      }
    } else {  // E4M3 pool
      uint32_t c[8];
      if constexpr (SRC == PKV_FP8_E4M3) {
        const uint2 x = *(const uint2*)((const uint8_t*)s + src);
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = ((j < 4 ? x.x : x.y) >> (8 * (j % 4))) & 0xFFu;
      } else {  // bf16 -> E4M3: y = x / scale[g], IEEE fp32 division
        const uint4 x = *(const uint4*)((const uint16_t*)s + src);
        const uint32_t w[4] = {x.x, x.y, x.z, x.w};
        const float sc = (which ? p.v_scale : p.k_scale)[g];
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = bf16_to_e4m3((w[j / 2] >> (16 * (j % 2))) & 0xFFFFu, sc);
      }
      uint8_t* pp = (uint8_t*)pool + tile;
      if (!which) {  // K: X = 16, this thread's 8 codes are half of a 16-byte group
        const uint2 packed = make_uint2(c[0] | c[1] << 8 | c[2] << 16 | c[3] << 24,
                                        c[4] | c[5] << 8 | c[6] << 16 | c[7] << 24);
        *(uint2*)(pp + ((size_t)(d0 / 16) * p.bs + off) * 16 + (d0 % 16)) = packed;
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) pp[(size_t)(d0 + j) * p.bs + off] = (uint8_t)c[j];
      }
    }
  }
}

template <int SRC, int DST>
hipError_t launch_t(const AppendArgs& a, hipStream_t s) {
  const long long total = (long long)a.T * a.H_kv * (a.D / 8);
  const long long grid = (total + 255) / 256;
  hipLaunchKernelGGL((kv_append_kernel<SRC, DST>), dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.src_dtype == PKV_F32 && a.pool_dtype == PKV_F32) return launch_t<PKV_F32, PKV_F32>(a, s);
  if (a.src_dtype == PKV_BF16 && a.pool_dtype == PKV_BF16) return launch_t<PKV_BF16, PKV_BF16>(a, s);
  if (a.src_dtype == PKV_BF16 && a.pool_dtype == PKV_FP8_E4M3) return launch_t<PKV_BF16, PKV_FP8_E4M3>(a, s);
  if (a.src_dtype == PKV_FP8_E4M3 && a.pool_dtype == PKV_FP8_E4M3)
    return launch_t<PKV_FP8_E4M3, PKV_FP8_E4M3>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
