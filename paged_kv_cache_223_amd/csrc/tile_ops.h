// Matrix-core tile operations shared by the paged decode and prefill kernels
// (gfx950): operand types, the bf16 and fp16 MFMAs, E4M3 -> bf16 and fp16
// conversions, the P regroup across lane groups, the maximum over lane groups,
// and the clamped block-table lookup.
//
// MFMA v_mfma_f32_16x16x32_bf16 lane layouts (checked on the device):
//   A[16][32]: lane l holds A[l % 16][8 * (l / 16) + j], j = 0..7
//   B[32][16]: lane l holds B[8 * (l / 16) + j][l % 16]
//   C[16][16]: lane l holds C[4 * (l / 16) + i][l % 16], i = 0..3
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "internal.h"

namespace pkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// physical block of logical block j (clamped to the sequence's last block; an
// id outside the pool is read as block 0 so that no access leaves the pool).
// The table is read through the constant address space: no kernel writes it, and
// so its wave-uniform reads stay scalar loads whatever else a kernel stores.
__device__ __forceinline__ int block_id(const int32_t* __restrict__ tab, int j, int last, int NB) {
  j = j > last ? last : j;
  const int id = ((const __attribute__((address_space(4))) int32_t*)tab)[j];
  return (unsigned)id < (unsigned)NB ? id : 0;
}

template <int KVT>
struct KvTraits;
template <>
struct KvTraits<PKV_BF16> {
  static constexpr int kBytes = 2;
};
template <>
struct KvTraits<PKV_FP8_E4M3> {
  static constexpr int kBytes = 1;
};

// head-dim offset of the 8 k-slots lane group kg feeds into QK MFMA number c
template <int KVT>
__device__ __forceinline__ constexpr int qk_dofs(int c, int kg) {
  return KVT == PKV_BF16 ? 32 * c + 8 * kg : 64 * (c / 2) + 16 * kg + 8 * (c % 2);
}

// E4M3 (OCP) pair -> bf16 pair, exact; `hi` picks bytes 2,3 instead of 0,1
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
  bf16x2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  return u32x4{e4m3x2_to_bf16x2(w0, false), e4m3x2_to_bf16x2(w0, true), e4m3x2_to_bf16x2(w1, false),
               e4m3x2_to_bf16x2(w1, true)};
}

// eight E4M3 codes (w0: codes 0-3, w1: codes 4-7) -> four fp16 pairs in order (exact: every E4M3
// value is an fp16 value)
__device__ __forceinline__ u32x4 e4m3x8_to_f16x8(uint32_t w0, uint32_t w1) {
  return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false)),
               __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true))};
}

// two fp32 -> packed fp16 pair, round to nearest even; x in the low half
__device__ __forceinline__ uint32_t pack_f16(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{x, y}), f16x2));
}

__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}

// Regroup the P operand across lane groups.  In: lane group r (lanes 16r ..
// 16r+15) holds, for its head, tokens 4r..4r+3 of the chunk's first half in
// words 0,1 and of the second half in words 2,3 (the QK^T accumulator rows).
// Out: lane group r holds tokens 8r .. 8r+7 in words 0..3, so that each
// lane's V operand is 8 consecutive tokens of one column.  With rows R0..R3
// of two registers X (half 0) and Y (half 1): permlane32_swap gives
// X' = [X0 X1 Y0 Y1], Y' = [X2 X3 Y2 Y3]; permlane16_swap then gives
// [X0 X2 Y0 Y2] (tokens 8r..8r+3) and [X1 X3 Y1 Y3] (tokens 8r+4..8r+7).
__device__ __forceinline__ u32x4 tokens_by_eight(u32x4 v) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const auto a = __builtin_amdgcn_permlane32_swap(v[w], v[w + 2], false, false);
    const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[1], false, false);
    r[w] = b[0];
    r[w + 2] = b[1];
  }
  return r;
}

// Maximum over the four lane groups, i.e. over lanes l, l ^ 16, l ^ 32 and
// l ^ 48, without a round trip through LDS: swapping a register with itself
// across halves (permlane32_swap) leaves each lane with its own value and
// that of lane l ^ 32 in the two results, and across adjacent rows
// (permlane16_swap) with that of lane l ^ 16.  The results are copied into
// scalars before the bit casts: this compiler reads element 0 for a
// __builtin_bit_cast of element 1 of the returned pair.
__device__ __forceinline__ float max_over_groups(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const uint32_t a0 = a[0], a1 = a[1];
  const float y = fmaxf(__builtin_bit_cast(float, a0), __builtin_bit_cast(float, a1));
  const uint32_t v = __builtin_bit_cast(uint32_t, y);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  const uint32_t b0 = b[0], b1 = b[1];
  return fmaxf(__builtin_bit_cast(float, b0), __builtin_bit_cast(float, b1));
}

}  // namespace
}  // namespace pkv
