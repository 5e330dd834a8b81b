// fp32 -> OCP E4M3FN encoding shared by the append kernel and the decode's fused append, so that
// both write the same codes for the same value.
//
// "Paged Attention and KV Cache Fragmentation" (inferenceengineering.co), section "Quantization as
// a way to stretch paged memory further": an FP8 cache stores each value in one byte.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace pkv {
namespace {

// fp32 -> OCP E4M3FN, round to nearest even; |y| >= 448 or inf saturates to
// +-448 (code 0x7E), NaN -> 0x7F with the input's sign.  Integer bit work for
// the normal range, an exact power-of-two scaling plus rint for subnormals.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __builtin_bit_cast(uint32_t, y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;   // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;  // >= 448 (and inf)
  const int e = (int)(a >> 23) - 127;
  if (e >= -6) {  // normal E4M3: keep 3 of the 23 mantissa bits, ties to even
    const uint32_t mant = a & 0x7FFFFFu;
    const uint32_t q = mant >> 20, rem = mant & 0xFFFFFu;
    uint32_t code = ((uint32_t)(e + 7) << 3) | q;
    if (rem > 0x80000u || (rem == 0x80000u && (q & 1u))) code += 1u;  // carry into the exponent is correct
    return sign | code;
  }
  // subnormal E4M3: value = k * 2^-9, k = rint(|y| * 2^9) in 0..8 (8 is the smallest normal)
  const float k = __builtin_rintf(__builtin_bit_cast(float, a) * 512.0f);
  return sign | (uint32_t)k;
}

// The code a bf16 element x (its 16 bits) takes in a pool with per-head scale sc: x / sc in IEEE
// fp32 division, then encoded.
__device__ __forceinline__ uint32_t bf16_to_e4m3(uint32_t x16, float sc) {
  return f32_to_e4m3(__builtin_bit_cast(float, x16 << 16) / sc);
}

}  // namespace
}  // namespace pkv
