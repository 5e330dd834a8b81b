// Device helpers shared by the two decode paths (matrix-core and vector).
#pragma once

#include <hip/hip_runtime.h>

#include "internal.h"

namespace pkv {

// A sequence's length as the decode uses it: negative lengths count as 0 and lengths above the
// launch's cap are cut to it.  Read through the constant address space (no kernel writes the
// lengths), which keeps wave-uniform reads scalar.
__device__ __forceinline__ int seq_len(const int32_t* __restrict__ lens, int b, int cap) {
  int n = ((const __attribute__((address_space(4))) int32_t*)lens)[b];
  return n < 0 ? 0 : (n > cap ? cap : n);
}

// The hole [lo, hi) of logical positions sequence b does not attend: without
// masks it is empty; with them, t < n is attended iff t < sink or t >= window.
__device__ __forceinline__ void seq_hole(const DecodeArgs& a, int b, int& lo, int& hi) {
  lo = 0;
  hi = 0;
  if (a.sink_lens) lo = max(a.sink_lens[b], 0);
  if (a.window_starts) hi = a.window_starts[b];
  hi = max(hi, lo);
}

}  // namespace pkv
