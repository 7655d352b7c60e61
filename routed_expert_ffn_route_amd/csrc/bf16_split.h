// bf16_split.h -- x as a pair of bf16 values for the MFMA paths: hi = RNE(x), lo = RNE(x - hi),
// so that hi + lo carries x to about 16 significant bits.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace moe {

__device__ __forceinline__ uint16_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Elements [i0, n) with stride `step`: hi[i], lo[i] of x[i].
__device__ __forceinline__ void split_x_range(const float* x, size_t n, uint16_t* hi,
                                              uint16_t* lo, size_t i0, size_t step) {
  for (size_t i = i0; i < n; i += step) {
    const float f = x[i];
    const uint16_t h = bf16_rne_bits(f);
    hi[i] = h;
    lo[i] = bf16_rne_bits(f - __uint_as_float((uint32_t)h << 16));
  }
}

}  // namespace moe
