// Device helpers for the fixed-order sums of per-run partials.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sd {

// Sum of p[u * stride] over u0 <= u < u1, added in order of u (the plain
// loop's sum, bit for bit) with 8 loads in flight at a time.
__device__ __forceinline__ float strided_sum_in_order(const float* p, int64_t stride, int u0, int u1) {
  float s = 0.f;
  for (int u = u0; u < u1; u += 8) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (u + j < u1) ? p[(int64_t)(u + j) * stride] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (u + j < u1) s += v[j];
  }
  return s;
}

}  // namespace sd
