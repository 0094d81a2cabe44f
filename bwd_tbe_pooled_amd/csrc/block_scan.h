// Workgroup-wide scans for 256-thread (4-wave) workgroups.
#pragma once

#include "device.h"

namespace tbe {

// Inclusive scan across the 64 lanes of a wave.
__device__ __forceinline__ int32_t wave_inclusive_scan(int32_t x) {
  const int lane = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Exclusive scan over the 256 threads of a workgroup; `total` receives the sum.
// `scratch` must hold 4 ints of LDS; the call contains two barriers.
__device__ __forceinline__ int32_t block256_exclusive_scan(int32_t x, int32_t* scratch,
                                                            int32_t& total) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int32_t inc = wave_inclusive_scan(x);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  int32_t base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int32_t v = scratch[w];
    if (w < wave) base += v;
    total += v;
  }
  __syncthreads();
  return base + inc - x;
}

}  // namespace tbe
