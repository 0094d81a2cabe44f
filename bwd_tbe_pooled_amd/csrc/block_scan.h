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

// Exclusive scan of v[0..n) in place by one 1024-thread workgroup; returns
// the total to every thread (`wsum`: 16 ints of LDS). The array goes in
// rounds of 1024 x 32 elements: each thread loads 32 consecutive ones into
// registers, sums them, the per-thread sums are scanned across the workgroup,
// and each thread writes its 32 prefixes. Few barriers and all loads of a
// round in flight at once, instead of one barrier-separated step per 1024.
// Calls `on_value(i, prefix)` for every element after writing it.
template <typename F>
__device__ int32_t block1024_scan_inplace(int32_t* __restrict__ v, int64_t n, int32_t* wsum,
                                          F on_value) {
  constexpr int kPer = 32;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  int32_t carry = 0;
  for (int64_t base = 0; base < n; base += (int64_t)1024 * kPer) {
    const int64_t a = base + (int64_t)threadIdx.x * kPer;
    int32_t x[kPer];
    int32_t s = 0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      x[k] = a + k < n ? v[a + k] : 0;
      s += x[k];
    }
    const int32_t inc = wave_inclusive_scan(s);
    if (lane == kWave - 1) wsum[wave] = inc;
    __syncthreads();
    int32_t pre = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int32_t y = wsum[w];
      if (w < wave) pre += y;
      tot += y;
    }
    __syncthreads();
    int32_t run = carry + pre + inc - s;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      if (a + k < n) {
        v[a + k] = run;
        on_value(a + k, run);
      }
      run += x[k];
    }
    carry += tot;
  }
  return carry;
}

}  // namespace tbe
