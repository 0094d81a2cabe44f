// Row-gather probe (measurement aid): reads n random rows of a float32
// matrix with the load shape of the library's gathers and sums them, so that
// bytes read over time gives the rate at which a device gathers rows that
// its L2 holds. See include/tbe_probe.h.
#include <hip/hip_runtime.h>

#include "device.h"
#include "internal.h"
#include "tbe_probe.h"

namespace tbe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 8;   // rows in flight per 16-lane slot
constexpr int kGrid = TBE_PROBE_SINK_FLOATS / kWaves;

// PASSES = row_floats / 64: a 16-lane slot reads 64 floats (256 bytes) per pass.
template <int PASSES>
__global__ __launch_bounds__(kThreads) void probe_gather_kernel(const float* __restrict__ src,
                                                                const int32_t* __restrict__ rows,
                                                                int64_t n,
                                                                float* __restrict__ sink) {
  const int lane = lane_id();
  const int slot = lane >> 4;
  const int col = lane & 15;
  constexpr int RF = PASSES * 64;
  float4 acc[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) acc[p] = float4{0.f, 0.f, 0.f, 0.f};
  const int64_t gwave = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  for (int64_t base = gwave * kWave; base < n; base += nwaves * kWave) {
    const int64_t i = base + lane;
    const int32_t my_row = i < n ? rows[i] : 0;
    const int cnt = n - base < kWave ? (int)(n - base) : kWave;
    for (int r0 = 0; r0 < cnt; r0 += 4 * kUnroll) {
      float4 buf[kUnroll][PASSES];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int r = r0 + u * 4 + slot;
        const int32_t row = __shfl(my_row, r & (kWave - 1));
        const float* rp = src + (int64_t)row * RF;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          if (r < cnt) buf[u][p] = *reinterpret_cast<const float4*>(rp + (p * 16 + col) * 4);
          else buf[u][p] = float4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
          acc[p].x += buf[u][p].x;
          acc[p].y += buf[u][p].y;
          acc[p].z += buf[u][p].z;
          acc[p].w += buf[u][p].w;
        }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int p = 0; p < PASSES; ++p) s += acc[p].x + acc[p].y + acc[p].z + acc[p].w;
  for (int m = 1; m < kWave; m <<= 1) s += __shfl_xor(s, m);
  if (lane == 0) sink[gwave] = s;
}

}  // namespace
}  // namespace tbe

extern "C" tbe_status tbe_probe_row_gather(const float* src, int64_t src_rows, int32_t row_floats,
                                           const int32_t* rows, int64_t n, float* sink,
                                           void* stream) {
  using namespace tbe;
  if (!src || !sink || src_rows < 1 || n < 0 || (!rows && n > 0)) return TBE_ERR_ARG;
  if (row_floats != 64 && row_floats != 128 && row_floats != 256) return TBE_ERR_ARG;
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (row_floats == 64)
    hipLaunchKernelGGL(probe_gather_kernel<1>, dim3(kGrid), dim3(kThreads), 0, s, src, rows, n, sink);
  else if (row_floats == 128)
    hipLaunchKernelGGL(probe_gather_kernel<2>, dim3(kGrid), dim3(kThreads), 0, s, src, rows, n, sink);
  else
    hipLaunchKernelGGL(probe_gather_kernel<4>, dim3(kGrid), dim3(kThreads), 0, s, src, rows, n, sink);
  return hipGetLastError() == hipSuccess ? TBE_OK : TBE_ERR_HIP;
}
