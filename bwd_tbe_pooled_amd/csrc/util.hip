// Small utility kernels: table-info upload through kernel arguments (no host
// memory copy, so callers may free their host array right after the call),
// and the opt-in validation of offsets and index ranges (page 1, checklist
// item 5 makes the bounds check optional and off by default).
#include <atomic>
#include <algorithm>

#include "device.h"
#include "internal.h"

namespace tbe {

struct TinfoChunk {
  int32_t toff[256];
  int32_t rows[256];
};

__global__ void fill_tinfo_kernel2(int32_t* tinfo, int32_t T, int32_t t0, int32_t n, TinfoChunk c) {
  const int i = threadIdx.x;
  if (i < n) {
    tinfo[t0 + i] = c.toff[i];
    tinfo[T + t0 + i] = c.rows[i];
  }
}

int device_cu_count() {
  // Cached per device: the attribute query is a host call, made once.
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

hipError_t launch_fill_tinfo(const Problem& p, const int64_t* rows_host, int32_t* tinfo,
                             hipStream_t s) {
  int64_t acc = 0;
  for (int32_t t0 = 0; t0 < p.T; t0 += 256) {
    TinfoChunk c;
    const int32_t n = std::min<int32_t>(256, p.T - t0);
    for (int32_t i = 0; i < n; ++i) {
      c.toff[i] = (int32_t)acc;
      c.rows[i] = (int32_t)rows_host[t0 + i];
      acc += rows_host[t0 + i];
    }
    hipLaunchKernelGGL(fill_tinfo_kernel2, dim3(1), dim3(256), 0, s, tinfo, p.T, t0, n, c);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

// flag[0] = 1 if offsets are not a valid table-major partition of [0, N) or an
// index lies outside its table.
__global__ __launch_bounds__(256) void validate_kernel(const int32_t* __restrict__ indices,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ trows,
                                                       int32_t B, int64_t nbags, int64_t N,
                                                       int32_t* __restrict__ flag) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0 && (offsets[0] != 0 || offsets[nbags] != N)) atomicOr(flag, 1);
  if (i >= nbags) return;
  const int32_t a = offsets[i], e = offsets[i + 1];
  if (a < 0 || e > N || a > e) {
    atomicOr(flag, 1);
    return;
  }
  const int32_t rows = trows[i / B];
  bool bad = false;
  for (int32_t j = a; j < e; ++j) bad |= (indices[j] < 0) | (indices[j] >= rows);
  if (bad) atomicOr(flag, 1);
}

hipError_t launch_validate(const Problem& p, const int32_t* indices, const int32_t* offsets,
                           const int32_t* tinfo, int32_t* flag, hipStream_t s) {
  hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(64), 0, s, flag, 1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t blocks = std::max<int64_t>(1, (p.nbags + 255) / 256);
  hipLaunchKernelGGL(validate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, indices, offsets,
                     tinfo + p.T, p.B, p.nbags, p.N, flag);
  return hipGetLastError();
}

// --- int64 index arrays (page 1, checklist item 6): a call is split into
// groups of whole tables whose linearized rows and lookups each stay below
// 2^31, and each group runs on int32 copies of its indices and offsets. ----

constexpr int64_t kI32Max = 0x7fffffff;

// out[t] = offsets[t*B] for t = 0..T: where each table's lookups begin.
__global__ void table_bounds_kernel(const int64_t* __restrict__ offsets, int32_t T, int32_t B,
                                    int64_t* __restrict__ out) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t <= T) out[t] = offsets[t * B];
}

// In-table rows narrowed to int32. A value outside [0, 2^31 - 1) becomes
// 2^31 - 1, which lies outside every table (each has fewer rows), so the
// bounds checks report it instead of a wrapped row.
__global__ __launch_bounds__(256) void narrow_indices_kernel(const int64_t* __restrict__ src,
                                                             int64_t n, int32_t* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = src[i];
    dst[i] = (v >= 0 && v < kI32Max) ? (int32_t)v : (int32_t)kI32Max;
  }
}

// Offsets of a group's bags relative to its first lookup, saturated to
// [-1, 2^31 - 1] so that a bad offset stays bad (the group has fewer lookups).
__global__ __launch_bounds__(256) void narrow_offsets_kernel(const int64_t* __restrict__ src,
                                                             int64_t n, int64_t base,
                                                             int32_t* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t v = src[i] - base;
    dst[i] = v < 0 ? -1 : (v > kI32Max ? (int32_t)kI32Max : (int32_t)v);
  }
}

hipError_t launch_table_bounds(const int64_t* offsets, int32_t T, int32_t B, int64_t* out,
                               hipStream_t s) {
  const unsigned blocks = (unsigned)(((int64_t)T + 1 + 255) / 256);
  hipLaunchKernelGGL(table_bounds_kernel, dim3(blocks), dim3(256), 0, s, offsets, T, B, out);
  return hipGetLastError();
}

hipError_t launch_narrow(const int64_t* indices, int64_t n_idx, const int64_t* offsets,
                         int64_t n_off, int64_t base, int32_t* idx32, int32_t* off32,
                         hipStream_t s) {
  const int64_t per_block = 256 * 8;
  if (n_idx > 0) {
    const int64_t blocks = std::min<int64_t>(16384, (n_idx + per_block - 1) / per_block);
    hipLaunchKernelGGL(narrow_indices_kernel, dim3((unsigned)blocks), dim3(256), 0, s, indices,
                       n_idx, idx32);
  }
  const int64_t blocks = std::min<int64_t>(16384, std::max<int64_t>(1, (n_off + per_block - 1) / per_block));
  hipLaunchKernelGGL(narrow_offsets_kernel, dim3((unsigned)blocks), dim3(256), 0, s, offsets,
                     n_off, base, off32);
  return hipGetLastError();
}

}  // namespace tbe
