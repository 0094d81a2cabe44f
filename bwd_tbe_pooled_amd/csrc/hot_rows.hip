// The hot-row plan: per table, the rows of up to K of its longest runs.
#include "hot_rows.h"
#include "internal.h"

namespace tbe {

namespace {

// One workgroup per table: the row index (in its table) of up to K of the
// table's longest runs, in hot_rows[t*K ..], the rest -1. Long runs of table
// t are a contiguous range of the long-run list (keys ascend, tables are key
// ranges); those with at least v lookups are taken, v the least length >= S
// that leaves at most K of them. Optionally also, for every long run l of the
// table, run_slot[l] = t*K + its slot, or -1 when it is not hot; and
// hot_min[t] = v, or INT32_MAX when the table has no hot run: a long run is
// hot exactly when its length is at least hot_min of its table; and
// hot_flag[t] = 0 (the backward of the hot rows sets it to send them back to
// the chunk path). The table's run lengths are read once into LDS (when there
// are at most kPlanCache long runs; otherwise each count rereads them), and v
// is found by bisection between S and the longest run.
constexpr int kPlanCache = 4096;
__global__ __launch_bounds__(256) void hot_plan_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ long_runs,
    const int32_t* __restrict__ run_offsets, const int32_t* __restrict__ run_keys,
    const int32_t* __restrict__ tinfo, int32_t T, int32_t K, int32_t S,
    int32_t* __restrict__ hot_rows, int32_t* __restrict__ run_slot,
    int32_t* __restrict__ hot_min, int32_t* __restrict__ hot_flag) {
  __shared__ int32_t s_range[2];
  __shared__ int32_t s_n;
  __shared__ int32_t red[256 / kWave];
  __shared__ int32_t s_len[kPlanCache];
  const int32_t t = blockIdx.x;
  const int64_t n_long = counts[2];
  const int32_t first = tinfo[t];
  for (int i = threadIdx.x; i < K; i += blockDim.x) hot_rows[(int64_t)t * K + i] = -1;
  {
    // The table's range of the long-run list: the first run at or above each
    // of its two bounding keys, by a 128-way search (threads 0-127 for the
    // first key, 128-255 for the second). Each round probes 128 evenly spaced
    // runs of [lo, hi); those below the key are a prefix of c probes, and the
    // answer lies after the last of them and at or before the next.
    const int half = threadIdx.x >> 7, j = threadIdx.x & 127;
    const int32_t key = half == 0 ? first : first + tinfo[T + t];
    int32_t lo = 0, hi = (int32_t)n_long;
    while (__syncthreads_or(lo < hi)) {
      const int32_t step = (hi - lo + 127) / 128;
      const int32_t q = lo + j * step;
      const bool below = lo < hi && q < hi && run_keys[long_runs[q]] < key;
      const int32_t c0 = __syncthreads_count(half == 0 && below);
      const int32_t c1 = __syncthreads_count(half == 1 && below);
      const int32_t c = half ? c1 : c0;
      if (lo < hi) {
        if (c == 0) {
          hi = lo;
        } else {
          const int32_t nhi = lo + c * step < hi ? lo + c * step : hi;
          lo = lo + (c - 1) * step + 1;
          hi = nhi;
        }
      }
    }
    if (j == 0) s_range[half] = lo;
  }
  if (threadIdx.x == 0) {
    s_n = 0;
    if (hot_flag) hot_flag[t] = 0;
  }
  __syncthreads();
  const int32_t l0 = s_range[0], l1 = s_range[1];
  const bool cached = l1 - l0 <= kPlanCache;
  auto len_global = [&](int32_t l) {
    const int32_t u = long_runs[l];
    return run_offsets[u + 1] - run_offsets[u];
  };
  auto len = [&](int32_t l) { return cached ? s_len[l - l0] : len_global(l); };
  // block-wide sum (op 0) or maximum (op 1) of one value per thread
  auto block_reduce = [&](int32_t c, int op) {
    for (int m = 1; m < kWave; m <<= 1) {
      const int32_t o = __shfl_xor(c, m);
      c = op ? (o > c ? o : c) : c + o;
    }
    __syncthreads();
    if (lane_id() == 0) red[threadIdx.x / kWave] = c;
    __syncthreads();
    int32_t tot = op ? red[0] : 0;
    for (int w = op ? 1 : 0; w < (int)(blockDim.x / kWave); ++w)
      tot = op ? (red[w] > tot ? red[w] : tot) : tot + red[w];
    return tot;
  };
  int32_t mx = 0;
  for (int32_t l = l0 + threadIdx.x; l < l1; l += blockDim.x) {
    const int32_t n = len_global(l);
    if (cached) s_len[l - l0] = n;
    mx = n > mx ? n : mx;
  }
  mx = block_reduce(mx, 1);  // its barriers also publish s_len
  auto count_ge = [&](int32_t v) {
    int32_t c = 0;
    for (int32_t l = l0 + threadIdx.x; l < l1; l += blockDim.x) c += len(l) >= v;
    return block_reduce(c, 0);
  };
  int32_t v = S;
  if (count_ge(v) > K) {
    // more than K runs reach S, so mx >= S and v is in (S, mx + 1]: above the
    // longest no run is counted (more than K runs tied at mx leave v = mx + 1)
    int32_t lo = v + 1, hi = mx < 0x7fffffff ? mx + 1 : mx;
    while (lo < hi) {
      const int32_t mid = lo + (hi - lo) / 2;
      if (count_ge(mid) <= K) hi = mid;
      else lo = mid + 1;
    }
    v = lo;
  }
  __syncthreads();  // hot_rows cleared before any slot is written
  for (int32_t l = l0 + threadIdx.x; l < l1; l += blockDim.x) {
    int32_t q = -1;
    if (len(l) >= v) {
      q = atomicAdd(&s_n, 1);  // slot order does not change any value computed
      if (q < K) hot_rows[(int64_t)t * K + q] = run_keys[long_runs[l]] - first;
      else q = -1;  // cannot happen: at most K runs reach v
    }
    if (run_slot) run_slot[l] = q < 0 ? -1 : t * K + q;
  }
  if (hot_min) {
    __syncthreads();  // every slot taken (ties at v-1 may leave none)
    if (threadIdx.x == 0) hot_min[t] = s_n > 0 ? v : 0x7fffffff;
  }
}

}  // namespace

hipError_t launch_hot_plan(const Problem& p, const tbe_meta& meta, const int32_t* tinfo, int32_t K,
                           int32_t* hot_rows, int32_t* run_slot, int32_t* hot_min,
                           int32_t* hot_flag, hipStream_t s) {
  hipLaunchKernelGGL(hot_plan_kernel, dim3((unsigned)p.T), dim3(256), 0, s, meta.counts,
                     meta.long_runs, meta.run_offsets, meta.run_keys, tinfo, p.T, K, p.S, hot_rows,
                     run_slot, hot_min, hot_flag);
  return hipGetLastError();
}

}  // namespace tbe
