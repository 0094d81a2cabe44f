// transpose_embedding_input, part 2, and segment-length routing (page 1,
// backward section): run-length encode the sorted keys into runs (one unique
// (table,row) and the sorted slots of all lookups touching it), then split the
// runs by segment length SL: SL < S goes to the short-run path, the rest to
// the chunked path with C lookups per chunk.
//
// All counts stay on the device: grids are sized from host-known upper bounds
// (N, min(N, sum E_t)) and workgroups past the device-side count exit.
#include "block_scan.h"
#include "device.h"
#include "internal.h"

namespace tbe {

namespace {

constexpr int kThreads = 256;
constexpr int kPer = kRleTile / kThreads;  // 16 consecutive elements per thread

// Run heads of the sorted keys. A wave walks 1024 consecutive slots in rounds
// of 64 (coalesced); the previous key comes from the neighbouring lane, from
// the last lane of the previous round, or (first round) from memory.
struct HeadScan {
  int32_t key[kPer];
  uint64_t heads[kPer];
};

__device__ __forceinline__ void find_heads(const int32_t* __restrict__ keys, int64_t N,
                                           int64_t wbase, HeadScan& h) {
  const int lane = lane_id();
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int64_t k = wbase + r * kWave + lane;
    h.key[r] = k < N ? keys[k] : 0;
  }
  int32_t carry = 0;
  if (wbase > 0 && wbase < N) carry = keys[wbase - 1];
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int64_t k = wbase + r * kWave + lane;
    int32_t prev = __shfl_up(h.key[r], 1);
    if (lane == 0) prev = carry;
    const bool head = k < N && (k == 0 || h.key[r] != prev);
    h.heads[r] = __ballot(head);
    carry = __shfl(h.key[r], kWave - 1);
  }
}

// tile_heads[g] = number of run heads in sorted slots [g*TILE, (g+1)*TILE).
__global__ __launch_bounds__(kThreads) void rle_count_kernel(const int32_t* __restrict__ keys,
                                                             int64_t N, int32_t* __restrict__ tile_heads) {
  __shared__ int32_t wcount[4];
  const int64_t tile = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const int64_t wbase = tile * kRleTile + (int64_t)wave * (kPer * kWave);
  HeadScan h;
  find_heads(keys, N, wbase, h);
  int32_t c = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) c += __popcll(h.heads[r]);
  if (lane_id() == 0) wcount[wave] = c;
  __syncthreads();
  if (threadIdx.x == 0) tile_heads[tile] = wcount[0] + wcount[1] + wcount[2] + wcount[3];
}

// Single workgroup: exclusive scan of `ncols` interleaved arrays vals[c*n + i]
// in place; totals[c] receives each sum. With `items` set, only the tiles
// that hold any of the *items elements are scanned (the rest are never read).
__global__ __launch_bounds__(1024) void scan_tiles_kernel(int32_t* __restrict__ vals, int64_t n,
                                                          int ncols, int32_t* __restrict__ totals,
                                                          const int32_t* __restrict__ items) {
  __shared__ int32_t wsum[16];
  int64_t m = n;
  if (items) {
    const int64_t used = ((int64_t)*items + kRleTile - 1) / kRleTile;
    m = used < n ? used : n;
  }
  for (int c = 0; c < ncols; ++c) {
    const int32_t tot =
        block1024_scan_inplace(vals + (int64_t)c * n, m, wsum, [](int64_t, int32_t) {});
    if (threadIdx.x == 0) totals[c] = tot;
  }
}

// After the head scan: U into counts[0] and run_offsets[U] = N.
__global__ void rle_finish_kernel(const int32_t* __restrict__ heads_total, int64_t N,
                                  int32_t* __restrict__ counts, int32_t* __restrict__ run_offsets) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const int32_t U = heads_total[0];
    counts[0] = U;
    run_offsets[U] = (int32_t)N;
  }
}

__global__ __launch_bounds__(kThreads) void rle_write_kernel(const int32_t* __restrict__ keys,
                                                             int64_t N,
                                                             const int32_t* __restrict__ tile_base,
                                                             int32_t* __restrict__ run_keys,
                                                             int32_t* __restrict__ run_offsets) {
  __shared__ int32_t wcount[4];
  const int64_t tile = blockIdx.x;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t wbase = tile * kRleTile + (int64_t)wave * (kPer * kWave);
  HeadScan h;
  find_heads(keys, N, wbase, h);
  int32_t c = 0;
#pragma unroll
  for (int r = 0; r < kPer; ++r) c += __popcll(h.heads[r]);
  if (lane == 0) wcount[wave] = c;
  __syncthreads();
  int32_t u = tile_base[tile];
  for (int w = 0; w < wave; ++w) u += wcount[w];
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    if ((h.heads[r] >> lane) & 1ull) {
      const int32_t uu = u + __popcll(h.heads[r] & lt);
      run_keys[uu] = h.key[r];
      run_offsets[uu] = (int32_t)(wbase + r * kWave + lane);
    }
    u += __popcll(h.heads[r]);
  }
}

// Per tile of runs: number of short runs, long runs and chunks.
__global__ __launch_bounds__(kThreads) void route_count_kernel(const int32_t* __restrict__ run_offsets,
                                                               const int32_t* __restrict__ counts,
                                                               int32_t S, int32_t C, int64_t ntiles,
                                                               int32_t* __restrict__ tsum) {
  __shared__ int32_t scratch[4];
  const int64_t U = counts[0];
  // Plain tile order: the grid covers the host's bound on the runs, and only
  // its first ceil(U / TILE) tiles hold any (an XCD split would put them all
  // on one XCD). Tiles past the runs are not scanned.
  const int64_t tile = blockIdx.x;
  if (tile * kRleTile >= U) return;
  const int64_t base = tile * kRleTile + (int64_t)threadIdx.x * kPer;
  int32_t ns = 0, nl = 0, nc = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t u = base + i;
    if (u < U) {
      const int32_t sl = run_offsets[u + 1] - run_offsets[u];
      if (sl < S) ++ns;
      else { ++nl; nc += (sl + C - 1) / C; }
    }
  }
  int32_t t0, t1, t2;
  block256_exclusive_scan(ns, scratch, t0);
  block256_exclusive_scan(nl, scratch, t1);
  block256_exclusive_scan(nc, scratch, t2);
  if (threadIdx.x == 0) {
    tsum[tile] = t0;
    tsum[ntiles + tile] = t1;
    tsum[2 * ntiles + tile] = t2;
  }
}

__global__ void route_finish_kernel(const int32_t* __restrict__ totals, int32_t* __restrict__ counts,
                                    int32_t* __restrict__ long_chunk_begin) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    counts[1] = totals[0];
    counts[2] = totals[1];
    counts[3] = totals[2];
    long_chunk_begin[totals[1]] = totals[2];
  }
}

__global__ __launch_bounds__(kThreads) void route_write_kernel(
    const int32_t* __restrict__ run_offsets, const int32_t* __restrict__ counts, int32_t S,
    int32_t C, int64_t ntiles, const int32_t* __restrict__ tsum, int32_t* __restrict__ short_runs,
    int32_t* __restrict__ long_runs, int32_t* __restrict__ long_chunk_begin,
    int32_t* __restrict__ chunk_run, int32_t* __restrict__ chunk_start) {
  __shared__ int32_t scratch[4];
  // Block-local long runs: their run id and first local chunk (exclusive prefix).
  __shared__ int32_t l_run[kRleTile];
  __shared__ int32_t l_cbeg[kRleTile + 1];
  const int64_t U = counts[0];
  const int64_t tile = blockIdx.x;
  const int64_t tile0 = tile * kRleTile;
  if (tile0 >= U) return;
  const int64_t base = tile0 + (int64_t)threadIdx.x * kPer;
  int32_t sl[kPer];
  int32_t ns = 0, nl = 0, nc = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int64_t u = base + i;
    sl[i] = u < U ? run_offsets[u + 1] - run_offsets[u] : -1;
    if (sl[i] >= 0) {
      if (sl[i] < S) ++ns;
      else { ++nl; nc += (sl[i] + C - 1) / C; }
    }
  }
  int32_t tn, tl, tc;
  int32_t xs = block256_exclusive_scan(ns, scratch, tn);
  int32_t xl = block256_exclusive_scan(nl, scratch, tl);
  int32_t xc = block256_exclusive_scan(nc, scratch, tc);
  const int32_t bs = tsum[tile];
  const int32_t bl = tsum[ntiles + tile];
  const int32_t bc = tsum[2 * ntiles + tile];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (sl[i] < 0) continue;
    const int32_t u = (int32_t)(base + i);
    if (sl[i] < S) {
      short_runs[bs + xs++] = u;
    } else {
      long_runs[bl + xl] = u;
      long_chunk_begin[bl + xl] = bc + xc;
      l_run[xl] = u;
      l_cbeg[xl] = xc;
      ++xl;
      xc += (sl[i] + C - 1) / C;
    }
  }
  if (threadIdx.x == 0) l_cbeg[tl] = tc;
  __syncthreads();
  // Fill the block's chunks cooperatively: chunk c belongs to the last local
  // long run whose first chunk is <= c.
  for (int32_t c = threadIdx.x; c < tc; c += kThreads) {
    int32_t lo = 0, hi = tl - 1;
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (l_cbeg[mid] <= c) lo = mid; else hi = mid - 1;
    }
    const int32_t u = l_run[lo];
    chunk_run[bc + c] = u;
    chunk_start[bc + c] = run_offsets[u] + (c - l_cbeg[lo]) * C;
  }
}

}  // namespace

hipError_t launch_rle_route(const Problem& p, const int32_t* sorted_keys, int32_t* rle_tiles,
                            int32_t* route_tiles, const tbe_meta& meta, hipStream_t s) {
  hipError_t err;
  const int64_t nt = (p.N + kRleTile - 1) / kRleTile;
  int32_t* heads = rle_tiles;           // [nt]
  int32_t* totals = rle_tiles + nt;     // [4]
  if (nt > 0) {
    hipLaunchKernelGGL(rle_count_kernel, dim3((unsigned)nt), dim3(kThreads), 0, s, sorted_keys,
                       p.N, heads);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(scan_tiles_kernel, dim3(1), dim3(1024), 0, s, heads, nt, 1, totals,
                     (const int32_t*)nullptr);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(rle_finish_kernel, dim3(1), dim3(64), 0, s, totals, p.N, meta.counts,
                     meta.run_offsets);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (nt > 0) {
    hipLaunchKernelGGL(rle_write_kernel, dim3((unsigned)nt), dim3(kThreads), 0, s, sorted_keys,
                       p.N, heads, meta.run_keys, meta.run_offsets);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  // Routing over at most cap_runs runs.
  const int64_t rt = (p.cap_runs + kRleTile - 1) / kRleTile;
  int32_t* tsum = route_tiles;          // [3 * rt]
  int32_t* rtot = route_tiles + 3 * rt; // [3]
  if (rt > 0) {
    hipLaunchKernelGGL(route_count_kernel, dim3((unsigned)rt), dim3(kThreads), 0, s,
                       meta.run_offsets, meta.counts, p.S, p.C, rt, tsum);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  hipLaunchKernelGGL(scan_tiles_kernel, dim3(1), dim3(1024), 0, s, tsum, rt, 3, rtot,
                     (const int32_t*)meta.counts);  // counts[0] = U runs
  if ((err = hipGetLastError()) != hipSuccess) return err;
  hipLaunchKernelGGL(route_finish_kernel, dim3(1), dim3(64), 0, s, rtot, meta.counts,
                     meta.long_chunk_begin);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (rt > 0) {
    hipLaunchKernelGGL(route_write_kernel, dim3((unsigned)rt), dim3(kThreads), 0, s,
                       meta.run_offsets, meta.counts, p.S, p.C, rt, tsum, meta.short_runs,
                       meta.long_runs, meta.long_chunk_begin, meta.chunk_run, meta.chunk_start);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace tbe
