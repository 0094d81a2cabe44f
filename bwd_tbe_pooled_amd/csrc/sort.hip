// transpose_embedding_input, part 1 (page 1, backward section): linearize the
// lookups and sort them stably by (table,row) key.
//
// The indices are table-major, so every lookup of table t sits in the segment
// [offsets[t*B], offsets[(t+1)*B]) and all keys of table t are below all keys
// of table t+1. A stable sort by key is therefore a stable sort of each table
// segment by its in-table row: the sort below is an LSD radix sort segmented by
// table, with tiles that never straddle a segment. It needs ceil(log2(max E_t))
// key bits instead of ceil(log2(sum E_t)) (21 instead of 26 bits at 32 tables
// of 2M rows: three 7-bit passes).
//
// Each pass is reduce-then-scan:
//   upsweep   per tile, count digits               -> digit_counts[d][tile]
//   scan      per (table, digit), exclusive scan over the table's tiles
//   downsweep per tile, rank elements stably (wave-level multisplit with
//             ballots: 64 lanes find equal digits with one ballot per key bit),
//             reorder the tile in LDS, then write each digit bucket with
//             consecutive lanes on consecutive addresses.
// Pass 0 reads indices directly and takes position and bag id as payload; the
// last pass writes the full key (toff[t] + row) and the metadata arrays.
#include "block_scan.h"
#include "device.h"
#include "internal.h"

namespace tbe {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = kSortTile / kThreads;   // 16 per lane
constexpr int kWaveSpan = kSortTile / 4;       // 1024 consecutive elements per wave

// bag_of[j] = bag of lookup j. A wave takes 64 consecutive bags, whose
// lookups are contiguous; each lane finds the bag of a position by binary
// search over the 65 staged offsets, so the writes are coalesced.
__global__ __launch_bounds__(256) void linearize_kernel(const int32_t* __restrict__ offsets,
                                                        int64_t nbags, int32_t* __restrict__ bag_of) {
  __shared__ int32_t s_off[4][kWave + 1];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t b0 = ((int64_t)blockIdx.x * 4 + wave) * kWave;
  if (b0 >= nbags) return;
  const int nb = nbags - b0 < kWave ? (int)(nbags - b0) : kWave;
  if (lane < nb) s_off[wave][lane] = offsets[b0 + lane];
  if (lane == 0) s_off[wave][nb] = offsets[b0 + nb];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const int32_t P0 = s_off[wave][0], P1 = s_off[wave][nb];
  for (int32_t q = P0 + lane; q < P1; q += kWave) {
    int lo = 0, hi = nb - 1;  // last bag i with s_off[i] <= q (empty bags share offsets)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_off[wave][mid] <= q) lo = mid; else hi = mid - 1;
    }
    bag_of[q] = (int32_t)(b0 + lo);
  }
}

// tile_base[t] = first tile of table t's segment; tile_base[T] = tile count.
__global__ __launch_bounds__(256) void sort_setup_kernel(const int32_t* __restrict__ offsets,
                                                         int32_t T, int32_t B,
                                                         int32_t* __restrict__ tile_base) {
  __shared__ int32_t scratch[4];
  int32_t carry = 0;
  for (int32_t t0 = 0; t0 < T; t0 += kThreads) {
    const int32_t t = t0 + threadIdx.x;
    int32_t tiles = 0;
    if (t < T) {
      const int64_t n = (int64_t)offsets[(int64_t)(t + 1) * B] - offsets[(int64_t)t * B];
      tiles = (int32_t)((n + kSortTile - 1) / kSortTile);
    }
    int32_t total;
    const int32_t ex = block256_exclusive_scan(tiles, scratch, total);
    if (t < T) tile_base[t] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) tile_base[T] = carry;
}

struct TileInfo {
  int32_t t, a, e;  // table, element range [a, e)
  bool valid;
};

// tile_desc[g] = (table, first element, end element, first element of the
// table's segment) of tile g, or table = -1 past the last tile. Computed once
// per sort so that each pass's workgroups read their tile with one load.
__global__ __launch_bounds__(256) void sort_tiles_kernel(const int32_t* __restrict__ tile_base,
                                                         const int32_t* __restrict__ offsets,
                                                         int32_t T, int32_t B, int64_t tiles_max,
                                                         int4* __restrict__ tile_desc) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= tiles_max) return;
  int4 d = make_int4(-1, 0, 0, 0);
  if (g < tile_base[T]) {
    int32_t lo = 0, hi = T - 1;  // last t with tile_base[t] <= g (empty tables share a base)
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (tile_base[mid] <= g) lo = mid; else hi = mid - 1;
    }
    const int32_t seg_a = offsets[(int64_t)lo * B];
    const int32_t seg_e = offsets[(int64_t)(lo + 1) * B];
    const int32_t a = seg_a + (int32_t)(g - tile_base[lo]) * kSortTile;
    d = make_int4(lo, a, a + kSortTile < seg_e ? a + kSortTile : seg_e, seg_a);
  }
  tile_desc[g] = d;
}

__device__ __forceinline__ TileInfo tile_info(int64_t g, const int4* __restrict__ tile_desc) {
  const int4 d = tile_desc[g];
  TileInfo ti;
  ti.valid = d.x >= 0;
  ti.t = d.x;
  ti.a = d.y;
  ti.e = d.z;
  return ti;
}

// Per-tile digit counts. Lanes with equal digits are found with one ballot per
// key bit and counted by one leader lane into its wave's histogram, so skewed
// keys (many equal digits) cause no LDS atomic contention.
__global__ __launch_bounds__(kThreads) void sort_upsweep_kernel(
    const int32_t* __restrict__ keys, const int4* __restrict__ tile_desc, int shift, int bits,
    int64_t tiles_max, int32_t* __restrict__ digit_counts) {
  __shared__ int32_t hist[4][256];
  const int64_t g = blockIdx.x;
  const TileInfo ti = tile_info(g, tile_desc);
  if (!ti.valid) return;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int radix = 1 << bits;
  const uint32_t mask = (uint32_t)radix - 1;
  for (int d = threadIdx.x; d < 4 * 256; d += kThreads) (&hist[0][0])[d] = 0;
  __syncthreads();
  const int32_t wbase = ti.a + wave * kWaveSpan;
  int32_t key[kItems];
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int32_t j = wbase + r * kWave + lane;
    key[r] = j < ti.e ? keys[j] : 0;
  }
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int32_t j = wbase + r * kWave + lane;
    const bool ok = j < ti.e;
    const uint32_t dig = ((uint32_t)key[r] >> shift) & mask;
    uint64_t m = __ballot(ok);
    for (int bi = 0; bi < bits; ++bi) {
      const bool bit = (dig >> bi) & 1u;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    if (ok && lane == __ffsll((unsigned long long)m) - 1) hist[wave][dig] += __popcll(m);
  }
  __syncthreads();
  for (int d = threadIdx.x; d < radix; d += kThreads)
    digit_counts[(int64_t)d * tiles_max + g] = hist[0][d] + hist[1][d] + hist[2][d] + hist[3][d];
}

// One workgroup per (table, digit): exclusive scan of the digit's counts over
// the table's tiles (in place); digit_tot[t*radix + d] = the table's total.
__global__ __launch_bounds__(kThreads) void sort_scan_kernel(int32_t* __restrict__ digit_counts,
                                                             const int32_t* __restrict__ tile_base,
                                                             int radix, int64_t tiles_max,
                                                             int32_t* __restrict__ digit_tot) {
  __shared__ int32_t scratch[4];
  const int32_t t = blockIdx.x / radix;
  const int32_t d = blockIdx.x % radix;
  const int32_t g0 = tile_base[t], g1 = tile_base[t + 1];
  int32_t* col = digit_counts + (int64_t)d * tiles_max;
  int32_t carry = 0;
  constexpr int kPer = 4;
  for (int32_t base = g0; base < g1; base += kThreads * kPer) {
    int32_t v[kPer];
    int32_t sum = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int32_t g = base + threadIdx.x * kPer + i;
      v[i] = g < g1 ? col[g] : 0;
      sum += v[i];
    }
    int32_t total;
    int32_t ex = block256_exclusive_scan(sum, scratch, total);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int32_t g = base + threadIdx.x * kPer + i;
      if (g < g1) col[g] = carry + ex;
      ex += v[i];
    }
    carry += total;
  }
  if (threadIdx.x == 0) digit_tot[(int64_t)t * radix + d] = carry;
}

// FIRST: keys_in = indices, positions are j, bags come from bag_of.
// LAST:  keys_out receives toff[t] + row (the linearized key).
template <bool FIRST, bool LAST, bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void sort_downsweep_kernel(
    const int32_t* __restrict__ keys_in, const int32_t* __restrict__ pos_in,
    const int32_t* __restrict__ bag_in, const float* __restrict__ psw_in,
    int32_t* __restrict__ keys_out, int32_t* __restrict__ pos_out, int32_t* __restrict__ bag_out,
    float* __restrict__ psw_out, const int4* __restrict__ tile_desc,
    const int32_t* __restrict__ toff, int shift, int bits, int64_t tiles_max,
    const int32_t* __restrict__ digit_counts, const int32_t* __restrict__ digit_tot) {
  __shared__ int32_t wave_hist[4][256];
  __shared__ int32_t digit_off[256];   // tile-local start of each digit
  __shared__ int32_t gdelta[256];      // global position minus tile-local position
  __shared__ int32_t stage[kSortTile];
  __shared__ int32_t scratch[4];

  const int64_t g = blockIdx.x;
  const int4 desc = tile_desc[g];
  const TileInfo ti = tile_info(g, tile_desc);
  if (!ti.valid) return;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int radix = 1 << bits;
  const uint32_t mask = (uint32_t)radix - 1;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

  for (int d = threadIdx.x; d < 4 * 256; d += kThreads) (&wave_hist[0][0])[d] = 0;
  __syncthreads();

  int32_t key[kItems], pos[kItems], bag[kItems], rank[kItems];
  float w[kItems];
  const int32_t wbase = ti.a + wave * kWaveSpan;
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int32_t j = wbase + r * kWave + lane;
    const bool ok = j < ti.e;
    key[r] = ok ? keys_in[j] : 0;
    if constexpr (FIRST) {
      pos[r] = j;
      bag[r] = ok ? bag_in[j] : 0;
    } else {
      pos[r] = ok ? pos_in[j] : 0;
      bag[r] = ok ? bag_in[j] : 0;
    }
    if constexpr (WEIGHTED) w[r] = ok ? psw_in[j] : 0.f;
  }

  // Stable ranking inside the wave, round by round in element order.
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int32_t j = wbase + r * kWave + lane;
    const bool ok = j < ti.e;
    const uint32_t dig = ((uint32_t)key[r] >> shift) & mask;
    uint64_t m = __ballot(ok);
    for (int bi = 0; bi < bits; ++bi) {
      const bool bit = (dig >> bi) & 1u;
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int leader = m ? (__ffsll((unsigned long long)m) - 1) : 0;
    int32_t old = 0;
    if (ok && lane == leader) {
      old = wave_hist[wave][dig];
      wave_hist[wave][dig] = old + __popcll(m);
    }
    old = __shfl(old, leader);
    rank[r] = old + __popcll(m & lt_mask);
  }
  __syncthreads();

  // Per digit: exclusive prefix over waves, tile-local digit starts, and the
  // global base = segment start + table-wide digit start + this tile's prefix.
  int32_t cnt = 0, tot = 0;
  const int d = threadIdx.x;
  if (d < radix) {
    int32_t run = 0;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const int32_t c = wave_hist[ww][d];
      wave_hist[ww][d] = run;
      run += c;
    }
    cnt = run;
    tot = digit_tot[(int64_t)ti.t * radix + d];
  }
  int32_t total;
  const int32_t local_start = block256_exclusive_scan(d < radix ? cnt : 0, scratch, total);
  const int32_t tot_start = block256_exclusive_scan(d < radix ? tot : 0, scratch, total);
  if (d < radix) {
    digit_off[d] = local_start;
    const int32_t seg_a = desc.w;
    gdelta[d] = seg_a + tot_start + digit_counts[(int64_t)d * tiles_max + g] - local_start;
  }
  __syncthreads();

  int32_t lp[kItems];
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int32_t j = wbase + r * kWave + lane;
    const uint32_t dig = ((uint32_t)key[r] >> shift) & mask;
    lp[r] = (j < ti.e) ? digit_off[dig] + wave_hist[wave][dig] + rank[r] : -1;
  }

  const int32_t nvalid = ti.e - ti.a;
  int32_t dest[kItems];
  // keys
#pragma unroll
  for (int r = 0; r < kItems; ++r)
    if (lp[r] >= 0) stage[lp[r]] = key[r];
  __syncthreads();
  const int32_t kt = LAST ? toff[ti.t] : 0;
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int32_t i = q * kThreads + threadIdx.x;
    if (i < nvalid) {
      const int32_t row = stage[i];
      const uint32_t dig = ((uint32_t)row >> shift) & mask;
      dest[q] = gdelta[dig] + i;
      keys_out[dest[q]] = LAST ? kt + row : row;
    }
  }
  // payloads, one array at a time through the same LDS stage
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kItems; ++r)
    if (lp[r] >= 0) stage[lp[r]] = pos[r];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int32_t i = q * kThreads + threadIdx.x;
    if (i < nvalid) pos_out[dest[q]] = stage[i];
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < kItems; ++r)
    if (lp[r] >= 0) stage[lp[r]] = bag[r];
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int32_t i = q * kThreads + threadIdx.x;
    if (i < nvalid) bag_out[dest[q]] = stage[i];
  }
  if constexpr (WEIGHTED) {
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kItems; ++r)
      if (lp[r] >= 0) stage[lp[r]] = __float_as_int(w[r]);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kItems; ++q) {
      const int32_t i = q * kThreads + threadIdx.x;
      if (i < nvalid) psw_out[dest[q]] = __int_as_float(stage[i]);
    }
  }
}

template <bool FIRST, bool LAST>
hipError_t launch_downsweep(bool weighted, dim3 grid, hipStream_t s, const int32_t* ki,
                            const int32_t* pi, const int32_t* bi, const float* wi, int32_t* ko,
                            int32_t* po, int32_t* bo, float* wo, const int4* tile_desc,
                            const int32_t* toff, int shift, int bits, int64_t tiles_max,
                            const int32_t* dc, const int32_t* dt) {
  if (weighted)
    hipLaunchKernelGGL((sort_downsweep_kernel<FIRST, LAST, true>), grid, dim3(kThreads), 0, s, ki,
                       pi, bi, wi, ko, po, bo, wo, tile_desc, toff, shift, bits, tiles_max, dc, dt);
  else
    hipLaunchKernelGGL((sort_downsweep_kernel<FIRST, LAST, false>), grid, dim3(kThreads), 0, s, ki,
                       pi, bi, wi, ko, po, bo, wo, tile_desc, toff, shift, bits, tiles_max, dc, dt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linearize(const Problem& p, const int32_t* offsets, int32_t* bag_of,
                            hipStream_t s) {
  if (p.nbags == 0) return hipSuccess;
  const int64_t blocks = (p.nbags + 255) / 256;
  hipLaunchKernelGGL(linearize_kernel, dim3((unsigned)blocks), dim3(256), 0, s, offsets, p.nbags,
                     bag_of);
  return hipGetLastError();
}

hipError_t launch_sort(const Problem& p, const int32_t* indices, const int32_t* offsets,
                       const float* psw, const int32_t* tinfo, const SortBuffers& b,
                       const tbe_meta& meta, tbe_timer* timer, hipStream_t s) {
  (void)timer;
  hipError_t err;
  hipLaunchKernelGGL(sort_setup_kernel, dim3(1), dim3(256), 0, s, offsets, p.T, p.B, b.tile_base);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if (p.N == 0) return hipSuccess;
  hipLaunchKernelGGL(sort_tiles_kernel, dim3((unsigned)((p.sort_tiles_max + 255) / 256)), dim3(256),
                     0, s, b.tile_base, offsets, p.T, p.B, p.sort_tiles_max, b.tile_desc);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  const dim3 tgrid((unsigned)p.sort_tiles_max);
  const int radix = 1 << p.sort_bits;
  const bool weighted = p.weighted;
  const int32_t* toff = tinfo;
  for (int pass = 0; pass < p.sort_passes; ++pass) {
    const bool first = pass == 0;
    const bool last = pass == p.sort_passes - 1;
    const int shift = pass * p.sort_bits;
    // source and destination buffers
    int32_t* const* src = (pass % 2 == 1) ? b.A : b.B;  // pass 1 reads A, pass 2 reads B, ...
    int32_t* const* dst = (pass % 2 == 0) ? b.A : b.B;  // pass 0 writes A, pass 1 writes B, ...
    const int32_t* ki = first ? indices : src[0];
    const int32_t* pi = first ? nullptr : src[1];
    const int32_t* bi = first ? b.bag_of : src[2];
    const float* wi = first ? psw : (const float*)src[3];
    int32_t* ko = last ? b.sorted_keys : dst[0];
    int32_t* po = last ? meta.sorted_pos : dst[1];
    int32_t* bo = last ? meta.sorted_bag : dst[2];
    float* wo = last ? meta.sorted_psw : (float*)dst[3];

    hipLaunchKernelGGL(sort_upsweep_kernel, tgrid, dim3(kThreads), 0, s, ki, b.tile_desc, shift,
                       p.sort_bits, p.sort_tiles_max, b.digit_counts);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(sort_scan_kernel, dim3((unsigned)(p.T * radix)), dim3(kThreads), 0, s,
                       b.digit_counts, b.tile_base, radix, p.sort_tiles_max, b.digit_tot);
    if ((err = hipGetLastError()) != hipSuccess) return err;
#define TBE_DOWNSWEEP(F, L)                                                                    \
  launch_downsweep<F, L>(weighted, tgrid, s, ki, pi, bi, wi, ko, po, bo, wo, b.tile_desc, toff, \
                         shift, p.sort_bits, p.sort_tiles_max, b.digit_counts, b.digit_tot)
    if (first && last) err = TBE_DOWNSWEEP(true, true);
    else if (first) err = TBE_DOWNSWEEP(true, false);
    else if (last) err = TBE_DOWNSWEEP(false, true);
    else err = TBE_DOWNSWEEP(false, false);
#undef TBE_DOWNSWEEP
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace tbe
