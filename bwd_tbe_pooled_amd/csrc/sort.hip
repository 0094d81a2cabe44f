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
// Pass 0 reads the indices directly; the bag of each lookup comes from the
// tile's bag offsets staged in LDS (no bag-id array is written or read). The
// payload is (bag, per-sample weight), plus the original position only when
// the caller asks for it (the backward does not need it). The last pass
// writes the linearized key toff[t] + row and the metadata arrays.
#include "block_scan.h"
#include "device.h"
#include "internal.h"

namespace tbe {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = kSortTile / kThreads;   // 16 per lane
constexpr int kWaveSpan = kSortTile / 4;       // 1024 consecutive elements per wave

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
  int32_t seg_a;    // first element of the table's segment
  int32_t bag0, bag1;  // bags containing elements a and e-1
  bool valid;
};

// Last bag i in [lo, hi] with offsets[i] <= x (empty bags share offsets, so
// this is the bag that contains position x).
__device__ __forceinline__ int32_t bag_of_position(const int32_t* __restrict__ offsets, int32_t lo,
                                                   int32_t hi, int32_t x) {
  while (lo < hi) {
    const int32_t mid = lo + (hi - lo + 1) / 2;
    if (offsets[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// tile_desc[g] = (table, first element, end element, segment start) and
// (first bag, last bag) of tile g; table = -1 past the last tile. Computed
// once per sort so that each pass's workgroups read their tile with two loads.
__global__ __launch_bounds__(256) void sort_tiles_kernel(const int32_t* __restrict__ tile_base,
                                                         const int32_t* __restrict__ offsets,
                                                         int32_t T, int32_t B, int64_t tiles_max,
                                                         int4* __restrict__ tile_desc) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= tiles_max) return;
  int4 d0 = make_int4(-1, 0, 0, 0), d1 = make_int4(0, 0, 0, 0);
  if (g < tile_base[T]) {
    int32_t lo = 0, hi = T - 1;  // last t with tile_base[t] <= g (empty tables share a base)
    while (lo < hi) {
      const int32_t mid = (lo + hi + 1) >> 1;
      if (tile_base[mid] <= g) lo = mid; else hi = mid - 1;
    }
    const int32_t seg_a = offsets[lo * B];
    const int32_t seg_e = offsets[(lo + 1) * B];
    const int32_t a = seg_a + (int32_t)(g - tile_base[lo]) * kSortTile;
    const int32_t e = a + kSortTile < seg_e ? a + kSortTile : seg_e;
    d0 = make_int4(lo, a, e, seg_a);
    d1 = make_int4(bag_of_position(offsets, lo * B, (lo + 1) * B - 1, a),
                   bag_of_position(offsets, lo * B, (lo + 1) * B - 1, e - 1), 0, 0);
  }
  tile_desc[2 * g] = d0;
  tile_desc[2 * g + 1] = d1;
}

__device__ __forceinline__ TileInfo tile_info(int64_t g, const int4* __restrict__ tile_desc) {
  const int4 d0 = tile_desc[2 * g];
  const int4 d1 = tile_desc[2 * g + 1];
  TileInfo ti;
  ti.valid = d0.x >= 0;
  ti.t = d0.x;
  ti.a = d0.y;
  ti.e = d0.z;
  ti.seg_a = d0.w;
  ti.bag0 = d1.x;
  ti.bag1 = d1.y;
  return ti;
}

// Per-tile digit counts (digits of at most 7 bits), one 128-bin LDS histogram
// per wave. A wave's 64 lanes hold 64 consecutive keys; after the lower
// digits' passes equal digits sit together, so only the first lane of each
// run of equal digits adds the run's length (one atomic per run, not per key).
__global__ __launch_bounds__(kThreads) void sort_upsweep_kernel(
    const int32_t* __restrict__ keys, const int4* __restrict__ tile_desc, int shift, int bits,
    int64_t tiles_max, int32_t* __restrict__ digit_counts, const int32_t* __restrict__ clamp_rows) {
  constexpr int kUpWaves = kThreads / kWave;
  __shared__ uint32_t hist[kUpWaves][128];
  const int64_t g = xcd_logical_block(tiles_max);
  if (g < 0) return;
  const TileInfo ti = tile_info(g, tile_desc);
  if (!ti.valid) return;
  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = lane_id();
  const uint32_t mask = (1u << bits) - 1u;
  for (int i = tid; i < kUpWaves * 128; i += kThreads) (&hist[0][0])[i] = 0u;
  int32_t key[kItems];
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const int32_t j = ti.a + q * kThreads + tid;
    key[q] = j < ti.e ? keys[j] : 0;
  }
  const uint32_t Et = clamp_rows ? (uint32_t)clamp_rows[ti.t] : 0u;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kItems; ++q) {
    const bool ok = ti.a + q * kThreads + tid < ti.e;
    // TBE_FLAG_CHECK (first pass): a row outside the table sorts as row 0
    const uint32_t k = (clamp_rows && (uint32_t)key[q] >= Et) ? 0u : (uint32_t)key[q];
    const int d = ok ? (int)((k >> shift) & mask) : -1;
    const int dp = __shfl_up(d, 1);
    const bool head = ok && (lane == 0 || dp != d);
    const uint64_t heads = __ballot(head);
    const uint64_t valid = __ballot(ok);
    if (head) {
      // the run ends at the next head or at the last valid lane
      const uint64_t after = lane == 63 ? 0ull : (heads | ~valid) & (~0ull << (lane + 1));
      const int end = after ? __builtin_ctzll(after) : 64;
      __hip_atomic_fetch_add(&hist[wave][d], (uint32_t)(end - lane), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  __syncthreads();
  if (tid < 128) {
    uint32_t c = 0u;
#pragma unroll
    for (int v = 0; v < kUpWaves; ++v) c += hist[v][tid];
    if (tid <= (int)mask) digit_counts[(int64_t)tid * tiles_max + g] = (int32_t)c;
  }
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

// FIRST: keys_in = indices, the position of an element is its index, and its
// bag is found among the tile's bag offsets. LAST: keys_out receives
// toff[t] + row. WITH_POS: the original position travels as payload.
// Without positions, four waves per SIMD (at most 128 VGPRs, a couple of them
// spilled for the weighted form) beat three: the pass is latency-bound, and it
// took the three passes from 1.70 to 1.63 ms at T=32, E=2M, B=131072. With
// positions the fourth wave would cost about 30 spilled registers.
template <bool FIRST, bool LAST, bool WEIGHTED, bool WITH_POS>
__global__ __launch_bounds__(kThreads, WITH_POS ? 3 : 4) void sort_downsweep_kernel(
    const int32_t* __restrict__ keys_in, const int32_t* __restrict__ pos_in,
    const int32_t* __restrict__ bag_in, const float* __restrict__ psw_in,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ keys_out,
    int32_t* __restrict__ pos_out, int32_t* __restrict__ bag_out, float* __restrict__ psw_out,
    const int4* __restrict__ tile_desc, const int32_t* __restrict__ toff, int shift, int bits,
    int64_t tiles_max, const int32_t* __restrict__ digit_counts,
    const int32_t* __restrict__ digit_tot, const int32_t* __restrict__ clamp_rows,
    int32_t* __restrict__ err) {
  __shared__ int32_t wave_hist[4][256];
  __shared__ int32_t digit_off[256];   // tile-local start of each digit
  __shared__ int32_t gdelta[256];      // global position minus tile-local position
  __shared__ int32_t stage[kSortTile + 1];
  __shared__ int32_t scratch[4];

  const int64_t g = xcd_logical_block(tiles_max);
  if (g < 0) return;
  const TileInfo ti = tile_info(g, tile_desc);
  if (!ti.valid) return;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int radix = 1 << bits;
  const uint32_t mask = (uint32_t)radix - 1;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

  for (int d = threadIdx.x; d < 4 * 256; d += kThreads) (&wave_hist[0][0])[d] = 0;
  // The tile's loads issue ahead of the ranking of the workgroups already
  // resident (1.596 -> 1.582 ms for the three passes at T=32, B=131072).
  __builtin_amdgcn_s_setprio(1);

  int32_t key[kItems], pos[kItems], bag[kItems], rank[kItems];
  float w[kItems];
  const int32_t wbase = ti.a + wave * kWaveSpan;
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const int32_t j = wbase + r * kWave + lane;
    const bool ok = j < ti.e;
    key[r] = ok ? keys_in[j] : 0;
    if constexpr (WITH_POS) pos[r] = FIRST ? j : (ok ? pos_in[j] : 0);
    if constexpr (!FIRST) bag[r] = ok ? bag_in[j] : 0;
    if constexpr (WEIGHTED) w[r] = ok ? psw_in[j] : 0.f;
  }
  __builtin_amdgcn_s_setprio(0);
  if (clamp_rows) {
    // Bounds check fused into the first pass: a row outside its table sorts
    // (and is later read and updated) as row 0, and the call reports it.
    const uint32_t Et = (uint32_t)clamp_rows[ti.t];
    bool bad = false;
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
      const bool out = wbase + r * kWave + lane < ti.e && (uint32_t)key[r] >= Et;
      bad |= out;
      key[r] = out ? 0 : key[r];
    }
    if (__ballot(bad) != 0 && lane == 0) atomicOr(err, (int32_t)TBE_ERROR_INDEX);
  }
  if constexpr (FIRST) {
    // Bag of every element of the tile: each thread takes bags of the tile and
    // writes the bag id into the LDS slots of its lookups.
    for (int32_t bg = ti.bag0 + threadIdx.x; bg <= ti.bag1; bg += kThreads) {
      const int32_t lo = offsets[bg] > ti.a ? offsets[bg] : ti.a;
      const int32_t hi = offsets[bg + 1] < ti.e ? offsets[bg + 1] : ti.e;
      for (int32_t j = lo; j < hi; ++j) stage[j - ti.a] = bg;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kItems; ++r) {
      const int32_t j = wbase + r * kWave + lane;
      bag[r] = j < ti.e ? stage[j - ti.a] : 0;
    }
  }
  __syncthreads();

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
    gdelta[d] = ti.seg_a + tot_start + digit_counts[(int64_t)d * tiles_max + g] - local_start;
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
  if constexpr (WITH_POS) {
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

struct PassArgs {
  const int32_t *ki, *pi, *bi;
  const float* wi;
  int32_t *ko, *po, *bo;
  float* wo;
};

template <bool FIRST, bool LAST>
hipError_t launch_downsweep(bool weighted, bool with_pos, dim3 grid, hipStream_t s,
                            const PassArgs& a, const int32_t* offsets, const int4* tile_desc,
                            const int32_t* toff, int shift, int bits, int64_t tiles_max,
                            const int32_t* dc, const int32_t* dt, const int32_t* clamp_rows,
                            int32_t* err) {
#define TBE_DS(W, P)                                                                           \
  hipLaunchKernelGGL((sort_downsweep_kernel<FIRST, LAST, W, P>), grid, dim3(kThreads), 0, s,   \
                     a.ki, a.pi, a.bi, a.wi, offsets, a.ko, a.po, a.bo, a.wo, tile_desc, toff, \
                     shift, bits, tiles_max, dc, dt, clamp_rows, err)
  if (weighted && with_pos) TBE_DS(true, true);
  else if (weighted) TBE_DS(true, false);
  else if (with_pos) TBE_DS(false, true);
  else TBE_DS(false, false);
#undef TBE_DS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sort_setup(const Problem& p, const int32_t* offsets, const SortBuffers& b,
                             hipStream_t s) {
  hipLaunchKernelGGL(sort_setup_kernel, dim3(1), dim3(256), 0, s, offsets, p.T, p.B, b.tile_base);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || p.N == 0) return err;
  hipLaunchKernelGGL(sort_tiles_kernel, dim3((unsigned)((p.sort_tiles_max + 255) / 256)), dim3(256),
                     0, s, b.tile_base, offsets, p.T, p.B, p.sort_tiles_max, b.tile_desc);
  return hipGetLastError();
}

hipError_t launch_sort(const Problem& p, const int32_t* indices, const int32_t* offsets,
                       const float* psw, const int32_t* tinfo, const SortBuffers& b,
                       const tbe_meta& meta, hipStream_t s) {
  hipError_t err;
  if (p.N == 0) return hipSuccess;
  // Consecutive tiles run on one XCD: the digit counts of neighbouring tiles
  // share cache lines, and so do the ends of their output buckets, which one
  // L2 then merges instead of eight writing back partial lines.
  const dim3 tgrid((unsigned)xcd_grid(p.sort_tiles_max));
  const int radix = 1 << p.sort_bits;
  const bool weighted = p.weighted;
  const bool with_pos = meta.sorted_pos != nullptr;
  const int32_t* toff = tinfo;
  for (int pass = 0; pass < p.sort_passes; ++pass) {
    const bool first = pass == 0;
    const bool last = pass == p.sort_passes - 1;
    const int shift = pass * p.sort_bits;
    // source and destination buffers: pass 0 writes A, pass 1 reads A and
    // writes B, pass 2 reads B, ...; the last pass writes the outputs.
    int32_t* const* src = (pass % 2 == 1) ? b.A : b.B;
    int32_t* const* dst = (pass % 2 == 0) ? b.A : b.B;
    PassArgs a;
    a.ki = first ? indices : src[0];
    a.pi = first ? nullptr : src[1];
    a.bi = first ? nullptr : src[2];
    a.wi = first ? psw : (const float*)src[3];
    a.ko = last ? b.sorted_keys : dst[0];
    a.po = last ? meta.sorted_pos : dst[1];
    a.bo = last ? meta.sorted_bag : dst[2];
    a.wo = last ? meta.sorted_psw : (float*)dst[3];

    // TBE_FLAG_CHECK: the first pass reads the indices, so it clamps them
    const int32_t* clamp_rows = (first && p.err) ? tinfo + p.T : nullptr;
    hipLaunchKernelGGL(sort_upsweep_kernel, tgrid, dim3(kThreads), 0, s, a.ki, b.tile_desc, shift,
                       p.sort_bits, p.sort_tiles_max, b.digit_counts, clamp_rows);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(sort_scan_kernel, dim3((unsigned)(p.T * radix)), dim3(kThreads), 0, s,
                       b.digit_counts, b.tile_base, radix, p.sort_tiles_max, b.digit_tot);
    if ((err = hipGetLastError()) != hipSuccess) return err;
#define TBE_DOWNSWEEP(F, L)                                                                     \
  launch_downsweep<F, L>(weighted, with_pos, tgrid, s, a, offsets, b.tile_desc, toff, shift,    \
                         p.sort_bits, p.sort_tiles_max, b.digit_counts, b.digit_tot, clamp_rows,  \
                         p.err)
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
