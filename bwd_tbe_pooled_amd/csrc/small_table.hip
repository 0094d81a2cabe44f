// Small-table path (page 1, "Forward state reuse and preprocessing" and
// checklist item 2: E <= 64, 64 <= D <= 128, L >= 64, f16 weights, no
// per-sample weights). With so few rows, a bag is better described by its row
// histogram H[bag][e] than by its index list, and pooling becomes a dense
// contraction:
//     forward   out[b, t-block] = H_t[b, :] . W_t            ([B x 64] x [64 x D])
//     backward  G_t = H_t^T . grad_t                         ([64 x B] x [B x D])
// both on the matrix cores (v_mfma_f32_32x32x16_f16: f16 inputs, f32
// accumulation). Counts are exact in f16 up to 2048. The backward scales each
// gradient column by a power of two 2^s that brings its magnitudes near
// [2^4, 2^5), splits the scaled value x into
// hi = f16(x) and lo = f16((x - hi) * 2^11), contracts H with both (the lo
// product with H * 2^-11, exact in f16) and unscales the sums by 2^-s at the
// end. That compensates the f16 rounding to about 2^-22 relative for every
// gradient down to 2^-18 of the column's first largest, whatever its magnitude.
// The scale of a column is set by its first tile with a nonzero gradient; a
// workgroup that meets a tile far outside it, or a non-finite gradient, flags
// its (table, split), and the f32 kernel then recomputes that partial. The
// forward saves
// the counts (uint8, saturating at 255 with a flag) and the backward reuses
// them; only the counts cross from forward to backward.
//
// MFMA operand layout used (lane l, i = l % 32, kb = l / 32):
//   A[i][kb*8 + j] and B[kb*8 + j][i] for j = 0..7 (the same k assignment on
//   both sides, so the contraction is over matching k), and
//   C[8*(r/4) + 4*kb + r%4][i] in accumulator register r = 0..15.
#include "adagrad.h"
#include "device.h"
#include "internal.h"

namespace tbe {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kBagTile = 64;            // bags per count tile
constexpr int kHStride = kSmallE + 4;   // LDS count row, padded: 16-byte aligned, banks rotate
constexpr int kFwdTiles = 4;            // bag tiles per recounting forward workgroup
constexpr int kPoolTiles = 8;           // bag tiles per pooling workgroup
constexpr int kCountTiles = 4;          // bag tiles per counting workgroup
constexpr int kMaxD = 128;              // widest row on this path
constexpr int kWStride = kMaxD + 8;     // staged W_t row (f16), same bytes as a count row
constexpr int kTStride = kBagTile + 8;  // transposed f16 count row (16-byte aligned)
static_assert(kSmallE * kWStride * 2 == kBagTile * kHStride * 4, "W_t stage aliases H");
constexpr uint32_t kExactCount = 2048;  // counts exact in f16 up to here

__device__ __forceinline__ float16v mfma32(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ _Float16 w_half(const f16_t* W, int64_t idx) {
  return __builtin_bit_cast(_Float16, W[idx].bits);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const uint32_t y = (uint32_t)__shfl_xor((int)x, m);
    x = y > x ? y : x;
  }
  return x;
}

// Count the lookups of bags [bag0, bag0 + nb) of one table into H. Wave w
// owns bags 16w .. 16w+15; a bag's lookups are contiguous, so its lanes read
// 64 of them with one coalesced load and add them to the bag's row with one
// LDS atomic, the bag known without any search. The first 64 lookups of
// INFLIGHT bags are loaded before any of them is counted; lookups past the
// 64th follow bag by bag, eight loads in flight.
// A lookup's row: without a bounds check (err null) the index is masked to
// the 64 rows the buffers hold; with one (TBE_FLAG_CHECK) an index outside
// the table's Et rows counts as row 0 and is reported.
template <bool CHECK>
__device__ __forceinline__ uint32_t count_row(int32_t v, uint32_t Et, bool& bad) {
  if constexpr (!CHECK) return (uint32_t)v & (kSmallE - 1);
  const bool out = (uint32_t)v >= Et;
  bad |= out;
  return out ? 0u : (uint32_t)v;
}

template <bool CHECK, int INFLIGHT = 4>
__device__ void count_tile_impl(uint32_t (*H)[kHStride], int32_t* s_off,
                                const int32_t* __restrict__ indices,
                                const int32_t* __restrict__ offsets, int64_t bag0, int nb,
                                uint32_t Et, int32_t* __restrict__ err) {
  constexpr int NBW = kBagTile / kWaves;
  __syncthreads();  // earlier readers of H and s_off are done
  uint4* h4 = reinterpret_cast<uint4*>(&H[0][0]);
  for (int q = threadIdx.x; q < kBagTile * kHStride / 4; q += kThreads) h4[q] = uint4{0, 0, 0, 0};
  if ((int)threadIdx.x <= nb) s_off[threadIdx.x] = offsets[bag0 + threadIdx.x];
  __syncthreads();
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int bw0 = wave * NBW;
  bool bad = false;
  for (int u0 = 0; u0 < NBW; u0 += INFLIGHT) {
    int32_t v[INFLIGHT];
    bool ok[INFLIGHT];
#pragma unroll
    for (int u = 0; u < INFLIGHT; ++u) {
      const int bl = bw0 + u0 + u;
      const int32_t a = bl < nb ? s_off[bl] : 0;
      const int32_t len = bl < nb ? s_off[bl + 1] - a : 0;
      ok[u] = lane < len;
      v[u] = ok[u] ? indices[a + lane] : 0;
    }
#pragma unroll
    for (int u = 0; u < INFLIGHT; ++u)
      if (ok[u]) atomicAdd(&H[bw0 + u0 + u][count_row<CHECK>(v[u], Et, bad)], 1u);
  }
  for (int u = 0; u < NBW; ++u) {
    const int bl = bw0 + u;
    if (bl >= nb) break;
    const int32_t a = s_off[bl];
    const int64_t len = (int64_t)s_off[bl + 1] - a;
    for (int64_t c = kWave; c < len; c += 8 * kWave) {
      int32_t x[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t r = c + q * kWave + lane;
        x[q] = r < len ? indices[a + r] : 0;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q)
        if (c + q * kWave + lane < len) atomicAdd(&H[bl][count_row<CHECK>(x[q], Et, bad)], 1u);
    }
  }
  if constexpr (CHECK) {
    if (__ballot(bad) != 0 && lane == 0) atomicOr(err, (int32_t)TBE_ERROR_INDEX);
  }
  __syncthreads();
}

// The recounting kernels are off the common path: one body, checked or not
// by the call's flag.
__device__ __forceinline__ void count_tile(uint32_t (*H)[kHStride], int32_t* s_off,
                                           const int32_t* __restrict__ indices,
                                           const int32_t* __restrict__ offsets, int64_t bag0,
                                           int nb, uint32_t Et, int32_t* __restrict__ err) {
  if (err) count_tile_impl<true>(H, s_off, indices, offsets, bag0, nb, Et, err);
  else count_tile_impl<false>(H, s_off, indices, offsets, bag0, nb, Et, err);
}

// Saturating uint8 counts of kCountTiles consecutive 64-bag tiles of one
// table, written to hist, and the flags: counts[4] when a count exceeds 255,
// counts[5] when one exceeds 2048. Grid (ceil(B / (64 * kCountTiles)), T).
// The tiles are pipelined: wave w owns bags 16w .. 16w+15 of each tile (its
// own rows of H), and the first 64 lookups of its bags in tile k+1 are loaded
// (one coalesced load per bag) before it counts tile k with LDS atomics; it
// then packs its rows into hist and clears them for the next tile. The waves
// share no rows, so after the first barrier they run without any.
template <bool CHECK>
// Seven waves per SIMD (72 registers): more bags' loads in flight per CU.
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(7))) void small_count_kernel(
    const int32_t* __restrict__ indices, const int32_t* __restrict__ offsets,
    uint8_t* __restrict__ hist, int32_t* __restrict__ counts, int32_t B,
    const int32_t* __restrict__ trows, int32_t* __restrict__ err) {
  constexpr int NBW = kBagTile / kWaves;
  __shared__ __align__(16) uint32_t H[kBagTile][kHStride];
  __shared__ int32_t s_off[kBagTile * kCountTiles + 1];
  __shared__ uint32_t s_wmax[kWaves];
  const int32_t t = blockIdx.y;
  const int32_t wb0 = (int32_t)blockIdx.x * kBagTile * kCountTiles;
  const int32_t wnb = B - wb0 < kBagTile * kCountTiles ? B - wb0 : kBagTile * kCountTiles;
  const int64_t wbag0 = (int64_t)t * B + wb0;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const uint32_t Et = (uint32_t)trows[t];
  bool bad = false;
  uint4* h4 = reinterpret_cast<uint4*>(&H[0][0]);
  for (int q = threadIdx.x; q < kBagTile * kHStride / 4; q += kThreads) h4[q] = uint4{0, 0, 0, 0};
  for (int q = threadIdx.x; q <= wnb; q += kThreads) s_off[q] = offsets[wbag0 + q];
  __syncthreads();

  int32_t v[NBW];
  bool ok[NBW];
  auto load_first = [&](int k) {  // first 64 lookups of this wave's bags in tile k
#pragma unroll
    for (int u = 0; u < NBW; ++u) {
      const int bl = k * kBagTile + wave * NBW + u;
      const int32_t a = bl < wnb ? s_off[bl] : 0;
      const int32_t len = bl < wnb ? s_off[bl + 1] - a : 0;
      ok[u] = lane < len;
      v[u] = ok[u] ? indices[a + lane] : 0;
    }
  };
  load_first(0);
  uint32_t mx = 0;
  for (int k = 0; k < kCountTiles; ++k) {
    const int tb0 = k * kBagTile;  // first bag of the tile, within the workgroup's range
    if (tb0 >= wnb) break;
    const int nb = wnb - tb0 < kBagTile ? wnb - tb0 : kBagTile;
    int32_t cv[NBW];
    bool cok[NBW];
#pragma unroll
    for (int u = 0; u < NBW; ++u) {
      cv[u] = v[u];
      cok[u] = ok[u];
    }
    if (k + 1 < kCountTiles) load_first(k + 1);
#pragma unroll
    for (int u = 0; u < NBW; ++u)
      if (cok[u]) atomicAdd(&H[wave * NBW + u][count_row<CHECK>(cv[u], Et, bad)], 1u);
    // lookups past the 64th of each bag, eight loads in flight
    for (int u = 0; u < NBW; ++u) {
      const int bl = wave * NBW + u;
      if (bl >= nb) break;
      const int32_t a = s_off[tb0 + bl];
      const int64_t len = (int64_t)s_off[tb0 + bl + 1] - a;
      for (int64_t c = kWave; c < len; c += 8 * kWave) {
        int32_t x[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int64_t r = c + q * kWave + lane;
          x[q] = r < len ? indices[a + r] : 0;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (c + q * kWave + lane < len) atomicAdd(&H[bl][count_row<CHECK>(x[q], Et, bad)], 1u);
      }
    }
    wave_lds_sync();  // this wave's atomics have landed
    const int64_t bag0 = wbag0 + tb0;
    for (int q = lane; q < NBW * (kSmallE / 4); q += kWave) {
      const int bl = wave * NBW + (q >> 4), e4 = (q & 15) * 4;
      if (bl >= nb) break;
      uint4* hp = reinterpret_cast<uint4*>(&H[bl][e4]);
      const uint4 c = *hp;
      *hp = uint4{0, 0, 0, 0};
      const uint32_t a = c.x > c.y ? c.x : c.y, b = c.z > c.w ? c.z : c.w;
      mx = mx > (a > b ? a : b) ? mx : (a > b ? a : b);
      const uint32_t packed = (c.x > 255u ? 255u : c.x) | (c.y > 255u ? 255u : c.y) << 8 |
                              (c.z > 255u ? 255u : c.z) << 16 | (c.w > 255u ? 255u : c.w) << 24;
      *reinterpret_cast<uint32_t*>(hist + (bag0 + bl) * kSmallE + e4) = packed;
    }
    wave_lds_sync();  // cleared before this wave's next atomics
  }
  if constexpr (CHECK) {
    if (__ballot(bad) != 0 && lane == 0) atomicOr(err, (int32_t)TBE_ERROR_INDEX);
  }
  mx = wave_max_u32(mx);
  if (lane == 0) s_wmax[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tmax = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tmax = s_wmax[w] > tmax ? s_wmax[w] : tmax;
    if (tmax > 255u) atomicOr(&counts[4], 1);
    if (tmax > kExactCount) atomicOr(&counts[5], 1);
  }
}

// Stage W_t (zero-padded to 64 x 128) in LDS with coalesced loads and pick a
// wave's B operands out of it: rows e(ks, kb, j) of the two 32-column tiles
// (w >> 1) and (w >> 1) + 2, for the k order the caller's A operands use.
template <typename EOF_>
__device__ void load_w_operands(const f16_t* __restrict__ Wt, int32_t Et, int32_t D,
                                _Float16 (*Ws)[kWStride], half8 (&bw)[kSmallE / 16][2],
                                EOF_ e_of) {
  for (int q = threadIdx.x; q < kSmallE * kMaxD; q += kThreads) {
    const int e = q / kMaxD, d = q % kMaxD;
    Ws[e][d] = (e < Et && d < D) ? w_half(Wt, (int64_t)e * D + d) : (_Float16)0.f;
  }
  __syncthreads();
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i = lane & 31, kb = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < kSmallE / 16; ++ks)
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int d = ((wave >> 1) + 2 * q) * 32 + i;
#pragma unroll
      for (int j = 0; j < 8; ++j) bw[ks][q][j] = Ws[e_of(ks, kb, j)][d];
    }
}

// Store a wave's two 32 x 32 output blocks (bag rows mt*32.., column tiles
// (w >> 1) and (w >> 1) + 2) of the tile at bag b0.
__device__ __forceinline__ void store_out_blocks(float* __restrict__ ot, int64_t ostride,
                                                 const float16v (&acc)[2], int32_t b0, int nb,
                                                 int32_t D) {
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i = lane & 31, kb = lane >> 5;
  const int mt = wave & 1;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int d = ((wave >> 1) + 2 * q) * 32 + i;
    if (d >= D) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int bl = mt * 32 + 8 * (r / 4) + 4 * kb + (r % 4);
      if (bl < nb) store_stream(&ot[(int64_t)(b0 + bl) * ostride + d], acc[q][r]);
    }
  }
}

// Forward contraction out[b, t-block] = H_t[b, :] . W_t from the saved uint8
// counts (all at most 255, so counts[4] is clear; else this grid exits and the
// recounting kernel below runs). A wave's A operand rows are its lanes' bags,
// read straight from hist: the contraction order over e is free as long as
// both operands use it, so lane (i, kb) takes e = kb*32 + ks*8 + j, i.e. 32
// consecutive count bytes, two 16-byte loads per tile. No LDS or barriers in
// the tile loop; the next tile's counts are loaded before this tile's MFMAs.
// Grid ceil(B / (kPoolTiles * 64)) * T, table = block % T.
__global__ __launch_bounds__(kThreads) void small_pool_kernel(
    const f16_t* __restrict__ W, const uint8_t* __restrict__ hist,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ toff,
    const int32_t* __restrict__ trows, float* __restrict__ out, int32_t T, int32_t B,
    int32_t D, int64_t ld) {
  __shared__ __align__(16) _Float16 Ws[kSmallE][kWStride];
  if (counts[4] != 0) return;
  const int32_t t = blockIdx.x % T;   // tables vary fastest: the resident
  const int32_t bx = blockIdx.x / T;  // workgroups write whole output rows
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i = lane & 31, kb = lane >> 5;
  const int mt = wave & 1;
  half8 bw[kSmallE / 16][2];
  load_w_operands(W + (int64_t)toff[t] * D, trows[t], D, Ws, bw,
                  [](int ks, int kb_, int j) { return kb_ * 32 + ks * 8 + j; });
  float* ot = out + (int64_t)t * D;
  const int64_t ostride = ld;
  const int32_t tb0 = bx * kPoolTiles * kBagTile;
  auto load_counts = [&](int32_t b0, uint4& h0, uint4& h1) {
    const int32_t b = b0 + mt * 32 + i;
    h0 = h1 = uint4{0, 0, 0, 0};
    if (b < B) {
      const uint4* p = reinterpret_cast<const uint4*>(hist + ((int64_t)t * B + b) * kSmallE + kb * 32);
      h0 = p[0];
      h1 = p[1];
    }
  };
  uint4 n0, n1;
  load_counts(tb0, n0, n1);
  for (int k = 0; k < kPoolTiles; ++k) {
    const int32_t b0 = tb0 + k * kBagTile;
    if (b0 >= B) break;
    const int nb = B - b0 < kBagTile ? B - b0 : kBagTile;
    const uint32_t w8[8] = {n0.x, n0.y, n0.z, n0.w, n1.x, n1.y, n1.z, n1.w};
    if (k + 1 < kPoolTiles && b0 + kBagTile < B) load_counts(b0 + kBagTile, n0, n1);
    float16v acc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kSmallE / 16; ++ks) {
      half8 a;
#pragma unroll
      for (int j = 0; j < 8; ++j)
        a[j] = (_Float16)(float)((w8[2 * ks + j / 4] >> (8 * (j % 4))) & 0xffu);
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q] = mfma32(a, bw[ks][q], acc[q]);
    }
    store_out_blocks(ot, ostride, acc, b0, nb, D);
  }
}

// Forward when some saved count saturated (counts[4] set; else this grid
// exits): recount each 64-bag tile exactly in LDS, then contract on the
// matrix cores, or in plain f32 for a tile with a count above 2048.
// Grid (ceil(B / (kFwdTiles * 64)), T).
__global__ __launch_bounds__(kThreads) void small_recount_forward_kernel(
    const f16_t* __restrict__ W, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ toff, const int32_t* __restrict__ trows, float* __restrict__ out,
    int32_t T, int32_t B, int32_t D, int64_t ld, int32_t* __restrict__ err) {
  __shared__ __align__(16) uint32_t H[kBagTile][kHStride];
  __shared__ int32_t s_off[kBagTile + 1];
  __shared__ uint32_t s_wmax[kWaves];
  if (counts[4] == 0) return;
  const int32_t t = blockIdx.y;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i = lane & 31, kb = lane >> 5;
  const int mt = wave & 1;
  const int32_t Et = trows[t];
  const f16_t* Wt = W + (int64_t)toff[t] * D;
  float* ot = out + (int64_t)t * D;
  const int64_t ostride = ld;
  half8 bw[kSmallE / 16][2];
  load_w_operands(Wt, Et, D, reinterpret_cast<_Float16(*)[kWStride]>(&H[0][0]), bw,
                  [](int ks, int kb_, int j) { return ks * 16 + kb_ * 8 + j; });

  for (int k = 0; k < kFwdTiles; ++k) {
    const int32_t b0 = ((int32_t)blockIdx.x * kFwdTiles + k) * kBagTile;
    if (b0 >= B) break;
    const int nb = B - b0 < kBagTile ? B - b0 : kBagTile;
    count_tile(H, s_off, indices, offsets, (int64_t)t * B + b0, nb, (uint32_t)Et, err);
    uint32_t mx = 0;
    for (int q = threadIdx.x; q < nb * (kSmallE / 4); q += kThreads) {
      const uint4 c = *reinterpret_cast<const uint4*>(&H[q >> 4][(q & 15) * 4]);
      const uint32_t a = c.x > c.y ? c.x : c.y, b = c.z > c.w ? c.z : c.w;
      mx = mx > (a > b ? a : b) ? mx : (a > b ? a : b);
    }
    mx = wave_max_u32(mx);
    if (lane == 0) s_wmax[wave] = mx;
    __syncthreads();
    uint32_t tmax = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) tmax = s_wmax[w] > tmax ? s_wmax[w] : tmax;

    if (tmax > kExactCount) {
      // Counts beyond f16's exact range: plain f32 dot products over the rows.
      for (int q = threadIdx.x; q < nb * D; q += kThreads) {
        const int bl = q / D, d = q % D;
        float acc = 0.f;
        for (int e = 0; e < Et && e < kSmallE; ++e)
          acc += (float)H[bl][e] * (float)w_half(Wt, (int64_t)e * D + d);
        ot[(int64_t)(b0 + bl) * ostride + d] = acc;
      }
      continue;
    }
    float16v acc[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < kSmallE / 16; ++ks) {
      const uint4* hp = reinterpret_cast<const uint4*>(&H[mt * 32 + i][ks * 16 + kb * 8]);
      const uint4 c0 = hp[0], c1 = hp[1];
      half8 a;
      a[0] = (_Float16)(float)c0.x; a[1] = (_Float16)(float)c0.y;
      a[2] = (_Float16)(float)c0.z; a[3] = (_Float16)(float)c0.w;
      a[4] = (_Float16)(float)c1.x; a[5] = (_Float16)(float)c1.y;
      a[6] = (_Float16)(float)c1.z; a[7] = (_Float16)(float)c1.w;
      // (operands of columns past D are zero: no test, so acc stays in AGPRs)
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q] = mfma32(a, bw[ks][q], acc[q]);
    }
    store_out_blocks(ot, ostride, acc, b0, nb, D);
  }
}

// One workgroup per (table, split of the batch): partial G = H^T . grad over
// the split's bags, written to partials[(t*splits + s)][64][D], and the
// split's per-row counts to part_counts[(t*splits + s)][64]. Wave w owns the
// 32 columns w*32.. and both 32-row halves of G. Runs only when every count
// is exact in f16 (counts[5] clear). Every workgroup writes wide[t*splits + s]:
// 1 when some gradient of its split is not finite (the Inf or NaN then reaches
// the rows as plain arithmetic carries it) or lies outside its column's
// scaled range, so that the f32 kernel launched next recomputes that partial;
// 0 otherwise.
// Three waves per SIMD (168 registers; the few spills are on the recount path).
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void small_backward_kernel(
    const float* __restrict__ grad, const uint8_t* __restrict__ hist,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ offsets, float* __restrict__ partials,
    int32_t* __restrict__ part_counts, int32_t* __restrict__ wide, int32_t T, int32_t B,
    int32_t D, int64_t ld, int32_t splits, int32_t bags_per_split,
    const int32_t* __restrict__ trows, int32_t* __restrict__ err) {
  __shared__ __align__(16) uint32_t H[kBagTile][kHStride];     // recounted counts
  __shared__ __align__(16) _Float16 HT[kSmallE][kTStride];     // counts, row-major by table row
  __shared__ int32_t s_off[kBagTile + 1];
  if (counts[5] != 0) return;
  const int32_t t = blockIdx.y;
  const int32_t s = blockIdx.x;
  const int32_t sb0 = s * bags_per_split < B ? s * bags_per_split : B;
  const int32_t sb1 = sb0 + bags_per_split < B ? sb0 + bags_per_split : B;
  const bool recount = counts[4] != 0;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i = lane & 31, kb = lane >> 5;
  const int nt = wave;
  const int NT = (D + 31) / 32;
  const int d = nt * 32 + i;
  const bool has_col = nt < NT && d < D;
  const float* gt = grad + (int64_t)t * D;
  const int64_t gstride = ld;
  // offset of (bag kb*8, column d) from a 16-bag group's first row; columns
  // past D read column D-1 and are zeroed after the load
  const int32_t lane_off = kb * 8 * (int32_t)gstride + (d < D ? d : D - 1);

  float16v acc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
  uint32_t cnt[2] = {0u, 0u};  // count of row q*32 + i over this lane's half of the bags
  bool big = false;            // some gradient this lane split is not finite or out of scale
  int sc = 0;                  // this column's scale: the sums are in units of 2^-sc
  bool has_sc = false;         // set by the first tile with a nonzero gradient

  // gradient of bag b0 + ks*16 + kb*8 + j at column d, in g[ks*8 + j]; the
  // next tile's are loaded while this one is split and contracted. Every
  // load is in bounds (a ragged tile rereads its last bag, a lane past D
  // reads column D-1), and the returned mask, applied where the values are
  // used, zeroes those: no select waits for the loads right after issue.
  float gn[kBagTile / 2], gnext[kBagTile / 2];
  auto load_grad = [&](int32_t b0, float (&g)[kBagTile / 2]) -> uint32_t {
    const int nb = sb1 - b0 < kBagTile ? sb1 - b0 : kBagTile;
    if (nb <= 0) return 0u;
    if (nb == kBagTile) {
#pragma unroll
      for (int ks = 0; ks < kBagTile / 16; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float* row = gt + (int64_t)(b0 + ks * 16 + j) * gstride;  // uniform
          g[ks * 8 + j] = row[lane_off];
        }
      return has_col ? 0xffffffffu : 0u;
    }
    uint32_t m = 0u;
    const int32_t dc = d < D ? d : D - 1;
#pragma unroll
    for (int ks = 0; ks < kBagTile / 16; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int bl = ks * 16 + kb * 8 + j;
        const int bc = bl < nb ? bl : nb - 1;
        g[ks * 8 + j] = gt[(int64_t)(b0 + bc) * gstride + dc];
        m |= (has_col && bl < nb ? 1u : 0u) << (ks * 8 + j);
      }
    return m;
  };

  typedef _Float16 half2v __attribute__((ext_vector_type(2)));
  const half2v ones = {(_Float16)1.f, (_Float16)1.f};

  // Saved counts of bag hb, rows h16..h16+15, one tile ahead like the
  // gradients and loaded before them (loads complete in order): a ragged
  // tile rereads its last bag, zeroed where used.
  const int hb = threadIdx.x >> 2, h16 = (threadIdx.x & 3) * 16;
  auto load_hist = [&](int32_t b0) -> uint4 {
    const int nb = sb1 - b0 < kBagTile ? sb1 - b0 : kBagTile;
    if (recount || nb <= 0) return uint4{0, 0, 0, 0};
    const int bc = hb < nb ? hb : nb - 1;
    return *reinterpret_cast<const uint4*>(hist + ((int64_t)t * B + b0 + bc) * kSmallE + h16);
  };
  uint4 hnext = load_hist(sb0);
  uint32_t mnext = load_grad(sb0, gnext);
  for (int32_t b0 = sb0; b0 < sb1; b0 += kBagTile) {
    const int nb = sb1 - b0 < kBagTile ? sb1 - b0 : kBagTile;
    const int64_t bag0 = (int64_t)t * B + b0;
    const uint4 hv = hb < nb ? hnext : uint4{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < kBagTile / 2; ++q) gn[q] = (mnext >> q) & 1u ? gnext[q] : 0.f;
    // this tile's values are taken before the next tile's loads are issued,
    // so that the wait for them does not also wait for those
#pragma unroll
    for (int q = 0; q < kBagTile / 2; ++q) asm volatile("" ::"v"(gn[q]));
    asm volatile("" ::"v"(hv.x), "v"(hv.y), "v"(hv.z), "v"(hv.w) : "memory");
    hnext = load_hist(b0 + kBagTile);
    mnext = load_grad(b0 + kBagTile, gnext);
    // B operands: this tile's gradients of column d times 2^sc, split into
    // hi = f16(x) and lo = f16((x - hi) * 2^11). sc is a power-of-two scale
    // per column (lanes i and i + 32 agree on it), set by the first tile with
    // a nonzero gradient so that its largest magnitude lands in [2^4, 2^5):
    // gradients far below 1 would otherwise fall into f16's subnormals, and
    // above 65504 overflow. The sums are in units of 2^-sc, unscaled once at
    // the end (exact). A later tile whose largest scaled magnitude leaves
    // [2^-14, 2^15) (1024 times the first tile's largest, or 2^18 times less)
    // marks the split for the f32 kernel, like a non-finite one.
    {
      float gmax = 0.f;
#pragma unroll
      for (int q = 0; q < kBagTile / 2; ++q) {
        const float a = __builtin_fabsf(gn[q]);
        big |= !(a <= 3.402823466e38f);  // Inf or NaN
        gmax = a > gmax && a <= 3.402823466e38f ? a : gmax;
      }
      gmax = fmaxf(gmax, __shfl_xor(gmax, 32));
      if (gmax > 0.f) {
        const int e = __builtin_amdgcn_frexp_expf(gmax);  // gmax in [2^(e-1), 2^e)
        if (!has_sc) {
          sc = 5 - e;
          has_sc = true;
        } else if (e + sc > 15 || e + sc < -13) {
          big = true;
        }
      }
    }
    half8 hi[kBagTile / 16], lo[kBagTile / 16];
#pragma unroll
    for (int ks = 0; ks < kBagTile / 16; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = __builtin_ldexpf(gn[ks * 8 + j], sc);
        const _Float16 h = (_Float16)x;
        hi[ks][j] = h;
        lo[ks][j] = (_Float16)((x - (float)h) * 2048.f);
      }

    if (recount) count_tile(H, s_off, indices, offsets, bag0, nb, (uint32_t)trows[t], err);
    else __syncthreads();  // earlier readers of HT are done
    {
      // Counts of bag bl, rows e16..e16+15, into HT[e][bl] as f16 (exact).
      const int bl = hb, e16 = h16;
      uint32_t c[16];
      if (recount) {
        const uint4* hp = reinterpret_cast<const uint4*>(&H[bl][e16]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint4 v = hp[q];
          c[4 * q] = v.x; c[4 * q + 1] = v.y; c[4 * q + 2] = v.z; c[4 * q + 3] = v.w;
        }
      } else {
        const uint32_t wds[4] = {hv.x, hv.y, hv.z, hv.w};
#pragma unroll
        for (int q = 0; q < 16; ++q) c[q] = (wds[q >> 2] >> (8 * (q & 3))) & 0xffu;
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) HT[e16 + q][bl] = (_Float16)(float)c[q];
    }
    __syncthreads();

#pragma unroll
    for (int ks = 0; ks < kBagTile / 16; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const half8 a_hi = *reinterpret_cast<const half8*>(&HT[mt * 32 + i][ks * 16 + kb * 8]);
        const half8 a_lo = a_hi * (_Float16)(1.f / 2048.f);  // exact: counts <= 2048
        float tc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const half2v pr = {a_hi[j], a_hi[j + 1]};
          tc = __builtin_amdgcn_fdot2(pr, ones, tc, false);
        }
        cnt[mt] += (uint32_t)tc;
        acc[mt] = mfma32(a_hi, hi[ks], acc[mt]);  // zero gradients past D
        acc[mt] = mfma32(a_lo, lo[ks], acc[mt]);
      }
    }
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[mt][r] = __builtin_ldexpf(acc[mt][r], -sc);

  const int any_big = __syncthreads_or(big ? 1 : 0);
  if (threadIdx.x == 0) wide[(int64_t)t * splits + s] = any_big ? 1 : 0;
  float* pt = partials + ((int64_t)t * splits + s) * kSmallE * D;
  if (has_col && !any_big) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = mt * 32 + 8 * (r / 4) + 4 * kb + (r % 4);
        pt[(int64_t)e * D + d] = acc[mt][r];
      }
  }
  if (wave == 0) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint32_t c = cnt[mt] + (uint32_t)__shfl_xor((int)cnt[mt], 32);
      if (kb == 0) part_counts[((int64_t)t * splits + s) * kSmallE + mt * 32 + i] = (int32_t)c;
    }
  }
}

// The same partial sums in plain f32 arithmetic, for problems where some
// count exceeds 2048 (counts[5] set; every split), or for the splits whose
// gradients the matrix-core kernel could not split into f16 halves
// (wide[t*splits + s] set): counts are recounted from the indices and each
// thread accumulates 32 (row, column) elements of G over the bags.
__global__ __launch_bounds__(kThreads) void small_backward_wide_kernel(
    const float* __restrict__ grad, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ indices, const int32_t* __restrict__ offsets,
    float* __restrict__ partials, int32_t* __restrict__ part_counts,
    const int32_t* __restrict__ wide, int32_t T, int32_t B, int32_t D, int64_t ld,
    int32_t splits, int32_t bags_per_split, const int32_t* __restrict__ trows,
    int32_t* __restrict__ err) {
  __shared__ __align__(16) uint32_t H[kBagTile][kHStride];
  __shared__ int32_t s_off[kBagTile + 1];
  const int32_t t = blockIdx.y;
  const int32_t s = blockIdx.x;
  if (counts[5] == 0 && wide[(int64_t)t * splits + s] == 0) return;
  const int32_t sb0 = s * bags_per_split < B ? s * bags_per_split : B;
  const int32_t sb1 = sb0 + bags_per_split < B ? sb0 + bags_per_split : B;
  const int d = threadIdx.x % kMaxD;
  const int e0 = (threadIdx.x / kMaxD) * (kSmallE / 2);  // rows e0 .. e0+31
  const float* gt = grad + (int64_t)t * D;
  const int64_t gstride = ld;
  float acc[kSmallE / 2];
#pragma unroll
  for (int r = 0; r < kSmallE / 2; ++r) acc[r] = 0.f;
  uint32_t cnt = 0;  // thread e < 64: count of row e
  for (int32_t b0 = sb0; b0 < sb1; b0 += kBagTile) {
    const int nb = sb1 - b0 < kBagTile ? sb1 - b0 : kBagTile;
    count_tile(H, s_off, indices, offsets, (int64_t)t * B + b0, nb, (uint32_t)trows[t], err);
    if (threadIdx.x < kSmallE)
      for (int bl = 0; bl < nb; ++bl) cnt += H[bl][threadIdx.x];
    if (d < D) {
      for (int bl = 0; bl < nb; ++bl) {
        const float g = gt[(int64_t)(b0 + bl) * gstride + d];
#pragma unroll
        for (int r = 0; r < kSmallE / 2; ++r) acc[r] += (float)H[bl][e0 + r] * g;
      }
    }
  }
  float* pt = partials + ((int64_t)t * splits + s) * kSmallE * D;
  if (d < D) {
#pragma unroll
    for (int r = 0; r < kSmallE / 2; ++r) pt[(int64_t)(e0 + r) * D + d] = acc[r];
  }
  if (threadIdx.x < kSmallE)
    part_counts[((int64_t)t * splits + s) * kSmallE + threadIdx.x] = (int32_t)cnt;
}

// Reduce the splits of each (table, row) in ascending split order and apply
// Adagrad to rows with a non-zero count. One 16-lane slot per row at D = 128.
template <int V, int PMAX>
__global__ __launch_bounds__(kThreads) void small_apply_kernel(
    f16_t* __restrict__ W, float* __restrict__ mom, const int32_t* __restrict__ toff,
    const int32_t* __restrict__ trows, const float* __restrict__ partials,
    const int32_t* __restrict__ part_counts, int32_t T, int32_t D, int32_t splits, int32_t G,
    int32_t log2G, int32_t P, float lr, float eps) {
  const int lane = lane_id();
  const int slot = lane >> log2G;
  const int col = lane & (G - 1);
  const int NS = kWave >> log2G;
  const int64_t row = ((int64_t)blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave) * NS + slot;
  if (row >= (int64_t)T * kSmallE) return;
  const int32_t t = (int32_t)(row / kSmallE), e = (int32_t)(row % kSmallE);
  if (e >= trows[t]) return;
  int64_t cnt = 0;
  for (int s = 0; s < splits; ++s) cnt += part_counts[((int64_t)t * splits + s) * kSmallE + e];
  if (cnt == 0) return;  // untouched row: no update
  float g[PMAX][V];
#pragma unroll
  for (int p = 0; p < PMAX; ++p)
#pragma unroll
    for (int v = 0; v < V; ++v) g[p][v] = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float* src = partials + (((int64_t)t * splits + s) * kSmallE + e) * D;
#pragma unroll
    for (int p = 0; p < PMAX; ++p) {
      const int c0 = (p * G + col) * V;
      if (p < P && c0 < D) {
#pragma unroll
        for (int v = 0; v < V; ++v) g[p][v] += src[c0 + v];
      }
    }
  }
  const int64_t key = (int64_t)toff[t] + e;
  adagrad_row<f16_t, float, V, PMAX>(W + key * D, mom + key, g, col, G, P, D, lr, eps);
}

__global__ void zero_counts_kernel(int32_t* counts) {
  if (threadIdx.x < 8) counts[threadIdx.x] = 0;
}

}  // namespace

int small_splits_for(int32_t T, int32_t B) {
  // About three workgroups per CU over the whole problem (the backward holds
  // three per CU: one round, no tail), at least 256 bags each.
  int64_t per_table = 3 * (int64_t)device_cu_count() / (T > 0 ? T : 1);
  if (per_table < 1) per_table = 1;
  int64_t max_splits = (B + 255) / 256;
  if (max_splits < 1) max_splits = 1;
  return (int)(per_table < max_splits ? per_table : max_splits);
}

hipError_t launch_small_count(const Problem& p, const int32_t* indices, const int32_t* offsets,
                              const int32_t* tinfo, uint8_t* hist, int32_t* counts,
                              hipStream_t s) {
  hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(64), 0, s, counts);
  if (p.B > 0) {
    const int64_t count_bags = (int64_t)kBagTile * kCountTiles;
    const dim3 grid((unsigned)((p.B + count_bags - 1) / count_bags), (unsigned)p.T);
    if (p.err)
      hipLaunchKernelGGL(small_count_kernel<true>, grid, dim3(kThreads), 0, s, indices, offsets,
                         hist, counts, p.B, tinfo + p.T, p.err);
    else
      hipLaunchKernelGGL(small_count_kernel<false>, grid, dim3(kThreads), 0, s, indices, offsets,
                         hist, counts, p.B, tinfo + p.T, p.err);
  }
  return hipGetLastError();
}

hipError_t launch_small_pool(const Problem& p, const void* W, const int32_t* indices,
                             const int32_t* offsets, const int32_t* tinfo, float* out,
                             const uint8_t* hist, const int32_t* counts, hipStream_t s) {
  if (p.B == 0) return hipSuccess;
  const int32_t* toff = tinfo;
  const int32_t* trows = tinfo + p.T;
  // Exactly one of the two computes the output, chosen on the device by counts[4].
  const int64_t pool_bags = (int64_t)kBagTile * kPoolTiles;
  hipLaunchKernelGGL(small_pool_kernel, dim3((unsigned)((p.B + pool_bags - 1) / pool_bags * p.T)),
                     dim3(kThreads), 0, s, (const f16_t*)W, hist, counts, toff, trows, out, p.T,
                     p.B, p.D, p.ld);
  const int64_t re_bags = (int64_t)kBagTile * kFwdTiles;
  hipLaunchKernelGGL(small_recount_forward_kernel,
                     dim3((unsigned)((p.B + re_bags - 1) / re_bags), (unsigned)p.T), dim3(kThreads), 0,
                     s, (const f16_t*)W, indices, offsets, counts, toff, trows, out, p.T, p.B, p.D,
                     p.ld, p.err);
  return hipGetLastError();
}

hipError_t launch_small_backward(const Problem& p, const float* grad, const uint8_t* hist,
                                 const int32_t* counts, const int32_t* indices,
                                 const int32_t* offsets, float* partials, int32_t* part_counts,
                                 int32_t* wide, const int32_t* tinfo, hipStream_t s) {
  const int splits = p.small_splits;
  int32_t per = (p.B + splits - 1) / splits;
  const dim3 grid((unsigned)splits, (unsigned)p.T);
  // Chosen on the device: with counts[5] set only the f32 kernel works; else
  // the matrix-core kernel computes every split and the f32 kernel redoes the
  // splits it flagged in `wide` (none, for finite gradients).
  hipLaunchKernelGGL(small_backward_kernel, grid, dim3(kThreads), 0, s, grad, hist, counts, indices,
                     offsets, partials, part_counts, wide, p.T, p.B, p.D, p.ld, splits, per,
                     tinfo + p.T, p.err);
  hipLaunchKernelGGL(small_backward_wide_kernel, grid, dim3(kThreads), 0, s, grad, counts, indices,
                     offsets, partials, part_counts, wide, p.T, p.B, p.D, p.ld, splits, per,
                     tinfo + p.T, p.err);
  return hipGetLastError();
}

hipError_t launch_small_apply(const Problem& p, void* W, float* m, const int32_t* tinfo,
                              const float* partials, const int32_t* part_counts, double lr,
                              double eps, hipStream_t s) {
  const RowShape rs = row_shape(p.D, 8);
  const int NS = kWave / rs.G;
  const int64_t rows = (int64_t)p.T * kSmallE;
  const int64_t blocks = (rows + NS * 4 - 1) / (NS * 4);
  const int32_t* toff = tinfo;
  const int32_t* trows = tinfo + p.T;
#define TBE_SMALL_APPLY(VV)                                                                     \
  hipLaunchKernelGGL((small_apply_kernel<VV, 1>), dim3((unsigned)blocks), dim3(kThreads), 0, s, \
                     (f16_t*)W, m, toff, trows, partials, part_counts, p.T, p.D,                \
                     p.small_splits, rs.G, rs.log2G, rs.P, (float)lr, (float)eps)
  if (rs.P != 1) return hipErrorInvalidValue;
  if (rs.V == 8) TBE_SMALL_APPLY(8);
  else if (rs.V == 4) TBE_SMALL_APPLY(4);
  else if (rs.V == 2) TBE_SMALL_APPLY(2);
  else TBE_SMALL_APPLY(1);
#undef TBE_SMALL_APPLY
  return hipGetLastError();
}

}  // namespace tbe
