// Backward of the hot rows on the matrix cores (page 1, "Forward state reuse
// and preprocessing": the transposed contraction with a compensated f16
// hi/lo split accumulated in f32; backward path 2 of "Backward kernel: three
// paths by segment length", whose output is one gradient row per unique row).
//
// A table's hot rows are the rows of its longest runs (the hot-row plan). For
// them the per-lookup gather of the chunk path reads each bag's gradient row
// once per hot lookup, about 15 times at the Zipf-skewed batch. Here each
// gradient row is read once instead: with H[s][b] the summed per-sample
// weight of hot slot s in bag b (the count when unweighted),
//     G[s, :] = sum_b H[s][b] * grad[b, t-block]         ([256 x B] x [B x D])
// is one dense contraction per table, tiled over 32-bag tiles and split over
// the batch into segments (one workgroup each). The chunk path keeps the
// other long runs; the apply then reduces each hot row's segment partials in
// segment order (deterministic) and applies its Adagrad step.
//
// Per tile (its gradients, indices and weights loaded during the previous
// tile's contraction):
//  A. H is cleared and each gradient column's largest magnitude found;
//  B. 16 threads per bag add each hot lookup's weight into H[slot][bag]
//     (the slot through the LDS hash) with f64 atomics: H holds sums of a
//     bag's few f32 weights, which are exact in f64, so the bits do not
//     depend on the order of the adds; each gradient column is scaled by its
//     power-of-two scale and split into f16 hi and lo (the B operands);
//  C. wave w multiplies hot slots 32w..32w+31 by the tile on
//     v_mfma_f32_32x32x16_f16, accumulating in f32.
//
// Precision: each gradient column is scaled by a power of two set by its
// first tile with a nonzero value (largest magnitude then in [2^4, 2^5)); x =
// g * 2^s is split into hi = f16(x) and lo = f16((x - hi) * 2^11), and the
// product takes H_hi * hi + (H_hi * 2^-11) * lo (+ H_res * hi when weighted,
// H_res = f16(H' - H_hi) with H' = H times its slot's power-of-two scale, set
// by the slot's first nonzero tile so that its largest sum lands in [1, 2)).
// That is about 2^-22 relative per term for every gradient down to 2^-18 of
// its column's scale. A gradient that is not finite or whose scaled value
// reaches 2^15 (1024 times the column's first largest), a weight sum 2^14
// times its slot's first, or a count above 2048 flags the table
// (hot_flag[t]); the schedule then sends that table's hot runs through the
// chunk path, which the apply reads for them instead.
//
// MFMA operand layout (lane l, i = l % 32, kb = l / 32): A[i][kb*8 + j] and
// B[kb*8 + j][i] for j = 0..7, C[8*(r/4) + 4*kb + r%4][i] in register r.
#include "device.h"
#include "hot_rows.h"
#include "internal.h"

namespace tbe {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float16v mfma32(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

constexpr int kHbThreads = 512;             // 8 waves: wave w owns hot slots 32w..32w+31
constexpr int kHbWaves = kHbThreads / kWave;
static_assert(kHbWaves * 32 == kHotMaxK, "one 32-slot block per wave");
constexpr int kHbBags = 32;                 // bags per tile: two 16-bag k-steps
static_assert(kHbBags * 16 == kHbThreads, "16 threads per bag");
constexpr int kHbHStride = kHbBags + 2;     // doubles per H row: 16-byte aligned, banks rotate
constexpr int kHbAhead = 2;                 // lookups per thread loaded a tile ahead

template <bool WEIGHTED, int NT>
__global__ __launch_bounds__(kHbThreads) void bwd_hot_kernel(
    const float* __restrict__ grad, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ offsets, const float* __restrict__ psw,
    const int32_t* __restrict__ hot_rows, const int32_t* __restrict__ tinfo,
    float* __restrict__ hot_parts, int32_t* __restrict__ hot_flag, int32_t T, int32_t B,
    int64_t ld, int32_t seg_bags) {
  constexpr int D = NT * 32;
  __shared__ __align__(16) int32_t s_key[kHotHash];
  __shared__ uint8_t s_slotof[kHotHash];
  __shared__ __align__(16) double s_H[kHotMaxK][kHbHStride];      // weight sums, exact
  __shared__ __align__(16) _Float16 s_gb[2][2][NT][kWave][8];     // [hi, lo][k-step][nt][lane][j]
  __shared__ uint32_t s_cmax[D];  // per column: bits of the tile's largest finite |g|
  __shared__ int32_t s_gsc[D];    // per column: scale exponent, for the unscaling
  __shared__ int32_t s_nhot;

  const int32_t t = blockIdx.y;
  const int32_t seg = blockIdx.x;
  const int32_t b_begin = seg * seg_bags;
  const int32_t b_end = b_begin + seg_bags < B ? b_begin + seg_bags : B;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i = lane & 31, kb = lane >> 5;
  const int32_t* __restrict__ hr = hot_rows + (int64_t)t * kHotMaxK;
  // an index outside the table is read as row 0, as the transpose keyed it
  const uint32_t Et = (uint32_t)tinfo[T + t];

  for (int q = threadIdx.x; q < kHotHash; q += kHbThreads) s_key[q] = -1;
  for (int d = threadIdx.x; d < D; d += kHbThreads) s_cmax[d] = 0u;
  if (threadIdx.x == 0) s_nhot = 0;
  __syncthreads();
  hot_hash_insert(s_key, s_slotof, hr, kHotMaxK);
  if (threadIdx.x < kHotMaxK && hr[threadIdx.x] >= 0) atomicMax(&s_nhot, (int)threadIdx.x + 1);
  __syncthreads();
  const int n_hot = s_nhot;  // slots 0..n_hot-1 are taken
  if (n_hot == 0) return;    // the whole workgroup: the table has no hot row
  const bool mine = wave * 32 < n_hot;  // this wave owns a taken slot

  // Lookups: 16 threads per bag of the tile, thread k of bag lb taking its
  // lookups k, k+16, ... Gradients: thread (g, c) holds column c of the 8
  // bags 8g..8g+7 (the j = 0..7 of one MFMA B operand lane).
  const int lb = threadIdx.x >> 4, lk = threadIdx.x & 15;
  const bool gthr = (int)threadIdx.x < 4 * D;
  const int gc = threadIdx.x % D, gg = threadIdx.x / D;
  const float* __restrict__ gcol = grad + (int64_t)t * D + gc;
  int gsc = 0;        // scale of column gc (the same in the 4 threads of a column)
  bool gset = false;
  int hsc = 0;        // scale of hot slot 32*wave + i (weighted)
  bool hset = false;
  bool bad = false;

  float16v acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[nt][r] = 0.f;

  const int32_t* __restrict__ ofs = offsets + (int64_t)t * B;
  auto tile_nb = [&](int32_t b0) { return b_end - b0 < kHbBags ? b_end - b0 : kHbBags; };
  // Global loads run ahead: the next-but-one tile's offsets, and the next
  // tile's gradients, indices and weights, issued before the matrix-core work.
  struct Off {
    int32_t q0, q1;  // this thread's bag's lookups [q0, q1); empty past the tile
  };
  struct Data {
    float g[8];
    int32_t idx[kHbAhead];
    float w[kHbAhead];
  };
  auto load_off = [&](int32_t b0, Off& o) {
    o.q0 = o.q1 = 0;
    if (b0 < b_end && lb < tile_nb(b0)) {
      o.q0 = ofs[b0 + lb];
      o.q1 = ofs[b0 + lb + 1];
    }
  };
  auto load_data = [&](int32_t b0, const Off& o, Data& x) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x.g[j] = 0.f;
#pragma unroll
    for (int r = 0; r < kHbAhead; ++r) {
      x.idx[r] = 0;
      x.w[r] = 0.f;
    }
    if (b0 >= b_end) return;
    const int nb = tile_nb(b0);
    if (gthr) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (gg * 8 + j < nb) x.g[j] = gcol[(int64_t)(b0 + gg * 8 + j) * ld];
    }
#pragma unroll
    for (int r = 0; r < kHbAhead; ++r) {
      const int32_t q = o.q0 + lk + r * 16;
      if (q < o.q1) {
        x.idx[r] = indices[q];
        if constexpr (WEIGHTED) x.w[r] = psw[q];
      }
    }
  };
  auto add_lookup = [&](int32_t idx, float w) {
    const int slot = hot_hash_find(s_key, s_slotof, (uint32_t)idx < Et ? idx : 0);
    // f64 sums of a bag's few f32 weights are exact, so the order in which
    // the atomics land does not change the bits
    if (slot >= 0) atomicAdd(&s_H[slot][lb], (double)w);
  };

  Off o_cur, o_nxt;
  Data dat;
  load_off(b_begin, o_cur);
  load_data(b_begin, o_cur, dat);
  load_off(b_begin + kHbBags, o_nxt);
  for (int32_t b0 = b_begin; b0 < b_end; b0 += kHbBags) {
    // --- A: H cleared; the gradients' per-column maximum -----------------
    for (int q = threadIdx.x; q < kHotMaxK * kHbHStride / 2; q += kHbThreads)
      reinterpret_cast<double2*>(&s_H[0][0])[q] = double2{0.0, 0.0};
    if (gthr) {
      float m = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float a = __builtin_fabsf(dat.g[j]);
        if (a <= 3.402823466e38f) m = a > m ? a : m;
        else bad = true;  // Inf or NaN
      }
      if (m > 0.f) atomicMax(&s_cmax[gc], __float_as_uint(m));
    }
    __syncthreads();

    // --- B: H[slot][bag] += weight of each hot lookup; the gradients scaled
    //        and split into the B operands ----------------------------------
#pragma unroll
    for (int r = 0; r < kHbAhead; ++r)
      if (o_cur.q0 + lk + r * 16 < o_cur.q1) add_lookup(dat.idx[r], WEIGHTED ? dat.w[r] : 1.f);
    for (int32_t q = o_cur.q0 + lk + kHbAhead * 16; q < o_cur.q1; q += 16)  // long bags
      add_lookup(indices[q], WEIGHTED ? psw[q] : 1.f);
    if (gthr) {
      const uint32_t mb = s_cmax[gc];
      if (mb != 0u) {
        const int e = __builtin_amdgcn_frexp_expf(__uint_as_float(mb));  // max in [2^(e-1), 2^e)
        if (!gset) {
          gsc = 5 - e;
          gset = true;
        } else if (e + gsc > 15) {
          bad = true;  // 1024 times the column's first largest: beyond f16 after scaling
        }
      }
      half8 h, l;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = __builtin_ldexpf(dat.g[j], gsc);
        h[j] = (_Float16)x;
        l[j] = (_Float16)((x - (float)h[j]) * 2048.f);
      }
      // B[kb*8 + j][i] of k-step gg/2: bag 8*gg + j, column gc = nt*32 + i
      const int bl = (gg & 1) * 32 + (gc & 31);
      *reinterpret_cast<half8*>(&s_gb[0][gg >> 1][gc >> 5][bl][0]) = h;
      *reinterpret_cast<half8*>(&s_gb[1][gg >> 1][gc >> 5][bl][0]) = l;
    }
    __syncthreads();

    // the next tile's loads, in flight during the contraction
    o_cur = o_nxt;
    load_data(b0 + kHbBags, o_cur, dat);
    load_off(b0 + 2 * kHbBags, o_nxt);

    // --- C: the contraction -------------------------------------------------
    if (mine) {
      const double* hrow = &s_H[wave * 32 + i][0];
      float hx[2][8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
          const double2 v = *reinterpret_cast<const double2*>(hrow + ks * 16 + kb * 8 + j);
          hx[ks][j] = (float)v.x;
          hx[ks][j + 1] = (float)v.y;
        }
      if constexpr (WEIGHTED) {
        float hm = 0.f;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int j = 0; j < 8; ++j) hm = fmaxf(hm, __builtin_fabsf(hx[ks][j]));
        hm = fmaxf(hm, __shfl_xor(hm, 32));
        if (hm > 0.f) {
          const int e = __builtin_amdgcn_frexp_expf(hm);
          if (!(hm <= 3.402823466e38f)) bad = true;
          else if (!hset) {
            hsc = 1 - e;  // the slot's first nonzero tile: largest sum in [1, 2)
            hset = true;
          } else if (e + hsc > 15) {
            bad = true;
          }
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        half8 a_hi, a_hs, a_res;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (WEIGHTED) {
            const float x = __builtin_ldexpf(hx[ks][j], hsc);
            const _Float16 h = (_Float16)x;
            a_hi[j] = h;
            a_res[j] = (_Float16)(x - (float)h);
          } else {
            bad |= hx[ks][j] > 2048.f;  // counts are exact in f16 up to 2048
            a_hi[j] = (_Float16)hx[ks][j];
          }
          a_hs[j] = a_hi[j] * (_Float16)(1.f / 2048.f);
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const half8 b_hi = *reinterpret_cast<const half8*>(&s_gb[0][ks][nt][lane][0]);
          const half8 b_lo = *reinterpret_cast<const half8*>(&s_gb[1][ks][nt][lane][0]);
          acc[nt] = mfma32(a_hi, b_hi, acc[nt]);
          acc[nt] = mfma32(a_hs, b_lo, acc[nt]);
          if constexpr (WEIGHTED) acc[nt] = mfma32(a_res, b_hi, acc[nt]);
        }
      }
    }
    for (int d = threadIdx.x; d < D; d += kHbThreads) s_cmax[d] = 0u;  // read in B, done
    __syncthreads();
  }

  // Column scales to LDS, then the unscaled partials of this segment.
  if (gthr && gg == 0) s_gsc[gc] = gsc;
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (any_bad) {
    if (threadIdx.x == 0) atomicOr(&hot_flag[t], 1);
    return;
  }
  if (!mine) return;
  float* __restrict__ out =
      hot_parts + ((int64_t)t * gridDim.x + seg) * kHotMaxK * D + (int64_t)wave * 32 * D;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int row = 8 * (r / 4) + 4 * kb + (r % 4);   // slot within this wave's block
    const int rs = WEIGHTED ? __shfl(hsc, row) : 0;   // that slot's scale (lane row holds it)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int d = nt * 32 + i;
      out[(int64_t)row * D + d] = __builtin_ldexpf(acc[nt][r], -(rs + s_gsc[d]));
    }
  }
}

}  // namespace

// Opt-in (TBE_FLAG_HOT_BACKWARD): at T=32, B=131072, D=128 bf16 on one
// MI355X the contraction takes 2.16 ms and the remaining long runs' chunks
// 0.85 ms, against 2.05 ms for the chunk path alone.
bool hot_backward_eligible(const Problem& p) {
  return p.hot_bwd_asked && !p.no_hot && p.path == TBE_PATH_GENERIC && p.wdtype != TBE_F32 &&
         p.D % 32 == 0 && p.D <= 128 && p.B >= 1 && p.cap_long > 0;
}

int32_t hot_backward_segments(const Problem& p) {
  // about one workgroup per CU over all tables, and at least 16 tiles (512
  // bags) per segment, so that small batches keep few partials
  const int64_t tiles = ((int64_t)p.B + kHbBags - 1) / kHbBags;
  int64_t nseg = (256 + p.T - 1) / p.T;
  const int64_t by_tiles = (tiles + 15) / 16;
  if (nseg > by_tiles) nseg = by_tiles;
  return (int32_t)(nseg < 1 ? 1 : nseg);
}

hipError_t launch_bwd_hot(const Problem& p, const float* grad, const int32_t* indices,
                          const int32_t* offsets, const float* psw, const int32_t* hot_rows,
                          const int32_t* tinfo, float* hot_parts, int32_t* hot_flag,
                          hipStream_t s) {
  const int32_t nseg = hot_backward_segments(p);
  const int64_t tiles = ((int64_t)p.B + kHbBags - 1) / kHbBags;
  const int32_t seg_bags = (int32_t)(((tiles + nseg - 1) / nseg) * kHbBags);
  const dim3 grid((unsigned)nseg, (unsigned)p.T);
#define TBE_HOT(WGT, NTT)                                                                   \
  hipLaunchKernelGGL((bwd_hot_kernel<WGT, NTT>), grid, dim3(kHbThreads), 0, s, grad, indices, \
                     offsets, psw, hot_rows, tinfo, hot_parts, hot_flag, p.T, p.B, p.ld, seg_bags)
#define TBE_HOT_NT(WGT)                       \
  switch (p.D / 32) {                         \
    case 1: TBE_HOT(WGT, 1); break;           \
    case 2: TBE_HOT(WGT, 2); break;           \
    case 3: TBE_HOT(WGT, 3); break;           \
    default: TBE_HOT(WGT, 4); break;          \
  }
  if (p.weighted) {
    TBE_HOT_NT(true)
  } else {
    TBE_HOT_NT(false)
  }
#undef TBE_HOT_NT
#undef TBE_HOT
  return hipGetLastError();
}

}  // namespace tbe
