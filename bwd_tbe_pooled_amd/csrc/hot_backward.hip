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
// is one dense contraction per table, tiled over 16-bag tiles and split over
// the batch into segments (one workgroup of four waves each, two per CU). The
// chunk path keeps the other long runs; the apply then reduces each hot row's
// segment partials in segment order (deterministic) and applies its Adagrad
// step.
//
// Per tile (its gradients, indices and weights loaded during the previous
// tile's contraction):
//  A. build: the cells of H the last tile set are cleared by the threads that
//     set them; 16 threads per bag add each hot lookup's weight into
//     H[slot][bag] (the slot through the LDS hash, two lookups probing
//     together) with f32 LDS atomics: all adds to one cell come from its
//     bag's 16 threads, which sit in one wave, in a fixed order of
//     instructions and lanes, so the sums are the same from run to run; two
//     threads per gradient column scale it by its power-of-two scale and
//     split it into f16 hi and lo (the B operands); then the next tile's
//     loads are issued;
//  B. wave w multiplies hot slots 64w..64w+63 (two 32-row blocks) by the tile
//     on v_mfma_f32_32x32x16_f16, accumulating in f32.
//
// Precision: each gradient column is scaled by a power of two set by its
// first tile with a nonzero value (largest magnitude then in [2^4, 2^5)); x =
// g * 2^s is split into hi = f16(x) and lo = f16((x - hi) * 2^11), and the
// product takes H_hi * hi + (H_hi * 2^-11) * lo (+ H_res * hi when weighted,
// H_res = f16(H' - H_hi) with H' = H times its slot's power-of-two scale, set
// by the slot's first nonzero tile so that its largest sum lands in [1, 2)).
// That is about 2^-22 relative per term for every gradient down to 2^-18 of
// its column's scale. A tile whose largest gradient or weight sum reaches
// 2^12 once scaled moves its column's or slot's scale back to the ranges
// above (the accumulated values are multiplied by the exact power of two
// between the two scales before the tile's products), so f16 never overflows. A gradient or
// weight sum that is not finite, or a count above 2048, flags the table
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

constexpr int kHbThreads = 256;             // 4 waves: wave w owns hot slots 64w..64w+63
constexpr int kHbWaves = kHbThreads / kWave;
static_assert(kHbWaves * 64 == kHotMaxK, "two 32-slot blocks per wave");
constexpr int kHbBags = 16;                 // bags per tile: one k-step of the 32x32x16 product
static_assert(kHbBags * 16 == kHbThreads, "16 threads per bag");
static_assert(kHbThreads == 2 * 128, "two threads per gradient column of 128");
constexpr int kHbHStride = kHbBags + 4;     // floats per H row: 16-byte aligned, banks rotate
constexpr int kHbAhead = 2;                 // lookups per thread loaded a tile ahead

template <bool WEIGHTED, int NT>
__global__ __launch_bounds__(kHbThreads) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_hot_kernel(
    const float* __restrict__ grad, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ offsets, const float* __restrict__ psw,
    const int32_t* __restrict__ hot_rows, const int32_t* __restrict__ tinfo,
    float* __restrict__ hot_parts, int32_t* __restrict__ hot_flag, int32_t T, int32_t B,
    int64_t ld, int32_t seg_bags, int64_t N) {
  constexpr int D = NT * 32;
  __shared__ __align__(16) int32_t s_key[kHotHash];  // packed hash: row << 8 | slot
  __shared__ __align__(16) float s_H[kHotMaxK][kHbHStride];   // weight sums
  __shared__ __align__(16) _Float16 s_gb[2][NT][kWave][8];    // [hi, lo][nt][lane][j]
  __shared__ int32_t s_gsc[D];    // per column: scale exponent, for the unscaling
  __shared__ int32_t s_gdelta[D]; // per column: exponent change in this tile (rescaled columns)
  __shared__ int32_t s_resc[2];   // per tile parity: some column was rescaled
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
  for (int q = threadIdx.x; q < kHotMaxK * kHbHStride / 4; q += kHbThreads)
    reinterpret_cast<float4*>(&s_H[0][0])[q] = float4{0.f, 0.f, 0.f, 0.f};
  if (threadIdx.x == 0) {
    s_nhot = 0;
    s_resc[0] = s_resc[1] = 0;
  }
  for (int d = threadIdx.x; d < D; d += kHbThreads) s_gdelta[d] = 0;
  __syncthreads();
  hot_hash_insert_packed(s_key, hr, kHotMaxK);
  if (threadIdx.x < kHotMaxK && hr[threadIdx.x] >= 0) atomicMax(&s_nhot, (int)threadIdx.x + 1);
  __syncthreads();
  const int n_hot = s_nhot;  // slots 0..n_hot-1 are taken
  if (n_hot == 0) return;    // the whole workgroup: the table has no hot row
  const bool mine = wave * 64 < n_hot;  // this wave owns a taken slot

  // Lookups: 16 threads per bag of the tile, thread k of bag lb taking its
  // lookups k, k+16, ... Gradients: threads 2c and 2c+1 hold column c of bags
  // 0..7 and 8..15 (lane kb*32 + c%32 of block c/32 of the B operand).
  const int lb = threadIdx.x >> 4, lk = threadIdx.x & 15;
  const int gc = threadIdx.x >> 1, gh = threadIdx.x & 1;
  const bool gthr = gc < D;
  int gsc = 0;        // scale of column gc (the same in both threads of a column)
  bool gset = false;
  int hsc[2] = {0, 0};  // scales of hot slots 64*wave + 32*mb + i (weighted)
  bool hset[2] = {false, false};
  bool bad = false;

  float16v acc[2][NT];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mb][nt][r] = 0.f;

  // Loads through buffer resources at 32-bit byte offsets (the launcher
  // checks the bounds): a lookup past its bag or a gradient row past the
  // tile reads as zero from an offset past the resource's end.
  constexpr uint32_t kNoRow = 0x80000000u;
  const __amdgpu_buffer_rsrc_t ridx = make_rsrc(indices, (uint32_t)N * 4u);
  const __amdgpu_buffer_rsrc_t rpsw = make_rsrc(WEIGHTED ? (const void*)psw : (const void*)indices, (uint32_t)N * 4u);
  const uint32_t ldb = (uint32_t)ld * 4u;                              // bytes per gradient row
  const uint32_t goff = (uint32_t)(gh * 8) * ldb + (uint32_t)gc * 4u;  // row 8*gh, column gc
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
    // gthr is the same in a whole wave (a wave's threads hold 32 columns)
    if (b0 < b_end && gthr) {
      const __amdgpu_buffer_rsrc_t rg =
          make_rsrc(grad + (int64_t)b0 * ld + (int64_t)t * D, (uint32_t)tile_nb(b0) * ldb);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x.g[j] = __builtin_bit_cast(float,
                                    __builtin_amdgcn_raw_buffer_load_b32(rg, goff + j * ldb, 0, 0));
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) x.g[j] = 0.f;
    }
#pragma unroll
    for (int r = 0; r < kHbAhead; ++r) {
      const int32_t q = o.q0 + lk + r * 16;
      const uint32_t off = q < o.q1 ? (uint32_t)q * 4u : kNoRow;
      x.idx[r] = __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(ridx, off, 0, 0));
      if constexpr (WEIGHTED)
        x.w[r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rpsw, off, 0, 0));
      else
        x.w[r] = 1.f;
    }
  };
  auto slot_of = [&](int32_t idx) {
    int s0, s1;
    hot_hash_find2_packed(s_key, (uint32_t)idx < Et ? idx : 0, true, 0, false, s0, s1);
    return s0;
  };

  // H cells this thread added to in the last tile, cleared before the next
  // tile's adds (by this same thread, or, after a bag longer than the
  // lookups staged ahead, by its bag's 16 threads over the whole column)
  int zslot[kHbAhead] = {-1, -1};
  bool zcol = false;
  bool gdirty = false;  // this thread wrote s_gdelta[gc] in the last tile
  int par = 0;          // tile parity: which s_resc flag this tile sets

  Off o_cur, o_nxt;
  Data dat;
  load_off(b_begin, o_cur);
  load_data(b_begin, o_cur, dat);
  load_off(b_begin + kHbBags, o_nxt);
  for (int32_t b0 = b_begin; b0 < b_end; b0 += kHbBags, par ^= 1) {
    // The build issues before the contraction on a SIMD that holds waves of
    // both phases (the two workgroups of a CU drift apart): the next tile's
    // loads and the LDS atomics start sooner, and the matrix-core work of the
    // other workgroup fills the gaps (1.36 -> 1.30 ms on the Zipf-skewed
    // batch; raising the contraction instead gave 1.31 ms).
    __builtin_amdgcn_s_setprio(1);
    // --- build: the last tile's H cells cleared, H[slot][bag] += weight of
    //     each hot lookup, the gradients scaled and split into the B operands
    if (zcol) {
      for (int s = lk; s < kHotMaxK; s += 16) s_H[s][lb] = 0.f;
    } else {
#pragma unroll
      for (int r = 0; r < kHbAhead; ++r)
        if (zslot[r] >= 0) s_H[zslot[r]][lb] = 0.f;
    }
    if (threadIdx.x == 0) s_resc[par ^ 1] = 0;  // read in the last tile's contraction
    if (gdirty) s_gdelta[gc] = 0;
    gdirty = false;
    // both staged lookups probe the hash together
    static_assert(kHbAhead == 2, "two staged lookups per thread");
    {
      const bool v0 = o_cur.q0 + lk < o_cur.q1, v1 = o_cur.q0 + lk + 16 < o_cur.q1;
      hot_hash_find2_packed(s_key, (uint32_t)dat.idx[0] < Et ? dat.idx[0] : 0, v0,
                            (uint32_t)dat.idx[1] < Et ? dat.idx[1] : 0, v1, zslot[0], zslot[1]);
    }
    {
      // the largest |g| as the largest bit pattern (finite values only)
      uint32_t mbits = 0u;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t a = __float_as_uint(dat.g[j]) & 0x7fffffffu;
        mbits = a > mbits ? a : mbits;
      }
      mbits = max(mbits, (uint32_t)__shfl_xor((int)mbits, 1));  // the column's other eight bags
      bad |= mbits >= 0x7f800000u;                             // Inf or NaN
      {
        // the column's first nonzero tile sets its scale (largest then in
        // [2^4, 2^5)); a later tile 2^12 above the scale moves it, and its
        // accumulators follow before this tile's products. Selects, no branch
        // but the rare rescale's.
        const int e = __builtin_amdgcn_frexp_expf(__uint_as_float(mbits));  // max in [2^(e-1), 2^e)
        const bool nz = mbits != 0u && mbits < 0x7f800000u;
        const bool resc = nz && gset && e + gsc > 12;
        const int nsc = 5 - e;
        if (resc && gh == 0) {
          s_gdelta[gc] = nsc - gsc;
          s_resc[par] = 1;
          gdirty = true;
        }
        gsc = nz && (!gset || resc) ? nsc : gsc;
        gset = gset || nz;
      }
      if (gthr) {
        half8 h, l;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = __builtin_ldexpf(dat.g[j], gsc);
          h[j] = (_Float16)x;
          l[j] = (_Float16)((x - (float)h[j]) * 2048.f);
        }
        // B[kb*8 + j][i] of block nt: bag 8*gh + j, column gc = nt*32 + i
        const int bl = gh * 32 + (gc & 31);
        *reinterpret_cast<half8*>(&s_gb[0][gc >> 5][bl][0]) = h;
        *reinterpret_cast<half8*>(&s_gb[1][gc >> 5][bl][0]) = l;
      }
    }
    // A cell's adds all come from the 16 threads of its bag, which are in one
    // wave, in a fixed order of instructions and lanes, so the f32 sums do not
    // change from run to run.
#pragma unroll
    for (int r = 0; r < kHbAhead; ++r) {
      if (zslot[r] >= 0) {
        if constexpr (WEIGHTED) bad |= !(__builtin_fabsf(dat.w[r]) <= 3.402823466e38f);
        atomicAdd(&s_H[zslot[r]][lb], dat.w[r]);
      }
    }
    zcol = o_cur.q1 - o_cur.q0 > kHbAhead * 16;
    for (int32_t q = o_cur.q0 + lk + kHbAhead * 16; q < o_cur.q1; q += 16) {  // long bags
      const int sl = slot_of(indices[q]);
      if (sl >= 0) {
        const float w = WEIGHTED ? psw[q] : 1.f;
        bad |= !(__builtin_fabsf(w) <= 3.402823466e38f);
        atomicAdd(&s_H[sl][lb], w);
      }
    }
    // the next tile's loads, issued as soon as this tile's registers are
    // consumed: in flight during the barrier and the contraction
    o_cur = o_nxt;
    load_data(b0 + kHbBags, o_cur, dat);
    load_off(b0 + 2 * kHbBags, o_nxt);
    __syncthreads();

    // --- the contraction ----------------------------------------------------
    __builtin_amdgcn_s_setprio(0);
    if (mine) {
      float hx[2][8];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const float* hrow = &s_H[wave * 64 + mb * 32 + i][kb * 8];
        const float4 v0 = *reinterpret_cast<const float4*>(hrow);
        const float4 v1 = *reinterpret_cast<const float4*>(hrow + 4);
        hx[mb][0] = v0.x; hx[mb][1] = v0.y; hx[mb][2] = v0.z; hx[mb][3] = v0.w;
        hx[mb][4] = v1.x; hx[mb][5] = v1.y; hx[mb][6] = v1.z; hx[mb][7] = v1.w;
      }
      // columns rescaled in this tile's build (workgroup-uniform flag)
      if (s_resc[par]) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int dg = s_gdelta[nt * 32 + i];
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[mb][nt][r] = __builtin_ldexpf(acc[mb][nt][r], dg);
        }
      }
      half8 a_hi[2], a_hs[2], a_res[2];
      int dsc[2] = {0, 0};  // exponent change of this lane's slot in block mb
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        if constexpr (WEIGHTED) {
          float hm = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j) hm = fmaxf(hm, __builtin_fabsf(hx[mb][j]));
          hm = fmaxf(hm, __shfl_xor(hm, 32));
          // the slot's first nonzero tile sets its scale (largest sum then in
          // [1, 2)); a later tile 2^12 above it moves the scale
          const int e = __builtin_amdgcn_frexp_expf(hm);
          const bool fin = hm <= 3.402823466e38f;
          bad |= !fin;
          const bool nz = hm > 0.f && fin;
          const bool resc = nz && hset[mb] && e + hsc[mb] > 12;
          const int nsc = 1 - e;
          dsc[mb] = resc ? nsc - hsc[mb] : 0;
          hsc[mb] = nz && (!hset[mb] || resc) ? nsc : hsc[mb];
          hset[mb] = hset[mb] || nz;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if constexpr (WEIGHTED) {
            const float x = __builtin_ldexpf(hx[mb][j], hsc[mb]);
            const _Float16 h = (_Float16)x;
            a_hi[mb][j] = h;
            a_res[mb][j] = (_Float16)(x - (float)h);
          } else {
            bad |= hx[mb][j] > 2048.f;  // counts are exact in f16 up to 2048
            a_hi[mb][j] = (_Float16)hx[mb][j];
          }
          a_hs[mb][j] = a_hi[mb][j] * (_Float16)(1.f / 2048.f);
        }
      }
      if constexpr (WEIGHTED) {
        // a rescaled slot's accumulator rows follow its new scale (lane `row`
        // holds the change of slot row; a wave-uniform test, rarely taken)
        if (__ballot(dsc[0] != 0 || dsc[1] != 0) != 0) {
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int d = __shfl(dsc[mb], 8 * (r / 4) + 4 * kb + (r % 4));
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) acc[mb][nt][r] = __builtin_ldexpf(acc[mb][nt][r], d);
            }
        }
      }
      half8 b_hi[NT], b_lo[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        b_hi[nt] = *reinterpret_cast<const half8*>(&s_gb[0][nt][lane][0]);
        b_lo[nt] = *reinterpret_cast<const half8*>(&s_gb[1][nt][lane][0]);
      }
      // products in rounds over the eight independent accumulators
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mb][nt] = mfma32(a_hi[mb], b_hi[nt], acc[mb][nt]);
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) acc[mb][nt] = mfma32(a_hs[mb], b_lo[nt], acc[mb][nt]);
      if constexpr (WEIGHTED) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mb][nt] = mfma32(a_res[mb], b_hi[nt], acc[mb][nt]);
      }
    }
    __syncthreads();  // H and the B operands read: the next tile may overwrite them
  }

  // Column scales to LDS, then the unscaled partials of this segment.
  if (gthr && gh == 0) s_gsc[gc] = gsc;
  const int any_bad = __syncthreads_or(bad ? 1 : 0);
  if (any_bad) {
    if (threadIdx.x == 0) atomicOr(&hot_flag[t], 1);
    return;
  }
  if (!mine) return;
  float* __restrict__ out =
      hot_parts + ((int64_t)t * gridDim.x + seg) * kHotMaxK * D + (int64_t)wave * 64 * D;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r / 4) + 4 * kb + (r % 4);      // slot within this 32-slot block
      const int rs = WEIGHTED ? __shfl(hsc[mb], row) : 0;  // that slot's scale (lane row holds it)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int d = nt * 32 + i;
        out[(int64_t)(mb * 32 + row) * D + d] = __builtin_ldexpf(acc[mb][nt][r], -(rs + s_gsc[d]));
      }
    }
}

}  // namespace

// Opt-in (TBE_FLAG_HOT_BACKWARD): at T=32, B=131072, D=128 bf16 on one
// MI355X the plan and the contraction take about 1.3 ms and the remaining long
// runs' chunks 0.43 ms, against 2.03 ms for the chunk path alone.
bool hot_backward_eligible(const Problem& p) {
  // 32-bit byte offsets: the lookups below 2^29, a 16-row gradient tile below 2^31 bytes;
  // the packed hash: tables of fewer than 2^24 - 1 rows
  return p.hot_bwd_asked && !p.no_hot && p.path == TBE_PATH_GENERIC && p.wdtype != TBE_F32 &&
         p.D % 32 == 0 && p.D <= 128 && p.B >= 1 && p.cap_long > 0 && p.N < (int64_t(1) << 29) &&
         p.ld < (int64_t(1) << 25) && p.max_rows < (int64_t(1) << 24) - 1;
}

int32_t hot_backward_segments(const Problem& p) {
  // two workgroups per CU over all tables, never more (a workgroup past the
  // ones that fit at once would start only when others end, and double the
  // time), and at least 32 tiles (512 bags) per segment, so that small
  // batches keep few partials
  const int64_t tiles = ((int64_t)p.B + kHbBags - 1) / kHbBags;
  int64_t nseg = kHotBwdWorkgroups / p.T;
  const int64_t by_tiles = (tiles + 31) / 32;
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
                     offsets, psw, hot_rows, tinfo, hot_parts, hot_flag, p.T, p.B, p.ld, seg_bags, p.N)
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
