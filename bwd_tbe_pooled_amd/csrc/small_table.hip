// Small-table path (page 1, "Forward state reuse and preprocessing" and
// checklist item 2: E <= 64, 64 <= D <= 128, L >= 64, f16 weights, no
// per-sample weights). With so few rows, a bag is better described by its row
// histogram H[bag][e] than by its index list, and pooling becomes a dense
// contraction:
//     forward   out[b, t-block] = H_t[b, :] . W_t            ([B x 64] x [64 x D])
//     backward  G_t = H_t^T . grad_t                         ([64 x B] x [B x D])
// both on the matrix cores (v_mfma_f32_32x32x16_f16: f16 inputs, f32
// accumulation). Counts are exact in f16 up to 2048. The backward splits the
// f32 upstream gradient into hi = f16(g) and lo = f16((g - hi) * 2^11) and
// contracts H with both (the lo product with H * 2^-11, exact in f16), which
// compensates the f16 rounding of g to about 2^-22 relative. The forward saves
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
constexpr int kBagTile = 64;            // bags per forward workgroup / backward stage
constexpr uint32_t kExactCount = 2048;  // counts exact in f16 up to here

__device__ __forceinline__ float16v mfma32(half8 a, half8 b, float16v c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ _Float16 w_half(const f16_t* W, int64_t idx) {
  return __builtin_bit_cast(_Float16, W[idx].bits);
}

// Build the counts of bags [b0, b0+nb) of table t in LDS (uint32 [64][64]).
__device__ void count_bags(uint32_t (*H)[kSmallE], const int32_t* __restrict__ indices,
                           const int32_t* __restrict__ offsets, int64_t bag0, int nb) {
  for (int i = threadIdx.x; i < kBagTile * kSmallE; i += kThreads) (&H[0][0])[i] = 0;
  __syncthreads();
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  for (int bl = wave; bl < nb; bl += kThreads / kWave) {
    const int32_t a = offsets[bag0 + bl], e = offsets[bag0 + bl + 1];
    for (int32_t j = a + lane; j < e; j += kWave)
      atomicAdd(&H[bl][indices[j] & (kSmallE - 1)], 1u);
  }
  __syncthreads();
}

template <bool WITH_OUT, bool WITH_HIST>
__global__ __launch_bounds__(kThreads) void small_forward_kernel(
    const f16_t* __restrict__ W, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ toff,
    const int32_t* __restrict__ trows, float* __restrict__ out, uint8_t* __restrict__ hist,
    int32_t* __restrict__ counts, int32_t T, int32_t B, int32_t D) {
  __shared__ uint32_t H[kBagTile][kSmallE];
  __shared__ uint32_t s_max;
  const int32_t t = blockIdx.y;
  const int32_t b0 = blockIdx.x * kBagTile;
  const int nb = B - b0 < kBagTile ? B - b0 : kBagTile;
  const int64_t bag0 = (int64_t)t * B + b0;
  if (threadIdx.x == 0) s_max = 0;
  count_bags(H, indices, offsets, bag0, nb);

  // Save the counts (uint8, saturating) and find the tile's largest count.
  uint32_t local_max = 0;
  for (int q = threadIdx.x; q < nb * (kSmallE / 4); q += kThreads) {
    const int bl = q / (kSmallE / 4), e4 = (q % (kSmallE / 4)) * 4;
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t c = H[bl][e4 + k];
      local_max = c > local_max ? c : local_max;
      packed |= (c > 255u ? 255u : c) << (8 * k);
    }
    if constexpr (WITH_HIST)
      *reinterpret_cast<uint32_t*>(hist + (bag0 + bl) * kSmallE + e4) = packed;
  }
  if (local_max > 0) atomicMax(&s_max, local_max);
  __syncthreads();
  if (WITH_HIST && threadIdx.x == 0 && s_max > 255u) atomicOr(&counts[4], 1);
  if constexpr (!WITH_OUT) return;

  const int32_t Et = trows[t];
  const f16_t* Wt = W + (int64_t)toff[t] * D;
  float* ot = out + (int64_t)t * D;
  const int64_t ostride = (int64_t)T * D;

  if (s_max > kExactCount) {
    // Counts beyond f16's exact range: plain f32 dot products over the rows.
    for (int q = threadIdx.x; q < nb * D; q += kThreads) {
      const int bl = q / D, d = q % D;
      float acc = 0.f;
      for (int e = 0; e < Et && e < kSmallE; ++e)
        acc += (float)H[bl][e] * (float)w_half(Wt, (int64_t)e * D + d);
      ot[(int64_t)(b0 + bl) * ostride + d] = acc;
    }
    return;
  }

  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i = lane & 31, kb = lane >> 5;
  const int mt = wave & 1;             // bag rows mt*32 .. +32
  const int NT = (D + 31) / 32;        // 32-column tiles
  float16v acc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
#pragma unroll
  for (int ks = 0; ks < kSmallE / 16; ++ks) {
    half8 a;
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = (_Float16)(float)H[mt * 32 + i][ks * 16 + kb * 8 + j];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int nt = (wave >> 1) + 2 * q;
      if (nt < NT) {
        const int d = nt * 32 + i;
        half8 bv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int e = ks * 16 + kb * 8 + j;
          bv[j] = (e < Et && d < D) ? w_half(Wt, (int64_t)e * D + d) : (_Float16)0.f;
        }
        acc[q] = mfma32(a, bv, acc[q]);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int nt = (wave >> 1) + 2 * q;
    if (nt >= NT) continue;
    const int d = nt * 32 + i;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 8 * (r / 4) + 4 * kb + (r % 4);
      const int bl = mt * 32 + row;
      if (bl < nb && d < D) ot[(int64_t)(b0 + bl) * ostride + d] = acc[q][r];
    }
  }
}

// One workgroup per (table, split of the batch): partial G = H^T . grad over
// the split's bags, written to partials[(t*splits + s)][64][D], and the
// split's per-row counts to part_counts[(t*splits + s)][64].
__global__ __launch_bounds__(kThreads) void small_backward_kernel(
    const float* __restrict__ grad, const uint8_t* __restrict__ hist,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ offsets, float* __restrict__ partials,
    int32_t* __restrict__ part_counts, int32_t T, int32_t B, int32_t D, int32_t splits,
    int32_t bags_per_split) {
  __shared__ uint32_t H[kBagTile][kSmallE];
  __shared__ uint32_t s_max;
  __shared__ float s_part[kSmallE][129];  // fallback accumulators (D <= 128)
  const int32_t t = blockIdx.y;
  const int32_t s = blockIdx.x;
  const int32_t sb0 = s * bags_per_split;
  const int32_t sb1 = sb0 + bags_per_split < B ? sb0 + bags_per_split : B;
  const bool recount = counts[4] != 0;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int i = lane & 31, kb = lane >> 5;
  const int nt = wave;                 // this wave's 32 columns
  const int NT = (D + 31) / 32;
  const int d = nt * 32 + i;
  const float* gt = grad + (int64_t)t * D;
  const int64_t gstride = (int64_t)T * D;

  float16v acc[2];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[q][r] = 0.f;
  for (int q = threadIdx.x; q < kSmallE * 129; q += kThreads) (&s_part[0][0])[q] = 0.f;
  uint32_t row_count = 0;  // thread e < 64 accumulates the count of row e

  for (int32_t b0 = sb0; b0 < sb1; b0 += kBagTile) {
    const int nb = sb1 - b0 < kBagTile ? sb1 - b0 : kBagTile;
    const int64_t bag0 = (int64_t)t * B + b0;
    __syncthreads();
    if (threadIdx.x == 0) s_max = 0;
    if (recount) {
      count_bags(H, indices, offsets, bag0, nb);
    } else {
      for (int q = threadIdx.x; q < kBagTile * (kSmallE / 4); q += kThreads) {
        const int bl = q / (kSmallE / 4), e4 = (q % (kSmallE / 4)) * 4;
        const uint32_t packed =
            bl < nb ? *reinterpret_cast<const uint32_t*>(hist + (bag0 + bl) * kSmallE + e4) : 0u;
#pragma unroll
        for (int k = 0; k < 4; ++k) H[bl][e4 + k] = (packed >> (8 * k)) & 0xffu;
      }
      __syncthreads();
    }
    uint32_t local_max = 0;
    for (int q = threadIdx.x; q < nb * kSmallE; q += kThreads) {
      const uint32_t c = (&H[0][0])[q];
      local_max = c > local_max ? c : local_max;
    }
    if (local_max > kExactCount) atomicMax(&s_max, local_max);
    if (threadIdx.x < kSmallE)
      for (int bl = 0; bl < nb; ++bl) row_count += H[bl][threadIdx.x];
    __syncthreads();

    if (s_max > kExactCount) {
      // f32 fallback for counts beyond f16's exact range.
      for (int q = threadIdx.x; q < kSmallE * D; q += kThreads) {
        const int e = q / D, dd = q % D;
        float a = 0.f;
        for (int bl = 0; bl < nb; ++bl)
          a += (float)H[bl][e] * gt[(int64_t)(b0 + bl) * gstride + dd];
        s_part[e][dd] += a;
      }
      continue;
    }
    if (nt >= NT) continue;
#pragma unroll
    for (int ks = 0; ks < kBagTile / 16; ++ks) {
      // B operand: the gradient of 8 bags at column d, split into hi/lo halves.
      half8 hi, lo;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int bl = ks * 16 + kb * 8 + j;
        const float g = (bl < nb && d < D) ? gt[(int64_t)(b0 + bl) * gstride + d] : 0.f;
        const _Float16 h = (_Float16)g;
        hi[j] = h;
        lo[j] = (_Float16)((g - (float)h) * 2048.f);
      }
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        half8 a_hi, a_lo;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float c = (float)H[ks * 16 + kb * 8 + j][mt * 32 + i];
          a_hi[j] = (_Float16)c;
          a_lo[j] = (_Float16)(c * (1.f / 2048.f));
        }
        acc[mt] = mfma32(a_hi, hi, acc[mt]);
        acc[mt] = mfma32(a_lo, lo, acc[mt]);
      }
    }
  }
  __syncthreads();
  float* pt = partials + ((int64_t)t * splits + s) * kSmallE * D;
  if (nt < NT) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int e = mt * 32 + 8 * (r / 4) + 4 * kb + (r % 4);
        if (d < D) s_part[e][d] += acc[mt][r];
      }
  }
  __syncthreads();
  for (int q = threadIdx.x; q < kSmallE * D; q += kThreads) pt[q] = s_part[q / D][q % D];
  if (threadIdx.x < kSmallE)
    part_counts[((int64_t)t * splits + s) * kSmallE + threadIdx.x] = (int32_t)row_count;
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
  // About 1024 workgroups over the whole problem, at least 256 bags each.
  int64_t per_table = 1024 / (T > 0 ? T : 1);
  if (per_table < 1) per_table = 1;
  int64_t max_splits = (B + 255) / 256;
  if (max_splits < 1) max_splits = 1;
  return (int)(per_table < max_splits ? per_table : max_splits);
}

hipError_t launch_small_forward(const Problem& p, const void* W, const int32_t* indices,
                                const int32_t* offsets, const int32_t* tinfo, float* out,
                                uint8_t* hist, int32_t* counts, hipStream_t s) {
  hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(64), 0, s, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (p.B == 0) return hipSuccess;
  const dim3 grid((unsigned)((p.B + kBagTile - 1) / kBagTile), (unsigned)p.T);
  const int32_t* toff = tinfo;
  const int32_t* trows = tinfo + p.T;
  if (out && hist)
    hipLaunchKernelGGL((small_forward_kernel<true, true>), grid, dim3(kThreads), 0, s,
                       (const f16_t*)W, indices, offsets, toff, trows, out, hist, counts, p.T,
                       p.B, p.D);
  else if (out)
    hipLaunchKernelGGL((small_forward_kernel<true, false>), grid, dim3(kThreads), 0, s,
                       (const f16_t*)W, indices, offsets, toff, trows, out, hist, counts, p.T,
                       p.B, p.D);
  else
    hipLaunchKernelGGL((small_forward_kernel<false, true>), grid, dim3(kThreads), 0, s,
                       (const f16_t*)W, indices, offsets, toff, trows, out, hist, counts, p.T,
                       p.B, p.D);
  return hipGetLastError();
}

hipError_t launch_small_backward(const Problem& p, const float* grad, const uint8_t* hist,
                                 const int32_t* counts, const int32_t* indices,
                                 const int32_t* offsets, float* partials, int32_t* part_counts,
                                 hipStream_t s) {
  const int splits = p.small_splits;
  int32_t per = (p.B + splits - 1) / splits;
  const dim3 grid((unsigned)splits, (unsigned)p.T);
  hipLaunchKernelGGL(small_backward_kernel, grid, dim3(kThreads), 0, s, grad, hist, counts, indices,
                     offsets, partials, part_counts, p.T, p.B, p.D, splits, per);
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
