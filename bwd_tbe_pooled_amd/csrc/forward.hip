// Generic forward: pooled (weighted) sums of embedding rows over T tables in
// one launch (page 1, backward section's notation; page 2 section 1, one fused
// lookup for all features instead of one launch per feature).
//
//   out[b, t*D + d] = sum_{j in bag (t,b)} s_j * W[toff[t] + indices[j], d]
//
// Mapping on gfx950: a wave owns NS = 64/G consecutive bags, one per "row
// slot" of G lanes; a slot reads a row with G lanes x V elements per pass
// (16-byte loads for 2-byte weights at D = 128: G = 16, V = 8), keeps UNROLL
// rows in flight and accumulates in registers (float for f16/bf16 weights,
// double for f32 weights, page 1 checklist item 1). The bags' indices and
// per-sample weights are staged once per wave in LDS with coalesced loads.
// Bags are table-major, and workgroups are remapped so that each XCD walks a
// contiguous range of bags, i.e. a subset of the tables: the hot rows of those
// tables stay in that XCD's L2.
#include "device.h"
#include "internal.h"

namespace tbe {

namespace {

constexpr int kFwdThreads = 256;
constexpr int kFwdWaves = kFwdThreads / kWave;
constexpr int kStage = 256;  // staged lookups per wave and window

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// CHECK: the bounds check fused into the gather (an index outside its table
// is read as row 0 and sets TBE_ERROR_INDEX in *err).
template <typename WT, int V, int PMAX, bool WEIGHTED, bool CHECK>
__global__ __launch_bounds__(kFwdThreads) void fwd_pool_kernel(
    const WT* __restrict__ W, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ offsets, const float* __restrict__ psw,
    const int32_t* __restrict__ toff, float* __restrict__ out, int32_t T, int32_t B, int32_t D,
    int32_t G, int32_t log2G, int32_t P, int64_t nbags, int64_t nblocks, int64_t ld,
    int32_t* __restrict__ err) {
  using ACC = typename acc_of<WT>::type;
  using RAW = typename raw_vec<WT, V>::type;
  constexpr int UNROLL = PMAX == 1 ? 4 : 1;
  __shared__ int32_t s_idx[kFwdWaves][kStage];
  __shared__ float s_w[kFwdWaves][WEIGHTED ? kStage : 1];

  const int64_t lb = xcd_logical_block(nblocks);
  if (lb < 0) return;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int slot = lane >> log2G;
  const int col = lane & (G - 1);
  const int NS = kWave >> log2G;

  const int64_t first_bag = (lb * kFwdWaves + wave) * NS;
  if (first_bag >= nbags) return;
  const int64_t last_bag = first_bag + NS < nbags ? first_bag + NS : nbags;  // exclusive
  const int64_t my_bag = first_bag + slot;
  const bool has_bag = my_bag < last_bag;
  const int32_t my_begin = has_bag ? offsets[my_bag] : 0;
  const int32_t my_end = has_bag ? offsets[my_bag + 1] : 0;
  const int32_t J0 = offsets[first_bag];
  const int32_t J1 = offsets[last_bag];
  const int32_t t = has_bag ? (int32_t)(my_bag / B) : 0;
  const int32_t b = has_bag ? (int32_t)(my_bag - (int64_t)t * B) : 0;
  const WT* __restrict__ Wt = W + (int64_t)(has_bag ? toff[t] : 0) * D;
  const uint32_t Et = CHECK ? (uint32_t)(has_bag ? toff[T + t] : 1) : 0u;  // tinfo rows follow
  bool bad = false;

  ACC acc[PMAX][V];
#pragma unroll
  for (int p = 0; p < PMAX; ++p)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[p][v] = (ACC)0;

  for (int32_t w0 = J0; w0 < J1; w0 += kStage) {
    const int32_t wn = J1 - w0 < kStage ? J1 - w0 : kStage;
    wave_lds_sync();
    for (int i = lane; i < wn; i += kWave) {
      s_idx[wave][i] = indices[w0 + i];
      if constexpr (WEIGHTED) s_w[wave][i] = psw[w0 + i];
    }
    wave_lds_sync();
    const int32_t lo = my_begin > w0 ? my_begin : w0;
    const int32_t hi = my_end < w0 + wn ? my_end : w0 + wn;
    for (int32_t j = lo; j < hi; j += UNROLL) {
      RAW buf[UNROLL][PMAX];
      float sc[UNROLL];
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const int32_t jj = j + u;
        const bool ok = jj < hi;
        const int32_t li = ok ? jj - w0 : 0;
        int32_t idx = s_idx[wave][li];
        if constexpr (CHECK) {
          const bool out = ok && (uint32_t)idx >= Et;
          bad |= out;
          idx = out ? 0 : idx;
        }
        if constexpr (WEIGHTED) sc[u] = ok ? s_w[wave][li] : 0.f;
        else sc[u] = ok ? 1.f : 0.f;
        const WT* row = Wt + (int64_t)idx * D;
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
          const int e = (p * G + col) * V;
          if (ok && p < P && e < D) buf[u][p] = load_vec<WT, V>(row + e);
          else buf[u][p] = RAW{};
        }
      }
#pragma unroll
      for (int u = 0; u < UNROLL; ++u) {
        const ACC s = (ACC)sc[u];
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
          ACC x[V];
          unpack<WT, V, ACC>(buf[u][p], x);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[p][v] += s * x[v];
        }
      }
    }
  }

  if constexpr (CHECK) {
    if (__ballot(bad) != 0 && lane == 0) atomicOr(err, (int32_t)TBE_ERROR_INDEX);
  }
  if (!has_bag) return;
  float* o = out + (int64_t)b * ld + (int64_t)t * D;
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
    const int e = (p * G + col) * V;
    if (p < P && e < D) {
      // written once: streamed past L2, which keeps the hot rows instead
      typename vec_bytes<V * 4>::type ov;
      float* of = reinterpret_cast<float*>(&ov);
#pragma unroll
      for (int v = 0; v < V; ++v) of[v] = (float)acc[p][v];
      store_stream(reinterpret_cast<decltype(ov)*>(o + e), ov);
    }
  }
}

template <typename WT, int V, int PMAX>
hipError_t launch_typed(const Problem& p, const RowShape& rs, const void* W, const int32_t* indices,
                        const int32_t* offsets, const float* psw, const int32_t* toff, float* out,
                        hipStream_t s) {
  const int NS = kWave / rs.G;
  const int64_t bags_per_block = (int64_t)NS * kFwdWaves;
  const int64_t nblocks = (p.nbags + bags_per_block - 1) / bags_per_block;
  if (nblocks == 0) return hipSuccess;
  const dim3 grid((unsigned)xcd_grid(nblocks));
#define TBE_FWD(WGT, CHK)                                                                      \
  hipLaunchKernelGGL((fwd_pool_kernel<WT, V, PMAX, WGT, CHK>), grid, dim3(kFwdThreads), 0, s,  \
                     (const WT*)W, indices, offsets, psw, toff, out, p.T, p.B, p.D, rs.G,      \
                     rs.log2G, rs.P, p.nbags, nblocks, p.ld, p.err)
  if (psw) {
    if (p.err) TBE_FWD(true, true);
    else TBE_FWD(true, false);
  } else {
    if (p.err) TBE_FWD(false, true);
    else TBE_FWD(false, false);
  }
#undef TBE_FWD
  return hipGetLastError();
}

template <typename WT>
hipError_t launch_for_type(const Problem& p, const void* W, const int32_t* indices,
                           const int32_t* offsets, const float* psw, const int32_t* toff,
                           float* out, hipStream_t s) {
  const RowShape rs = row_shape(p.D, 8);
#define TBE_FWD_CASE(VV)                                                                     \
  if (rs.V == VV) {                                                                          \
    if (rs.P == 1) return launch_typed<WT, VV, 1>(p, rs, W, indices, offsets, psw, toff, out, s); \
    return launch_typed<WT, VV, 4>(p, rs, W, indices, offsets, psw, toff, out, s);           \
  }
  TBE_FWD_CASE(8)
  TBE_FWD_CASE(4)
  TBE_FWD_CASE(2)
  TBE_FWD_CASE(1)
#undef TBE_FWD_CASE
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_forward_pool(const Problem& p, const void* W, const int32_t* indices,
                               const int32_t* offsets, const float* psw, const int32_t* tinfo,
                               float* out, hipStream_t s) {
  switch (p.wdtype) {
    case TBE_F32: return launch_for_type<float>(p, W, indices, offsets, psw, tinfo, out, s);
    case TBE_F16: return launch_for_type<f16_t>(p, W, indices, offsets, psw, tinfo, out, s);
    case TBE_BF16: return launch_for_type<bf16_t>(p, W, indices, offsets, psw, tinfo, out, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tbe
