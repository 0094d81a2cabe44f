// Row-wise Adagrad step shared by the generic and small-table paths (page 1:
// "exact row-wise Adagrad", one update per touched row):
//     m' = m + (1/D) * sum_d g_d^2,   w' = w - lr * g / (sqrt(m') + eps)
// in the accumulator precision (float for f16/bf16 weights, double for f32).
#pragma once

#include "device.h"

namespace tbe {

// One row held by the G lanes of a slot (every lane of
// the slot holds its V*PMAX elements of g). The updated row and state are
// written once per step, so they are streamed past L2.
template <typename WT, typename ACC, int V, int PMAX>
__device__ __forceinline__ void adagrad_row(WT* __restrict__ wrow, float* __restrict__ mrow,
                                            ACC (&g)[PMAX][V], int col, int G, int P, int D,
                                            ACC lr, ACC eps) {
  using RAW = typename raw_vec<WT, V>::type;
  ACC sq = (ACC)0;
#pragma unroll
  for (int p = 0; p < PMAX; ++p)
#pragma unroll
    for (int v = 0; v < V; ++v) sq += g[p][v] * g[p][v];
  sq = group_sum<ACC>(sq, G);
  const ACC m1 = (ACC)(*mrow) + sq / (ACC)D;
  const ACC scale = lr / (sqrt(m1) + eps);
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
    const int e = (p * G + col) * V;
    if (p < P && e < D) {
      const RAW raw = load_vec<WT, V>(wrow + e);
      ACC w[V];
      unpack<WT, V, ACC>(raw, w);
      RAW outv;
      WT* o = reinterpret_cast<WT*>(&outv);
#pragma unroll
      for (int v = 0; v < V; ++v) store_w(&o[v], w[v] - g[p][v] * scale);
      store_stream(reinterpret_cast<RAW*>(wrow + e), outv);
    }
  }
  if (col == 0) store_stream(mrow, (float)m1);
}

// The same step split in two, so that the row's weights and state can be
// loaded before its gradient is complete (their latency then overlaps the
// gradient gather).
template <typename WT, int V, int PMAX>
struct RowState {
  typename raw_vec<WT, V>::type w[PMAX];
  float m;
};

template <typename WT, int V, int PMAX>
__device__ __forceinline__ void load_row_state(const WT* __restrict__ wrow,
                                               const float* __restrict__ mrow, int col, int G,
                                               int P, int D, RowState<WT, V, PMAX>& st) {
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
    const int e = (p * G + col) * V;
    if (p < P && e < D) st.w[p] = load_vec<WT, V>(wrow + e);
  }
  st.m = *mrow;
}

template <typename WT, typename ACC, int V, int PMAX>
__device__ __forceinline__ void apply_row_state(WT* __restrict__ wrow, float* __restrict__ mrow,
                                                const RowState<WT, V, PMAX>& st,
                                                ACC (&g)[PMAX][V], int col, int G, int P, int D,
                                                ACC lr, ACC eps) {
  using RAW = typename raw_vec<WT, V>::type;
  ACC sq = (ACC)0;
#pragma unroll
  for (int p = 0; p < PMAX; ++p)
#pragma unroll
    for (int v = 0; v < V; ++v) sq += g[p][v] * g[p][v];
  sq = group_sum<ACC>(sq, G);
  const ACC m1 = (ACC)st.m + sq / (ACC)D;
  const ACC scale = lr / (sqrt(m1) + eps);
#pragma unroll
  for (int p = 0; p < PMAX; ++p) {
    const int e = (p * G + col) * V;
    if (p < P && e < D) {
      ACC w[V];
      unpack<WT, V, ACC>(st.w[p], w);
      RAW outv;
      WT* o = reinterpret_cast<WT*>(&outv);
#pragma unroll
      for (int v = 0; v < V; ++v) store_w(&o[v], w[v] - g[p][v] * scale);
      store_stream(reinterpret_cast<RAW*>(wrow + e), outv);
    }
  }
  if (col == 0) store_stream(mrow, (float)m1);
}

}  // namespace tbe
