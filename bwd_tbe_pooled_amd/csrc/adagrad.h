// Row-wise Adagrad step shared by the generic and small-table paths (page 1:
// "exact row-wise Adagrad", one update per touched row):
//     m' = m + (1/D) * sum_d g_d^2,   w' = w - lr * g / (sqrt(m') + eps)
// in the accumulator precision (float for f16/bf16 weights, double for f32).
#pragma once

#include "device.h"

namespace tbe {

// One row held by the G lanes of a slot (every lane of
// the slot holds its V*PMAX elements of g). Plain stores.
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
      *reinterpret_cast<RAW*>(wrow + e) = outv;
    }
  }
  if (col == 0) *mrow = (float)m1;
}

}  // namespace tbe
