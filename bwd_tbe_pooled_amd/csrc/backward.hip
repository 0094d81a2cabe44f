// Backward with the optimizer applied in place (page 1, backward section): for
// each run (unique (table,row)), sum the upstream gradient rows of all its
// lookups, each scaled by the lookup's per-sample weight on weighted tables,
// then apply exactly one row-wise Adagrad step to the row:
//     m' = m + mean_d(g_d^2),   w' = w - lr * g / (sqrt(m') + eps).
//
// Three kernels, following the page's routing by segment length:
//   short  (SL < S): one row slot (G lanes of a wave) owns a whole run: it
//          gathers the run's gradient rows, accumulates in registers, applies
//          Adagrad and stores the row with plain stores; no atomics, since no
//          other slot touches the row.
//   long   (SL >= S): one wave per chunk of C lookups writes the chunk's
//          partial sum to the workspace.
//   apply  one wave per long run reduces its chunk partials in a fixed order
//          and applies Adagrad.
// Accumulation is float for f16/bf16 weights and double for f32 weights (page
// 1, checklist item 1); nothing is accumulated with atomics, so results are
// deterministic run to run.
//
// The gradient row of lookup k is grad[b, t*D .. t*D+D-1] where sorted_bag[k]
// = t*B + b; every lookup of a run shares its table t.
//
// Memory access on gfx950:
// - Gradient rows are f32 and read at random; a lane reads 16 contiguous bytes
//   and consecutive lanes read consecutive bytes, so each load instruction
//   covers whole 128-byte lines (D = 128: 16 lanes x 16 B x 2 passes per row).
//   Random 512-byte rows served from L2 move about twice as fast this way as
//   with 32 bytes per lane split over two instructions.
// - Long-run chunks are executed in a schedule, not in chunk order: chunks are
//   bucketed per XCD (a contiguous block of tables per XCD), and within an
//   XCD's list taken two tables at a time, each pair ordered by the batch
//   position of the middle of the chunk's lookups. Lookups of a run are in batch order,
//   so concurrent chunks on one XCD read gradient rows of nearby bags (and
//   the two tables' rows of one bag are adjacent in memory), which its L2
//   keeps. Each chunk still writes its own partial, so the result does
//   not depend on the schedule.
#include <algorithm>
#include <type_traits>

#include "adagrad.h"
#include "block_scan.h"
#include "device.h"
#include "internal.h"

namespace tbe {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <typename ACC, int V, int PMAX>
__device__ __forceinline__ void zero_acc(ACC (&acc)[PMAX][V]) {
#pragma unroll
  for (int p = 0; p < PMAX; ++p)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[p][v] = (ACC)0;
}

// All row slots of a wave accumulate sorted slots [k0, k1) of one run of table
// t: slot s takes k0+s, k0+s+NS, ...; bag ids and weights of 64 slots at a
// time are loaded coalesced and handed to the slots with shuffles. On return
// every slot holds the wave's sum (fixed butterfly over the slots).
// Rows in flight per slot: UNROLL (4 by default, 8 in the long kernels at
// D = 128).
template <int V, int PMAX, typename ACC, bool WEIGHTED, int UNROLL = (PMAX <= 2 ? 4 : 1)>
__device__ __forceinline__ void wave_accumulate(const float* __restrict__ grad,
                                                const int32_t* __restrict__ sorted_bag,
                                                const float* __restrict__ sorted_psw, int32_t k0,
                                                int32_t k1, int64_t ld, int32_t B, int32_t D,
                                                int G, int log2G, int P, ACC (&acc)[PMAX][V]) {
  using GRAW = typename raw_vec<float, V>::type;
  const int lane = lane_id();
  const int slot = lane >> log2G;
  const int col = lane & (G - 1);
  const int NS = kWave >> log2G;
  const int32_t t = sorted_bag[k0] / B;
  const float* __restrict__ gt = grad + (int64_t)t * D;
  const int32_t tB = t * B;
  zero_acc<ACC, V, PMAX>(acc);
  // bag ids and weights of the next 64 slots are loaded while the current
  // 64 rows are gathered
  int32_t nx_bag = k0 + lane < k1 ? sorted_bag[k0 + lane] : tB;
  float nx_s = 0.f;
  if constexpr (WEIGHTED) nx_s = k0 + lane < k1 ? sorted_psw[k0 + lane] : 0.f;
  for (int32_t base = k0; base < k1; base += kWave) {
    const int n = k1 - base < kWave ? k1 - base : kWave;
    const int32_t my_bag = nx_bag;
    const float my_s = nx_s;
    {
      const int32_t nk = base + kWave + lane;
      nx_bag = nk < k1 ? sorted_bag[nk] : tB;
      if constexpr (WEIGHTED) nx_s = nk < k1 ? sorted_psw[nk] : 0.f;
    }
    for (int r0 = 0; r0 < n; r0 += NS * UNROLL) {
      GRAW buf[UNROLL][PMAX];
      float sc[UNROLL];
#pragma unroll
      for (int uu = 0; uu < UNROLL; ++uu) {
        const int r = r0 + uu * NS + slot;
        const bool ok = r < n;
        const int32_t bag = __shfl(my_bag, r & (kWave - 1));
        if constexpr (WEIGHTED) {
          const float sv = __shfl(my_s, r & (kWave - 1));
          sc[uu] = ok ? sv : 0.f;
        } else {
          sc[uu] = ok ? 1.f : 0.f;
        }
        // Slots past the end of the range load nothing: their zero weight
        // would turn an Inf or NaN in some other bag's row into a NaN here.
        const float* row = gt + (int64_t)(ok ? bag - tB : 0) * ld;
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
          const int e = (p * G + col) * V;
          if (ok && p < P && e < D) buf[uu][p] = load_vec<float, V>(row + e);
          else buf[uu][p] = GRAW{};
        }
      }
#pragma unroll
      for (int uu = 0; uu < UNROLL; ++uu) {
        const ACC s = (ACC)sc[uu];
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
          const float* x = reinterpret_cast<const float*>(&buf[uu][p]);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[p][v] += s * (ACC)x[v];
        }
      }
    }
  }
#pragma unroll
  for (int p = 0; p < PMAX; ++p)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[p][v] = across_slots_sum<ACC>(acc[p][v], G);
}

// Short runs. A wave takes 64 entries of the short-run list at a time:
// - runs of at most kTinyMax lookups are owned by one row slot each (four runs
//   in flight per wave, all their rows loaded at once);
// - longer short runs are owned by the whole wave in turn, four slots sharing
//   the rows, so a run of a few hundred lookups does not hold three idle slots.
// Either way one owner updates the row, with plain stores. The row's weights
// and state are loaded before its gradient gather completes.
constexpr int kTinyMax = 4;

template <typename WT, int V, int PMAX, bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void bwd_short_kernel(
    WT* __restrict__ W, float* __restrict__ mom, const float* __restrict__ grad,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ short_runs,
    const int32_t* __restrict__ run_keys, const int32_t* __restrict__ run_offsets,
    const int32_t* __restrict__ sorted_bag, const float* __restrict__ sorted_psw, int64_t ld,
    int32_t B, int32_t D, int32_t G, int32_t log2G, int32_t P,
    typename acc_of<WT>::type lr, typename acc_of<WT>::type eps) {
  using ACC = typename acc_of<WT>::type;
  using GRAW = typename raw_vec<float, V>::type;
  __shared__ int32_t s_src[kWaves][kWave];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int slot = lane >> log2G;
  const int col = lane & (G - 1);
  const int NS = kWave >> log2G;
  const uint64_t lt = lane == 0 ? 0ull : (~0ull >> (kWave - lane));
  const int64_t n_short = counts[1];
  const int64_t gwave = (int64_t)blockIdx.x * kWaves + wave;
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;

  for (int64_t tile = gwave * kWave; tile < n_short; tile += nwaves * kWave) {
    const int64_t i = tile + lane;
    const bool valid = i < n_short;
    const int32_t u = valid ? short_runs[i] : 0;
    const int32_t k0 = valid ? run_offsets[u] : 0;
    const int32_t k1 = valid ? run_offsets[u + 1] : 0;
    const int32_t key = valid ? run_keys[u] : 0;
    const bool tiny = valid && k1 - k0 <= kTinyMax;
    const uint64_t tmask = __ballot(tiny);
    uint64_t mmask = __ballot(valid && !tiny);
    wave_lds_sync();
    if (tiny) s_src[wave][__popcll(tmask & lt)] = lane;
    wave_lds_sync();

    // tiny runs, one per slot
    const int ntiny = __popcll(tmask);
    for (int q = 0; q < ntiny; q += NS) {
      const bool act = q + slot < ntiny;
      const int src = act ? s_src[wave][q + slot] : 0;
      const int32_t a = __shfl(k0, src), e = __shfl(k1, src), rkey = __shfl(key, src);
      RowState<WT, V, PMAX> st;
      if (act) load_row_state<WT, V, PMAX>(W + (int64_t)rkey * D, mom + rkey, col, G, P, D, st);
      // Only the run's own lookups are loaded: a run of one lookup issues one
      // row load, not kTinyMax loads of the same row.
      int32_t bag[kTinyMax];
      float sc[kTinyMax];
      bool ok[kTinyMax];
#pragma unroll
      for (int r = 0; r < kTinyMax; ++r) {
        ok[r] = act && a + r < e;
        bag[r] = act ? sorted_bag[ok[r] ? a + r : a] : 0;
        if constexpr (WEIGHTED) sc[r] = ok[r] ? sorted_psw[a + r] : 0.f;
        else sc[r] = ok[r] ? 1.f : 0.f;
      }
      const int32_t t = bag[0] / (B > 0 ? B : 1);
      const float* __restrict__ gt = grad + (int64_t)t * D;
      GRAW buf[kTinyMax][PMAX];
#pragma unroll
      for (int r = 0; r < kTinyMax; ++r) {
        const float* row = gt + (int64_t)(bag[r] - t * B) * ld;
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
          const int ee = (p * G + col) * V;
          if (ok[r] && p < P && ee < D) buf[r][p] = load_vec<float, V>(row + ee);
          else buf[r][p] = GRAW{};
        }
      }
      ACC acc[PMAX][V];
      zero_acc<ACC, V, PMAX>(acc);
#pragma unroll
      for (int r = 0; r < kTinyMax; ++r) {
        const ACC sv = (ACC)sc[r];
#pragma unroll
        for (int p = 0; p < PMAX; ++p) {
          const float* x = reinterpret_cast<const float*>(&buf[r][p]);
#pragma unroll
          for (int v = 0; v < V; ++v) acc[p][v] += sv * (ACC)x[v];
        }
      }
      if (act)  // whole slots are active or not, so the slot's reductions stay within it
        apply_row_state<WT, ACC, V, PMAX>(W + (int64_t)rkey * D, mom + rkey, st, acc, col, G, P,
                                          D, lr, eps);
    }

    // longer short runs, one per wave
    while (mmask) {
      const int src = __ffsll((unsigned long long)mmask) - 1;
      mmask &= mmask - 1;
      const int32_t a = __shfl(k0, src), e = __shfl(k1, src), rkey = __shfl(key, src);
      RowState<WT, V, PMAX> st;
      if (slot == 0) load_row_state<WT, V, PMAX>(W + (int64_t)rkey * D, mom + rkey, col, G, P, D, st);
      ACC acc[PMAX][V];
      wave_accumulate<V, PMAX, ACC, WEIGHTED>(grad, sorted_bag, sorted_psw, a, e, ld, B, D, G,
                                              log2G, P, acc);
      if (slot == 0)
        apply_row_state<WT, ACC, V, PMAX>(W + (int64_t)rkey * D, mom + rkey, st, acc, col, G, P,
                                          D, lr, eps);
    }
  }
}

// Per-XCD work queue of the long kernels: a wave takes the next item of its
// XCD's list, so the chunks in flight stay a narrow window of the list. A
// fixed stride lets waves that draw slow chunks fall behind, which widens the
// set of gradient rows the XCD's L2 must hold: at T=32, B=131072, D=128 the
// long kernel took 3.05 ms with a fixed stride and 2.74 ms with the queue at
// two workgroups per CU (one MI355X).
constexpr int kQueueStride = 32;  // ints between the XCDs' counters: one 128-byte line each
// Every wave adds one more after the list is exhausted; a list within a few
// hundred items of 2^31 would wrap the counter, so callers also stop on a
// negative value (all valid items are below 2^31).
__device__ __forceinline__ int64_t next_item(int32_t* q) {
  int32_t it = 0;
  if (lane_id() == 0) it = __hip_atomic_fetch_add(q, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return (int64_t)__shfl(it, 0);
}

// Rows in flight per slot in the long kernels (the short kernel keeps 4).
template <int PMAX>
constexpr int kLongUnroll = PMAX <= 2 ? 8 : 1;

// Workgroup w serves the schedule list of XCD (w mod 8); the grid is a
// multiple of 8, so every list is served whatever the dispatch order.
template <int V, int PMAX, typename ACC, bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void bwd_long_kernel(
    const float* __restrict__ grad, const int32_t* __restrict__ chunk_run,
    const int32_t* __restrict__ chunk_start, const int32_t* __restrict__ run_offsets,
    const int32_t* __restrict__ sorted_bag, const float* __restrict__ sorted_psw,
    const int32_t* __restrict__ order, const int32_t* __restrict__ list_begin,
    int32_t* __restrict__ queue, ACC* __restrict__ partials, int64_t ld, int32_t B, int32_t D,
    int32_t C, int32_t G, int32_t log2G, int32_t P) {
  const int lane = lane_id();
  const int slot = lane >> log2G;
  const int col = lane & (G - 1);
  const int x = blockIdx.x % kXcds;
  const int64_t first = list_begin[x];
  const int64_t n_items = list_begin[x + 1] - first;
  for (;;) {
    const int64_t it = next_item(queue + x * kQueueStride);
    if (it < 0 || it >= n_items) break;  // past the end (or wrapped past 2^31)
    const int32_t c = order[first + it];
    const int32_t u = chunk_run[c];
    const int32_t k0 = chunk_start[c];
    const int32_t kend = run_offsets[u + 1];
    const int32_t k1 = k0 + C < kend ? k0 + C : kend;
    ACC acc[PMAX][V];
    wave_accumulate<V, PMAX, ACC, WEIGHTED, kLongUnroll<PMAX>>(grad, sorted_bag, sorted_psw, k0,
                                                               k1, ld, B, D, G, log2G, P, acc);
    if (slot == 0) {
      ACC* out = partials + (int64_t)c * D;
#pragma unroll
      for (int p = 0; p < PMAX; ++p) {
        const int e = (p * G + col) * V;
        if (p < P && e < D) {
#pragma unroll
          for (int v = 0; v < V; ++v) out[e + v] = acc[p][v];
        }
      }
    }
  }
}

// Sum of the n partials part[0], part[stride], ... of one long run (its
// chunks' partials, or its segment partials from the hot rows' contraction),
// then its Adagrad step. Slot s sums partials s, s+NS, ... in ascending order
// and the slots are combined by a fixed butterfly, so the order is the same
// every call; the apply kernel and the fused long kernel both reduce through
// this function with the same row shape, so they give the same bits.
template <typename WT, typename ACC, int V, int PMAX>
__device__ __forceinline__ void reduce_apply_run(WT* __restrict__ W, float* __restrict__ mom,
                                                 const ACC* __restrict__ part, int64_t stride,
                                                 int32_t n, int32_t key, int32_t D, int G,
                                                 int log2G, int P, ACC lr, ACC eps) {
  const int lane = lane_id();
  const int slot = lane >> log2G;
  const int col = lane & (G - 1);
  const int NS = kWave >> log2G;
  using RAW = typename raw_vec<ACC, V>::type;
  constexpr int UNROLL = 4;  // chunks in flight per slot: a run's chain of loads is the latency
  ACC acc[PMAX][V];
  zero_acc<ACC, V, PMAX>(acc);
  for (int32_t cb = slot; cb < n; cb += NS * UNROLL) {
    RAW buf[UNROLL][PMAX];
#pragma unroll
    for (int uu = 0; uu < UNROLL; ++uu) {
      const int32_t c = cb + uu * NS;
      const ACC* src = part + (int64_t)(c < n ? c : 0) * stride;
#pragma unroll
      for (int p = 0; p < PMAX; ++p) {
        const int e = (p * G + col) * V;
        if (p < P && e < D) buf[uu][p] = load_vec<ACC, V>(src + e);
        else buf[uu][p] = RAW{};  // columns past the row stay zero (they enter the sum of squares)
      }
    }
#pragma unroll
    for (int uu = 0; uu < UNROLL; ++uu) {
      if (cb + uu * NS >= n) break;
#pragma unroll
      for (int p = 0; p < PMAX; ++p) {
        const ACC* x = reinterpret_cast<const ACC*>(&buf[uu][p]);
#pragma unroll
        for (int v = 0; v < V; ++v) acc[p][v] += x[v];
      }
    }
  }
#pragma unroll
  for (int p = 0; p < PMAX; ++p)
#pragma unroll
    for (int v = 0; v < V; ++v) acc[p][v] = across_slots_sum<ACC>(acc[p][v], G);
  if (slot == 0)
    adagrad_row<WT, ACC, V, PMAX>(W + (int64_t)key * D, mom + key, acc, col, G, P, D, lr, eps);
}

// A hot run (run_slot[l] = t*256 + slot, its table not flagged back to the
// chunk path) sums its nseg segment partials hot_parts[t][seg][slot][:], the
// other long runs their chunks' partials.
template <typename WT, int V, int PMAX>
__global__ __launch_bounds__(kThreads) void bwd_apply_kernel(
    WT* __restrict__ W, float* __restrict__ mom, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ long_runs, const int32_t* __restrict__ long_chunk_begin,
    const int32_t* __restrict__ run_keys, const typename acc_of<WT>::type* __restrict__ partials,
    const int32_t* __restrict__ run_slot, const int32_t* __restrict__ hot_flag,
    const typename acc_of<WT>::type* __restrict__ hot_parts, int32_t nseg, int32_t D, int32_t G,
    int32_t log2G, int32_t P, typename acc_of<WT>::type lr, typename acc_of<WT>::type eps) {
  using ACC = typename acc_of<WT>::type;
  const int64_t n_long = counts[2];
  const int64_t gwave = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  const int64_t nwaves = (int64_t)gridDim.x * kWaves;
  for (int64_t l = gwave; l < n_long; l += nwaves) {
    const int32_t q = run_slot ? run_slot[l] : -1;
    const int32_t key = run_keys[long_runs[l]];
    if (q >= 0 && hot_flag[q / 256] == 0) {
      const int32_t t = q / 256, sl = q % 256;
      reduce_apply_run<WT, ACC, V, PMAX>(W, mom, hot_parts + ((int64_t)t * nseg * 256 + sl) * D,
                                         (int64_t)256 * D, nseg, key, D, G, log2G, P, lr, eps);
    } else {
      const int32_t c0 = long_chunk_begin[l];
      reduce_apply_run<WT, ACC, V, PMAX>(W, mom, partials + (int64_t)c0 * D, D,
                                         long_chunk_begin[l + 1] - c0, key, D, G, log2G, P, lr,
                                         eps);
    }
  }
}

// The long path in one launch: each chunk writes its partial, makes it visible
// device-wide (agent-scope release) and counts itself in on its run; the wave
// that arrives last (acquire) reduces the run's partials and applies Adagrad.
// No wave waits for another, so the kernel cannot stall on a missing chunk.
// arrivals[first chunk of the run] must be zero at launch. On gfx950 the
// agent-scope release writes back the XCD's L2 and the acquire invalidates it.
template <typename WT, int V, int PMAX, bool WEIGHTED>
__global__ __launch_bounds__(kThreads) void bwd_long_fused_kernel(
    WT* __restrict__ W, float* __restrict__ mom, const float* __restrict__ grad,
    const int32_t* __restrict__ chunk_run, const int32_t* __restrict__ chunk_start,
    const int32_t* __restrict__ run_offsets, const int32_t* __restrict__ run_keys,
    const int32_t* __restrict__ sorted_bag, const float* __restrict__ sorted_psw,
    const int32_t* __restrict__ order, const int32_t* __restrict__ list_begin,
    int32_t* __restrict__ queue, typename acc_of<WT>::type* __restrict__ partials,
    int32_t* __restrict__ arrivals, int64_t ld, int32_t B, int32_t D, int32_t C, int32_t G,
    int32_t log2G, int32_t P, typename acc_of<WT>::type lr, typename acc_of<WT>::type eps) {
  using ACC = typename acc_of<WT>::type;
  const int lane = lane_id();
  const int slot = lane >> log2G;
  const int col = lane & (G - 1);
  const int x = blockIdx.x % kXcds;
  const int64_t first = list_begin[x];
  const int64_t n_items = list_begin[x + 1] - first;
  for (;;) {
    const int64_t it = next_item(queue + x * kQueueStride);
    if (it < 0 || it >= n_items) break;  // past the end (or wrapped past 2^31)
    const int32_t c = order[first + it];
    const int32_t u = chunk_run[c];
    const int32_t k0 = chunk_start[c];
    const int32_t ks = run_offsets[u];
    const int32_t kend = run_offsets[u + 1];
    const int32_t k1 = k0 + C < kend ? k0 + C : kend;
    ACC acc[PMAX][V];
    wave_accumulate<V, PMAX, ACC, WEIGHTED, kLongUnroll<PMAX>>(grad, sorted_bag, sorted_psw, k0,
                                                               k1, ld, B, D, G, log2G, P, acc);
    if (slot == 0) {
      ACC* out = partials + (int64_t)c * D;
#pragma unroll
      for (int p = 0; p < PMAX; ++p) {
        const int e = (p * G + col) * V;
        if (p < P && e < D) {
#pragma unroll
          for (int v = 0; v < V; ++v) out[e + v] = acc[p][v];
        }
      }
    }
    // The whole wave executes the fence, so every lane's partial stores are
    // complete and visible device-wide before lane 0's increment is issued.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const int32_t c_first = c - (k0 - ks) / C;
    const int32_t nch = (kend - ks + C - 1) / C;
    int32_t prev = 0;
    if (lane == 0)
      prev = __hip_atomic_fetch_add(arrivals + c_first, 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    prev = __shfl(prev, 0);
    if (prev != nch - 1) continue;  // another chunk of the run is still to come
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    reduce_apply_run<WT, ACC, V, PMAX>(W, mom, partials + (int64_t)c_first * D, D, nch, run_keys[u], D,
                                       G, log2G, P, lr, eps);
  }
}

// --- long-chunk schedule: bucket = (XCD of the chunk's table block, group of
// kSchedTables tables within the block, middle bag of the chunk); counting
// sort of chunk ids into buckets. An XCD thus walks its tables two at a time,
// each pair in bag order. A chunk is placed by the middle of its bag span:
// a dense chunk's span is short either way, and a sparse one then runs while
// the dense chunks around it read the middle of its rows, not its first ones
// (2.04 ms against 2.26 ms by first bag, 2.24 ms by last bag and 2.08 ms at a
// quarter of the span, with the queue below). With T=32, E=2M, D=128, B=131072 and Zipf-Mandelbrot rows the long
// kernel took 3.04 ms with pairs, 3.19 ms with the whole 4-table block at
// once, 3.38 ms one table at a time, 4.1 ms when every XCD took an eighth of
// each table's bags (tables in order) and 5.2 ms with an eighth of the bags
// of all tables at once (one MI355X, fixed-stride waves, first-bag order).
// With the work queue and middle-bag order: 2.04 ms with pairs, 2.27 ms with
// the block, 2.08 ms one table at a time. ------------------------------------
constexpr int kSchedBuckets = 4096;  // per XCD
constexpr int kSchedTables = 2;      // tables of a block walked together

__global__ void sched_zero_kernel(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// With the backward of the hot rows (hot_min non-null), the chunks of a hot
// run (length >= hot_min of its table) are left out of the lists, unless the
// table's hot_flag sent its hot runs back to the chunk path.
__global__ __launch_bounds__(256) void sched_count_kernel(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ chunk_start,
    const int32_t* __restrict__ sorted_bag, const int32_t* __restrict__ chunk_run,
    const int32_t* __restrict__ run_offsets, int32_t C, int32_t B, int32_t T,
    const int32_t* __restrict__ hot_min, const int32_t* __restrict__ hot_flag,
    int32_t* __restrict__ hist, int32_t* __restrict__ bucket_of, int32_t* __restrict__ arrivals) {
  const int64_t n = counts[3];
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n;
       c += (int64_t)gridDim.x * blockDim.x) {
    arrivals[c] = 0;  // arrival counters of the fused long kernel
    // the chunk's place in batch order: the middle of its bag span
    const int32_t k0 = chunk_start[c];
    const int32_t u = chunk_run[c];
    const int32_t ke = run_offsets[u + 1];
    const int32_t klast = (k0 + C < ke ? k0 + C : ke) - 1;
    const int32_t bag0 = sorted_bag[k0], bag1 = sorted_bag[klast];
    const int32_t bag = bag0 + (bag1 - bag0) / 2;
    const int32_t t = bag / B, b = bag - t * B;
    if (hot_min && ke - run_offsets[u] >= hot_min[t] && hot_flag[t] == 0) {
      bucket_of[c] = -1;  // summed by the hot rows' contraction
      continue;
    }
    int bk;
    if (T % kXcds == 0) {
      // T/8 whole tables per XCD, walked kSchedTables at a time in bag order
      const int x = (int)(((int64_t)t * kXcds) / T);
      const int t0 = (int)(((int64_t)x * T + kXcds - 1) / kXcds);  // first table of block x
      const int t1 = (int)(((int64_t)(x + 1) * T + kXcds - 1) / kXcds);
      const int ngrp = (t1 - t0 + kSchedTables - 1) / kSchedTables;
      const int per = kSchedBuckets / ngrp;  // buckets per table group (0 past 4096 groups)
      const int g = (t - t0) / kSchedTables;
      bk = x * kSchedBuckets + g * per + (int)(((int64_t)b * per) / B);
    } else {
      // Otherwise whole tables per XCD would leave XCDs idle (T < 8) or give
      // some twice the work of others (e.g. 13 tables: blocks of 2 and 1).
      // Each chunk gets a position on the tables laid end to end, t + b / B,
      // scaled to 8 XCDs: XCD x takes positions [x, x + 1), so a table's bags
      // are split over XCDs in proportion, walked in position order.
      const int64_t pos = (((int64_t)t * B + b) * kXcds * kSchedBuckets) / ((int64_t)T * B);
      bk = (int)pos;  // = x * kSchedBuckets + bucket within XCD x
    }
    bucket_of[c] = bk;
    atomicAdd(&hist[bk], 1);
  }
}

// Single workgroup: exclusive scan of the bucket counts in place; list_begin[x]
// = first slot of XCD x's list, list_begin[8] = number of chunks.
__global__ __launch_bounds__(1024) void sched_scan_kernel(int32_t* __restrict__ hist,
                                                          int32_t* __restrict__ list_begin) {
  __shared__ int32_t wsum[16];
  const int32_t tot = block1024_scan_inplace(
      hist, (int64_t)kXcds * kSchedBuckets, wsum, [&](int64_t i, int32_t prefix) {
        if (i % kSchedBuckets == 0) list_begin[i / kSchedBuckets] = prefix;
      });
  if (threadIdx.x == 0) list_begin[kXcds] = tot;
}

__global__ __launch_bounds__(256) void sched_scatter_kernel(const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ bucket_of,
                                                            int32_t* __restrict__ cursor,
                                                            int32_t* __restrict__ order) {
  const int64_t n = counts[3];
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < n;
       c += (int64_t)gridDim.x * blockDim.x) {
    const int32_t bk = bucket_of[c];
    if (bk < 0) continue;
    const int32_t pos = atomicAdd(&cursor[bk], 1);
    order[pos] = (int32_t)c;
  }
}

// Layout of the long-chunk schedule in its workspace (int32 units): chunk
// order, bucket of each chunk, bucket counts, list starts (padded), work-queue
// counters, arrival counters of the fused kernel.
struct SchedLayout {
  int32_t *order, *bucket_of, *hist, *list_begin, *queue, *arrivals;
};
constexpr int kListPad = 64;
inline SchedLayout sched_layout(int32_t* sched, int64_t cap) {
  SchedLayout L;
  L.order = sched;
  L.bucket_of = L.order + cap;
  L.hist = L.bucket_of + cap;
  L.list_begin = L.hist + kXcds * kSchedBuckets;
  L.queue = L.list_begin + kListPad;
  L.arrivals = L.queue + kXcds * kQueueStride;
  return L;
}

inline int64_t persistent_blocks(int64_t work_waves) {
  // Enough workgroups to fill 256 CUs several times over; the kernels stride.
  int64_t cap = 256 * 16;
  int64_t need = (work_waves + kWaves - 1) / kWaves;
  if (need < 1) need = 1;
  return need < cap ? need : cap;
}

template <typename WT, int V, int PMAX>
hipError_t short_typed(const Problem& p, const RowShape& rs, void* W, float* m, const float* grad,
                       const tbe_meta& meta, double lr, double eps, hipStream_t s) {
  using ACC = typename acc_of<WT>::type;
  // One 64-run tile per wave where the grid allows, so the dispatcher
  // balances tiles of very different cost (tiny runs against runs of a few
  // hundred lookups); past 65536 workgroups the waves stride. The run count
  // is only known on the device, and workgroups beyond it exit at once. At
  // T=32, B=131072, D=128 (3.0M short runs, capacity 64M) the kernel took
  // 1.40, 1.30 and 1.30 ms with 4096, 16384 and 65536 workgroups and 2.07 ms
  // with one per tile of the capacity; with uniform rows (46.7M short runs)
  // 12.5, 12.0, 10.5 and 11.1 ms (one MI355X).
  const int64_t tiles = (p.cap_runs + kWave - 1) / kWave;
  const dim3 grid((unsigned)std::max<int64_t>(
      1, std::min<int64_t>(65536, (tiles + kWaves - 1) / kWaves)));
  if (p.weighted)
    hipLaunchKernelGGL((bwd_short_kernel<WT, V, PMAX, true>), grid, dim3(kThreads), 0, s, (WT*)W, m,
                       grad, meta.counts, meta.short_runs, meta.run_keys, meta.run_offsets,
                       meta.sorted_bag, meta.sorted_psw, p.ld, p.B, p.D, rs.G, rs.log2G, rs.P,
                       (ACC)lr, (ACC)eps);
  else
    hipLaunchKernelGGL((bwd_short_kernel<WT, V, PMAX, false>), grid, dim3(kThreads), 0, s, (WT*)W,
                       m, grad, meta.counts, meta.short_runs, meta.run_keys, meta.run_offsets,
                       meta.sorted_bag, meta.sorted_psw, p.ld, p.B, p.D, rs.G, rs.log2G, rs.P,
                       (ACC)lr, (ACC)eps);
  return hipGetLastError();
}

// Three workgroups (twelve waves) per CU. More chunks in flight widen the
// window of bags whose gradient rows the XCD's L2 must hold at once; fewer
// leave too few loads in flight. With T=32, E=2M, D=128, B=131072 and
// Zipf-Mandelbrot rows (287,766 chunks) on one MI355X, with the work queue:
// 2, 3 and 4 workgroups per CU took 2.74, 2.29 and 2.37 ms at 4 rows in
// flight per slot; 3 per CU took 2.62, 2.29 and 2.25 ms at 2, 4 and 8 rows
// (first-bag order). In middle-bag order: 2.29, 2.04 and 2.07 ms at 2, 3 and
// 4 per CU with 8 rows, and 2.09 ms at 3 per CU with 4 rows.
// (Before the queue, with a fixed stride, 1, 2, 3, 4 and 8 per CU took
// 4.87, 3.21, 3.43, 3.80 and 4.01 ms.)
inline dim3 long_grid(const Problem& p) {
  const int64_t per_xcd = 3 * std::max(1, device_cu_count() / kXcds);
  int64_t blocks = (persistent_blocks(p.cap_chunks) + kXcds - 1) / kXcds * kXcds;
  if (blocks > per_xcd * kXcds) blocks = per_xcd * kXcds;
  return dim3((unsigned)blocks);
}

template <typename ACC, int V, int PMAX>
hipError_t long_typed(const Problem& p, const RowShape& rs, const float* grad, const tbe_meta& meta,
                      void* partials, int32_t* sched, hipStream_t s) {
  const SchedLayout L = sched_layout(sched, p.cap_chunks);
  const dim3 grid = long_grid(p);
  if (p.weighted)
    hipLaunchKernelGGL((bwd_long_kernel<V, PMAX, ACC, true>), grid, dim3(kThreads), 0, s, grad,
                       meta.chunk_run, meta.chunk_start, meta.run_offsets, meta.sorted_bag,
                       meta.sorted_psw, L.order, L.list_begin, L.queue, (ACC*)partials, p.ld, p.B,
                       p.D, p.C, rs.G, rs.log2G, rs.P);
  else
    hipLaunchKernelGGL((bwd_long_kernel<V, PMAX, ACC, false>), grid, dim3(kThreads), 0, s, grad,
                       meta.chunk_run, meta.chunk_start, meta.run_offsets, meta.sorted_bag,
                       meta.sorted_psw, L.order, L.list_begin, L.queue, (ACC*)partials, p.ld, p.B,
                       p.D, p.C, rs.G, rs.log2G, rs.P);
  return hipGetLastError();
}

template <typename WT, int V, int PMAX>
hipError_t long_fused_typed(const Problem& p, const RowShape& rs, void* W, float* m,
                            const float* grad, const tbe_meta& meta, void* partials,
                            int32_t* sched, double lr, double eps, hipStream_t s) {
  using ACC = typename acc_of<WT>::type;
  const SchedLayout L = sched_layout(sched, p.cap_chunks);
  const dim3 grid = long_grid(p);
  if (p.weighted)
    hipLaunchKernelGGL((bwd_long_fused_kernel<WT, V, PMAX, true>), grid, dim3(kThreads), 0, s,
                       (WT*)W, m, grad, meta.chunk_run, meta.chunk_start, meta.run_offsets,
                       meta.run_keys, meta.sorted_bag, meta.sorted_psw, L.order, L.list_begin,
                       L.queue, (ACC*)partials, L.arrivals, p.ld, p.B, p.D, p.C, rs.G, rs.log2G, rs.P,
                       (ACC)lr, (ACC)eps);
  else
    hipLaunchKernelGGL((bwd_long_fused_kernel<WT, V, PMAX, false>), grid, dim3(kThreads), 0, s,
                       (WT*)W, m, grad, meta.chunk_run, meta.chunk_start, meta.run_offsets,
                       meta.run_keys, meta.sorted_bag, meta.sorted_psw, L.order, L.list_begin,
                       L.queue, (ACC*)partials, L.arrivals, p.ld, p.B, p.D, p.C, rs.G, rs.log2G, rs.P,
                       (ACC)lr, (ACC)eps);
  return hipGetLastError();
}

template <typename WT, int V, int PMAX>
hipError_t apply_typed(const Problem& p, const RowShape& rs, void* W, float* m,
                       const tbe_meta& meta, const void* partials, const HotBwd& hot, double lr,
                       double eps, hipStream_t s) {
  using ACC = typename acc_of<WT>::type;
  const dim3 grid((unsigned)persistent_blocks(p.cap_long));
  // hot partials are f32: the backward of the hot rows runs for f16/bf16 weights only
  const ACC* hot_parts = std::is_same<ACC, float>::value ? (const ACC*)hot.parts : nullptr;
  hipLaunchKernelGGL((bwd_apply_kernel<WT, V, PMAX>), grid, dim3(kThreads), 0, s, (WT*)W, m,
                     meta.counts, meta.long_runs, meta.long_chunk_begin, meta.run_keys,
                     (const ACC*)partials, hot_parts ? hot.run_slot : nullptr, hot.hot_flag,
                     hot_parts, hot.nseg, p.D, rs.G, rs.log2G, rs.P, (ACC)lr, (ACC)eps);
  return hipGetLastError();
}

#define TBE_DISPATCH_P(VV, RS, CALL_V)          \
  do {                                           \
    if ((RS).P == 1) return CALL_V(VV, 1);       \
    if ((RS).P == 2) return CALL_V(VV, 2);       \
    return CALL_V(VV, 4);                        \
  } while (0)
#define TBE_DISPATCH_V(RS, CALL_V)                           \
  do {                                                       \
    if ((RS).V == 8) TBE_DISPATCH_P(8, RS, CALL_V);          \
    if ((RS).V == 4) TBE_DISPATCH_P(4, RS, CALL_V);          \
    if ((RS).V == 2) TBE_DISPATCH_P(2, RS, CALL_V);          \
    TBE_DISPATCH_P(1, RS, CALL_V);                           \
  } while (0)

// Row shape for f32 gradient rows: 16 bytes per lane, consecutive lanes on
// consecutive bytes (whole lines per load instruction), at most 16 lanes per
// row so that four rows are in flight per wave; wider rows take more passes.
inline RowShape grad_row_shape(int D) {
  int V = 4;
  while (V > 1 && D % V != 0) V >>= 1;
  const int per = (D + V - 1) / V;
  int G = 1, lg = 0;
  while (G < per && G < 16) { G <<= 1; ++lg; }
  int P = (D + G * V - 1) / (G * V);
  while (P > 4 && G < 64) { G <<= 1; ++lg; P = (D + G * V - 1) / (G * V); }
  if (P > 4) return row_shape(D, 8);
  RowShape r;
  r.V = V;
  r.G = G;
  r.log2G = lg;
  r.P = P;
  return r;
}

template <typename WT>
hipError_t short_for(const Problem& p, void* W, float* m, const float* grad, const tbe_meta& meta,
                     double lr, double eps, hipStream_t s) {
  const RowShape rs = grad_row_shape(p.D);
#define CALL(VV, PP) short_typed<WT, VV, PP>(p, rs, W, m, grad, meta, lr, eps, s)
  TBE_DISPATCH_V(rs, CALL);
#undef CALL
}

template <typename ACC>
hipError_t long_for(const Problem& p, const float* grad, const tbe_meta& meta, void* partials,
                    int32_t* sched, hipStream_t s) {
  const RowShape rs = grad_row_shape(p.D);
#define CALL(VV, PP) long_typed<ACC, VV, PP>(p, rs, grad, meta, partials, sched, s)
  TBE_DISPATCH_V(rs, CALL);
#undef CALL
}

template <typename WT>
hipError_t long_fused_for(const Problem& p, void* W, float* m, const float* grad,
                          const tbe_meta& meta, void* partials, int32_t* sched, double lr,
                          double eps, hipStream_t s) {
  const RowShape rs = grad_row_shape(p.D);
#define CALL(VV, PP) \
  long_fused_typed<WT, VV, PP>(p, rs, W, m, grad, meta, partials, sched, lr, eps, s)
  TBE_DISPATCH_V(rs, CALL);
#undef CALL
}

// The apply reduces with the row shape of the long kernel, so that the fused
// long kernel (which reduces in the same wave that accumulated) matches it.
template <typename WT>
hipError_t apply_for(const Problem& p, void* W, float* m, const tbe_meta& meta,
                     const void* partials, const HotBwd& hot, double lr, double eps,
                     hipStream_t s) {
  const RowShape rs = grad_row_shape(p.D);
#define CALL(VV, PP) apply_typed<WT, VV, PP>(p, rs, W, m, meta, partials, hot, lr, eps, s)
  TBE_DISPATCH_V(rs, CALL);
#undef CALL
}

}  // namespace

hipError_t launch_bwd_short(const Problem& p, void* W, float* m, const float* grad,
                            const tbe_meta& meta, const int32_t* tinfo, double lr, double eps,
                            hipStream_t s) {
  (void)tinfo;
  if (p.cap_runs == 0) return hipSuccess;
  switch (p.wdtype) {
    case TBE_F32: return short_for<float>(p, W, m, grad, meta, lr, eps, s);
    case TBE_F16: return short_for<f16_t>(p, W, m, grad, meta, lr, eps, s);
    case TBE_BF16: return short_for<bf16_t>(p, W, m, grad, meta, lr, eps, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_long_schedule(const Problem& p, const tbe_meta& meta, int32_t* sched,
                                const HotBwd& hot, hipStream_t s) {
  if (p.cap_chunks == 0) return hipSuccess;
  const SchedLayout L = sched_layout(sched, p.cap_chunks);
  // bucket counts, list starts and queue counters are contiguous: clear them together
  hipLaunchKernelGGL(sched_zero_kernel, dim3(32), dim3(256), 0, s, L.hist,
                     (int)(L.arrivals - L.hist));
  hipLaunchKernelGGL(sched_count_kernel, dim3(1024), dim3(256), 0, s, meta.counts, meta.chunk_start,
                     meta.sorted_bag, meta.chunk_run, meta.run_offsets, p.C, p.B, p.T, hot.hot_min,
                     hot.hot_flag, L.hist, L.bucket_of, L.arrivals);
  hipLaunchKernelGGL(sched_scan_kernel, dim3(1), dim3(1024), 0, s, L.hist, L.list_begin);
  hipLaunchKernelGGL(sched_scatter_kernel, dim3(1024), dim3(256), 0, s, meta.counts, L.bucket_of,
                     L.hist, L.order);
  return hipGetLastError();
}

hipError_t launch_bwd_long(const Problem& p, const float* grad, const tbe_meta& meta,
                           void* partials, int32_t* sched, hipStream_t s) {
  if (p.cap_chunks == 0) return hipSuccess;
  if (p.wdtype == TBE_F32) return long_for<double>(p, grad, meta, partials, sched, s);
  return long_for<float>(p, grad, meta, partials, sched, s);
}

hipError_t launch_bwd_long_fused(const Problem& p, void* W, float* m, const float* grad,
                                 const tbe_meta& meta, void* partials, int32_t* sched, double lr,
                                 double eps, hipStream_t s) {
  if (p.cap_chunks == 0) return hipSuccess;
  switch (p.wdtype) {
    case TBE_F32: return long_fused_for<float>(p, W, m, grad, meta, partials, sched, lr, eps, s);
    case TBE_F16: return long_fused_for<f16_t>(p, W, m, grad, meta, partials, sched, lr, eps, s);
    case TBE_BF16: return long_fused_for<bf16_t>(p, W, m, grad, meta, partials, sched, lr, eps, s);
  }
  return hipErrorInvalidValue;
}

size_t long_schedule_ints(const Problem& p) {
  // order, bucket of each chunk, bucket counts, list starts, queue counters,
  // arrival counters (sched_layout)
  return 3 * (size_t)p.cap_chunks + kXcds * kSchedBuckets + kListPad + kXcds * kQueueStride;
}

hipError_t launch_bwd_apply(const Problem& p, void* W, float* m, const tbe_meta& meta,
                            const void* partials, const HotBwd& hot, double lr, double eps,
                            hipStream_t s) {
  if (p.cap_long == 0) return hipSuccess;
  switch (p.wdtype) {
    case TBE_F32: return apply_for<float>(p, W, m, meta, partials, hot, lr, eps, s);
    case TBE_F16: return apply_for<f16_t>(p, W, m, meta, partials, hot, lr, eps, s);
    case TBE_BF16: return apply_for<bf16_t>(p, W, m, meta, partials, hot, lr, eps, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace tbe
