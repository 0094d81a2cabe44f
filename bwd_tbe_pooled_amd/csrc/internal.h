// Host-side internals shared by the API layer and the kernel launchers:
// problem geometry, the row decomposition of a D-wide row over wave lanes,
// workspace carving, and the launcher entry points of each kernel file.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tbe.h"

namespace tbe {

constexpr int kDefaultShortMax = 256;  // SL < 256 is short (page 1, routing)
constexpr int kDefaultChunk = 256;     // 256-lookup chunks (page 1, routing)
constexpr int kSmallE = 64;            // small-table path row limit and hist stride

// Sort geometry.
constexpr int kSortTile = 4096;        // elements per radix tile (256 threads x 16)
constexpr int kRleTile = 4096;         // elements per RLE / routing tile

// How one D-wide row maps onto the lanes of a wave: V consecutive elements
// per lane per pass, G lanes per row (power of two), P passes; 64/G rows are
// in flight per wave ("row slots").
struct RowShape {
  int V, G, P, log2G;
};
RowShape row_shape(int D, int max_v);

// Everything the launchers need, derived once per call on the host.
struct Problem {
  int32_t T, D, B;
  int64_t N;
  int64_t nbags;       // T*B
  int64_t sum_rows;    // sum(E_t)
  int64_t max_rows;    // max(E_t)
  tbe_dtype wdtype;
  bool weighted;
  int32_t S, C;        // short/long threshold and chunk length
  int path;            // TBE_PATH_*
  // radix sort
  int sort_passes, sort_bits;   // bits per pass
  int64_t sort_tiles_max;       // upper bound of tiles over all table segments
  // capacities
  int64_t cap_runs, cap_long, cap_chunks;
  // small-table backward split
  int small_splits;
  // TBE_FLAG_CHECK: where kernels that read indices report a bad one (else null)
  int32_t* err;
  // TBE_FLAG_FUSED_LONG: long runs reduced and applied by the long kernel
  bool fused_long;
  // TBE_FLAG_NO_HOT_ROWS (implied by TBE_FLAG_FUSED_LONG): no hot-row paths
  bool no_hot;
  // TBE_FLAG_HOT_BACKWARD: the hot rows' backward on the matrix cores, asked for
  bool hot_bwd_asked;
  // Forward after the transpose: hot rows per table kept in LDS (0 = the
  // plain gather) and bags per workgroup of that kernel.
  int32_t hot_k, hot_bags;
  // Backward of the hot rows on the matrix cores (TBE_FLAG_HOT_BACKWARD,
  // generic path, f16/bf16 weights, D a multiple of 32 up to 128): segments of
  // the batch per table.
  bool hot_bwd;
  int32_t hot_nseg;
  // Row stride (floats) of the pooled output and of the upstream gradient:
  // T*D, or the whole problem's T*D when this problem is one group of tables
  // of a larger call.
  int64_t ld;
};

tbe_status make_problem(const tbe_desc* d, int64_t N, int weighted, Problem* p);

// Workspace carving: every region 256-byte aligned.
struct WsLayout {
  size_t total;
  // common
  size_t tinfo;        // int32 toff[T], int32 rows[T]
  size_t flags;        // int32[16]
  // generic preprocessing
  size_t sortA[4];     // key, pos, bag, psw  (int32/float [N] each)
  size_t sortB[4];
  size_t sorted_keys;  // int32[N]
  size_t tile_base;    // int32[T+1]
  size_t tile_desc;    // int4[2 * sort_tiles_max]
  size_t digit_counts; // int32[radix * sort_tiles_max]
  size_t digit_tot;    // int32[T * radix]
  size_t rle_tiles;    // int32[2 * n_rle_tiles]
  size_t route_tiles;  // int32[6 * n_route_tiles]
  // carved metadata (backward without a caller meta)
  size_t meta[TBE_META_NUM_ARRAYS];
  // backward
  size_t partials;     // long-run chunk partials / small-table partials
  size_t part_counts;  // small-table per-split row counts
  size_t part_wide;    // small-table per-split flag: gradients outside the f16 split's range
  size_t hist;         // small-table counts of a forward given no metadata
  size_t sched;        // long-chunk schedule (order, buckets, list bounds)
  size_t hot_rows;     // forward after the transpose: hot rows per table, int32[T * hot_k]
  // backward of the hot rows: hot rows int32[T * 256], slot of each long run
  // int32[cap_long], shortest hot run and fallback flag per table int32[T] each,
  // segment partials float[T * nseg * 256 * D]
  size_t hb_rows, hb_run_slot, hb_min, hb_flag, hb_parts;
  bool has_pre, has_meta, has_partials;
};

WsLayout ws_layout(const Problem& p, tbe_op op);
void meta_caps(const Problem& p, int64_t caps[TBE_META_NUM_ARRAYS]);

// Stage timer (opaque to callers).
struct StageTimer;
void timer_begin(tbe_timer* t, int stage, hipStream_t s);
void timer_end(tbe_timer* t, int stage, hipStream_t s);

// --- launchers (return hipSuccess or the first launch error) ----------------
// Compute units of the current device (queried once per device).
int device_cu_count();

hipError_t launch_fill_tinfo(const Problem& p, const int64_t* rows_host, int32_t* tinfo,
                             hipStream_t s);
hipError_t launch_validate(const Problem& p, const int32_t* indices, const int32_t* offsets,
                           const int32_t* tinfo, int32_t* flag, hipStream_t s);

hipError_t launch_forward_pool(const Problem& p, const void* W, const int32_t* indices,
                               const int32_t* offsets, const float* psw, const int32_t* tinfo,
                               float* out, hipStream_t s);
void choose_hot(Problem* p);
hipError_t launch_hot_plan(const Problem& p, const tbe_meta& meta, const int32_t* tinfo, int32_t K,
                           int32_t* hot_rows, int32_t* run_slot, int32_t* hot_min,
                           int32_t* hot_flag, hipStream_t s);
bool hot_backward_eligible(const Problem& p);
// workgroups the hot rows' contraction runs over all tables (two per CU of
// an MI355X): T * segments <= max(T, kHotBwdWorkgroups)
constexpr int kHotBwdWorkgroups = 512;
int32_t hot_backward_segments(const Problem& p);
hipError_t launch_bwd_hot(const Problem& p, const float* grad, const int32_t* indices,
                          const int32_t* offsets, const float* psw, const int32_t* hot_rows,
                          const int32_t* tinfo, float* hot_parts, int32_t* hot_flag,
                          hipStream_t s);
// The hot rows' plan, flags and partials as the chunk schedule and the apply
// read them (all null when the backward takes no hot rows).
struct HotBwd {
  const int32_t* run_slot;   // per long run: t*256 + slot, or -1
  const int32_t* hot_min;    // per table: the shortest hot run's length
  const int32_t* hot_flag;   // per table: 1 = its hot runs take the chunk path
  const float* parts;        // [T][nseg][256][D]
  int32_t nseg;
};
hipError_t launch_forward_pool_hot(const Problem& p, const void* W, const int32_t* indices,
                                   const int32_t* offsets, const float* psw, const int32_t* tinfo,
                                   const int32_t* hot_rows, float* out, hipStream_t s);

struct SortBuffers {
  int32_t* A[4];       // key, pos, bag, psw after even passes
  int32_t* B[4];       // ... after odd passes
  int32_t* sorted_keys;
  int32_t* tile_base;
  int4* tile_desc;     // two int4 per tile
  int32_t* digit_counts;
  int32_t* digit_tot;
};
hipError_t launch_sort_setup(const Problem& p, const int32_t* offsets, const SortBuffers& b,
                             hipStream_t s);
hipError_t launch_sort(const Problem& p, const int32_t* indices, const int32_t* offsets,
                       const float* psw, const int32_t* tinfo, const SortBuffers& b,
                       const tbe_meta& meta, hipStream_t s);
hipError_t launch_rle_route(const Problem& p, const int32_t* sorted_keys, int32_t* rle_tiles,
                            int32_t* route_tiles, const tbe_meta& meta, hipStream_t s);

hipError_t launch_bwd_short(const Problem& p, void* W, float* m, const float* grad,
                            const tbe_meta& meta, const int32_t* tinfo, double lr, double eps,
                            hipStream_t s);
hipError_t launch_long_schedule(const Problem& p, const tbe_meta& meta, int32_t* sched,
                                const HotBwd& hot, hipStream_t s);
hipError_t launch_bwd_long(const Problem& p, const float* grad, const tbe_meta& meta,
                           void* partials, int32_t* sched, hipStream_t s);
hipError_t launch_bwd_long_fused(const Problem& p, void* W, float* m, const float* grad,
                                 const tbe_meta& meta, void* partials, int32_t* sched, double lr,
                                 double eps, hipStream_t s);
size_t long_schedule_ints(const Problem& p);  // workspace ints of the chunk schedule
hipError_t launch_bwd_apply(const Problem& p, void* W, float* m, const tbe_meta& meta,
                            const void* partials, const HotBwd& hot, double lr, double eps,
                            hipStream_t s);

// int64 index arrays: table start offsets (T+1) and int32 copies of one
// group of tables.
hipError_t launch_table_bounds(const int64_t* offsets, int32_t T, int32_t B, int64_t* out,
                               hipStream_t s);
hipError_t launch_narrow(const int64_t* indices, int64_t n_idx, const int64_t* offsets,
                         int64_t n_off, int64_t base, int32_t* idx32, int32_t* off32,
                         hipStream_t s);

hipError_t launch_small_count(const Problem& p, const int32_t* indices, const int32_t* offsets,
                              const int32_t* tinfo, uint8_t* hist, int32_t* counts,
                              hipStream_t s);
hipError_t launch_small_pool(const Problem& p, const void* W, const int32_t* indices,
                             const int32_t* offsets, const int32_t* tinfo, float* out,
                             const uint8_t* hist, const int32_t* counts, hipStream_t s);
hipError_t launch_small_backward(const Problem& p, const float* grad, const uint8_t* hist,
                                 const int32_t* counts, const int32_t* indices,
                                 const int32_t* offsets, float* partials, int32_t* part_counts,
                                 int32_t* wide, const int32_t* tinfo, hipStream_t s);
hipError_t launch_small_apply(const Problem& p, void* W, float* m, const int32_t* tinfo,
                              const float* partials, const int32_t* part_counts, double lr,
                              double eps, hipStream_t s);

}  // namespace tbe
