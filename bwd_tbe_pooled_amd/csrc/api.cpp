// C ABI of the TBE library: argument validation (host, before any launch),
// path selection, workspace carving and the launch sequence of each call on
// the caller's stream. No allocation of device memory; the only global state
// is the per-thread text of the last HIP failure.
#include <cstdio>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "internal.h"

namespace tbe {

int small_splits_for(int32_t T, int32_t B);

RowShape row_shape(int D, int max_v) {
  RowShape r;
  int V = max_v;
  while (V > 1 && D % V != 0) V >>= 1;
  const int per = (D + V - 1) / V;
  int G = 1, lg = 0;
  while (G < per && G < 64) { G <<= 1; ++lg; }
  r.V = V;
  r.G = G;
  r.log2G = lg;
  r.P = (D + G * V - 1) / (G * V);
  return r;
}

constexpr int64_t kI32Lim = (int64_t(1) << 31) - 1;

static bool small_eligible(const tbe_desc* d, int64_t N, int weighted, int64_t max_rows) {
  // Page 1, checklist item 2: E <= 64, 64 <= D <= 128, L >= 64, f16, unweighted.
  if (d->flags & TBE_FLAG_FORCE_GENERIC) return false;
  if (weighted || d->wdtype != TBE_F16) return false;
  if (max_rows > kSmallE || d->D < 64 || d->D > 128) return false;
  if ((int64_t)d->T * d->D >= (int64_t(1) << 27)) return false;  // gradient offsets stay int32
  const int64_t nbags = (int64_t)d->T * d->B;
  if (nbags == 0) return false;
  return N >= 64 * nbags;  // average bag length N / (T*B) >= 64
}

// Checks shared by the int32 and int64 entry points: everything but the
// int32 size limits. Sets *sum and *mx to the sum and maximum of the rows.
static tbe_status check_desc(const tbe_desc* d, int64_t N, int64_t* sum, int64_t* mx) {
  if (!d || !d->rows) return TBE_ERR_ARG;
  if (d->T < 1 || d->D < 1 || d->B < 0 || N < 0) return TBE_ERR_ARG;
  if (d->wdtype != TBE_F32 && d->wdtype != TBE_F16 && d->wdtype != TBE_BF16) return TBE_ERR_UNSUPPORTED;
  if (d->flags &
      ~(TBE_FLAG_VALIDATE | TBE_FLAG_FORCE_GENERIC | TBE_FLAG_CHECK | TBE_FLAG_FUSED_LONG |
        TBE_FLAG_NO_HOT_ROWS | TBE_FLAG_HOT_BACKWARD))
    return TBE_ERR_ARG;
  if ((d->flags & TBE_FLAG_CHECK) && !d->error_flags) return TBE_ERR_ARG;
  if (d->short_max < 0 || d->chunk < 0) return TBE_ERR_ARG;
  int64_t s = 0, m = 0;
  for (int32_t t = 0; t < d->T; ++t) {
    if (d->rows[t] < 1) return TBE_ERR_ARG;
    if (d->rows[t] >= kI32Lim) return TBE_ERR_UNSUPPORTED;  // in-table rows stay int32
    s += d->rows[t];
    m = std::max<int64_t>(m, d->rows[t]);
  }
  const RowShape rs = row_shape(d->D, 8);
  if (rs.P > 4) return TBE_ERR_UNSUPPORTED;
  *sum = s;
  *mx = m;
  return TBE_OK;
}

// Sizes derived from T, D, B, N, nbags, sum_rows, max_rows, S and C.
static void derive_sizes(Problem* p) {
  int nbits = 0;
  while ((int64_t(1) << nbits) < p->max_rows) ++nbits;
  p->sort_passes = std::max(1, (nbits + 6) / 7);  // digits of at most 7 bits
  p->sort_bits = std::max(1, (nbits + p->sort_passes - 1) / p->sort_passes);
  p->sort_tiles_max = (p->N + kSortTile - 1) / kSortTile + p->T;
  p->cap_runs = std::min<int64_t>(p->N, p->sum_rows);
  p->cap_long = p->N / p->S;
  p->cap_chunks = p->cap_long ? p->N / p->C + p->cap_long : 0;
  p->small_splits = small_splits_for(p->T, p->B);
  p->ld = (int64_t)p->T * p->D;
  choose_hot(p);
  p->hot_bwd = hot_backward_eligible(*p);  // reads no_hot, hot_bwd_asked: set before this
  p->hot_nseg = p->hot_bwd ? hot_backward_segments(*p) : 0;
}

tbe_status make_problem(const tbe_desc* d, int64_t N, int weighted, Problem* p) {
  if (!p) return TBE_ERR_ARG;
  int64_t sum = 0, mx = 0;
  const tbe_status st = check_desc(d, N, &sum, &mx);
  if (st != TBE_OK) return st;
  // int32 keys, positions and bags (checklist item 6); larger problems use
  // the int64 entry points
  if (sum >= kI32Lim || N >= kI32Lim || (int64_t)d->T * d->B >= kI32Lim) return TBE_ERR_UNSUPPORTED;

  p->T = d->T;
  p->D = d->D;
  p->B = d->B;
  p->N = N;
  p->nbags = (int64_t)d->T * d->B;
  p->sum_rows = sum;
  p->max_rows = mx;
  p->wdtype = d->wdtype;
  p->weighted = weighted != 0;
  p->S = d->short_max ? d->short_max : kDefaultShortMax;
  p->C = d->chunk ? d->chunk : kDefaultChunk;
  p->path = small_eligible(d, N, weighted, mx) ? TBE_PATH_SMALL_TABLE : TBE_PATH_GENERIC;
  p->fused_long = (d->flags & TBE_FLAG_FUSED_LONG) != 0;
  p->no_hot = (d->flags & (TBE_FLAG_NO_HOT_ROWS | TBE_FLAG_FUSED_LONG)) != 0;
  p->hot_bwd_asked = (d->flags & TBE_FLAG_HOT_BACKWARD) != 0;
  derive_sizes(p);
  p->err = (d->flags & TBE_FLAG_CHECK) ? d->error_flags : nullptr;
  return TBE_OK;
}

void meta_caps(const Problem& p, int64_t c[TBE_META_NUM_ARRAYS]) {
  for (int i = 0; i < TBE_META_NUM_ARRAYS; ++i) c[i] = 0;
  c[TBE_META_COUNTS] = 8;
  if (p.path == TBE_PATH_SMALL_TABLE) {
    c[TBE_META_HIST] = p.nbags * kSmallE;
    return;
  }
  c[TBE_META_RUN_KEYS] = p.cap_runs;
  c[TBE_META_RUN_OFFSETS] = p.cap_runs + 1;
  c[TBE_META_SORTED_POS] = p.N;
  c[TBE_META_SORTED_BAG] = p.N;
  c[TBE_META_SORTED_PSW] = p.weighted ? p.N : 0;
  c[TBE_META_SHORT_RUNS] = p.cap_runs;
  c[TBE_META_LONG_RUNS] = p.cap_long;
  c[TBE_META_LONG_CHUNK_BEGIN] = p.cap_long + 1;
  c[TBE_META_CHUNK_RUN] = p.cap_chunks;
  c[TBE_META_CHUNK_START] = p.cap_chunks;
}

static size_t meta_elem_bytes(int i) { return i == TBE_META_HIST ? 1 : 4; }

WsLayout ws_layout(const Problem& p, tbe_op op) {
  WsLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~size_t(255);
    return at;
  };
  L.tinfo = take(sizeof(int32_t) * 2 * (size_t)p.T);
  L.flags = take(sizeof(int32_t) * 16);
  const bool generic = p.path == TBE_PATH_GENERIC;
  const bool pre = (op == TBE_OP_FORWARD_PREPROCESS || op == TBE_OP_PREPROCESS ||
                    op == TBE_OP_BACKWARD_SELF);
  L.has_pre = pre && generic;
  if (L.has_pre) {
    const size_t n4 = sizeof(int32_t) * (size_t)p.N;
    const int sets = p.sort_passes >= 3 ? 2 : (p.sort_passes == 2 ? 1 : 0);
    for (int k = 0; k < 4; ++k) {
      const bool need = k < 3 || p.weighted;
      L.sortA[k] = (sets >= 1 && need) ? take(n4) : 0;
      L.sortB[k] = (sets >= 2 && need) ? take(n4) : 0;
    }
    L.sorted_keys = take(n4);
    L.tile_base = take(sizeof(int32_t) * ((size_t)p.T + 1));
    L.tile_desc = take(sizeof(int32_t) * 8 * (size_t)p.sort_tiles_max);
    const int64_t radix = int64_t(1) << p.sort_bits;
    L.digit_counts = take(sizeof(int32_t) * (size_t)(radix * p.sort_tiles_max));
    L.digit_tot = take(sizeof(int32_t) * (size_t)(radix * p.T));
    const int64_t nt = (p.N + kRleTile - 1) / kRleTile;
    L.rle_tiles = take(sizeof(int32_t) * (size_t)(nt + 4));
    const int64_t rt = (p.cap_runs + kRleTile - 1) / kRleTile;
    L.route_tiles = take(sizeof(int32_t) * (size_t)(3 * rt + 4));
  }
  if (!generic && op == TBE_OP_FORWARD) L.hist = take((size_t)p.nbags * kSmallE);
  if (generic && op == TBE_OP_FORWARD_PREPROCESS && p.hot_k > 0)
    L.hot_rows = take(sizeof(int32_t) * (size_t)p.T * (size_t)p.hot_k);
  L.has_meta = op == TBE_OP_BACKWARD_SELF;
  if (L.has_meta) {
    int64_t caps[TBE_META_NUM_ARRAYS];
    meta_caps(p, caps);
    caps[TBE_META_SORTED_POS] = 0;  // the backward never reads positions: none sorted
    for (int i = 0; i < TBE_META_NUM_ARRAYS; ++i)
      L.meta[i] = caps[i] ? take(meta_elem_bytes(i) * (size_t)caps[i]) : 0;
  }
  L.has_partials = op == TBE_OP_BACKWARD || op == TBE_OP_BACKWARD_SELF;
  if (L.has_partials) {
    if (generic) {
      const size_t acc = p.wdtype == TBE_F32 ? 8 : 4;
      L.partials = take(acc * (size_t)p.cap_chunks * (size_t)p.D);
      L.sched = take(sizeof(int32_t) * long_schedule_ints(p));
      if (p.hot_bwd) {
        L.hb_rows = take(sizeof(int32_t) * (size_t)p.T * 256);
        L.hb_run_slot = take(sizeof(int32_t) * (size_t)p.cap_long);
        L.hb_min = take(sizeof(int32_t) * (size_t)p.T);
        L.hb_flag = take(sizeof(int32_t) * (size_t)p.T);
        L.hb_parts = take(sizeof(float) * (size_t)p.T * (size_t)p.hot_nseg * 256 * (size_t)p.D);
      }
    } else {
      const size_t parts = (size_t)p.T * (size_t)p.small_splits * kSmallE;
      L.partials = take(sizeof(float) * parts * (size_t)p.D);
      L.part_counts = take(sizeof(int32_t) * parts);
      L.part_wide = take(sizeof(int32_t) * (size_t)p.T * (size_t)p.small_splits);
    }
  }
  L.total = off;
  return L;
}

// --- stage timer -------------------------------------------------------------

struct StageTimer {
  int32_t capacity;
  std::vector<hipEvent_t> ev[TBE_NUM_STAGES];  // 2 per interval
  int32_t used[TBE_NUM_STAGES];
  bool open[TBE_NUM_STAGES];
};

}  // namespace tbe

struct tbe_timer {
  tbe::StageTimer st;
};

namespace tbe {

void timer_begin(tbe_timer* t, int stage, hipStream_t s) {
  if (!t) return;
  StageTimer& st = t->st;
  st.open[stage] = false;
  if (st.used[stage] >= st.capacity) return;
  (void)hipEventRecord(st.ev[stage][2 * st.used[stage]], s);
  st.open[stage] = true;
}

void timer_end(tbe_timer* t, int stage, hipStream_t s) {
  if (!t) return;
  StageTimer& st = t->st;
  if (!st.open[stage]) return;
  (void)hipEventRecord(st.ev[stage][2 * st.used[stage] + 1], s);
  st.used[stage] += 1;
  st.open[stage] = false;
}

}  // namespace tbe

using namespace tbe;

namespace {

thread_local char g_last_error[256] = "";

tbe_status hip_failure(hipError_t e, const char* what) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s (%s) in %s", hipGetErrorName(e),
                hipGetErrorString(e), what);
  return TBE_ERR_HIP;
}

#define TBE_TRY_HIP(expr)                                  \
  do {                                                     \
    const hipError_t tbe_e_ = (expr);                      \
    if (tbe_e_ != hipSuccess) return hip_failure(tbe_e_, #expr); \
  } while (0)

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

bool meta_ok_generic(const tbe_meta* m, bool weighted) {
  return m && m->counts && m->run_keys && m->run_offsets && m->sorted_bag &&
         (!weighted || m->sorted_psw) && m->short_runs && m->long_runs && m->long_chunk_begin &&
         m->chunk_run && m->chunk_start;
}

bool meta_ok_small(const tbe_meta* m) {
  return m && m->counts && m->hist && ((uintptr_t)m->hist & 15) == 0;  // 16-byte count loads
}

tbe_meta carve_meta(void* ws, const WsLayout& L) {
  tbe_meta m{};
  auto ptr = [&](int i) -> void* { return L.meta[i] ? at<char>(ws, L.meta[i]) : nullptr; };
  m.counts = (int32_t*)ptr(TBE_META_COUNTS);
  m.run_keys = (int32_t*)ptr(TBE_META_RUN_KEYS);
  m.run_offsets = (int32_t*)ptr(TBE_META_RUN_OFFSETS);
  m.sorted_pos = (int32_t*)ptr(TBE_META_SORTED_POS);
  m.sorted_bag = (int32_t*)ptr(TBE_META_SORTED_BAG);
  m.sorted_psw = (float*)ptr(TBE_META_SORTED_PSW);
  m.short_runs = (int32_t*)ptr(TBE_META_SHORT_RUNS);
  m.long_runs = (int32_t*)ptr(TBE_META_LONG_RUNS);
  m.long_chunk_begin = (int32_t*)ptr(TBE_META_LONG_CHUNK_BEGIN);
  m.chunk_run = (int32_t*)ptr(TBE_META_CHUNK_RUN);
  m.chunk_start = (int32_t*)ptr(TBE_META_CHUNK_START);
  m.hist = (uint8_t*)ptr(TBE_META_HIST);
  // Arrays the path does not use (positions, the psw of unweighted problems,
  // the generic arrays on the small-table path and the reverse) stay NULL.
  return m;
}

// Common prologue: table info upload and optional validation.
tbe_status prologue(const tbe_desc* d, const Problem& p, const int32_t* indices,
                    const int32_t* offsets, void* ws, const WsLayout& L, hipStream_t s) {
  // The launchers report hipGetLastError(); clear what an earlier runtime
  // call of the caller's may have left there, so that only this call's own
  // launch errors are reported.
  (void)hipGetLastError();
  int32_t* tinfo = at<int32_t>(ws, L.tinfo);
  TBE_TRY_HIP(launch_fill_tinfo(p, d->rows, tinfo, s));
  if (d->flags & TBE_FLAG_VALIDATE) {
    int32_t* flag = at<int32_t>(ws, L.flags);
    timer_begin(d->timer, TBE_STAGE_VALIDATE, s);
    TBE_TRY_HIP(launch_validate(p, indices, offsets, tinfo, flag, s));
    timer_end(d->timer, TBE_STAGE_VALIDATE, s);
    int32_t host_flag = 0;
    TBE_TRY_HIP(hipMemcpyAsync(&host_flag, flag, sizeof host_flag, hipMemcpyDeviceToHost, s));
    TBE_TRY_HIP(hipStreamSynchronize(s));
    if (host_flag) return TBE_ERR_INDEX_RANGE;
  }
  return TBE_OK;
}

tbe_status run_preprocess(const tbe_desc* d, const Problem& p, const int32_t* indices,
                          const int32_t* offsets, const float* psw, const tbe_meta& meta,
                          void* ws, const WsLayout& L, hipStream_t s) {
  const int32_t* tinfo = at<int32_t>(ws, L.tinfo);
  SortBuffers b{};
  for (int k = 0; k < 4; ++k) {
    b.A[k] = L.sortA[k] ? at<int32_t>(ws, L.sortA[k]) : nullptr;
    b.B[k] = L.sortB[k] ? at<int32_t>(ws, L.sortB[k]) : nullptr;
  }
  b.sorted_keys = at<int32_t>(ws, L.sorted_keys);
  b.tile_base = at<int32_t>(ws, L.tile_base);
  b.tile_desc = at<int4>(ws, L.tile_desc);
  b.digit_counts = at<int32_t>(ws, L.digit_counts);
  b.digit_tot = at<int32_t>(ws, L.digit_tot);
  timer_begin(d->timer, TBE_STAGE_LINEARIZE, s);
  TBE_TRY_HIP(launch_sort_setup(p, offsets, b, s));
  timer_end(d->timer, TBE_STAGE_LINEARIZE, s);
  timer_begin(d->timer, TBE_STAGE_SORT, s);
  TBE_TRY_HIP(launch_sort(p, indices, offsets, psw, tinfo, b, meta, s));
  timer_end(d->timer, TBE_STAGE_SORT, s);
  timer_begin(d->timer, TBE_STAGE_RLE_ROUTE, s);
  TBE_TRY_HIP(launch_rle_route(p, b.sorted_keys, at<int32_t>(ws, L.rle_tiles),
                               at<int32_t>(ws, L.route_tiles), meta, s));
  timer_end(d->timer, TBE_STAGE_RLE_ROUTE, s);
  return TBE_OK;
}

tbe_status check_ws(const Problem& p, tbe_op op, void* ws, size_t ws_bytes, WsLayout* L) {
  *L = ws_layout(p, op);
  if (!ws || ws_bytes < L->total) return TBE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return TBE_ERR_ARG;
  return TBE_OK;
}

tbe_status forward_impl(const tbe_desc* desc, const Problem& p, const void* W,
                        const int32_t* indices, const int32_t* offsets, const float* psw,
                        float* out, tbe_meta* meta, void* ws, size_t ws_bytes, hipStream_t s) {
  tbe_status st;
  const tbe_op op = meta ? TBE_OP_FORWARD_PREPROCESS : TBE_OP_FORWARD;
  if (meta && !(p.path == TBE_PATH_SMALL_TABLE ? meta_ok_small(meta) : meta_ok_generic(meta, p.weighted)))
    return TBE_ERR_ARG;
  WsLayout L;
  if ((st = check_ws(p, op, ws, ws_bytes, &L)) != TBE_OK) return st;
  if ((st = prologue(desc, p, indices, offsets, ws, L, s)) != TBE_OK) return st;
  const int32_t* tinfo = at<int32_t>(ws, L.tinfo);
  if (p.path == TBE_PATH_SMALL_TABLE) {
    int32_t* counts = meta ? meta->counts : at<int32_t>(ws, L.flags) + 8;
    uint8_t* hist = meta ? meta->hist : at<uint8_t>(ws, L.hist);
    timer_begin(desc->timer, TBE_STAGE_SMALL_COUNT, s);
    TBE_TRY_HIP(launch_small_count(p, indices, offsets, tinfo, hist, counts, s));
    timer_end(desc->timer, TBE_STAGE_SMALL_COUNT, s);
    timer_begin(desc->timer, TBE_STAGE_SMALL_FWD, s);
    TBE_TRY_HIP(launch_small_pool(p, W, indices, offsets, tinfo, out, hist, counts, s));
    timer_end(desc->timer, TBE_STAGE_SMALL_FWD, s);
    return TBE_OK;
  }
  if (meta && p.hot_k > 0) {
    // the transpose first: its longest runs are the rows the pool then reads
    // from LDS (same values, same order: the same output bits)
    if ((st = run_preprocess(desc, p, indices, offsets, psw, *meta, ws, L, s)) != TBE_OK) return st;
    int32_t* hot = at<int32_t>(ws, L.hot_rows);
    timer_begin(desc->timer, TBE_STAGE_HOT_PLAN, s);
    TBE_TRY_HIP(launch_hot_plan(p, *meta, tinfo, p.hot_k, hot, nullptr, nullptr, nullptr, s));
    timer_end(desc->timer, TBE_STAGE_HOT_PLAN, s);
    timer_begin(desc->timer, TBE_STAGE_FWD_POOL, s);
    TBE_TRY_HIP(launch_forward_pool_hot(p, W, indices, offsets, psw, tinfo, hot, out, s));
    timer_end(desc->timer, TBE_STAGE_FWD_POOL, s);
    return TBE_OK;
  }
  timer_begin(desc->timer, TBE_STAGE_FWD_POOL, s);
  TBE_TRY_HIP(launch_forward_pool(p, W, indices, offsets, psw, tinfo, out, s));
  timer_end(desc->timer, TBE_STAGE_FWD_POOL, s);
  if (meta) return run_preprocess(desc, p, indices, offsets, psw, *meta, ws, L, s);
  return TBE_OK;
}


tbe_status backward_impl(const tbe_desc* desc, const Problem& p, void* W, float* momentum,
                         const float* grad_out, const int32_t* indices, const int32_t* offsets,
                         const float* psw, const tbe_meta* meta, double lr, double eps, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  tbe_status st;
  const tbe_op op = meta ? TBE_OP_BACKWARD : TBE_OP_BACKWARD_SELF;
  if (meta && !(p.path == TBE_PATH_SMALL_TABLE ? meta_ok_small(meta) : meta_ok_generic(meta, p.weighted)))
    return TBE_ERR_ARG;
  WsLayout L;
  if ((st = check_ws(p, op, ws, ws_bytes, &L)) != TBE_OK) return st;
  if ((st = prologue(desc, p, indices, offsets, ws, L, s)) != TBE_OK) return st;
  const int32_t* tinfo = at<int32_t>(ws, L.tinfo);
  tbe_meta m = meta ? *meta : carve_meta(ws, L);

  if (p.path == TBE_PATH_SMALL_TABLE) {
    if (!meta) {
      timer_begin(desc->timer, TBE_STAGE_SMALL_COUNT, s);
      TBE_TRY_HIP(launch_small_count(p, indices, offsets, tinfo, m.hist, m.counts, s));
      timer_end(desc->timer, TBE_STAGE_SMALL_COUNT, s);
    }
    float* parts = at<float>(ws, L.partials);
    int32_t* pcounts = at<int32_t>(ws, L.part_counts);
    timer_begin(desc->timer, TBE_STAGE_SMALL_BWD, s);
    TBE_TRY_HIP(launch_small_backward(p, grad_out, m.hist, m.counts, indices, offsets, parts,
                                      pcounts, at<int32_t>(ws, L.part_wide), tinfo, s));
    timer_end(desc->timer, TBE_STAGE_SMALL_BWD, s);
    timer_begin(desc->timer, TBE_STAGE_SMALL_APPLY, s);
    TBE_TRY_HIP(launch_small_apply(p, W, momentum, tinfo, parts, pcounts, lr, eps, s));
    timer_end(desc->timer, TBE_STAGE_SMALL_APPLY, s);
    return TBE_OK;
  }

  if (!meta) {
    if ((st = run_preprocess(desc, p, indices, offsets, psw, m, ws, L, s)) != TBE_OK) return st;
  }
  void* parts = at<void>(ws, L.partials);
  timer_begin(desc->timer, TBE_STAGE_BWD_SHORT, s);
  TBE_TRY_HIP(launch_bwd_short(p, W, momentum, grad_out, m, tinfo, lr, eps, s));
  timer_end(desc->timer, TBE_STAGE_BWD_SHORT, s);
  HotBwd hot{};
  if (p.hot_bwd) {
    // the hot rows' plan, then their contraction; tables it flags go back to
    // the chunk path below
    int32_t* hb_rows = at<int32_t>(ws, L.hb_rows);
    int32_t* hb_flag = at<int32_t>(ws, L.hb_flag);
    float* hb_parts = at<float>(ws, L.hb_parts);
    hot.run_slot = at<int32_t>(ws, L.hb_run_slot);
    hot.hot_min = at<int32_t>(ws, L.hb_min);
    hot.hot_flag = hb_flag;
    hot.parts = hb_parts;
    hot.nseg = p.hot_nseg;
    timer_begin(desc->timer, TBE_STAGE_BWD_HOT_PLAN, s);
    TBE_TRY_HIP(launch_hot_plan(p, m, tinfo, 256, hb_rows, at<int32_t>(ws, L.hb_run_slot),
                                at<int32_t>(ws, L.hb_min), hb_flag, s));
    timer_end(desc->timer, TBE_STAGE_BWD_HOT_PLAN, s);
    timer_begin(desc->timer, TBE_STAGE_BWD_HOT, s);
    TBE_TRY_HIP(launch_bwd_hot(p, grad_out, indices, offsets, psw, hb_rows, tinfo, hb_parts,
                               hb_flag, s));
    timer_end(desc->timer, TBE_STAGE_BWD_HOT, s);
  }
  timer_begin(desc->timer, TBE_STAGE_LONG_SCHEDULE, s);
  TBE_TRY_HIP(launch_long_schedule(p, m, at<int32_t>(ws, L.sched), hot, s));
  timer_end(desc->timer, TBE_STAGE_LONG_SCHEDULE, s);
  timer_begin(desc->timer, TBE_STAGE_BWD_LONG, s);
  if (p.fused_long) {
    TBE_TRY_HIP(launch_bwd_long_fused(p, W, momentum, grad_out, m, parts,
                                      at<int32_t>(ws, L.sched), lr, eps, s));
    timer_end(desc->timer, TBE_STAGE_BWD_LONG, s);
    return TBE_OK;
  }
  TBE_TRY_HIP(launch_bwd_long(p, grad_out, m, parts, at<int32_t>(ws, L.sched), s));
  timer_end(desc->timer, TBE_STAGE_BWD_LONG, s);
  timer_begin(desc->timer, TBE_STAGE_BWD_APPLY, s);
  TBE_TRY_HIP(launch_bwd_apply(p, W, momentum, m, parts, hot, lr, eps, s));
  timer_end(desc->timer, TBE_STAGE_BWD_APPLY, s);
  return TBE_OK;
}


// --- int64 indices and offsets ---------------------------------------------
// A call with int64 index arrays runs as a sequence of calls over groups of
// consecutive tables, each small enough for int32 keys, positions and bags
// (page 1, checklist item 6: int32 wherever the linearized range allows it).
// Every step of the method works table by table, so the split changes no
// result. The groups follow from where each table's lookups begin, which the
// host reads back (T+1 values, one synchronisation per call).

struct TableGroup {
  int32_t t0, t1;     // tables [t0, t1)
  int64_t base, n;    // lookups [base, base + n)
};

bool small_possible(const tbe_desc* d, int weighted) {
  if ((d->flags & TBE_FLAG_FORCE_GENERIC) || weighted || d->wdtype != TBE_F16) return false;
  if (d->D < 64 || d->D > 128) return false;
  for (int32_t t = 0; t < d->T; ++t)
    if (d->rows[t] <= kSmallE) return true;
  return false;
}

// A problem at least as large, in every size the workspace depends on, as
// any group of this call.
Problem bound_problem(const tbe_desc* d, int64_t N, int weighted, int64_t sum, int64_t mx,
                      int path) {
  Problem p{};
  p.T = d->T;
  p.D = d->D;
  p.B = d->B;
  p.N = std::min<int64_t>(N, kI32Lim - 1);
  p.nbags = std::min<int64_t>((int64_t)d->T * d->B, kI32Lim - 1);
  p.sum_rows = std::min<int64_t>(sum, kI32Lim - 1);
  p.max_rows = mx;
  p.wdtype = d->wdtype;
  p.weighted = weighted != 0;
  p.S = d->short_max ? d->short_max : kDefaultShortMax;
  p.C = d->chunk ? d->chunk : kDefaultChunk;
  p.path = path;
  p.fused_long = (d->flags & TBE_FLAG_FUSED_LONG) != 0;
  p.no_hot = (d->flags & (TBE_FLAG_NO_HOT_ROWS | TBE_FLAG_FUSED_LONG)) != 0;
  p.hot_bwd_asked = (d->flags & TBE_FLAG_HOT_BACKWARD) != 0;
  derive_sizes(&p);
  p.sort_bits = 7;  // a group with fewer rows can take fewer, wider digits
  // a group of T_g tables takes T_g * max(1, floor(W / T_g)) <= T + W - 1
  // segments in all (W = kHotBwdWorkgroups)
  if (p.hot_bwd) p.hot_nseg = (int32_t)((p.T + kHotBwdWorkgroups - 1 + p.T - 1) / p.T);
  if (path == TBE_PATH_SMALL_TABLE) {  // split partials: T_g * splits(T_g) at most
    int64_t parts = 0;
    for (int32_t tg = 1; tg <= d->T; ++tg)
      parts = std::max<int64_t>(parts, (int64_t)tg * small_splits_for(tg, d->B));
    p.small_splits = (int)((parts + d->T - 1) / d->T);
  }
  return p;
}

struct I64Layout {
  size_t bounds, idx32, off32, group, total;
};

I64Layout i64_layout(const tbe_desc* d, int64_t N, int weighted, tbe_op op, int64_t sum,
                     int64_t mx) {
  I64Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) & ~size_t(255);
    return at;
  };
  L.bounds = take(sizeof(int64_t) * ((size_t)d->T + 1));
  L.idx32 = take(sizeof(int32_t) * (size_t)std::min<int64_t>(N, kI32Lim - 1));
  L.off32 = take(sizeof(int32_t) * ((size_t)std::min<int64_t>((int64_t)d->T * d->B, kI32Lim - 1) + 1));
  size_t g = ws_layout(bound_problem(d, N, weighted, sum, mx, TBE_PATH_GENERIC), op).total;
  if (small_possible(d, weighted))
    g = std::max(g, ws_layout(bound_problem(d, N, weighted, sum, mx, TBE_PATH_SMALL_TABLE), op).total);
  L.group = take(g);
  L.total = off;
  return L;
}

tbe_status plan_groups(const tbe_desc* d, const std::vector<int64_t>& tb, int64_t N,
                       std::vector<TableGroup>* out) {
  const int32_t T = d->T;
  if (tb[0] != 0 || tb[T] != N) return TBE_ERR_INDEX_RANGE;
  TableGroup g{0, 0, 0, 0};
  int64_t rows = 0;
  for (int32_t t = 0; t < T; ++t) {
    const int64_t n = tb[t + 1] - tb[t];
    if (n < 0) return TBE_ERR_INDEX_RANGE;
    if (n >= kI32Lim || (int64_t)d->B >= kI32Lim) return TBE_ERR_UNSUPPORTED;
    const bool fits = rows + d->rows[t] < kI32Lim && g.n + n < kI32Lim &&
                      (int64_t)(g.t1 - g.t0 + 1) * d->B < kI32Lim;
    if (g.t1 > g.t0 && !fits) {
      out->push_back(g);
      g = TableGroup{t, t, tb[t], 0};
      rows = 0;
    }
    g.t1 = t + 1;
    g.n += n;
    rows += d->rows[t];
  }
  out->push_back(g);
  return TBE_OK;
}

// The description of one group, and its problem with the whole call's row
// stride for the pooled output and the upstream gradient.
tbe_status group_problem(const tbe_desc* d, const TableGroup& g, int weighted, tbe_desc* sub,
                         Problem* p) {
  *sub = *d;
  sub->T = g.t1 - g.t0;
  sub->rows = d->rows + g.t0;
  tbe_status st = make_problem(sub, g.n, weighted, p);
  if (st != TBE_OK) return st;
  // the small-table backward keeps 8-row gradient offsets in int32
  if (p->path == TBE_PATH_SMALL_TABLE && (int64_t)d->T * d->D >= (int64_t(1) << 27)) {
    sub->flags |= TBE_FLAG_FORCE_GENERIC;
    if ((st = make_problem(sub, g.n, weighted, p)) != TBE_OK) return st;
  }
  p->ld = (int64_t)d->T * d->D;
  return TBE_OK;
}

tbe_status run_i64(bool backward, const tbe_desc* d, void* W, float* momentum,
                   const float* grad_out, const int64_t* indices, const int64_t* offsets,
                   int64_t N, const float* psw, float* out, double lr, double eps, void* ws,
                   size_t ws_bytes, hipStream_t s) {
  int64_t sum = 0, mx = 0;
  tbe_status st = check_desc(d, N, &sum, &mx);
  if (st != TBE_OK) return st;
  const int weighted = psw != nullptr;
  const int64_t nbags = (int64_t)d->T * d->B;
  if (!W || !offsets || (!indices && N > 0)) return TBE_ERR_ARG;
  if (backward && (!momentum || (!grad_out && nbags > 0) || !(lr >= 0.0) || !(eps >= 0.0)))
    return TBE_ERR_ARG;
  if (!backward && !out && nbags > 0) return TBE_ERR_ARG;
  const tbe_op op = backward ? TBE_OP_BACKWARD_SELF : TBE_OP_FORWARD;
  const I64Layout L = i64_layout(d, N, weighted, op, sum, mx);
  if (!ws || ws_bytes < L.total) return TBE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) return TBE_ERR_ARG;

  (void)hipGetLastError();
  int64_t* dbounds = at<int64_t>(ws, L.bounds);
  TBE_TRY_HIP(launch_table_bounds(offsets, d->T, d->B, dbounds, s));
  std::vector<int64_t> tb((size_t)d->T + 1);
  TBE_TRY_HIP(hipMemcpyAsync(tb.data(), dbounds, sizeof(int64_t) * tb.size(),
                             hipMemcpyDeviceToHost, s));
  TBE_TRY_HIP(hipStreamSynchronize(s));
  std::vector<TableGroup> groups;
  if ((st = plan_groups(d, tb, N, &groups)) != TBE_OK) return st;
  std::vector<int64_t> roff((size_t)d->T + 1, 0);
  for (int32_t t = 0; t < d->T; ++t) roff[t + 1] = roff[t] + d->rows[t];

  int32_t* idx32 = at<int32_t>(ws, L.idx32);
  int32_t* off32 = at<int32_t>(ws, L.off32);
  void* gws = at<char>(ws, L.group);
  const size_t gws_bytes = L.total - L.group;
  auto narrow = [&](const TableGroup& g, int32_t Tg) {
    return launch_narrow(indices ? indices + g.base : nullptr, g.n, offsets + (int64_t)g.t0 * d->B,
                         (int64_t)Tg * d->B + 1, g.base, idx32, off32, s);
  };
  if (d->flags & TBE_FLAG_VALIDATE) {  // every group is checked before any work
    for (const TableGroup& g : groups) {
      tbe_desc sub;
      Problem p;
      if ((st = group_problem(d, g, weighted, &sub, &p)) != TBE_OK) return st;
      TBE_TRY_HIP(narrow(g, sub.T));
      WsLayout Lg;
      if ((st = check_ws(p, op, gws, gws_bytes, &Lg)) != TBE_OK) return st;
      if ((st = prologue(&sub, p, idx32, off32, gws, Lg, s)) != TBE_OK) return st;
    }
  }
  const size_t wbytes = d->wdtype == TBE_F32 ? 4 : 2;
  for (const TableGroup& g : groups) {
    tbe_desc sub;
    Problem p;
    if ((st = group_problem(d, g, weighted, &sub, &p)) != TBE_OK) return st;
    sub.flags &= ~TBE_FLAG_VALIDATE;
    TBE_TRY_HIP(narrow(g, sub.T));
    char* Wg = static_cast<char*>(W) + roff[g.t0] * d->D * (int64_t)wbytes;
    const float* psw_g = psw ? psw + g.base : nullptr;
    // out and grad_out may be NULL when there are no bags
    const int64_t col = (int64_t)g.t0 * d->D;
    if (backward)
      st = backward_impl(&sub, p, Wg, momentum + roff[g.t0], grad_out ? grad_out + col : nullptr,
                         idx32, off32, psw_g, nullptr, lr, eps, gws, gws_bytes, s);
    else
      st = forward_impl(&sub, p, Wg, idx32, off32, psw_g, out ? out + col : nullptr, nullptr,
                        gws, gws_bytes, s);
    if (st != TBE_OK) return st;
  }
  return TBE_OK;
}

// --- the backward without allocation ---------------------------------------
// Scratch of tbe_backward_adagrad_noalloc, one copy per device, held until the
// process ends. Host code never passes the name `scratch` itself to a kernel
// or a copy: on the host it is only a stand-in for the device symbol. Each
// device's address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is used.
static __device__ __align__(256) unsigned char scratch[TBE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address, or null after setting the last-error
// text.
void* device_scratch() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_failure(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    std::snprintf(g_last_error, sizeof g_last_error,
                  "device %d is beyond the %d devices the scratch table holds", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      hip_failure(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

tbe_status tbe_backward_adagrad_noalloc(const tbe_desc* desc, void* W, float* momentum,
                                        const float* grad_out, const int32_t* indices,
                                        const int32_t* offsets, int64_t N, const float* psw,
                                        const tbe_meta* meta, double lr, double eps,
                                        void* stream) {
  Problem p;
  tbe_status st = make_problem(desc, N, psw != nullptr, &p);
  if (st != TBE_OK) return st;
  if (!meta || !W || !momentum || (!grad_out && p.nbags > 0) || !offsets || (!indices && N > 0))
    return TBE_ERR_ARG;
  if (!(lr >= 0.0) || !(eps >= 0.0)) return TBE_ERR_ARG;
  const size_t need = ws_layout(p, TBE_OP_BACKWARD).total;
  if (need > TBE_NOALLOC_SCRATCH_BYTES) {
    std::snprintf(g_last_error, sizeof g_last_error,
                  "the problem needs %zu bytes of scratch; the built-in scratch holds %zu",
                  need, (size_t)TBE_NOALLOC_SCRATCH_BYTES);
    return TBE_ERR_WORKSPACE;
  }
  void* ws = device_scratch();
  if (!ws) return TBE_ERR_HIP;
  return backward_impl(desc, p, W, momentum, grad_out, indices, offsets, psw, meta, lr, eps, ws,
                       TBE_NOALLOC_SCRATCH_BYTES, static_cast<hipStream_t>(stream));
}

const char* tbe_last_error(void) { return g_last_error; }

const char* tbe_status_str(tbe_status s) {
  switch (s) {
    case TBE_OK: return "ok";
    case TBE_ERR_ARG: return "invalid argument";
    case TBE_ERR_UNSUPPORTED: return "unsupported problem shape or type";
    case TBE_ERR_WORKSPACE: return "workspace missing or too small";
    case TBE_ERR_INDEX_RANGE: return "offsets or indices out of range";
    case TBE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

int32_t tbe_select_path(const tbe_desc* desc, int64_t N, int32_t weighted) {
  Problem p;
  const tbe_status st = make_problem(desc, N, weighted, &p);
  if (st != TBE_OK) return -(int32_t)st;
  return p.path;
}

tbe_status tbe_meta_capacity(const tbe_desc* desc, int64_t N, int32_t weighted, int64_t* caps) {
  if (!caps) return TBE_ERR_ARG;
  Problem p;
  const tbe_status st = make_problem(desc, N, weighted, &p);
  if (st != TBE_OK) return st;
  meta_caps(p, caps);
  return TBE_OK;
}

size_t tbe_workspace_bytes(const tbe_desc* desc, int64_t N, int32_t weighted, tbe_op op) {
  Problem p;
  if (make_problem(desc, N, weighted, &p) != TBE_OK) return 0;
  if (op < TBE_OP_FORWARD || op > TBE_OP_BACKWARD_SELF) return 0;
  return ws_layout(p, op).total;
}

tbe_status tbe_forward(const tbe_desc* desc, const void* W, const int32_t* indices,
                       const int32_t* offsets, int64_t N, const float* psw, float* out,
                       tbe_meta* meta, void* ws, size_t ws_bytes, void* stream) {
  Problem p;
  tbe_status st = make_problem(desc, N, psw != nullptr, &p);
  if (st != TBE_OK) return st;
  if (!W || !offsets || (!indices && N > 0) || (!out && p.nbags > 0)) return TBE_ERR_ARG;
  return forward_impl(desc, p, W, indices, offsets, psw, out, meta, ws, ws_bytes,
                      static_cast<hipStream_t>(stream));
}

tbe_status tbe_preprocess(const tbe_desc* desc, const int32_t* indices, const int32_t* offsets,
                          int64_t N, const float* psw, tbe_meta* meta, void* ws, size_t ws_bytes,
                          void* stream) {
  Problem p;
  tbe_status st = make_problem(desc, N, psw != nullptr, &p);
  if (st != TBE_OK) return st;
  if (!offsets || (!indices && N > 0)) return TBE_ERR_ARG;
  if (!(p.path == TBE_PATH_SMALL_TABLE ? meta_ok_small(meta) : meta_ok_generic(meta, p.weighted)))
    return TBE_ERR_ARG;
  WsLayout L;
  if ((st = check_ws(p, TBE_OP_PREPROCESS, ws, ws_bytes, &L)) != TBE_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = prologue(desc, p, indices, offsets, ws, L, s)) != TBE_OK) return st;
  if (p.path == TBE_PATH_SMALL_TABLE) {
    timer_begin(desc->timer, TBE_STAGE_SMALL_COUNT, s);
    TBE_TRY_HIP(launch_small_count(p, indices, offsets, at<int32_t>(ws, L.tinfo), meta->hist,
                                   meta->counts, s));
    timer_end(desc->timer, TBE_STAGE_SMALL_COUNT, s);
    return TBE_OK;
  }
  return run_preprocess(desc, p, indices, offsets, psw, *meta, ws, L, s);
}

tbe_status tbe_backward_adagrad(const tbe_desc* desc, void* W, float* momentum,
                                const float* grad_out, const int32_t* indices,
                                const int32_t* offsets, int64_t N, const float* psw,
                                const tbe_meta* meta, double lr, double eps, void* ws,
                                size_t ws_bytes, void* stream) {
  Problem p;
  tbe_status st = make_problem(desc, N, psw != nullptr, &p);
  if (st != TBE_OK) return st;
  if (!W || !momentum || (!grad_out && p.nbags > 0) || !offsets || (!indices && N > 0))
    return TBE_ERR_ARG;
  if (!(lr >= 0.0) || !(eps >= 0.0)) return TBE_ERR_ARG;
  return backward_impl(desc, p, W, momentum, grad_out, indices, offsets, psw, meta, lr, eps, ws,
                       ws_bytes, static_cast<hipStream_t>(stream));
}

size_t tbe_workspace_bytes_i64(const tbe_desc* desc, int64_t N, int32_t weighted, tbe_op op) {
  if (op != TBE_OP_FORWARD && op != TBE_OP_BACKWARD_SELF) return 0;
  int64_t sum = 0, mx = 0;
  if (check_desc(desc, N, &sum, &mx) != TBE_OK) return 0;
  return i64_layout(desc, N, weighted, op, sum, mx).total;
}

tbe_status tbe_forward_i64(const tbe_desc* desc, const void* W, const int64_t* indices,
                           const int64_t* offsets, int64_t N, const float* psw, float* out,
                           void* ws, size_t ws_bytes, void* stream) {
  return run_i64(false, desc, const_cast<void*>(W), nullptr, nullptr, indices, offsets, N, psw,
                 out, 0.0, 0.0, ws, ws_bytes, static_cast<hipStream_t>(stream));
}

tbe_status tbe_backward_adagrad_i64(const tbe_desc* desc, void* W, float* momentum,
                                    const float* grad_out, const int64_t* indices,
                                    const int64_t* offsets, int64_t N, const float* psw,
                                    double lr, double eps, void* ws, size_t ws_bytes,
                                    void* stream) {
  return run_i64(true, desc, W, momentum, grad_out, indices, offsets, N, psw, nullptr, lr, eps,
                 ws, ws_bytes, static_cast<hipStream_t>(stream));
}

tbe_status tbe_timer_create(int32_t capacity, tbe_timer** out) {
  if (!out || capacity < 1) return TBE_ERR_ARG;
  tbe_timer* t = new (std::nothrow) tbe_timer;
  if (!t) return TBE_ERR_ARG;
  t->st.capacity = capacity;
  for (int s = 0; s < TBE_NUM_STAGES; ++s) {
    t->st.used[s] = 0;
    t->st.open[s] = false;
    t->st.ev[s].assign(2 * (size_t)capacity, nullptr);
    for (auto& e : t->st.ev[s]) {
      if (hipEventCreate(&e) != hipSuccess) {
        tbe_timer_destroy(t);
        return TBE_ERR_HIP;
      }
    }
  }
  *out = t;
  return TBE_OK;
}

tbe_status tbe_timer_reset(tbe_timer* t) {
  if (!t) return TBE_ERR_ARG;
  for (int s = 0; s < TBE_NUM_STAGES; ++s) {
    t->st.used[s] = 0;
    t->st.open[s] = false;
  }
  return TBE_OK;
}

tbe_status tbe_timer_read(tbe_timer* t, float* ms, int32_t* intervals) {
  if (!t || !ms || !intervals) return TBE_ERR_ARG;
  for (int s = 0; s < TBE_NUM_STAGES; ++s) {
    float total = 0.f;
    for (int32_t i = 0; i < t->st.used[s]; ++i) {
      hipEvent_t a = t->st.ev[s][2 * i], b = t->st.ev[s][2 * i + 1];
      if (hipEventSynchronize(b) != hipSuccess) return TBE_ERR_HIP;
      float x = 0.f;
      if (hipEventElapsedTime(&x, a, b) != hipSuccess) return TBE_ERR_HIP;
      total += x;
    }
    ms[s] = total;
    intervals[s] = t->st.used[s];
  }
  return TBE_OK;
}

void tbe_timer_destroy(tbe_timer* t) {
  if (!t) return;
  for (int s = 0; s < TBE_NUM_STAGES; ++s)
    for (auto& e : t->st.ev[s])
      if (e) (void)hipEventDestroy(e);
  delete t;
}

}  // extern "C"
