/*
 * tbe.h — C ABI of the MI355X (gfx950) table-batched embedding (TBE) library.
 *
 * The library runs the training hot path of a pooled embedding lookup over T
 * tables: the forward sum / per-sample-weighted sum of rows (one launch for
 * all tables), the batch transpose (stable sort of linearized (table,row) keys
 * plus run-length encoding), routing of runs by segment length, the per-row
 * gradient sum and exactly one row-wise Adagrad step per touched row; plus the
 * small-table histogram path whose contraction runs on the matrix cores.
 * Sources: the FBTriton TBE tutorial (page 1) — "Forward state reuse and
 * preprocessing", "Backward kernel: three paths by segment length" with its
 * notation list, and the decision checklist items 1-6; the TorchEasyRec
 * article (page 2) section 1 for the jagged (KeyedJaggedTensor-like) layout.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Plain C types only. Pointers marked "device" are HIP device pointers;
 *   pointers marked "host" are ordinary host memory, read during the call only.
 * - The caller owns every buffer. The library never allocates or frees device
 *   memory and keeps no state between calls (a timer, when passed, is the
 *   caller's object) beyond host-side caches: the text behind tbe_last_error
 *   (per calling thread), each device's compute-unit count, queried once, and
 *   each device's address of the built-in scratch of
 *   tbe_backward_adagrad_noalloc (the one device array the library holds
 *   itself). Calls on different streams with disjoint buffers may run
 *   concurrently, except tbe_backward_adagrad_noalloc calls on one device.
 * - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued on it
 *   and the call returns without waiting, except under TBE_FLAG_VALIDATE.
 *   Buffers must stay alive until the stream has passed the call.
 * - Argument errors are detected on the host before anything is enqueued; the
 *   call then returns an error code and leaves every buffer untouched.
 *   TBE_ERR_HIP reports a failed launch (work enqueued before it may have run).
 *   No C++ exception crosses this boundary.
 * - Indices, offsets and linearized keys are int32: the library requires the
 *   total row count sum(E_t) and the lookup count N to be below 2^31
 *   (checklist item 6 of page 1), else TBE_ERR_UNSUPPORTED. The _i64 entry
 *   points take int64 indices and offsets and lift both limits.
 *
 * Data layout (device)
 * --------------------
 *   W        [sum(E_t), D] row-major, tables stacked in table order; element
 *            type per `wdtype` (f32, f16 or bf16 bit patterns).
 *   indices  int32 [N]: row inside its own table.
 *   offsets  int32 [T*B + 1]: table-major bags; bag i = t*B + b holds
 *            indices[offsets[i] .. offsets[i+1]-1]. offsets[0] = 0,
 *            offsets[T*B] = N, non-decreasing.
 *   psw      float32 [N] per-sample weights, or NULL for plain sums.
 *   out      float32 [B, T*D]: bag (t,b) pools into row b, columns t*D..t*D+D-1.
 *   grad_out float32 [B, T*D]: upstream gradient of `out`, same layout.
 *   momentum float32 [sum(E_t)]: row-wise Adagrad state, one scalar per row.
 *
 * Precision (checklist item 1 of page 1): f16/bf16 weights accumulate in
 * float32 and their Adagrad arithmetic is float32; f32 weights accumulate in
 * float64 and their Adagrad arithmetic is float64. Updated weights are rounded
 * to nearest even into their storage type, the state into float32.
 */
#ifndef TBE_H
#define TBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TBE_OK = 0,
    TBE_ERR_ARG = 1,          /* null/inconsistent argument, bad flag bits */
    TBE_ERR_UNSUPPORTED = 2,  /* shape outside what the library handles */
    TBE_ERR_WORKSPACE = 3,    /* workspace null or smaller than required */
    TBE_ERR_INDEX_RANGE = 4,  /* TBE_FLAG_VALIDATE found bad offsets/indices */
    TBE_ERR_HIP = 5           /* a HIP runtime call or launch failed */
} tbe_status;

typedef enum { TBE_F32 = 0, TBE_F16 = 1, TBE_BF16 = 2 } tbe_dtype;

/* flags */
#define TBE_FLAG_VALIDATE      0x1u  /* check offsets and index ranges on the
                                        device before any other work; waits
                                        for the check (host synchronisation) */
#define TBE_FLAG_FORCE_GENERIC 0x2u  /* never take the small-table path */
#define TBE_FLAG_CHECK         0x4u  /* bounds check fused into the kernels
                                        that read indices (page 1, checklist
                                        item 5): an index outside [0, E_t)
                                        is read as row 0 and sets
                                        TBE_ERROR_INDEX in *desc->error_flags;
                                        no extra pass, no host synchronisation */
#define TBE_FLAG_FUSED_LONG    0x8u  /* long runs in one launch (page 1,
                                        backward section, the third of the
                                        paths by segment length, figure 3):
                                        each chunk publishes its partial with
                                        a device-scope release and counts
                                        itself in; the last chunk of a run
                                        reduces the run's partials in chunk
                                        order and applies Adagrad. Implies
                                        TBE_FLAG_NO_HOT_ROWS; same bits as
                                        the two launches (chunk partials,
                                        then apply) under that flag. */
#define TBE_FLAG_NO_HOT_ROWS   0x10u /* no hot-row paths: the forward after the
                                        transpose gathers every row through
                                        the plain gather (by default it reads
                                        the rows of each table's longest runs
                                        from LDS, when every table has fewer
                                        than 2^24 - 1 rows), and
                                        TBE_FLAG_HOT_BACKWARD is ignored */
#define TBE_FLAG_HOT_BACKWARD  0x20u /* the backward sums the gradients of
                                        each table's up to 256 longest runs
                                        as one matrix-core contraction that
                                        reads every gradient row once (page
                                        1, the compensated f16 hi/lo
                                        contraction; f16/bf16 weights, D a
                                        multiple of 32 up to 128, fewer than
                                        2^29 lookups, every table fewer than
                                        2^24 - 1 rows; otherwise ignored),
                                        the other long runs on the chunk
                                        path. Opt-in; at the Zipf-skewed
                                        batch on gfx950 the faster of the
                                        two (0.3 ms a step at 32 tables) */

/* Bits OR-ed into *tbe_desc.error_flags under TBE_FLAG_CHECK. */
#define TBE_ERROR_INDEX 0x1u   /* some index was outside its table */

/* Execution paths chosen on the host (tbe_select_path). */
#define TBE_PATH_GENERIC     0
#define TBE_PATH_SMALL_TABLE 1

/* Stages a timer can attribute device time to. */
typedef enum {
    TBE_STAGE_FWD_POOL = 0,     /* generic forward gather-and-pool (after the
                                   transpose: the gather that reads the hot
                                   rows from LDS)                            */
    TBE_STAGE_LINEARIZE = 1,    /* sort setup: table segments and tiles       */
    TBE_STAGE_SORT = 2,         /* radix passes                               */
    TBE_STAGE_RLE_ROUTE = 3,    /* run-length encoding and routing            */
    TBE_STAGE_BWD_SHORT = 4,    /* short runs: accumulate + Adagrad + store   */
    TBE_STAGE_BWD_LONG = 5,     /* long-run chunks: partial sums to workspace
                                   (under TBE_FLAG_FUSED_LONG also the reduce
                                   and Adagrad of the long runs)             */
    TBE_STAGE_BWD_APPLY = 6,    /* long runs: reduce partials + Adagrad       */
    TBE_STAGE_SMALL_FWD = 7,    /* small-table contraction (forward output)   */
    TBE_STAGE_SMALL_BWD = 8,    /* small-table transposed contraction         */
    TBE_STAGE_SMALL_APPLY = 9,  /* small-table reduce + Adagrad               */
    TBE_STAGE_VALIDATE = 10,    /* TBE_FLAG_VALIDATE check                    */
    TBE_STAGE_LONG_SCHEDULE = 11, /* per-XCD order of the long-run chunks     */
    TBE_STAGE_SMALL_COUNT = 12, /* small-table per-bag row counts             */
    TBE_STAGE_BWD_HOT = 13,     /* hot rows: the matrix-core contraction      */
    TBE_STAGE_HOT_PLAN = 14,    /* the forward's hot-row plan (after the
                                   transpose, when the hot rows are on)       */
    TBE_STAGE_BWD_HOT_PLAN = 15, /* the backward's hot-row plan (under
                                   TBE_FLAG_HOT_BACKWARD)                     */
    TBE_NUM_STAGES = 16
} tbe_stage;

typedef struct tbe_timer tbe_timer;   /* opaque; see tbe_timer_create */

/*
 * Problem description (host struct, read during each call only).
 * T, E_t, D, B follow the notation list of page 1's backward section.
 */
typedef struct {
    int32_t T;              /* number of tables, >= 1 */
    int32_t D;              /* embedding dimension (same for every table), >= 1 */
    int32_t B;              /* bags per table (batch size), >= 0 */
    const int64_t* rows;    /* host [T]: E_t rows of table t, each >= 1 */
    tbe_dtype wdtype;       /* element type of W */
    int32_t short_max;      /* S: runs with SL < S are short; 0 means 256 */
    int32_t chunk;          /* C: lookups per long-run chunk; 0 means 256 */
    uint32_t flags;         /* TBE_FLAG_* */
    tbe_timer* timer;       /* optional stage timer, NULL for none */
    int32_t* error_flags;   /* device int32, required with TBE_FLAG_CHECK
                               (else ignored): TBE_ERROR_* bits are OR-ed in
                               by the kernels; the library never clears it.
                               Offsets must still be valid: only
                               TBE_FLAG_VALIDATE checks them. */
} tbe_desc;

/*
 * Transpose metadata (all device pointers, caller-allocated; element counts
 * from tbe_meta_capacity). Written by tbe_forward (when given a meta) or
 * tbe_preprocess, read by tbe_backward_adagrad. Page 1 ("Forward state reuse
 * and preprocessing") hoists this work into the forward and reuses it in the
 * backward; the small-table path keeps per-bag row counts instead.
 *
 * Generic path, with U runs (unique keys) over N lookups:
 *   counts[0] = U, counts[1] = n_short, counts[2] = n_long, counts[3] = n_chunks
 *   (counts[4..7] are not written on this path);
 *   run_keys[u]       linearized key of run u, strictly increasing;
 *   run_offsets[u]    first sorted slot of run u; run_offsets[U] = N;
 *   sorted_pos[k]     lookup position at sorted slot k (stable order); optional:
 *                     when NULL the sort does not carry positions (the
 *                     backward does not need them) and writes none;
 *   sorted_bag[k]     bag id t*B+b of that lookup;
 *   sorted_psw[k]     its per-sample weight (only if weighted; may be NULL
 *                     for unweighted problems);
 *   short_runs[i]     runs with SL < S, ascending;
 *   long_runs[l]      runs with SL >= S, ascending;
 *   long_chunk_begin[l] first chunk of long run l; [n_long] = n_chunks;
 *   chunk_run[c], chunk_start[c]: chunk c covers sorted slots
 *                     chunk_start[c] .. min(chunk_start[c]+C, end of its run)-1.
 * Small-table path:
 *   hist[(t*B + b)*64 + e] = min(255, count of row e in bag (t,b)), uint8,
 *                     16-byte aligned (else TBE_ERR_ARG);
 *   counts[4] flags saturation (the backward then recounts from indices);
 *   counts[5] flags counts beyond f16's exact integers (the backward then
 *   contracts in f32 arithmetic instead of on the matrix cores).
 * Pointers the chosen path does not use may be NULL.
 */
typedef struct {
    int32_t* counts;
    int32_t* run_keys;
    int32_t* run_offsets;
    int32_t* sorted_pos;
    int32_t* sorted_bag;
    float* sorted_psw;
    int32_t* short_runs;
    int32_t* long_runs;
    int32_t* long_chunk_begin;
    int32_t* chunk_run;
    int32_t* chunk_start;
    uint8_t* hist;
} tbe_meta;

/* Index of each array in the capacity vector of tbe_meta_capacity. */
enum {
    TBE_META_COUNTS = 0, TBE_META_RUN_KEYS, TBE_META_RUN_OFFSETS, TBE_META_SORTED_POS,
    TBE_META_SORTED_BAG, TBE_META_SORTED_PSW, TBE_META_SHORT_RUNS, TBE_META_LONG_RUNS,
    TBE_META_LONG_CHUNK_BEGIN, TBE_META_CHUNK_RUN, TBE_META_CHUNK_START, TBE_META_HIST,
    TBE_META_NUM_ARRAYS
};

/* Operations, for tbe_workspace_bytes. */
typedef enum {
    TBE_OP_FORWARD = 0,            /* tbe_forward with meta == NULL */
    TBE_OP_FORWARD_PREPROCESS = 1, /* tbe_forward with a meta */
    TBE_OP_PREPROCESS = 2,         /* tbe_preprocess */
    TBE_OP_BACKWARD = 3,           /* tbe_backward_adagrad with a meta */
    TBE_OP_BACKWARD_SELF = 4       /* tbe_backward_adagrad with meta == NULL */
} tbe_op;

/* Human-readable name of a status code (static string). */
const char* tbe_status_str(tbe_status s);

/*
 * After a call returned TBE_ERR_HIP: the HIP error and the step that failed;
 * after tbe_backward_adagrad_noalloc returned TBE_ERR_WORKSPACE: the scratch
 * the problem needs and the scratch there is. Text owned by the library (per
 * calling thread, valid until that thread's next failing call; empty before
 * any).
 */
const char* tbe_last_error(void);

/*
 * Which path a call with this description, lookup count and weighting takes:
 * TBE_PATH_SMALL_TABLE when every table has E_t <= 64, 64 <= D <= 128, the
 * average bag length N/(T*B) >= 64, wdtype is f16, the problem is unweighted
 * and TBE_FLAG_FORCE_GENERIC is clear (page 1, checklist item 2); else
 * TBE_PATH_GENERIC. Host only. Returns -(tbe_status) on a bad description.
 */
int32_t tbe_select_path(const tbe_desc* desc, int64_t N, int32_t weighted);

/*
 * Element counts of the tbe_meta arrays (caps[TBE_META_NUM_ARRAYS], host),
 * for the path this problem takes; 0 for arrays the path does not use. hist
 * is in bytes. Host only; returns TBE_ERR_ARG/TBE_ERR_UNSUPPORTED on a bad
 * description.
 */
tbe_status tbe_meta_capacity(const tbe_desc* desc, int64_t N, int32_t weighted,
                             int64_t* caps);

/*
 * Workspace bytes `op` needs for this problem (0 on a bad description). The
 * workspace is scratch device memory owned by the caller, 256-byte aligned;
 * its contents need not be preserved between calls. Host only.
 */
size_t tbe_workspace_bytes(const tbe_desc* desc, int64_t N, int32_t weighted, tbe_op op);

/*
 * Forward: out = pooled sums (page 1, backward section's notation; page 2,
 * section 1's fused lookup of all features). With meta != NULL it also runs
 * the preprocessing of tbe_preprocess (page 1, "Forward state reuse and
 * preprocessing": sort/RLE hoisted into the forward) or, on the small-table
 * path, saves the per-bag row counts. W, indices, offsets, psw: device, read
 * only. out: device, overwritten. ws: device workspace of at least
 * tbe_workspace_bytes(op = FORWARD or FORWARD_PREPROCESS).
 */
tbe_status tbe_forward(const tbe_desc* desc, const void* W, const int32_t* indices,
                       const int32_t* offsets, int64_t N, const float* psw, float* out,
                       tbe_meta* meta, void* ws, size_t ws_bytes, void* stream);

/*
 * Preprocessing alone (transpose_embedding_input of page 1): linearize, stable
 * sort by key, run-length encode, route runs by segment length; or, on the
 * small-table path, the per-bag row counts. Writes `meta` (device).
 */
tbe_status tbe_preprocess(const tbe_desc* desc, const int32_t* indices,
                          const int32_t* offsets, int64_t N, const float* psw,
                          tbe_meta* meta, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward with the optimizer applied in place (page 1, backward section: for
 * each unique (table,row) touched by the batch, sum the upstream gradient
 * rows of every lookup touching it, scaled by the lookup's per-sample weight
 * for weighted tables, then apply exactly one row-wise Adagrad step):
 *     g     = sum over the row's lookups of psw_j * grad_out[b_j, t*D .. t*D+D-1]
 *     m'    = m + (1/D) * sum_d g_d^2
 *     w'    = w - lr * g / (sqrt(m') + eps)
 * Rows no lookup touches are not written. W (device, in/out) and momentum
 * (device, in/out) are updated in place; grad_out, indices, offsets, psw are
 * read only. meta: the metadata a tbe_forward/tbe_preprocess call produced for
 * the same indices/offsets/psw and description, or NULL to preprocess here
 * into the workspace. ws: at least tbe_workspace_bytes(BACKWARD or
 * BACKWARD_SELF).
 */
tbe_status tbe_backward_adagrad(const tbe_desc* desc, void* W, float* momentum,
                                const float* grad_out, const int32_t* indices,
                                const int32_t* offsets, int64_t N, const float* psw,
                                const tbe_meta* meta, double lr, double eps,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * int64 indices and offsets (page 1, checklist item 6: int32 index arrays
 * halve index storage and sort-key width while the linearized range stays
 * below 2^31; beyond it they must be 64-bit). `indices` and `offsets` are
 * int64 device arrays with the same meaning and layout as above; everything
 * else is as for tbe_forward / tbe_backward_adagrad. The sum of the rows and
 * N may reach 2^63 - 1. Each table must have fewer than 2^31 - 1 rows and
 * fewer than 2^31 - 1 lookups, and B must be below 2^31 - 1; otherwise
 * TBE_ERR_UNSUPPORTED.
 *
 * The call runs as a sequence of int32 calls over groups of consecutive
 * tables whose rows, lookups and bags each stay below 2^31 - 1. Every step of
 * the method is per table, so the result is that of one call. To form the
 * groups the host reads where each table's lookups begin (T+1 offsets: one
 * synchronisation of `stream` per call). offsets[0] must be 0 and
 * offsets[T*B] must equal N, and the per-table counts must be >= 0; else
 * TBE_ERR_INDEX_RANGE. An index outside [0, 2^31 - 1) is narrowed to
 * 2^31 - 1, which lies outside every table, so TBE_FLAG_CHECK and
 * TBE_FLAG_VALIDATE report it. Under TBE_FLAG_VALIDATE every group is checked
 * before any group is computed.
 *
 * There is no metadata form: the backward preprocesses each group into the
 * workspace (the int32 calls' meta == NULL behaviour). ws: device, 256-byte
 * aligned, at least tbe_workspace_bytes_i64(op = TBE_OP_FORWARD or
 * TBE_OP_BACKWARD_SELF), which bounds the workspace of every group
 * (0 for other ops or a bad description).
 */
size_t tbe_workspace_bytes_i64(const tbe_desc* desc, int64_t N, int32_t weighted, tbe_op op);
tbe_status tbe_forward_i64(const tbe_desc* desc, const void* W, const int64_t* indices,
                           const int64_t* offsets, int64_t N, const float* psw, float* out,
                           void* ws, size_t ws_bytes, void* stream);
tbe_status tbe_backward_adagrad_i64(const tbe_desc* desc, void* W, float* momentum,
                                    const float* grad_out, const int64_t* indices,
                                    const int64_t* offsets, int64_t N, const float* psw,
                                    double lr, double eps, void* ws, size_t ws_bytes,
                                    void* stream);

/*
 * The backward with metadata (as tbe_backward_adagrad with meta != NULL), for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving or training loops, harnesses that forbid allocation. It
 * takes no workspace: its scratch (table info, chunk partials, the long-run
 * schedule and its work-queue counters, small-table split partials) is a
 * static device array of TBE_NOALLOC_SCRATCH_BYTES that the library holds on
 * each device it runs on, from the first kernel launch of the library on
 * that device until the process ends. The call allocates nothing, neither
 * on the device nor on the host.
 *
 * Limits: the problem's backward workspace, tbe_workspace_bytes(desc, N,
 * weighted, TBE_OP_BACKWARD), must be at most TBE_NOALLOC_SCRATCH_BYTES; a
 * larger one returns TBE_ERR_WORKSPACE before anything is enqueued, with the
 * sizes in tbe_last_error(). (Generic path at D = 128: about 14M lookups with
 * f16/bf16 weights, 7M with f32 weights; the small-table path at T = 64,
 * B = 32768, D = 128 takes 34 MB.) meta must not be NULL (TBE_ERR_ARG).
 *
 * All calls on one device share that device's scratch, and each call leaves
 * its contents behind; the call rewrites or clears everything it reads
 * before reading it. Two calls that may run at the same time on one device
 * (different streams, or host threads) race on the scratch and give wrong
 * results: the caller must order them, e.g. on one stream. Everything else
 * is as for tbe_backward_adagrad, with the same results bit for bit.
 */
#define TBE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
tbe_status tbe_backward_adagrad_noalloc(const tbe_desc* desc, void* W, float* momentum,
                                        const float* grad_out, const int32_t* indices,
                                        const int32_t* offsets, int64_t N, const float* psw,
                                        const tbe_meta* meta, double lr, double eps,
                                        void* stream);

/*
 * Stage timer. When desc->timer is set, each stage a call runs is bracketed by
 * HIP events recorded on the call's stream; tbe_timer_read waits for the
 * recorded events and returns, per stage, the summed device milliseconds and
 * the number of bracketed intervals since the last reset. `capacity` bounds
 * the intervals kept per stage (further ones are not recorded).
 */
tbe_status tbe_timer_create(int32_t capacity, tbe_timer** out);
tbe_status tbe_timer_reset(tbe_timer* timer);
tbe_status tbe_timer_read(tbe_timer* timer, float* ms, int32_t* intervals);
void tbe_timer_destroy(tbe_timer* timer);

#ifdef __cplusplus
}
#endif

#endif /* TBE_H */
