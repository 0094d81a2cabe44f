/*
 * CPU oracle for the table-batched embedding (TBE) training hot path.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code, header or table with the HIP library.
 *
 * It is written to be read against the FBTriton TBE tutorial (page 1 of the
 * sources) and checked by eye: one thread, plain loops, every floating-point
 * quantity in double, the C library's qsort as the sorting primitive.
 *
 * What it computes (page 1, "Backward kernel" section and its notation list;
 * page 2, section 1 for the jagged layout):
 *   - linearize:  key_j = first row of table t + indices[j], bag_j = t*B + b,
 *                 after checking offsets and index ranges;
 *   - forward:    out[b, t*D + d] = sum over j in bag (t,b) of s_j * W[key_j, d]
 *                 with s_j the per-sample weight or 1 (weighted tables scale the
 *                 gradient row by the same per-sample weight, "Weighted tables");
 *   - sort:       the stable ascending order of lookups by key
 *                 ("transpose_embedding_input");
 *   - rle:        runs of equal keys: unique key, start offset, segment length;
 *   - route:      runs with SL < S are short; the others are long and are cut
 *                 into consecutive chunks of C lookups (page 1, the three
 *                 routing paths; S = C = 256 on the page);
 *   - backward:   per run, g = sum of s_k * (upstream gradient row of the bag of
 *                 lookup k), then exactly one row-wise Adagrad step on that row
 *                 (page 1, the core statement of the backward and the opening
 *                 paragraph on exact row-wise Adagrad):
 *                     m' = m + (1/D) * sum_d g_d^2
 *                     w' = w - lr * g / (sqrt(m') + eps)
 *   - histogram:  per bag, how many of its lookups hit each row (the counts the
 *                 small-table path keeps from the forward, page 1, first
 *                 section and decision item 2).
 * The formula of the Adagrad step is not printed on the pages; the reading
 * used here (mean of squares, eps outside the root, updated m in the
 * denominator) is the one a one-column row reduces to torch.optim.Adagrad.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG 1
#define OR_ERR_OFFSETS 2
#define OR_ERR_INDEX 3
#define OR_ERR_ROW_MISSING 4
#define OR_ERR_NOMEM 5

#define OR_F32 0
#define OR_F16 1
#define OR_BF16 2

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* Value of an IEEE binary16 bit pattern. */
static double half_bits_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (exp == 0)
        v = ldexp((double)man, -24);                 /* subnormal: man * 2^-24 */
    else if (exp == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(man + 1024), exp - 25);   /* (1.man) * 2^(exp-15) */
    return sign ? -v : v;
}

/* Value of a bfloat16 bit pattern: the top half of a binary32. */
static double bf16_bits_to_double(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void *base, int dtype, int64_t i) {
    if (dtype == OR_F32) return (double)((const float *)base)[i];
    if (dtype == OR_F16) return half_bits_to_double(((const uint16_t *)base)[i]);
    return bf16_bits_to_double(((const uint16_t *)base)[i]);
}

/*
 * Round x to the nearest value of a binary format with `p` significand bits
 * (implicit bit included), minimum normal exponent `emin` and largest finite
 * value `maxv`; ties go to the even neighbour. The quantum at x's binade is
 * 2^(e - p + 1) (fixed at the subnormal quantum below emin); x / quantum is
 * exact in double, and rint() rounds half to even in the default mode.
 */
static double round_to_format(double x, int p, int emin, double maxv) {
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e = ilogb(x);
    if (e < emin) e = emin;
    double q = ldexp(1.0, e - p + 1);
    double r = rint(x / q) * q;
    if (fabs(r) > maxv) return r > 0 ? INFINITY : -INFINITY;
    return r;
}

double or_round(double x, int dtype) {
    if (dtype == OR_F16) return round_to_format(x, 11, -14, 65504.0);
    if (dtype == OR_BF16)
        return round_to_format(x, 8, -126, ldexp(255.0, 120));   /* (2-2^-7)*2^127 */
    return round_to_format(x, 24, -126, ldexp(16777215.0, 104)); /* FLT_MAX */
}

void or_round_array(const double *x, int64_t n, int dtype, double *y) {
    for (int64_t i = 0; i < n; i++) y[i] = or_round(x[i], dtype);
}

void or_decode_array(const void *src, int64_t n, int dtype, double *y) {
    for (int64_t i = 0; i < n; i++) y[i] = load_elem(src, dtype, i);
}

/* ------------------------------------------------------------------------ */
/* Row store: weights (and optimizer state) addressed by linearized key.     */
/* If `keys` is NULL, row r of `data` is key r. Otherwise `keys` is sorted   */
/* ascending and row r of `data` belongs to keys[r] (lets a caller hand over */
/* only the rows a sample touches).                                          */
/* ------------------------------------------------------------------------ */
static int64_t store_row(const int32_t *keys, int64_t n, int32_t key) {
    if (!keys) return key;
    int64_t lo = 0, hi = n - 1;
    while (lo <= hi) {
        int64_t mid = lo + (hi - lo) / 2;
        if (keys[mid] == key) return mid;
        if (keys[mid] < key) lo = mid + 1; else hi = mid - 1;
    }
    return -1;
}

/* ------------------------------------------------------------------------ */
/* Step 1: validate and linearize.                                          */
/* ------------------------------------------------------------------------ */
int or_linearize(int32_t T, int32_t B, const int64_t *rows, int64_t N,
                 const int32_t *indices, const int32_t *offsets,
                 int32_t *keys, int32_t *bags) {
    if (T <= 0 || B < 0 || N < 0) return OR_ERR_ARG;
    int64_t nbags = (int64_t)T * B;
    if (offsets[0] != 0 || offsets[nbags] != N) return OR_ERR_OFFSETS;
    for (int64_t i = 0; i < nbags; i++)
        if (offsets[i + 1] < offsets[i]) return OR_ERR_OFFSETS;
    int64_t first_row = 0;
    for (int32_t t = 0; t < T; t++) {
        for (int64_t b = 0; b < B; b++) {
            int64_t bag = (int64_t)t * B + b;
            for (int64_t j = offsets[bag]; j < offsets[bag + 1]; j++) {
                if (indices[j] < 0 || indices[j] >= rows[t]) return OR_ERR_INDEX;
                keys[j] = (int32_t)(first_row + indices[j]);
                bags[j] = (int32_t)bag;
            }
        }
        first_row += rows[t];
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 2: forward pooling of selected bags.                                 */
/* out_row[s*D + d] = sum_{j in bag bag_ids[s]} s_j * W[key_j, d]            */
/* ------------------------------------------------------------------------ */
int or_forward_bags(int32_t D, int dtype, const int32_t *offsets,
                    const int32_t *keys, const float *psw,
                    const int32_t *wkeys, int64_t nw, const void *wdata,
                    int64_t nsel, const int32_t *bag_ids, double *out) {
    for (int64_t s = 0; s < nsel; s++) {
        double *o = out + s * D;
        for (int32_t d = 0; d < D; d++) o[d] = 0.0;
        int32_t bag = bag_ids[s];
        for (int64_t j = offsets[bag]; j < offsets[bag + 1]; j++) {
            int64_t r = store_row(wkeys, nw, keys[j]);
            if (r < 0) return OR_ERR_ROW_MISSING;
            double sj = psw ? (double)psw[j] : 1.0;
            for (int32_t d = 0; d < D; d++)
                o[d] += sj * load_elem(wdata, dtype, r * D + d);
        }
    }
    return OR_OK;
}

/* Whole forward: out is [B, T*D]; bag i = t*B + b lands in row b, columns t*D... */
int or_forward(int32_t T, int32_t B, int32_t D, int dtype, const int32_t *offsets,
               const int32_t *keys, const float *psw,
               const int32_t *wkeys, int64_t nw, const void *wdata, double *out) {
    for (int32_t t = 0; t < T; t++) {
        for (int32_t b = 0; b < B; b++) {
            int32_t bag = t * B + b;
            int rc = or_forward_bags(D, dtype, offsets, keys, psw, wkeys, nw, wdata,
                                     1, &bag, out + ((int64_t)b * T + t) * D);
            if (rc) return rc;
        }
    }
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 3: stable sort of lookups by key. Sorting (key, position) pairs      */
/* lexicographically is a total order, so the result is the stable order.   */
/* ------------------------------------------------------------------------ */
typedef struct { int32_t key; int32_t pos; } or_pair;

static int cmp_pair(const void *a, const void *b) {
    const or_pair *x = (const or_pair *)a, *y = (const or_pair *)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    if (x->pos != y->pos) return x->pos < y->pos ? -1 : 1;
    return 0;
}

int or_sort(int64_t N, const int32_t *keys, int32_t *sorted_pos) {
    or_pair *p = (or_pair *)malloc((size_t)(N > 0 ? N : 1) * sizeof *p);
    if (!p) return OR_ERR_NOMEM;
    for (int64_t j = 0; j < N; j++) { p[j].key = keys[j]; p[j].pos = (int32_t)j; }
    qsort(p, (size_t)N, sizeof *p, cmp_pair);
    for (int64_t k = 0; k < N; k++) sorted_pos[k] = p[k].pos;
    free(p);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 4: run-length encoding of the sorted keys.                           */
/* Returns U; run u holds sorted slots run_offsets[u] .. run_offsets[u+1]-1. */
/* Also permutes bag ids and per-sample weights into sorted order.           */
/* ------------------------------------------------------------------------ */
int64_t or_rle(int64_t N, const int32_t *keys, const int32_t *sorted_pos,
               const int32_t *bags, const float *psw,
               int32_t *run_keys, int32_t *run_offsets,
               int32_t *sorted_bag, float *sorted_psw) {
    int64_t U = 0;
    for (int64_t k = 0; k < N; k++) {
        int32_t key = keys[sorted_pos[k]];
        if (k == 0 || key != run_keys[U - 1]) {
            run_keys[U] = key;
            run_offsets[U] = (int32_t)k;
            U++;
        }
        sorted_bag[k] = bags[sorted_pos[k]];
        if (psw && sorted_psw) sorted_psw[k] = psw[sorted_pos[k]];
    }
    run_offsets[U] = (int32_t)N;
    return U;
}

/* ------------------------------------------------------------------------ */
/* Step 5: routing by segment length.                                        */
/* counts_out = {n_short, n_long, n_chunks}. long_chunk_begin[l] is the      */
/* first chunk of long run l (and long_chunk_begin[n_long] = n_chunks).      */
/* ------------------------------------------------------------------------ */
int or_route(int64_t U, const int32_t *run_offsets, int32_t S, int32_t C,
             int32_t *short_runs, int32_t *long_runs, int32_t *long_chunk_begin,
             int32_t *chunk_run, int32_t *chunk_start, int64_t *counts_out) {
    if (S < 1 || C < 1) return OR_ERR_ARG;
    int64_t ns = 0, nl = 0, nc = 0;
    for (int64_t u = 0; u < U; u++) {
        int64_t sl = (int64_t)run_offsets[u + 1] - run_offsets[u];
        if (sl < S) {
            short_runs[ns++] = (int32_t)u;
        } else {
            long_chunk_begin[nl] = (int32_t)nc;
            long_runs[nl++] = (int32_t)u;
            for (int64_t a = run_offsets[u]; a < run_offsets[u + 1]; a += C) {
                chunk_run[nc] = (int32_t)u;
                chunk_start[nc] = (int32_t)a;
                nc++;
            }
        }
    }
    long_chunk_begin[nl] = (int32_t)nc;
    counts_out[0] = ns;
    counts_out[1] = nl;
    counts_out[2] = nc;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Step 6+7: per-run gradient and one row-wise Adagrad step per run.         */
/* grad is the upstream gradient [B, T*D]; the bag i = t*B + b of a lookup   */
/* selects row b, columns t*D .. t*D+D-1.                                    */
/* Writes, per run u: g[u, :] (optional), the updated row w_new[u, :] and    */
/* state m_new[u], all unrounded doubles. Untouched rows are never visited.  */
/* m_data[r] is the state of store row r (same addressing as the weights).   */
/* ------------------------------------------------------------------------ */
int or_backward_adagrad(int32_t T, int32_t B, int32_t D, int dtype,
                        int64_t U, const int32_t *run_keys, const int32_t *run_offsets,
                        const int32_t *sorted_bag, const float *sorted_psw,
                        const float *grad,
                        const int32_t *wkeys, int64_t nw, const void *wdata,
                        const float *m_data, double lr, double eps,
                        double *g_out, double *w_new, double *m_new) {
    double *g = (double *)malloc((size_t)(D > 0 ? D : 1) * sizeof *g);
    if (!g) return OR_ERR_NOMEM;
    for (int64_t u = 0; u < U; u++) {
        for (int32_t d = 0; d < D; d++) g[d] = 0.0;
        for (int64_t k = run_offsets[u]; k < run_offsets[u + 1]; k++) {
            int64_t bag = sorted_bag[k];
            int64_t t = bag / B, b = bag % B;
            const float *row = grad + (b * T + t) * D;
            double s = sorted_psw ? (double)sorted_psw[k] : 1.0;
            for (int32_t d = 0; d < D; d++) g[d] += s * (double)row[d];
        }
        int64_t r = store_row(wkeys, nw, run_keys[u]);
        if (r < 0) { free(g); return OR_ERR_ROW_MISSING; }
        double sumsq = 0.0;
        for (int32_t d = 0; d < D; d++) sumsq += g[d] * g[d];
        double m1 = (double)m_data[r] + sumsq / D;
        double denom = sqrt(m1) + eps;
        for (int32_t d = 0; d < D; d++) {
            double w0 = load_elem(wdata, dtype, r * D + d);
            w_new[u * D + d] = w0 - lr * g[d] / denom;
            if (g_out) g_out[u * D + d] = g[d];
        }
        m_new[u] = m1;
    }
    free(g);
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* Small-table counts: H[(t*B + b)*E + e] = #lookups of bag (t,b) on row e.  */
/* ------------------------------------------------------------------------ */
int or_histogram(int32_t T, int32_t B, int32_t E, const int64_t *rows,
                 const int32_t *indices, const int32_t *offsets, int32_t *H) {
    int64_t nbags = (int64_t)T * B;
    for (int64_t i = 0; i < nbags * E; i++) H[i] = 0;
    for (int64_t bag = 0; bag < nbags; bag++) {
        int64_t t = bag / B;
        for (int64_t j = offsets[bag]; j < offsets[bag + 1]; j++) {
            if (indices[j] < 0 || indices[j] >= rows[t] || indices[j] >= E)
                return OR_ERR_INDEX;
            H[bag * E + indices[j]] += 1;
        }
    }
    return OR_OK;
}
