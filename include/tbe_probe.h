/*
 * tbe_probe.h — measurement aid of the TBE library (not part of the method).
 *
 * The forward gather and the backward's gradient gathers each read one row
 * per lookup at random; on a skewed batch most of those rows come from L2,
 * so their speed is bounded by the rate at which the compute units can
 * gather rows that L2 holds, not by HBM. This probe measures that rate on
 * the running device: it reads `n` rows of `row_floats` float32 values,
 * row rows[i] of `src` for i = 0 .. n-1, with the same load shape as the
 * library's gathers (16 bytes per lane, 16 lanes per 256-byte line pair,
 * eight rows in flight per 16-lane slot), sums them and writes one float per
 * wave to `sink`. With `src` small enough to stay in every XCD's L2 (a few MB)
 * and n large, n * row_floats * 4 bytes over the launch time is the L2
 * row-gather ceiling for that row size.
 *
 *   src      device float32 [src_rows, row_floats], read only
 *   rows     device int32 [n], each in [0, src_rows); not checked
 *   sink     device float32 [TBE_PROBE_SINK_FLOATS], overwritten
 *   row_floats  64, 128 or 256 (256, 512 or 1024 bytes), else TBE_ERR_ARG
 *
 * Enqueued on `stream`, no host synchronisation; allocates nothing.
 */
#ifndef TBE_PROBE_H
#define TBE_PROBE_H

#include "tbe.h"

#ifdef __cplusplus
extern "C" {
#endif

#define TBE_PROBE_SINK_FLOATS 16384

tbe_status tbe_probe_row_gather(const float* src, int64_t src_rows, int32_t row_floats,
                                const int32_t* rows, int64_t n, float* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TBE_PROBE_H */
