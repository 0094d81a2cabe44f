// A table's hot rows: the rows of its longest runs, known once the transpose
// has run (page 1, the segment-length distribution: at the Zipf-skewed batch
// the 256 longest runs of a table hold about three quarters of its lookups).
// The forward after the transpose reads them from LDS, and the backward sums
// their gradients on the matrix cores. Both find a lookup's hot slot through
// an LDS hash of the table's hot rows, built here.
#pragma once

#include "device.h"

namespace tbe {

constexpr int kHotMaxK = 256;         // hot rows per table at most (slots fit a byte)
constexpr int kHotBuckets = 256;      // hash buckets of 4 rows
constexpr int kHotHash = 4 * kHotBuckets;

// Bucket of a row: the top 8 bits of a multiplicative hash. A bucket holds 4
// rows (one 16-byte LDS read); a full bucket spills into the next one, so a
// lookup stops at the first bucket that holds it or has an empty entry.
__device__ __forceinline__ uint32_t hot_bucket(int32_t row) {
  return ((uint32_t)row * 0x9E3779B1u) >> 24;
}

// The hash (s_key[kHotHash], 16-byte aligned) packs each entry as
// row << 8 | slot, for tables of fewer than 2^24 - 1 rows, so the read of a
// bucket yields the slot as well, with no second, dependent read. With
// rk = row << 8, the entry minus rk (mod 2^32) is the slot (below 256) for the
// row's own entry, and at least 256 for another row's entry (rows differ by a
// nonzero multiple of 256 below 2^32) and for an empty one (-1 minus rk is at
// least 511 when row <= 2^24 - 2). Filled from rows[0..K) (entries < 0 being
// empty slots, the others below 2^24 - 1) by every thread of the workgroup
// between two barriers: s_key must be all -1 before (the caller clears it and
// synchronises), and is complete after the caller's next barrier.
__device__ __forceinline__ void hot_hash_insert_packed(int32_t* s_key,
                                                       const int32_t* __restrict__ rows, int K) {
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    const int32_t r = rows[k];
    if (r < 0) continue;
    const int32_t entry = (int32_t)(((uint32_t)r << 8) | (uint32_t)k);
    uint32_t h = hot_bucket(r) * 4;
    for (;;) {  // at most 256 rows in 1024 entries: a free entry exists
      if (atomicCAS(&s_key[h], -1, entry) == -1) break;
      h = (h + 1) & (kHotHash - 1);
    }
  }
}

// The slot held for rk = row << 8 in bucket q, or a value >= 256.
__device__ __forceinline__ uint32_t hot_packed_match(const int4& q, uint32_t rk) {
  const uint32_t d0 = (uint32_t)q.x - rk, d1 = (uint32_t)q.y - rk;
  const uint32_t d2 = (uint32_t)q.z - rk, d3 = (uint32_t)q.w - rk;
  return min(min(d0, d1), min(d2, d3));
}

// Slots of two rows in the packed hash (-1: not hot, or `go` false).
__device__ __forceinline__ void hot_hash_find2_packed(const int32_t* s_key, int32_t r0, bool go0,
                                                      int32_t r1, bool go1, int& slot0,
                                                      int& slot1) {
  uint32_t b0 = hot_bucket(r0), b1 = hot_bucket(r1);
  const uint32_t k0 = (uint32_t)r0 << 8, k1 = (uint32_t)r1 << 8;
  const bool v0 = go0, v1 = go1;
  uint32_t m0, m1;
  {  // the first probe of both, without branches: most searches end there
    int4 q0 = reinterpret_cast<const int4*>(s_key)[b0];
    int4 q1 = reinterpret_cast<const int4*>(s_key)[b1];
    // all eight words as loaded, so that the compares are not turned into a
    // second, dependent read of the words past the first
    asm volatile("" : "+v"(q0.x), "+v"(q0.y), "+v"(q0.z), "+v"(q0.w));
    asm volatile("" : "+v"(q1.x), "+v"(q1.y), "+v"(q1.z), "+v"(q1.w));
    m0 = hot_packed_match(q0, k0);
    m1 = hot_packed_match(q1, k1);
    go0 = go0 && m0 >= 256u && q0.w != -1;  // entries fill in order: an empty one ends the search
    go1 = go1 && m1 >= 256u && q1.w != -1;
  }
  while (go0 || go1) {  // a full bucket: the search goes on in the next
    if (go0) {
      b0 = (b0 + 1) & (kHotBuckets - 1);
      const int4 q = reinterpret_cast<const int4*>(s_key)[b0];
      m0 = hot_packed_match(q, k0);
      go0 = m0 >= 256u && q.w != -1;
    }
    if (go1) {
      b1 = (b1 + 1) & (kHotBuckets - 1);
      const int4 q = reinterpret_cast<const int4*>(s_key)[b1];
      m1 = hot_packed_match(q, k1);
      go1 = m1 >= 256u && q.w != -1;
    }
  }
  slot0 = v0 && m0 < 256u ? (int)m0 : -1;
  slot1 = v1 && m1 < 256u ? (int)m1 : -1;
}

}  // namespace tbe
