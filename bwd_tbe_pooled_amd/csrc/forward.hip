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
#include <algorithm>
#include <type_traits>

#include "device.h"
#include "hot_rows.h"
#include "internal.h"

namespace tbe {

namespace {

constexpr int kFwdThreads = 256;
constexpr int kFwdWaves = kFwdThreads / kWave;
constexpr int kStage = 256;  // staged lookups per wave and window

// CHECK: the bounds check fused into the gather (an index outside its table
// is read as row 0 and sets TBE_ERROR_INDEX in *err).
//
// The gather is bound by vector-ALU issue (each row piece costs an unpack and
// an FMA per element, and a wave64 instruction holds its SIMD for 4 cycles),
// so the row loop is kept to those: when a wave's bags lie in one table and
// the table is under 4 GiB (`fast`), rows are read with buffer loads at 32-bit
// byte offsets from the table's base (one address instruction per row), the
// staged indices and weights are read at fixed offsets past the slot's
// position (the staging arrays are padded for that), and rows past a bag's end
// are neither loaded nor added, so nothing is zeroed. Other waves take the
// general loop.
template <typename WT, int V, int PMAX, bool WEIGHTED, bool CHECK>
__global__ __launch_bounds__(kFwdThreads) void fwd_pool_kernel(
    const WT* __restrict__ W, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ offsets, const float* __restrict__ psw,
    const int32_t* __restrict__ toff, float* __restrict__ out, int32_t T, int32_t B, int32_t D,
    int32_t G, int32_t log2G, int32_t P, int64_t nbags, int64_t nblocks, int64_t ld,
    int32_t fast, int32_t rb_shift, int32_t* __restrict__ err) {
  using ACC = typename acc_of<WT>::type;
  using RAW = typename raw_vec<WT, V>::type;
  constexpr int UNROLL = PMAX == 1 ? 4 : 1;
  __shared__ int32_t s_idx[kFwdWaves][kStage + UNROLL];
  __shared__ float s_w[kFwdWaves][WEIGHTED ? kStage + UNROLL : 1];

  const int64_t lb = xcd_logical_block(nblocks);
  if (lb < 0) return;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
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

  // one table for the whole wave: its base and size as a buffer resource
  const int32_t tw = (int32_t)(first_bag / B);
  const bool one_table = PMAX == 1 && fast && tw == (int32_t)((last_bag - 1) / B);
  const uint32_t row_bytes = (uint32_t)D * (uint32_t)sizeof(WT);
  const uint32_t Ew = one_table ? (uint32_t)toff[T + tw] : 0u;
  const __amdgpu_buffer_rsrc_t rsrc =
      make_rsrc(W + (int64_t)(one_table ? toff[tw] : 0) * D, Ew * row_bytes);
  const uint32_t eoff = (uint32_t)(col * V) * (uint32_t)sizeof(WT);

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
    if constexpr (PMAX == 1) {
      if (one_table) {
        // row offsets by a shift (power-of-two row bytes) or a multiply,
        // chosen once per window rather than per row
        auto rows = [&](auto shift) {
          for (int32_t j = lo; j < hi; j += UNROLL) {
            const int li = j - w0;
            int32_t ix[UNROLL];
            float sc[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
              ix[u] = s_idx[wave][li + u];  // past the bag's end: read, not used
              if constexpr (WEIGHTED) sc[u] = s_w[wave][li + u];
              else sc[u] = 1.f;
              if constexpr (CHECK) {
                const bool o = j + u < hi && (uint32_t)ix[u] >= Ew;
                bad |= o;
                ix[u] = o ? 0 : ix[u];
              }
            }
            RAW buf[UNROLL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
              if (j + u < hi) {
                const uint32_t roff = decltype(shift)::value ? (uint32_t)ix[u] << rb_shift
                                                             : (uint32_t)ix[u] * row_bytes;
                buf[u] = buffer_load_raw<RAW>(rsrc, roff + eoff);
              }
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
              if (j + u < hi) {
                const ACC sv = (ACC)sc[u];
                ACC x[V];
                unpack<WT, V, ACC>(buf[u], x);
#pragma unroll
                for (int v = 0; v < V; ++v) acc[0][v] += sv * x[v];
              }
            }
          }
        };
        if (rb_shift >= 0) rows(std::true_type{});
        else rows(std::false_type{});
        continue;
      }
    }
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

// --- the forward with the transpose's hottest rows in LDS ----------------------
// When the forward runs after the transpose (tbe_forward with metadata), the
// longest runs of each table are known: those rows are read by most bags
// (page 1, the segment-length distribution; at the Zipf-skewed batch the 256
// longest runs of a table hold about three quarters of its lookups). The
// plain gather is bound by the vector memory pipeline, and LDS reads do not
// use it. So each workgroup takes hot_bags consecutive bags of one table,
// copies that table's hot rows (at most kHotBytes) into LDS once with an LDS
// hash from row to slot, and then:
// - stages a window of up to 128 lookups of its wave's bags, two per lane,
//   and splits it by ballot into a cold list (row indices) and a hot list
//   (LDS slots), both in lookup order;
// - per bag (row slot), issues up to kColdUnroll cold rows from global
//   memory first, sums its hot rows from LDS while they are in flight, then
//   adds the cold rows, so one memory latency covers most bags;
// - loads the next group's indices and offsets while this one is summed.
// A bag's sum is taken hot rows first, then cold rows, each in lookup order:
// another order than fwd_pool_kernel's, so the two agree to rounding.
constexpr int kHotBytes = 65536;      // LDS for the hot rows and one row of zeros
constexpr int kHotThreads = 512;
constexpr int kHotWaves = kHotThreads / kWave;
constexpr int kHotStage = 2 * kWave;  // staged lookups per wave and window
// rows in flight per row slot: cold 5 of 16-byte pieces (a batch is issued
// whole, and a bag averages about six cold rows at the Zipf-skewed batch:
// 3, 4, 6, 7 and 8 measured slower), 4 of 32-byte pieces (f32 rows of 128 or
// more); hot 2 of 16 or 32 bytes, 4 of smaller ones
template <int RAW_BYTES> constexpr int kColdUnroll = RAW_BYTES > 16 ? 4 : 5;
template <int RAW_BYTES> constexpr int kHotUnroll = RAW_BYTES >= 16 ? 2 : 4;
// bf16 hot rows are held in LDS widened to f32 (a bf16 is the upper half of an
// f32), so the hot lookups cost one multiply-add per element and no unpack;
// half as many rows fit. f16 rows convert inside the multiply-add anyway.
template <typename WT> constexpr bool kHotWiden = std::is_same<WT, bf16_t>::value;
template <typename WT> constexpr int kHotLdsElem = kHotWiden<WT> ? 4 : (int)sizeof(WT);

// Bits of m below this lane's (v_mbcnt: two instructions).
__device__ __forceinline__ int count_below_lane(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

template <typename WT, int V, bool WEIGHTED, bool CHECK>
__global__ __launch_bounds__(kHotThreads) __attribute__((amdgpu_waves_per_eu(4)))
void fwd_pool_hot_kernel(
    const WT* __restrict__ W, const int32_t* __restrict__ indices,
    const int32_t* __restrict__ offsets, const float* __restrict__ psw,
    const int32_t* __restrict__ tinfo, const int32_t* __restrict__ hot_rows,
    float* __restrict__ out, int32_t T, int32_t B, int32_t D, int32_t G, int32_t log2G,
    int32_t K, int32_t hot_bags, int64_t nblocks, int64_t ld, int32_t* __restrict__ err) {
  using ACC = typename acc_of<WT>::type;
  using RAW = typename raw_vec<WT, V>::type;
  constexpr bool WIDEN = kHotWiden<WT>;
  using HRAW = typename vec_bytes<V * kHotLdsElem<WT>>::type;  // a lane's piece of an LDS row
  constexpr int CU = kColdUnroll<(int)sizeof(RAW)>;
  constexpr int HU = kHotUnroll<(int)sizeof(HRAW)>;
  // hot rows in slots 0..K-1, then slot K, a row of zeros that padded lanes read
  __shared__ __align__(16) unsigned char s_rows[kHotBytes];
  __shared__ __align__(16) int32_t s_key[kHotHash];  // packed hash: row << 8 | slot
  __shared__ int32_t s_cidx[kHotWaves][kHotStage];   // cold lookups' rows, in lookup order
  __shared__ uint8_t s_hslot[kHotWaves][kHotStage];  // hot lookups' LDS slots, in lookup order
  // weights: cold lookups from the front, hot lookups from the back
  __shared__ float s_w[kHotWaves][WEIGHTED ? kHotStage : 1];
  // cold lookups before window position i, for i in [0, window length]
  __shared__ uint8_t s_cpre[kHotWaves][kHotStage + 4];

  const int64_t lb = xcd_logical_block(nblocks);
  if (lb < 0) return;
  const int64_t per_table = (B + hot_bags - 1) / hot_bags;
  const int32_t t = (int32_t)(lb / per_table);
  const int32_t bb0 = (int32_t)(lb - (int64_t)t * per_table) * hot_bags;
  const int32_t bb1 = bb0 + hot_bags < B ? bb0 + hot_bags : B;
  const int32_t first_row = tinfo[t];
  const uint32_t Et = (uint32_t)tinfo[T + t];
  const WT* __restrict__ Wt = W + (int64_t)first_row * D;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int slot = lane >> log2G;
  const int col = lane & (G - 1);
  const int NS = kWave >> log2G;
  const int last_slot_lane = (NS - 1) << log2G;
  const int row_bytes = D * (int)sizeof(WT);
  const int e = col * V;
  const bool col_ok = e < D;
  // Cold rows come through a buffer resource over the table (at most 2 GiB and
  // 2^24 rows, so a row's offset is a 24-bit product): a lane with nothing to
  // load gives an offset past the end, and the load returns zeros.
  const __amdgpu_buffer_rsrc_t wres = make_rsrc(Wt, Et * (uint32_t)row_bytes);
  constexpr uint32_t kNoRow = 0x80000000u;
  const uint32_t eb = (uint32_t)(e * (int)sizeof(WT));
  const uint32_t lrow = (uint32_t)(D * kHotLdsElem<WT>);  // LDS bytes per hot row
  const uint32_t eb_lds = col_ok ? (uint32_t)(e * kHotLdsElem<WT>) : 0u;  // lanes past the row read column 0
  const uint32_t zero_slot = (uint32_t)K;

  // hash of the table's hot rows, then the rows themselves
  for (int i = threadIdx.x; i < kHotHash; i += kHotThreads) s_key[i] = -1;
  __syncthreads();
  hot_hash_insert_packed(s_key, hot_rows + (int64_t)t * K, K);
  {
    const int n16 = K * row_bytes / 16;  // 16-byte pieces of the hot rows in memory
    for (int q = threadIdx.x; q < n16; q += kHotThreads) {
      const int k = q / (row_bytes / 16), o = q % (row_bytes / 16);
      const int32_t r = hot_rows[(int64_t)t * K + k];
      if (r >= 0) {
        const uint4 x = reinterpret_cast<const uint4*>(Wt + (int64_t)r * D)[o];
        if constexpr (WIDEN) {  // eight bf16 become eight f32: piece q lands at 32q
          reinterpret_cast<uint4*>(s_rows)[2 * q] =
              uint4{x.x << 16, x.x & 0xffff0000u, x.y << 16, x.y & 0xffff0000u};
          reinterpret_cast<uint4*>(s_rows)[2 * q + 1] =
              uint4{x.z << 16, x.z & 0xffff0000u, x.w << 16, x.w & 0xffff0000u};
        } else {
          reinterpret_cast<uint4*>(s_rows)[q] = x;
        }
      }
    }
    for (int q = threadIdx.x; q < (int)lrow / 16; q += kHotThreads)
      reinterpret_cast<uint4*>(s_rows + (size_t)K * lrow)[q] = uint4{0u, 0u, 0u, 0u};
  }
  __syncthreads();

  bool bad = false;
  const int32_t stride = kHotWaves * NS;

  // Offsets of the group of bags at g: slot s gets offsets[g+min(s,gn)] and
  // offsets[g+min(s+1,gn)], so slots past the group's end hold an empty range
  // and the last slot's end is the group's end. No group: all zero.
  auto load_offsets = [&](int32_t g, int32_t& ob, int32_t& oe) {
    ob = 0;
    oe = 0;
    if (g < bb1) {
      const int32_t gn = bb1 - g < NS ? bb1 - g : NS;
      const int64_t base = (int64_t)t * B + g;
      ob = offsets[base + (slot < gn ? slot : gn)];
      oe = offsets[base + (slot + 1 < gn ? slot + 1 : gn)];
    }
  };
  auto load_window = [&](int32_t w0, int32_t wn, int32_t (&ri)[2], float (&rw)[2]) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + r * kWave;
      ri[r] = i < wn ? indices[w0 + i] : 0;
      if constexpr (WEIGHTED) rw[r] = i < wn ? psw[w0 + i] : 0.f;
      else rw[r] = 1.f;
    }
  };
  // Split a window held in registers into the cold and hot lists, and count
  // the cold lookups before each position (s_cpre).
  auto stage = [&](const int32_t (&ri)[2], const float (&rw)[2], int32_t wn) {
    uint64_t cm[2], hm[2];  // cold and hot lookups' bits: position i at bit i % 64 of [i / 64]
    int32_t hs[2], id[2];
    // Wait for the window's loads here, outside any branch: a wait inside a
    // branch leaves the registers pending after it, and the next window's
    // loads into them would then wait for every load in flight.
    asm volatile("" ::"v"(ri[0]), "v"(ri[1]), "v"(rw[0]), "v"(rw[1]));
    bool valid[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      valid[r] = lane + r * kWave < wn;
      int32_t idx = ri[r];
      if constexpr (CHECK) {
        const bool o = valid[r] && (uint32_t)idx >= Et;
        bad |= o;
        idx = o ? 0 : idx;
      }
      id[r] = idx;
    }
    // both lookups probe the hash together, a bucket per LDS read that also
    // holds the slot
    hot_hash_find2_packed(s_key, id[0], valid[0], id[1], valid[1], hs[0], hs[1]);
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      cm[r] = __ballot(valid[r] && hs[r] < 0);
      hm[r] = __ballot(valid[r] && hs[r] >= 0);
    }
    wave_lds_sync();  // the previous window's lists have been read
    if (lane == 0) s_cpre[wave][wn] = (uint8_t)(__popcll(cm[0]) + __popcll(cm[1]));
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = lane + r * kWave;
      if (i < wn) {
        const int cpos = (r ? __popcll(cm[0]) : 0) + count_below_lane(cm[r]);  // cold before i
        s_cpre[wave][i] = (uint8_t)cpos;
        if (hs[r] < 0) {
          s_cidx[wave][cpos] = id[r];
          if constexpr (WEIGHTED) s_w[wave][cpos] = rw[r];
        } else {
          const int hpos = (r ? __popcll(hm[0]) : 0) + count_below_lane(hm[r]);
          s_hslot[wave][hpos] = (uint8_t)hs[r];
          if constexpr (WEIGHTED) s_w[wave][kHotStage - 1 - hpos] = rw[r];
        }
      }
    }
    wave_lds_sync();
  };
  // The list entries are all read before the first row load is issued (the
  // empty asm keeps the reads out of the loads' branches), so that one LDS
  // round trip, not one per row, precedes the loads.
  auto cold_batch = [&](int c, int c1, RAW (&cb)[CU], float (&cs)[CU]) {
    int32_t idx[CU];
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const int k = c + u;
      const bool ok = k < c1;
      const int kk = ok ? k : 0;
      idx[u] = s_cidx[wave][kk];
      if constexpr (WEIGHTED) cs[u] = s_w[wave][kk];
    }
    // idx and the weights are read unconditionally (the padded lanes' select
    // comes after), so the loads are not split into exec-masked ones
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      asm volatile("" ::"v"(idx[u]));
      if constexpr (WEIGHTED) asm volatile("" : "+v"(cs[u]));
    }
    if constexpr (WEIGHTED) {
#pragma unroll
      for (int u = 0; u < CU; ++u) cs[u] = c + u < c1 ? cs[u] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < CU; ++u) {
      const uint32_t off = __umul24((uint32_t)idx[u], (uint32_t)row_bytes) + eb;
      cb[u] = buffer_load_raw<RAW>(wres, c + u < c1 && col_ok ? off : kNoRow);
    }
  };
  auto add_rows = [&](ACC (&acc)[V], const auto* rb, const float* rs, auto n) {
    using R = std::remove_cv_t<std::remove_pointer_t<decltype(rb)>>;
#pragma unroll
    for (int u = 0; u < decltype(n)::value; ++u) {
      const ACC sv = (ACC)rs[u];
      ACC x[V];
      if constexpr (std::is_same<R, RAW>::value) {
        unpack<WT, V, ACC>(rb[u], x);
      } else {  // an LDS row widened to f32
        const float* f = reinterpret_cast<const float*>(&rb[u]);
#pragma unroll
        for (int v = 0; v < V; ++v) x[v] = (ACC)f[v];
      }
#pragma unroll
      for (int v = 0; v < V; ++v) {
        if constexpr (WEIGHTED) acc[v] += sv * x[v];
        else acc[v] += x[v];  // padded lanes hold zeros
      }
    }
  };
  // One window of the slot's bag [ob, oe): `pre` (the next group's loads),
  // the first cold batch, the hot rows while it is in flight, then the cold
  // batch and any further ones.
  auto window = [&](int32_t w0, int32_t wn, int32_t ob, int32_t oe, ACC (&acc)[V], auto&& pre) {
    int32_t lo = ob - w0, hi = oe - w0;
    lo = lo < 0 ? 0 : (lo > wn ? wn : lo);
    hi = hi < lo ? lo : (hi > wn ? wn : hi);
    const int c0 = s_cpre[wave][lo], c1 = s_cpre[wave][hi];
    const int h0 = lo - c0, h1 = hi - c1;
    pre();  // before the cold rows: waiting for those then covers these too
    RAW cb[CU];
    float cs[CU] = {};
    cold_batch(c0, c1, cb, cs);
    for (int k = h0; k < h1; k += HU) {
      HRAW hb[HU];
      float hsc[HU] = {};
      int hslot[HU];
#pragma unroll
      for (int u = 0; u < HU; ++u) {
        const int kk = k + u;
        const int q = kk < h1 ? kk : 0;
        hslot[u] = s_hslot[wave][q];
        if constexpr (WEIGHTED) hsc[u] = s_w[wave][kHotStage - 1 - q];
      }
      // read unconditionally (the padded lanes' select comes after), so the
      // reads are not split into exec-masked ones
#pragma unroll
      for (int u = 0; u < HU; ++u) {
        asm volatile("" ::"v"(hslot[u]));
        if constexpr (WEIGHTED) asm volatile("" : "+v"(hsc[u]));
      }
      if constexpr (WEIGHTED) {
#pragma unroll
        for (int u = 0; u < HU; ++u) hsc[u] = k + u < h1 ? hsc[u] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < HU; ++u) {
        const uint32_t sl = k + u < h1 ? hslot[u] : zero_slot;
        const unsigned char* q = s_rows + (__umul24(sl, lrow) + eb_lds);
        if constexpr (sizeof(HRAW) == 32) {  // two 16-byte LDS reads, not eight of 4
          hb[u].a = reinterpret_cast<const uint4*>(q)[0];
          hb[u].b = reinterpret_cast<const uint4*>(q)[1];
        } else {
          hb[u] = *reinterpret_cast<const HRAW*>(q);
        }
      }
      add_rows(acc, hb, hsc, std::integral_constant<int, HU>{});
    }
    add_rows(acc, cb, cs, std::integral_constant<int, CU>{});
    for (int c = c0 + CU; c < c1; c += CU) {
      cold_batch(c, c1, cb, cs);
      add_rows(acc, cb, cs, std::integral_constant<int, CU>{});
    }
  };

  const int32_t g_first = bb0 + wave * NS;
  int32_t cur_b, cur_e, nxt_b, nxt_e;
  load_offsets(g_first, cur_b, cur_e);
  load_offsets(g_first + stride, nxt_b, nxt_e);
  int32_t ri[2];
  float rw[2];
  {
    const int32_t J0 = __builtin_amdgcn_readlane(cur_b, 0);
    const int32_t J1 = __builtin_amdgcn_readlane(cur_e, last_slot_lane);
    load_window(J0, J1 - J0 < kHotStage ? J1 - J0 : kHotStage, ri, rw);
    // waited for here, so that inside the loop they are never the last loads
    // in flight (the wait in `stage` would then also wait for the stores)
    asm volatile("" ::"v"(ri[0]), "v"(ri[1]), "v"(rw[0]), "v"(rw[1]));
  }
  for (int32_t g = g_first; g < bb1; g += stride) {
    const int32_t J0 = __builtin_amdgcn_readlane(cur_b, 0);
    const int32_t J1 = __builtin_amdgcn_readlane(cur_e, last_slot_lane);
    const int32_t nJ0 = __builtin_amdgcn_readlane(nxt_b, 0);
    const int32_t nJ1 = __builtin_amdgcn_readlane(nxt_e, last_slot_lane);
    ACC acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = (ACC)0;
    const int32_t wn0 = J1 - J0 < kHotStage ? J1 - J0 : kHotStage;
    stage(ri, rw, wn0);
    int32_t n2_b, n2_e;
    window(J0, wn0, cur_b, cur_e, acc, [&]() {
      load_window(nJ0, nJ1 - nJ0 < kHotStage ? nJ1 - nJ0 : kHotStage, ri, rw);
      load_offsets(g + 2 * stride, n2_b, n2_e);
    });
    for (int32_t w0 = J0 + kHotStage; w0 < J1; w0 += kHotStage) {  // bags longer than a window
      const int32_t wn = J1 - w0 < kHotStage ? J1 - w0 : kHotStage;
      int32_t xi[2];
      float xw[2];
      load_window(w0, wn, xi, xw);
      stage(xi, xw, wn);
      window(w0, wn, cur_b, cur_e, acc, []() {});
    }
    const int32_t gn = bb1 - g < NS ? bb1 - g : NS;
    if (slot < gn && col_ok) {
      float* o = out + (int64_t)(g + slot) * ld + (int64_t)t * D;
      typename vec_bytes<V * 4>::type ov;
      float* of = reinterpret_cast<float*>(&ov);
#pragma unroll
      for (int v = 0; v < V; ++v) of[v] = (float)acc[v];
      store_stream(reinterpret_cast<decltype(ov)*>(o + e), ov);
    }
    cur_b = nxt_b;
    cur_e = nxt_e;
    nxt_b = n2_b;
    nxt_e = n2_e;
  }
  if constexpr (CHECK) {
    if (__ballot(bad) != 0 && lane == 0) atomicOr(err, (int32_t)TBE_ERROR_INDEX);
  }
}

template <typename WT, int V>
hipError_t launch_hot_typed(const Problem& p, const RowShape& rs, const void* W,
                            const int32_t* indices, const int32_t* offsets, const float* psw,
                            const int32_t* tinfo, const int32_t* hot_rows, float* out,
                            hipStream_t s) {
  const int64_t lrow = (int64_t)p.D * kHotLdsElem<WT>;
  // the hot rows and the zero row after them fit the kernel's LDS
  if ((int64_t)(p.hot_k + 1) * lrow > kHotBytes || p.hot_k > kHotMaxK || p.hot_k < 1)
    return hipErrorInvalidValue;
  const int64_t per_table = (p.B + p.hot_bags - 1) / p.hot_bags;
  const int64_t nblocks = per_table * p.T;
  if (nblocks == 0) return hipSuccess;
  const dim3 grid((unsigned)xcd_grid(nblocks));
#define TBE_FWD_HOT(WGT, CHK)                                                                   \
  hipLaunchKernelGGL((fwd_pool_hot_kernel<WT, V, WGT, CHK>), grid, dim3(kHotThreads), 0, s,     \
                     (const WT*)W, indices, offsets, psw, tinfo, hot_rows, out, p.T, p.B, p.D,  \
                     rs.G, rs.log2G, p.hot_k, p.hot_bags, nblocks, p.ld, p.err)
  if (psw) {
    if (p.err) TBE_FWD_HOT(true, true);
    else TBE_FWD_HOT(true, false);
  } else {
    if (p.err) TBE_FWD_HOT(false, true);
    else TBE_FWD_HOT(false, false);
  }
#undef TBE_FWD_HOT
  return hipGetLastError();
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
  // every table's bytes addressable with 32-bit offsets
  const int32_t fast = p.max_rows * p.D * (int64_t)sizeof(WT) <= (int64_t)0xffffffff ? 1 : 0;
  const int64_t rb = (int64_t)p.D * (int64_t)sizeof(WT);
  int32_t rb_shift = -1;  // log2 of the row bytes when a power of two
  for (int sh = 0; sh < 31; ++sh)
    if (((int64_t)1 << sh) == rb) rb_shift = sh;
#define TBE_FWD(WGT, CHK)                                                                      \
  hipLaunchKernelGGL((fwd_pool_kernel<WT, V, PMAX, WGT, CHK>), grid, dim3(kFwdThreads), 0, s,  \
                     (const WT*)W, indices, offsets, psw, toff, out, p.T, p.B, p.D, rs.G,      \
                     rs.log2G, rs.P, p.nbags, nblocks, p.ld, fast, rb_shift, p.err)
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

// 16-byte pieces per lane: 8 elements of 2 bytes, 4 of f32 (32-byte pieces of
// f32 rows would not fit the unrolled loads in 128 registers)
constexpr int hot_max_v(size_t elem_bytes) { return elem_bytes == 4 ? 4 : 8; }

template <typename WT>
hipError_t launch_hot_for_type(const Problem& p, const void* W, const int32_t* indices,
                               const int32_t* offsets, const float* psw, const int32_t* tinfo,
                               const int32_t* hot_rows, float* out, hipStream_t s) {
  const RowShape rs = row_shape(p.D, hot_max_v(sizeof(WT)));
  if (rs.P != 1) return hipErrorInvalidValue;
  if constexpr (sizeof(WT) == 2) {
    if (rs.V == 8) return launch_hot_typed<WT, 8>(p, rs, W, indices, offsets, psw, tinfo, hot_rows, out, s);
  }
  if (rs.V == 4) return launch_hot_typed<WT, 4>(p, rs, W, indices, offsets, psw, tinfo, hot_rows, out, s);
  if (rs.V == 2) return launch_hot_typed<WT, 2>(p, rs, W, indices, offsets, psw, tinfo, hot_rows, out, s);
  return launch_hot_typed<WT, 1>(p, rs, W, indices, offsets, psw, tinfo, hot_rows, out, s);
}

}  // namespace

// Hot rows per table for the forward after the transpose: as many as fit in
// kHotBytes of LDS (bf16 rows widened to f32) with a row of zeros after them,
// at most 256 (the hash stays at most a quarter full); 0 when the row is not
// one pass of 16-byte multiples or the grid would be too small.
void choose_hot(Problem* p) {
  p->hot_k = 0;
  p->hot_bags = 0;
  const int64_t wbytes = p->wdtype == TBE_F32 ? 4 : 2;
  const int64_t row = p->D * wbytes;
  if (p->no_hot || p->path != TBE_PATH_GENERIC || row % 16 != 0 || row_shape(p->D, hot_max_v(wbytes)).P != 1)
    return;
  // cold rows are read at 32-bit offsets below 2^31, rows numbered in 24 bits
  // (below 2^24 - 1: the hash packs row << 8 | slot in 32 bits)
  if (p->max_rows >= (int64_t(1) << 24) - 1 || p->max_rows * row >= (int64_t(1) << 31)) return;
  const int64_t lrow = p->D * (p->wdtype == TBE_BF16 ? kHotLdsElem<bf16_t> : wbytes);
  const int64_t k = std::min<int64_t>(256, kHotBytes / lrow - 1);  // and the zero row
  if (k < 16 || p->B < 1) return;
  int32_t bags = 2048;  // halve until the grid holds about four workgroups per CU
  while (bags > 256 && (int64_t)p->T * ((p->B + bags - 1) / bags) < 1024) bags /= 2;
  if ((int64_t)p->T * ((p->B + bags - 1) / bags) < 256) return;
  p->hot_k = (int32_t)k;
  p->hot_bags = bags;
}

hipError_t launch_forward_pool_hot(const Problem& p, const void* W, const int32_t* indices,
                                   const int32_t* offsets, const float* psw, const int32_t* tinfo,
                                   const int32_t* hot_rows, float* out, hipStream_t s) {
  switch (p.wdtype) {
    case TBE_F32: return launch_hot_for_type<float>(p, W, indices, offsets, psw, tinfo, hot_rows, out, s);
    case TBE_F16: return launch_hot_for_type<f16_t>(p, W, indices, offsets, psw, tinfo, hot_rows, out, s);
    case TBE_BF16: return launch_hot_for_type<bf16_t>(p, W, indices, offsets, psw, tinfo, hot_rows, out, s);
  }
  return hipErrorInvalidValue;
}

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
