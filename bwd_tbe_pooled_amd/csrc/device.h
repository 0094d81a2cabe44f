// Device-side helpers shared by the gfx950 kernels: element conversions,
// vector row loads/stores, wavefront reductions (DPP inside 16-lane rows,
// cross-row shuffles) and the XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tbe {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Element types. f16 and bf16 weights are handled as raw 16-bit patterns.
// ---------------------------------------------------------------------------
struct f16_t { uint16_t bits; };
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_float(f16_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, h.bits);
  return (float)v;
}
__device__ __forceinline__ float to_float(bf16_t h) {
  return __uint_as_float((uint32_t)h.bits << 16);
}
__device__ __forceinline__ float to_float(float f) { return f; }

__device__ __forceinline__ double to_double(f16_t h) { return (double)to_float(h); }
__device__ __forceinline__ double to_double(bf16_t h) { return (double)to_float(h); }
__device__ __forceinline__ double to_double(float f) { return (double)f; }

// Round-to-nearest-even narrowing conversions.
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32 honours the default RNE mode
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  uint32_t lsb = (u >> 16) & 1u;
  return (uint16_t)((u + 0x7fffu + lsb) >> 16);
}

// Accumulator type per weight type: f16/bf16 -> float, f32 -> double.
template <typename WT> struct acc_of { using type = float; };
template <> struct acc_of<float> { using type = double; };

template <typename ACC> __device__ __forceinline__ ACC cvt_acc(float x) { return (ACC)x; }

// Store an updated value (accumulator precision) into the weight type.
__device__ __forceinline__ void store_w(float* p, double v) { *p = (float)v; }
__device__ __forceinline__ void store_w(f16_t* p, float v) { p->bits = f32_to_f16_bits(v); }
__device__ __forceinline__ void store_w(bf16_t* p, float v) { p->bits = f32_to_bf16_bits(v); }

// ---------------------------------------------------------------------------
// Vector loads of V consecutive elements (V*sizeof(T) bytes, naturally
// aligned by construction: rows start at multiples of D elements and V | D).
// ---------------------------------------------------------------------------
template <int BYTES> struct vec_bytes;
template <> struct vec_bytes<2> { using type = uint16_t; };
template <> struct vec_bytes<4> { using type = uint32_t; };
template <> struct vec_bytes<8> { using type = uint2; };
template <> struct vec_bytes<16> { using type = uint4; };
template <> struct vec_bytes<32> { struct type { uint4 a, b; }; };
template <> struct vec_bytes<64> { struct type { uint4 a, b, c, d; }; };

template <typename T, int V>
struct raw_vec {
  using type = typename vec_bytes<V * (int)sizeof(T)>::type;
};

// Nontemporal store for data written once and not read again by the same
// kernel (pooled outputs, updated rows): it leaves the L2 to the rows that
// are re-read.
template <typename R>
__device__ __forceinline__ void store_stream(R* p, const R& v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  if constexpr (sizeof(R) == 32) {
    const u32x4* s = reinterpret_cast<const u32x4*>(&v);
    __builtin_nontemporal_store(s[0], reinterpret_cast<u32x4*>(p));
    __builtin_nontemporal_store(s[1], reinterpret_cast<u32x4*>(p) + 1);
  } else if constexpr (sizeof(R) == 16) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4*>(p));
  } else if constexpr (sizeof(R) == 8) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x2, v), reinterpret_cast<u32x2*>(p));
  } else if constexpr (sizeof(R) == 4) {
    __builtin_nontemporal_store(__builtin_bit_cast(uint32_t, v), reinterpret_cast<uint32_t*>(p));
  } else {
    static_assert(sizeof(R) == 2, "store_stream: 2, 4, 8, 16 or 32 bytes");
    __builtin_nontemporal_store(__builtin_bit_cast(uint16_t, v), reinterpret_cast<uint16_t*>(p));
  }
}

// Plain (cached) load: weight rows and gradient rows are both re-read many
// times per batch (hot rows, and every lookup of a bag), so they go through L2.
template <typename T, int V>
__device__ __forceinline__ typename raw_vec<T, V>::type load_vec(const T* p) {
  using R = typename raw_vec<T, V>::type;
  return *reinterpret_cast<const R*>(p);
}

// Buffer resource over `bytes` bytes from `base` (raw, stride 0). A load at
// an offset at or past `bytes` returns zeros instead of faulting.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// Raw buffer load of 2 to 32 bytes at byte offset `off` of the resource.
template <typename R>
__device__ __forceinline__ R buffer_load_raw(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (sizeof(R) == 32) {
    struct P { uint4 a, b; };
    static_assert(sizeof(P) == 32, "32-byte piece");
    P p;
    p.a = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    p.b = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0));
    return __builtin_bit_cast(R, p);
  } else if constexpr (sizeof(R) == 16) {
    return __builtin_bit_cast(R, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
  } else if constexpr (sizeof(R) == 8) {
    return __builtin_bit_cast(R, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
  } else if constexpr (sizeof(R) == 4) {
    return __builtin_bit_cast(R, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  } else {
    static_assert(sizeof(R) == 2, "buffer_load_raw: 2, 4, 8, 16 or 32 bytes");
    return __builtin_bit_cast(R, __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0));
  }
}

// A wave's LDS writes are visible to all its lanes after this (the wave's
// lanes exchange data through LDS without a workgroup barrier).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Unpack V elements from a raw vector into accumulator values.
template <typename T, int V, typename ACC>
__device__ __forceinline__ void unpack(const typename raw_vec<T, V>::type& r, ACC (&out)[V]) {
  const T* e = reinterpret_cast<const T*>(&r);
#pragma unroll
  for (int v = 0; v < V; ++v) out[v] = (ACC)to_float(e[v]);
}

// ---------------------------------------------------------------------------
// Wavefront reductions.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum over each 16-lane DPP row; every lane of the row receives the sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  x += dpp_f32<0x140>(x);  // row_mirror
  return x;
}

__device__ __forceinline__ double shfl_xor_d(double x, int m) {
  int lo = __double2loint(x), hi = __double2hiint(x);
  lo = __shfl_xor(lo, m);
  hi = __shfl_xor(hi, m);
  return __hiloint2double(hi, lo);
}
__device__ __forceinline__ float shfl_xor_any(float x, int m) { return __shfl_xor(x, m); }
__device__ __forceinline__ double shfl_xor_any(double x, int m) { return shfl_xor_d(x, m); }

// Sum over aligned groups of G lanes (G a power of two <= 64).
template <typename ACC>
__device__ __forceinline__ ACC group_sum(ACC x, int G) {
  for (int m = 1; m < G; m <<= 1) x += shfl_xor_any(x, m);
  return x;
}
template <>
__device__ __forceinline__ float group_sum<float>(float x, int G) {
  if (G == 16) return row16_sum(x);
  for (int m = 1; m < G; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// Sum across the row slots of a wave: lanes that share (lane mod G).
template <typename ACC>
__device__ __forceinline__ ACC across_slots_sum(ACC x, int G) {
  for (int m = G; m < kWave; m <<= 1) x += shfl_xor_any(x, m);
  return x;
}

// ---------------------------------------------------------------------------
// XCD-aware workgroup order. Workgroups of one dispatch go round-robin to the
// 8 XCDs (each with its own L2); remapping makes XCD x process the x-th
// contiguous slice of the logical work, so neighbouring work (e.g. bags of the
// same tables) shares one L2. Returns -1 for padding workgroups.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t xcd_logical_block(int64_t nlogical) {
  int64_t bid = blockIdx.x;
  int64_t per = (nlogical + kXcds - 1) / kXcds;
  int64_t logical = (bid % kXcds) * per + bid / kXcds;
  return logical < nlogical ? logical : -1;
}
inline int64_t xcd_grid(int64_t nlogical) {
  int64_t per = (nlogical + kXcds - 1) / kXcds;
  return per * kXcds;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace tbe
