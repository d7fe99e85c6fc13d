// Device-side helpers shared by the Prefix Sliding kernels (gfx950 only).
//
// Ring slot map and Continue-PE rotation: blog "Prefix Sliding 完全拆解"
// (pinghaoyang.com.cn), section "核心机制：注意力掩码上的两个区间" (hidden
// tokens are not kept; the cache never exceeds L + W tokens) and section
// "位置编码：Reset PE 还是 Continue PE？" (tokens keep their absolute position;
// cached keys are rotated once and reused).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "prefix_sliding.h"

namespace ps {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16-byte register type for global/LDS traffic (a native vector, so copies stay in registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRegionSlots = 64;   // slots per cache region (page size of paged mode)
constexpr int kMaxGroup = 16;      // query heads per KV head handled by one decode work item
constexpr int kMaxHalfDim = 64;    // head_dim <= 128

// Ring slot of absolute position n (prefix positions stay put; window
// positions cycle through the W slots after the prefix).
__host__ __device__ inline int32_t ring_slot(int64_t n, int32_t prefix_len, int32_t window) {
  return n < prefix_len ? (int32_t)n : (int32_t)(prefix_len + (n - prefix_len) % window);
}

// Geometry of one layer's cache (see the layout notes in prefix_sliding.h).
struct CacheGeom {
  int32_t paged;          // 0: contiguous ring per (sequence, KV head); 1: block table
  int32_t hkv;
  int32_t head_dim;
  int32_t window;
  int32_t slot_capacity;  // multiple of 64
  int32_t max_pages;      // paged: row length of the block table
  int64_t num_pages;      // paged: pool size
};

// Element offset of the 64-slot region that holds slot `slot` of
// (sequence s, KV head h); -1 when the block table names a page outside the pool.
__device__ inline int64_t region_offset(const CacheGeom& g, const int32_t* __restrict__ block_table,
                                        int32_t s, int32_t h, int32_t slot) {
  const int32_t seg = slot >> 6;
  int64_t region;
  if (!g.paged) {
    region = ((int64_t)s * g.hkv + h) * (g.slot_capacity >> 6) + seg;
  } else {
    const int32_t page = block_table[(int64_t)s * g.max_pages + seg];
    if (page < 0 || (int64_t)page >= g.num_pages) return -1;
    region = (int64_t)page * g.hkv + h;
  }
  return region * (int64_t)(kRegionSlots * g.head_dim);
}

// Offsets of slot j, dim d inside a region.
__host__ __device__ inline int32_t k_in_region(int32_t j, int32_t d, int32_t dim) {
  return (j & 63) * dim + d;
}
__host__ __device__ inline int32_t v_in_region(int32_t j, int32_t d, int32_t dim) {
  return ((j & 63) >> 3) * 8 * dim + d * 8 + (j & 7);
}

// Rotary inverse frequencies theta^(-2i/D), formed once on the host in double
// precision and passed by value; enabled == 0 means "inputs already rotated".
struct RopeFreq {
  double inv_freq[kMaxHalfDim];
  int32_t enabled;
};

// cos/sin of pos * inv_freq: the angle is formed and reduced modulo 2*pi in
// double precision (an fp32 angle at position 131072 would be off by ~0.016 rad),
// then evaluated in fp32.
__device__ inline void rope_cos_sin(int64_t pos, double inv_freq, float& c, float& s) {
  const double a = (double)pos * inv_freq;
  const double two_pi_hi = 6.283185307179586232;       // 2*pi rounded to double
  const double two_pi_lo = 2.4492935982947064e-16;     // 2*pi - two_pi_hi
  const double k = rint(a * 0.15915494309189535);      // a / (2*pi)
  const double r = fma(-k, two_pi_lo, fma(-k, two_pi_hi, a));
  sincosf((float)r, &s, &c);
}

// Rotate-half pair (x1, x2) -> (x1 c - x2 s, x2 c + x1 s).  Every kernel that
// stores a rotated key into the cache uses this one expression (explicit fused
// multiply-adds, no compiler contraction), so a key is bit-identical whichever
// kernel wrote it.
__device__ inline void rotate_pair(float x1, float x2, float c, float s, float& y1, float& y2) {
#pragma clang fp contract(off)
  y1 = __builtin_fmaf(x1, c, -(x2 * s));
  y2 = __builtin_fmaf(x2, c, x1 * s);
}

__device__ inline float bf16_to_f32(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

__device__ inline uint16_t f32_to_bf16_bits(float f) {
  bf16 b = (bf16)f;  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(uint16_t, b);
}

// Low/high bf16 of a packed dword, as float.
__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ inline uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

// Cross-lane reductions with the gfx950 lane-swap instructions (VALU, no LDS
// round trip): both lanes of a pair receive (value of the lower lane, value of
// the upper lane), for partners lane^32 and lane^16 respectively.
__device__ inline float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ inline float load(const float* p) { return *p; }
  static __device__ inline void store(float* p, float v) { *p = v; }
};
template <>
struct Elem<uint16_t> {  // bf16 storage
  static __device__ inline float load(const uint16_t* p) { return bf16_to_f32(*p); }
  static __device__ inline void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

}  // namespace ps
