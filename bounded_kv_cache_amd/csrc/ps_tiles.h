// Tile helpers shared by the prefill-family kernels (forward, chunk, backward).
#pragma once

#include "ps_common.h"

namespace ps {

__host__ __device__ inline int32_t nk_padded(int32_t nk) { return (nk + 63) / 64 * 64; }

// Position of index k inside its 16-wide group of a d-major ("transposed")
// operand row.  Stored order per group: 0-3, 8-11, 4-7, 12-15, so that the 8
// indices one 32x32x16 MFMA lane needs for a k-step (16j + 8*(e/4) + 4*half +
// e%4, e = 0..7) -- the order in which an S / S^T accumulator holds them --
// are 16 contiguous bytes.
__host__ __device__ inline int32_t vt_slot(int32_t k) {
  const int32_t kl = k & 15;
  return (k & ~15) | (((kl >> 2) & 1) << 3) | ((kl >> 3) << 2) | (kl & 3);
}

// n contiguous elements <-> floats, 16-byte loads / stores (kNT: non-temporal,
// for data streamed once that should not displace cached data)
template <typename T, bool kNT = false>
__device__ inline void load_vec(const T* p, float* x, int n) {
  constexpr int E = 16 / sizeof(T);
  for (int c = 0; c < n; c += E) {
    const u32x4 w = kNT ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + c))
                        : *reinterpret_cast<const u32x4*>(p + c);
    if (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c + 2 * e] = lo_bf16(w[e]);
        x[c + 2 * e + 1] = hi_bf16(w[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[c + e] = __uint_as_float(w[e]);
    }
  }
}
template <typename T, bool kNT = false>
__device__ inline void store_vec(T* p, const float* x, int n) {
  constexpr int E = 16 / sizeof(T);
  for (int c = 0; c < n; c += E) {
    u32x4 w;
    if (sizeof(T) == 2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(x[c + 2 * e], x[c + 2 * e + 1]);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(x[c + e]);
    }
    if (kNT)
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p + c));
    else
      *reinterpret_cast<u32x4*>(p + c) = w;
  }
}

// 16-byte chunk swizzle of an LDS tile with CH chunks per row (8 or 16): chunk
// c of row r lives at chunk c ^ chunk_swizzle<CH>(r), so that 16 consecutive
// rows read at one logical chunk fall in distinct LDS banks
template <int CH>
__device__ inline int chunk_swizzle(int row) {   // CH 16-byte chunks per row (8 or 16)
  return (row / (16 / CH)) & (CH - 1);
}

// Workgroup barrier that orders LDS only: global loads in flight stay in
// flight (__syncthreads would wait for them too).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// One wave load of 64 x 16 bytes into 1 KB of LDS at byte address `lds`
// (wave-uniform; lane i -> lds + 16 i), issued as inline assembly so that the
// compiler neither tracks it nor inserts waits for it: the kernel waits for
// these loads itself, with explicit vector-memory counts (the loads complete
// in issue order).  M0 carries the LDS address; nothing else in the kernels
// that use this sets or reads M0.
__device__ inline void dma_to_lds(const void* src, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(__builtin_amdgcn_readfirstlane(lds))
      : "memory");
}
// s_waitcnt operand: at most n vector memory operations outstanding, the LDS and export counters not waited on
constexpr int vmcnt_only(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
__device__ inline uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

}  // namespace ps
