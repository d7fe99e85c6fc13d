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

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane j receives element j % 4 of the 8-byte pieces addressed by lanes
// 4e + j / 4 of its group, e = 0..3.  So when lane s of a group addresses row
// r0 + s / 4, columns c0 + 4 (s % 4) .. + 3 of a row-major 16-bit tile, lane j
// receives column c0 + j of rows r0 .. r0 + 3: a column gather in one read.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ inline s16x4 read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const __attribute__((address_space(3))) void*)p);
}

// A operand of a 32x32x16 bf16 MFMA taken from a row-major 16-bit tile with D
// columns (16-byte chunks swizzled by chunk_swizzle<D / 8>): A[m][k] =
// tile[16 j + k'][32 mt + m], with the k order of an S / S^T accumulator (element
// e of lane half hf <-> row 16 j + 8 (e / 4) + 4 hf + e % 4).  Two transposing
// reads: lane group G of 16 covers columns 32 mt + 16 (G % 2) + [0, 16) and
// rows 16 j + 4 (G / 2) + [0, 4), then the same 8 rows further down.
template <int D>
__device__ inline bf16x8 gather_cols(const uint16_t* tile, int mt, int j, int lane) {
  const int c = 32 * mt + 4 * (lane & 3) + 16 * ((lane >> 4) & 1);   // this lane's 4 columns as a source
  const int r0 = 16 * j + ((lane & 15) >> 2) + 4 * (lane >> 5), r1 = r0 + 8;
  const s16x4 lo = read_tr16(&tile[r0 * D + (((c >> 3) ^ chunk_swizzle<D / 8>(r0)) * 8) + (c & 7)]);
  const s16x4 hi = read_tr16(&tile[r1 * D + (((c >> 3) ^ chunk_swizzle<D / 8>(r1)) * 8) + (c & 7)]);
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8, u32x4{l2.x, l2.y, h2.x, h2.y});
}

}  // namespace ps
