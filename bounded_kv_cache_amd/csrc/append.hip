// Append kernel: write new tokens' K (RoPE-rotated once, at the absolute
// position) and V into their ring slots.
//
// Blog "Prefix Sliding 完全拆解" (pinghaoyang.com.cn): section
// "核心机制：注意力掩码上的两个区间" (tokens outside prefix and window are not
// kept, so a slot is reused once its token leaves the window) and section
// "位置编码：Reset PE 还是 Continue PE？" (Continue PE: the rotated key is
// cached and never rotated again).
#include "ps_internal.h"
#include "ps_tiles.h"

namespace ps {
namespace {

// calls appending at least this many tokens per sequence take the block path
constexpr int32_t kBulkAppendTokens = 16;
// LDS bytes of the block path's V stage: the 8 tokens' V rows of every KV head
constexpr size_t kAppendStage = 8192;

// One wavefront per (sequence, token).  Each lane rotates rotate-half pairs
// (i, i + D/2) of one KV head; V is copied into the 8-slot d-major blocks.
template <typename T>
__global__ __launch_bounds__(64) void append_kernel(AppendArgs a) {
  const int64_t item = blockIdx.x;
  const int32_t s = (int32_t)(item / a.tokens_per_seq);
  const int32_t t = (int32_t)(item % a.tokens_per_seq);
  int32_t n_tok = a.seq_tokens ? a.seq_tokens[s] : a.tokens_per_seq;
  n_tok = n_tok < a.tokens_per_seq ? n_tok : a.tokens_per_seq;
  if (t >= n_tok) return;
  const CacheGeom& g = a.geom;
  const int32_t L = a.prefix_len[s];
  const int64_t start = a.start_pos[s];
  if (L < 0 || start < 0) return;  // invalid sequence: dropped
  const int64_t j = start + t;
  const int64_t last = start + n_tok - 1;
  // a token this same call would already evict is skipped (no two writes per slot)
  if (!(j < L || j > last - g.window)) return;
  const int32_t slot = ring_slot(j, L, g.window);
  if (slot >= g.slot_capacity) return;  // the ring is too small for this position: dropped
  const int32_t D = g.head_dim;
  const int32_t half = D >> 1;
  const T* kn = static_cast<const T*>(a.k_new) + ((int64_t)s * a.tokens_per_seq + t) * g.hkv * D;
  const T* vn = static_cast<const T*>(a.v_new) + ((int64_t)s * a.tokens_per_seq + t) * g.hkv * D;
  T* kc = static_cast<T*>(a.k_cache);
  T* vc = static_cast<T*>(a.v_cache);
  for (int32_t idx = threadIdx.x; idx < g.hkv * half; idx += 64) {
    const int32_t h = idx / half;
    const int32_t i = idx % half;
    const int64_t base = region_offset(g, a.block_table, s, h, slot);
    if (base < 0) continue;  // page outside the pool: dropped
    float x1 = Elem<T>::load(kn + h * D + i);
    float x2 = Elem<T>::load(kn + h * D + i + half);
    float y1 = x1, y2 = x2;
    if (a.rope.enabled) {
      float c, sn;
      if (a.rope_cs) {
        const float2 w = reinterpret_cast<const float2*>(a.rope_cs)[((int64_t)s * a.tokens_per_seq + t) * half + i];
        c = w.x;
        sn = w.y;
      } else {
        rope_cos_sin(j, a.rope.inv_freq[i], c, sn);
      }
      rotate_pair(x1, x2, c, sn, y1, y2);
    }
    Elem<T>::store(kc + base + k_in_region(slot, i, D), y1);
    Elem<T>::store(kc + base + k_in_region(slot, i + half, D), y2);
    vc[base + v_in_region(slot, i, D)] = vn[h * D + i];
    vc[base + v_in_region(slot, i + half, D)] = vn[h * D + i + half];
  }
  if (threadIdx.x == 0 && a.slot_pos) a.slot_pos[(int64_t)s * g.slot_capacity + slot] = (int32_t)j;
}

// Bulk path (many tokens per sequence): one wavefront per (sequence, 8-slot
// block).  Each slot of the block finds in O(1) which token of this call it
// keeps (the last position that maps to it, if that position stays visible),
// so a V block [D][8] is written as one 16-byte store per dim instead of 8
// scattered 2-byte stores.  Same rules and results as append_kernel.
template <typename T>
__global__ __launch_bounds__(64) void append_block_kernel(AppendArgs a) {
  const CacheGeom& g = a.geom;
  const int32_t nblk = g.slot_capacity >> 3;
  const int32_t s = (int32_t)(blockIdx.x / nblk);
  const int32_t kb = (int32_t)(blockIdx.x % nblk);
  const int lane = threadIdx.x;
  const int32_t L = a.prefix_len[s];
  const int64_t start = a.start_pos[s];
  if (L < 0 || start < 0) return;  // invalid sequence: dropped
  int32_t n_tok = a.seq_tokens ? a.seq_tokens[s] : a.tokens_per_seq;
  n_tok = n_tok < a.tokens_per_seq ? n_tok : a.tokens_per_seq;
  if (n_tok <= 0) return;
  const int64_t last = start + n_tok - 1;
  // lanes 0..7: the position this call leaves in slot 8 kb + lane, or -1
  int64_t src = -1;
  if (lane < 8) {
    const int32_t slot = 8 * kb + lane;
    if (slot < L) {
      if (slot >= start && slot <= last) src = slot;
    } else if ((int64_t)slot < (int64_t)L + g.window && last >= L) {
      const int64_t r = slot - L;
      int64_t back = ((last - L) - r) % g.window;
      if (back < 0) back += g.window;
      const int64_t j = last - back;   // the last position <= last that maps to this slot
      if (j >= L && j >= start) src = j;
    }
  }
  int64_t pos[8];
  int32_t written = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    pos[k] = __shfl(src, k);
    written += pos[k] >= 0;
  }
  if (written == 0) return;
  if (a.slot_pos && lane < 8 && src >= 0) a.slot_pos[(int64_t)s * g.slot_capacity + 8 * kb + lane] = (int32_t)src;
  const int32_t D = g.head_dim, half = D >> 1;
  // the new tokens and the cache never overlap: restrict lets every load of
  // the block be issued ahead of its stores
  const T* __restrict__ kn = static_cast<const T*>(a.k_new);
  const T* __restrict__ vn = static_cast<const T*>(a.v_new);
  T* __restrict__ kc = static_cast<T*>(a.k_cache);
  T* __restrict__ vc = static_cast<T*>(a.v_cache);
  const int64_t tok0 = (int64_t)s * a.tokens_per_seq - start;   // token row of position j: tok0 + j
  // K: rotate each kept token at its position (cos/sin shared by the KV heads);
  // a lane takes 16-byte runs of both halves of a row: E rotation pairs
  constexpr int E = 16 / sizeof(T);
  const int32_t runs = half / E;   // runs per half row
  for (int32_t task = lane; task < 8 * g.hkv * runs; task += 64) {
    const int k = task / (g.hkv * runs);
    const int32_t h = (task / runs) % g.hkv, i0 = (task % runs) * E;
    if (pos[k] < 0) continue;
    const int32_t slot = 8 * kb + k;
    const int64_t base = region_offset(g, a.block_table, s, h, slot);
    if (base < 0) continue;  // page outside the pool: dropped
    const T* row = kn + ((tok0 + pos[k]) * g.hkv + h) * D;
    float x1[E], x2[E], y1[E], y2[E];
    load_vec(row + i0, x1, E);
    load_vec(row + half + i0, x2, E);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      float c = 1.f, sn = 0.f;
      if (a.rope.enabled && a.rope_cs) {   // the caller's table row of this token
        const float2 w = reinterpret_cast<const float2*>(a.rope_cs)[(tok0 + pos[k]) * half + i0 + e];
        c = w.x;
        sn = w.y;
      } else if (a.rope.enabled) {
        rope_cos_sin(pos[k], a.rope.inv_freq[i0 + e], c, sn);
      }
      rotate_pair(x1[e], x2[e], c, sn, y1[e], y2[e]);
    }
    store_vec(kc + base + k_in_region(slot, i0, D), y1, E);
    store_vec(kc + base + k_in_region(slot, half + i0, D), y2, E);
  }
  // V: per (KV head, dim) the block's 8 slots are 8 contiguous elements.  With
  // all 8 slots written and the rows fitting the LDS stage, the 8 tokens' rows
  // come in with 16-byte loads and each (head, dim) column is read back from
  // LDS; otherwise column by column from global memory.
  __shared__ T vstage[kAppendStage / sizeof(T)];
  if (written == 8 && (size_t)8 * g.hkv * D * sizeof(T) <= kAppendStage) {
    const int32_t row_runs = g.hkv * D / E;
    for (int32_t task = lane; task < 8 * row_runs; task += 64) {
      const int k = task / row_runs, r = task % row_runs;
      *reinterpret_cast<u32x4*>(&vstage[(k * row_runs + r) * E]) =
          *reinterpret_cast<const u32x4*>(vn + (tok0 + pos[k]) * g.hkv * D + r * E);
    }
    // (one wave: its LDS accesses complete in program order)
    for (int32_t hd = lane; hd < g.hkv * D; hd += 64) {
      const int32_t h = hd / D, d = hd % D;
      const int64_t base = region_offset(g, a.block_table, s, h, 8 * kb);
      if (base < 0) continue;
      T* dst = vc + base + v_in_region(8 * kb, d, D);   // slot 8 kb + k at dst[k]
      T val[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) val[k] = vstage[k * g.hkv * D + hd];
      if constexpr (sizeof(T) == 2) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          w[e] = (uint32_t)__builtin_bit_cast(uint16_t, val[2 * e]) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, val[2 * e + 1]) << 16);
        *reinterpret_cast<u32x4*>(dst) = w;
      } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[k] = val[k];
      }
    }
    return;
  }
  for (int32_t hd = lane; hd < g.hkv * D; hd += 64) {
    const int32_t h = hd / D, d = hd % D;
    const int64_t base = region_offset(g, a.block_table, s, h, 8 * kb);
    if (base < 0) continue;
    T* dst = vc + base + v_in_region(8 * kb, d, D);   // slot 8 kb + k at dst[k]
    T val[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) val[k] = pos[k] >= 0 ? vn[((tok0 + pos[k]) * g.hkv + h) * D + d] : dst[k];
    // (a slot no token of this call keeps holds its previous value)
    if constexpr (sizeof(T) == 2) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = (uint32_t)__builtin_bit_cast(uint16_t, val[2 * e]) |
               ((uint32_t)__builtin_bit_cast(uint16_t, val[2 * e + 1]) << 16);
      *reinterpret_cast<u32x4*>(dst) = w;
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) dst[k] = val[k];
    }
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.num_seqs * a.tokens_per_seq;
  if (items == 0) return hipSuccess;
  if (a.tokens_per_seq >= kBulkAppendTokens) {
    const dim3 grid((uint32_t)((int64_t)a.num_seqs * (a.geom.slot_capacity >> 3))), block(64);
    if (a.dtype == PS_BF16)
      hipLaunchKernelGGL(append_block_kernel<uint16_t>, grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL(append_block_kernel<float>, grid, block, 0, stream, a);
    return hipGetLastError();
  }
  const dim3 grid((uint32_t)items), block(64);
  if (a.dtype == PS_BF16)
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<float>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace ps
