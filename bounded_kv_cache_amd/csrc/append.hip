// Append kernel: write new tokens' K (RoPE-rotated once, at the absolute
// position) and V into their ring slots.
//
// Blog "Prefix Sliding 完全拆解" (pinghaoyang.com.cn): section
// "核心机制：注意力掩码上的两个区间" (tokens outside prefix and window are not
// kept, so a slot is reused once its token leaves the window) and section
// "位置编码：Reset PE 还是 Continue PE？" (Continue PE: the rotated key is
// cached and never rotated again).
#include "ps_internal.h"

namespace ps {
namespace {

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
      rope_cos_sin(j, a.rope.inv_freq[i], c, sn);
      y1 = x1 * c - x2 * sn;
      y2 = x2 * c + x1 * sn;
    }
    Elem<T>::store(kc + base + k_in_region(slot, i, D), y1);
    Elem<T>::store(kc + base + k_in_region(slot, i + half, D), y2);
    vc[base + v_in_region(slot, i, D)] = vn[h * D + i];
    vc[base + v_in_region(slot, i + half, D)] = vn[h * D + i + half];
  }
  if (threadIdx.x == 0 && a.slot_pos) a.slot_pos[(int64_t)s * g.slot_capacity + slot] = (int32_t)j;
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t stream) {
  const int64_t items = (int64_t)a.num_seqs * a.tokens_per_seq;
  if (items == 0) return hipSuccess;
  const dim3 grid((uint32_t)items), block(64);
  if (a.dtype == PS_BF16)
    hipLaunchKernelGGL(append_kernel<uint16_t>, grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL(append_kernel<float>, grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace ps
