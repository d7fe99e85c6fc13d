// Reset PE paying the cost the blog attributes to it (section "位置编码：Reset PE
// 还是 Continue PE？"): renumbering the visible window to follow the prefix
// changes every window key's position at every step, so keys are cached
// un-rotated and, before each decode step, every visible key is rotated at its
// renumbered position into a scratch copy that the ordinary decode kernel then
// reads.  The identity used by pe_mode PS_PE_RESET gives the same scores
// without any of this; the two are measured side by side.
//
// Renumbering (0-indexed): prefix slot j keeps position j; the window token at
// absolute position n, n in [w_lo, p] with w_lo = max(L, p - W + 1), becomes
// L + (n - w_lo).  Its ring slot is L + (n - L) mod W, so slot j >= L holds
// renumbered position L + ((j - w_lo) mod W); the query takes min(p, L + W - 1).
#include "ps_reset.h"
#include "ps_tiles.h"

namespace ps {
namespace {

// cos/sin of every renumbered position [0, slot_capacity) and frequency.  For
// bf16 keys the pairs are stored as fp16 (their rounding, 2^-11 relative, is
// below that of the bf16 keys they produce, and half the bytes of an fp32
// table keep it resident in L2 while the keys stream through); the fp32 path
// keeps fp32 pairs.
__device__ inline uint32_t pack_f16x2(float lo, float hi) {
  const _Float16 l = (_Float16)lo, h = (_Float16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, l) | ((uint32_t)__builtin_bit_cast(uint16_t, h) << 16);
}
__device__ inline float f16_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu)); }
__device__ inline float f16_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }

template <typename T>
__global__ __launch_bounds__(256) void reset_table_kernel(ResetArgs a) {
  const int32_t half = a.geom.head_dim / 2;
  const int64_t n = (int64_t)a.geom.slot_capacity * half;
  for (int64_t idx = blockIdx.x * 256ll + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    float c = 1.f, s = 0.f;
    if (a.rope.enabled) rope_cos_sin(idx / half, a.rope.inv_freq[idx % half], c, s);
    if (sizeof(T) == 2)
      static_cast<uint32_t*>(a.table)[idx] = pack_f16x2(c, s);
    else
      static_cast<float2*>(a.table)[idx] = make_float2(c, s);
  }
}

// Workgroups of 256 threads per (sequence, KV head), kSegGroups of them, each
// walking every kSegGroups-th 64-slot segment; four threads per slot, each
// rotating a quarter of the rotate-half pairs (i, i + D/2).
constexpr int kSegGroups = 4;

__device__ inline void rotate(float& x1, float& x2, float c, float s) {
  const float y1 = x1 * c - x2 * s, y2 = x2 * c + x1 * s;
  x1 = y1;
  x2 = y2;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void reset_rerotate_kernel(ResetArgs a) {
  constexpr int HALF = D / 2, PQ = HALF / 4;
  const CacheGeom& g = a.geom;
  const int32_t sg = (int32_t)(blockIdx.x % kSegGroups);
  const int32_t h = (int32_t)((blockIdx.x / kSegGroups) % g.hkv);
  const int32_t s = (int32_t)(blockIdx.x / kSegGroups / g.hkv);
  const int32_t L = a.prefix_len[s];
  const int64_t p = a.pos[s];
  const int64_t W = g.window;
  if (sg == 0 && h == 0 && threadIdx.x == 0)
    a.pos_out[s] = (L < 0 || p < 0) ? p : (p < (int64_t)L + W - 1 ? p : (int64_t)L + W - 1);
  if (L < 0 || p < 0) return;
  const int64_t nvis = p + 1 < (int64_t)L + W ? p + 1 : (int64_t)L + W;
  if (nvis > g.slot_capacity) return;   // unservable: the decode kernel reports it
  const int64_t wlo = (int64_t)L > p - W + 1 ? (int64_t)L : p - W + 1;
  // window slot j = L + t holds renumbered position L + ((t - u) mod W), u = (wlo - L) mod W
  const int32_t u = (int32_t)((wlo - L) % W);
  const int q4 = threadIdx.x & 3;
  for (int32_t j = (sg * 64) + (int32_t)(threadIdx.x >> 2); j < nvis; j += kSegGroups * 64) {
    const int32_t t = j - L;
    const int32_t r = j < L ? j : L + t - u + (t < u ? (int32_t)W : 0);
    const int64_t off = region_offset(g, nullptr, s, h, j) + k_in_region(j, 0, D);
    const T* src = static_cast<const T*>(a.k_cache) + off;
    T* dst = static_cast<T*>(a.k_out) + off;
    float x1[PQ], x2[PQ];
    load_vec<T, true>(src + PQ * q4, x1, PQ);   // keys stream through once; the table stays cached
    load_vec<T, true>(src + HALF + PQ * q4, x2, PQ);
    if (sizeof(T) == 2) {
      const u32x4* cs = reinterpret_cast<const u32x4*>(static_cast<const uint32_t*>(a.table) + (int64_t)r * HALF +
                                                       PQ * q4);   // four (cos, sin) pairs per load
#pragma unroll
      for (int e = 0; e < PQ; e += 4) {
        const u32x4 cw = cs[e / 4];
#pragma unroll
        for (int k = 0; k < 4; ++k) rotate(x1[e + k], x2[e + k], f16_lo(cw[k]), f16_hi(cw[k]));
      }
    } else {
      const float4* cs = reinterpret_cast<const float4*>(static_cast<const float2*>(a.table) + (int64_t)r * HALF +
                                                         PQ * q4);   // two (cos, sin) pairs per load
#pragma unroll
      for (int e = 0; e < PQ; e += 2) {
        const float4 cw = cs[e / 2];
        rotate(x1[e], x2[e], cw.x, cw.y);
        rotate(x1[e + 1], x2[e + 1], cw.z, cw.w);
      }
    }
    store_vec(dst + PQ * q4, x1, PQ);
    store_vec(dst + HALF + PQ * q4, x2, PQ);
  }
}

template <typename T, int D>
hipError_t launch_t(const ResetArgs& a, hipStream_t stream) {
  const int64_t n = (int64_t)a.geom.slot_capacity * (D / 2);
  const int64_t tb = (n + 255) / 256;
  hipLaunchKernelGGL(reset_table_kernel<T>, dim3((uint32_t)(tb < 1024 ? tb : 1024)), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((uint32_t)((int64_t)a.num_seqs * a.geom.hkv * kSegGroups));
  hipLaunchKernelGGL((reset_rerotate_kernel<T, D>), grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reset_rerotate(const ResetArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  if (a.dtype == PS_BF16)
    return a.geom.head_dim == 64 ? launch_t<uint16_t, 64>(a, stream) : launch_t<uint16_t, 128>(a, stream);
  return a.geom.head_dim == 64 ? launch_t<float, 64>(a, stream) : launch_t<float, 128>(a, stream);
}

}  // namespace ps
