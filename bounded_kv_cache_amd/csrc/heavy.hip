// Prefix + heavy hitters + window: the bookkeeping around a decode step.
//
// Blog "Prefix Sliding 完全拆解" (pinghaoyang.com.cn), section comparing the
// method with H2O: H2O keeps the tokens that have drawn the most attention so
// far, Prefix Sliding pins the prefix; the two can be stacked -- prefix,
// heavily attended middle tokens and the window.  The pages give no algorithm,
// so the rule here is the plain reading (stated with the C ABI):
//   * per (sequence, KV head) up to H heavy slots right after the window's W
//     ring slots, so the visible slots stay one range [0, L + W + count);
//   * a token's score is the attention it has received while cached, summed
//     over the query heads of its KV head;
//   * when a token leaves the window it joins the heavy set if a slot is
//     free, or replaces the weakest member (smallest score, oldest on ties) if
//     its own score is strictly larger; otherwise it is dropped.
// Kernels: retire (one wave per (sequence, KV head): admission, the K/V copy
// into the heavy slot, then the step's token appended into the ring slot it
// frees) and accumulate (after a
// decode kernel that wrote its statistics and each row's log2-sum-exp2 to the
// workspace; when they fit in LDS the decode kernel adds the mass itself).
#include "ps_internal.h"

namespace ps {
namespace {

template <typename T>
__global__ __launch_bounds__(64) void heavy_retire_kernel(HeavyArgs a) {
  const CacheGeom& g = a.geom;
  const int32_t h = (int32_t)(blockIdx.x % g.hkv);
  const int32_t s = (int32_t)(blockIdx.x / g.hkv);
  const int lane = threadIdx.x;
  const int32_t L = a.prefix_len[s];
  const int64_t p = a.pos[s];
  const int32_t H = a.heavy_slots;
  if (L < 0 || p < 0) return;   // invalid sequence: nothing is written (the decode rows are NaN)
  const int64_t e = p - g.window;   // the token leaving the window at this step
  const int32_t se = ring_slot(e, L, g.window);
  const int64_t sh = (int64_t)s * g.hkv + h;
  T* kc = static_cast<T*>(a.k_cache);
  T* vc = static_cast<T*>(a.v_cache);
  if ((int64_t)L + g.window + H <= g.slot_capacity && e >= L) {
    float* score = a.score + sh * g.slot_capacity;
    int64_t* hpos = a.heavy_pos + sh * H;
    const float cand = score[se];
    const int32_t base = L + g.window;
    const int32_t cnt = a.heavy_count[sh];
    int32_t dst = -1;
    if (H > 0) {
      if (cnt < H) {
        dst = cnt;
      } else {
        // the weakest member: smallest score, then oldest position
        float best = INFINITY;
        int64_t bpos = INT64_MAX;
        int32_t bidx = -1;
        for (int32_t i = lane; i < H; i += 64) {
          const float sc = score[base + i];
          const int64_t hp = hpos[i];
          if (sc < best || (sc == best && hp < bpos)) {
            best = sc;
            bpos = hp;
            bidx = i;
          }
        }
        for (int off = 32; off > 0; off >>= 1) {
          const float ob = __shfl_xor(best, off);
          const int64_t op = __shfl_xor(bpos, off);
          const int32_t oi = __shfl_xor(bidx, off);
          if (ob < best || (ob == best && op < bpos)) {
            best = ob;
            bpos = op;
            bidx = oi;
          }
        }
        if (cand > best) dst = bidx;
      }
    }
    if (dst >= 0) {
      const int32_t sd = base + dst;
      const int64_t re = region_offset(g, a.block_table, s, h, se);
      const int64_t rd = region_offset(g, a.block_table, s, h, sd);
      if (re >= 0 && rd >= 0) {
        for (int32_t d = lane; d < g.head_dim; d += 64) {
          kc[rd + k_in_region(sd, d, g.head_dim)] = kc[re + k_in_region(se, d, g.head_dim)];
          vc[rd + v_in_region(sd, d, g.head_dim)] = vc[re + v_in_region(se, d, g.head_dim)];
        }
      }
      if (lane == 0) {
        score[sd] = cand;
        hpos[dst] = e;
        if (dst == cnt) a.heavy_count[sh] = cnt + 1;
      }
    }
    if (lane == 0) score[se] = 0.f;   // the slot receives position p next
  }
  // the step's token for this KV head into its ring slot (after the copy above
  // has read the slot's previous token): K rotated at p, V as given
  const int32_t slot = ring_slot(p, L, g.window);
  if (slot >= g.slot_capacity) return;   // the ring is too small for this position: dropped
  const int64_t rb = region_offset(g, a.block_table, s, h, slot);
  if (rb < 0) return;                    // page outside the pool: dropped
  const int32_t D = g.head_dim, half = D >> 1;
  const T* kn = static_cast<const T*>(a.k_new) + sh * D;
  const T* vn = static_cast<const T*>(a.v_new) + sh * D;
  for (int32_t i = lane; i < half; i += 64) {
    const float x1 = Elem<T>::load(kn + i), x2 = Elem<T>::load(kn + i + half);
    float y1 = x1, y2 = x2;
    if (a.rope.enabled) {
      float c, sn;
      rope_cos_sin(p, a.rope.inv_freq[i], c, sn);
      rotate_pair(x1, x2, c, sn, y1, y2);
    }
    Elem<T>::store(kc + rb + k_in_region(slot, i, D), y1);
    Elem<T>::store(kc + rb + k_in_region(slot, i + half, D), y2);
    vc[rb + v_in_region(slot, i, D)] = vn[i];
    vc[rb + v_in_region(slot, i + half, D)] = vn[i + half];
  }
}

// score[j] += sum over the group's query heads of exp2(s_j - lse2), j in [L, n_vis)
// (bf16 path: s_j = (s_j - m) + m from the fp16 slot value and its chunk's max)
__global__ __launch_bounds__(256) void heavy_accumulate_kernel(HeavyArgs a) {
  const CacheGeom& g = a.geom;
  const int32_t h = (int32_t)(blockIdx.x % g.hkv);
  const int32_t s = (int32_t)(blockIdx.x / g.hkv);
  const int32_t L = a.prefix_len[s];
  const int64_t p = a.pos[s];
  if (L < 0 || p < 0 || (int64_t)L + g.window + a.heavy_slots > g.slot_capacity) return;
  const int64_t sh = (int64_t)s * g.hkv + h;
  const int64_t lw = (int64_t)L + g.window;
  const int64_t nvis = (p + 1 < lw ? p + 1 : lw) + a.heavy_count[sh];
  if (nvis > g.slot_capacity) return;
  float lse2[kMaxGroup];
  for (int n = 0; n < a.group; ++n) lse2[n] = a.stat_lse2[(int64_t)s * a.hq + h * a.group + n];
  float* score = a.score + sh * g.slot_capacity;
  if (a.stat_max) {   // bf16 path: fp16 s - m per slot, m per 32-key chunk, chunk-major
    // 8 consecutive slots per thread (16-byte loads of each head's row; the
    // capacity is a multiple of 64, so a group never crosses a chunk or the end)
    const _Float16* st = static_cast<const _Float16*>(a.stat_scores) + sh * a.group * g.slot_capacity;
    const float* mx = a.stat_max + sh * a.group * (g.slot_capacity / 32);
    for (int64_t j0 = (L & ~7) + 8 * threadIdx.x; j0 < nvis; j0 += 8 * 256) {
      const int64_t c = j0 >> 5;
      float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      for (int n = 0; n < a.group; ++n) {
        const uint4 w = *reinterpret_cast<const uint4*>(st + (c * a.group + n) * 32 + (j0 & 31));
        const float off = mx[c * a.group + n] - lse2[n];
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const auto x = __builtin_bit_cast(_Float16 __attribute__((ext_vector_type(2))), ww[e]);
          m[2 * e] += __builtin_amdgcn_exp2f((float)x[0] + off);
          m[2 * e + 1] += __builtin_amdgcn_exp2f((float)x[1] + off);
        }
      }
      float4* sp = reinterpret_cast<float4*>(score + j0);
      float4 s0 = sp[0], s1 = sp[1];
      float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (j0 + i >= L && j0 + i < nvis) sv[i] += m[i];
      sp[0] = make_float4(sv[0], sv[1], sv[2], sv[3]);
      sp[1] = make_float4(sv[4], sv[5], sv[6], sv[7]);
    }
  } else {            // fp32 path: the scores themselves
    const float* st = static_cast<const float*>(a.stat_scores) + sh * a.group * g.slot_capacity;
    for (int64_t j = L + threadIdx.x; j < nvis; j += 256) {
      float m = 0.f;
      for (int n = 0; n < a.group; ++n) m += __builtin_amdgcn_exp2f(st[(int64_t)n * g.slot_capacity + j] - lse2[n]);
      score[j] += m;
    }
  }
}

}  // namespace

hipError_t launch_heavy_retire(const HeavyArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  const dim3 grid((uint32_t)((int64_t)a.num_seqs * a.geom.hkv));
  if (a.dtype == PS_BF16)
    hipLaunchKernelGGL(heavy_retire_kernel<uint16_t>, grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(heavy_retire_kernel<float>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_heavy_accumulate(const HeavyArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  const dim3 grid((uint32_t)((int64_t)a.num_seqs * a.geom.hkv));
  hipLaunchKernelGGL(heavy_accumulate_kernel, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ps
