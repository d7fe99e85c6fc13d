// Masked prefill / training-forward attention with tile skipping.
//
// Blog "Prefix Sliding 完全拆解" (pinghaoyang.com.cn): section
// "Kernel 实现：两层级过滤" (skip tiles with no visible pair; element masks only
// on partly visible tiles; walk the prefix tiles and the window tiles) and
// section "超长 rollouts 的反向传播：截断回传" (a chunk of the trace behind
// the prefix is attended to as a whole).
//
// Pipeline of one call:
//   1. prep kernel: rotate K at its absolute positions into a per-(batch, KV
//      head) contiguous copy, write V transposed ([D][keys], keys padded to a
//      multiple of 64 with zeros, permuted inside each 16-key group -- see
//      vt_slot) and a cos/sin table for the query positions.
//   2. attention kernel: one workgroup per (batch, query head, BM-query tile),
//      walking the scheduled key tiles (ps_sched.h).
// The bf16 kernel uses v_mfma_f32_32x32x16_bf16.  It computes S^T = K Q^T so
// each lane owns one query column: softmax reductions are in-lane plus one
// exchange between the two lane halves, and the S^T registers, rounded to bf16,
// are directly the B operand of O^T += V^T P^T (V^T staged through LDS).
#include "ps_internal.h"
#include "ps_sched.h"
#include "ps_tiles.h"

namespace ps {
namespace {

constexpr float kLn2 = 0.69314718055994531f;
// Lazy softmax rescaling: the reference max of a query only moves when a tile's
// max exceeds it by more than this (log2 units), so probabilities stay <= 2^8
// and the accumulator is rescaled rarely.  Exact: numerator and denominator
// share the reference.
constexpr float kRebase = 8.f;
#ifndef PS_PREFILL_MIN_BLOCKS
#define PS_PREFILL_MIN_BLOCKS 2
#endif
constexpr float kRebaseLow = 64.f;

template <typename T>
struct PfTraits;
template <>
struct PfTraits<uint16_t> {
  static constexpr int BM = 128, BN = 64;
};
template <>
struct PfTraits<float> {
  static constexpr int BM = 64, BN = 64;
};

// ---------------------------------------------------------------------------
// 1. prep: rotated K [b][hkv][nkp][D], V^T [b][hkv][D][nkp], query cos/sin table
// ---------------------------------------------------------------------------
// One workgroup per (batch, 64-key tile).  Each thread owns a quarter of one
// key row (16-byte loads and stores) and forms the cos/sin of its own dims
// once for every KV head; the loads of two KV heads are in flight together.
// V is transposed through LDS so the V^T rows are written contiguously.  Keys
// past num_k are written as zeros.
template <typename T, int D>
__global__ __launch_bounds__(256) void prefill_prep_kernel(PrefillArgs a) {
  constexpr int TK = 64;
  constexpr int HALF = D / 2;
  constexpr int PQ = HALF / 4;   // rotation pairs per thread
  constexpr int DQ = D / 4;      // V dims per thread
  constexpr int KH = 2;          // KV heads per pass
  __shared__ T vt_lds[KH][D][TK + 8];
  PrefillGeom geo{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, a.bm, a.bn};
  const int32_t nkp = a.nkp;
  const int32_t nkt = nkp / TK;
  const int tid = threadIdx.x;
  const int j = tid >> 2, qq = tid & 3;   // key row of the tile, quarter of the row
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  T* kr = static_cast<T*>(a.k_rot);
  T* vt = kr + (int64_t)a.batch * a.hkv * nkp * D;

  for (int64_t blk = blockIdx.x; blk < (int64_t)a.batch * nkt; blk += gridDim.x) {
    const int32_t kt = (int32_t)(blk % nkt);
    const int32_t b = (int32_t)(blk / nkt);
    const int32_t key = kt * TK + j;
    const bool live = key < a.num_k;
    float cs_c[PQ], cs_s[PQ];
    {
      const int64_t pos = live ? pf_key_pos(geo, key) : 0;
#pragma unroll
      for (int e = 0; e < PQ; ++e) {
        cs_c[e] = 1.f;
        cs_s[e] = 0.f;
        if (a.rope.enabled && live) rope_cos_sin(pos, a.rope.inv_freq[PQ * qq + e], cs_c[e], cs_s[e]);
      }
    }
    for (int32_t h0 = 0; h0 < a.hkv; h0 += KH) {
      float x1[KH][PQ], x2[KH][PQ], vv[KH][DQ];
#pragma unroll
      for (int hh = 0; hh < KH; ++hh) {
        if (live && h0 + hh < a.hkv) {
          const int64_t src = (((int64_t)b * a.num_k + key) * a.hkv + h0 + hh) * D;
          load_vec(k + src + PQ * qq, x1[hh], PQ);
          load_vec(k + src + HALF + PQ * qq, x2[hh], PQ);
          load_vec(v + src + DQ * qq, vv[hh], DQ);
        } else {
#pragma unroll
          for (int e = 0; e < PQ; ++e) x1[hh][e] = x2[hh][e] = 0.f;
#pragma unroll
          for (int e = 0; e < DQ; ++e) vv[hh][e] = 0.f;
        }
      }
      const int js = vt_slot(j);
#pragma unroll
      for (int hh = 0; hh < KH; ++hh) {
        if (h0 + hh >= a.hkv) break;
        const int64_t bh = (int64_t)b * a.hkv + h0 + hh;
#pragma unroll
        for (int e = 0; e < PQ; ++e) {
          const float y1 = x1[hh][e] * cs_c[e] - x2[hh][e] * cs_s[e];
          const float y2 = x2[hh][e] * cs_c[e] + x1[hh][e] * cs_s[e];
          x1[hh][e] = y1;
          x2[hh][e] = y2;
        }
        T* krow = kr + (bh * nkp + key) * D;
        store_vec(krow + PQ * qq, x1[hh], PQ);
        store_vec(krow + HALF + PQ * qq, x2[hh], PQ);
#pragma unroll
        for (int e = 0; e < DQ; ++e) {
          T tv;
          if (sizeof(T) == 2)
            tv = (T)f32_to_bf16_bits(vv[hh][e]);   // exact: vv holds bf16 values
          else
            tv = (T)vv[hh][e];
          vt_lds[hh][DQ * qq + e][js] = tv;
        }
      }
      __syncthreads();
      // V^T rows: D rows x 64 keys per head, 16-byte pieces
      constexpr int EP = 16 / sizeof(T);
      const int nh = a.hkv - h0 < KH ? a.hkv - h0 : KH;
      for (int idx = tid; idx < nh * D * (TK / EP); idx += 256) {
        const int hh = idx / (D * (TK / EP));
        const int rem = idx % (D * (TK / EP));
        const int d = rem / (TK / EP), c = rem % (TK / EP);
        u32x4 w;
        if (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)(uint16_t)vt_lds[hh][d][c * EP + 2 * e] |
                   ((uint32_t)(uint16_t)vt_lds[hh][d][c * EP + 2 * e + 1] << 16);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = __float_as_uint((float)vt_lds[hh][d][c * EP + e]);
        }
        const int64_t bh = (int64_t)b * a.hkv + h0 + hh;
        *reinterpret_cast<u32x4*>(vt + (bh * D + d) * nkp + kt * TK + c * EP) = w;
      }
      __syncthreads();
    }
  }
  // cos/sin of every query position (shared by batch and heads)
  const int64_t tq = (int64_t)a.num_q * HALF;
  for (int64_t idx = blockIdx.x * 256ll + tid; idx < tq; idx += (int64_t)gridDim.x * 256) {
    const int32_t i = (int32_t)(idx % HALF);
    const int32_t t = (int32_t)(idx / HALF);
    float c = 1.f, sn = 0.f;
    if (a.rope.enabled) rope_cos_sin(pf_query_pos(geo, t), a.rope.inv_freq[i], c, sn);
    a.rope_cs[idx * 2 + 0] = c;
    a.rope_cs[idx * 2 + 1] = sn;
  }
}

// Work-item decode shared by the attention kernels: workgroups are spread so
// that each XCD (hardware round-robin on blockIdx) gets a contiguous run of
// items ordered (batch, KV head, q-tile, head-in-group): concurrently running
// workgroups of one XCD then share the same K/V tiles in that XCD's L2.
struct Item {
  int32_t b, hq, qt;
  bool valid;
};
__device__ inline Item decode_item(const PrefillArgs& a, int32_t n_qt) {
  // the host keeps the item count below 2^31, so 32-bit unsigned arithmetic
  // is exact (64-bit divisions would cost hundreds of scalar instructions)
  const uint32_t total = (uint32_t)a.batch * (uint32_t)a.hq * (uint32_t)n_qt;
  const uint32_t per = (total + 7) / 8;
  const uint32_t lin = (blockIdx.x % 8) * per + blockIdx.x / 8;
  const uint32_t group = (uint32_t)a.group, nq = (uint32_t)n_qt, hkv = (uint32_t)a.hkv;
  Item it;
  it.valid = lin < total;
  const uint32_t hg = lin % group;
  uint32_t rest = lin / group;
  it.qt = (int32_t)(rest % nq);
  rest /= nq;
  const uint32_t kvh = rest % hkv;
  it.b = (int32_t)(rest / hkv);
  it.hq = (int32_t)(kvh * group + hg);
  return it;
}

// Geometry of a chunk that continues a cached trace.  Sequence b holds
// positions [0, P) in its ring and the chunk is positions [P, P + T).  Its key
// array is the pinned positions [0, min(L, P + T)) followed by the contiguous
// run [w0, P + T), w0 = max(L, P - W + 1): every key any chunk query can see
// (blog "Prefix Sliding 完全拆解", section "核心机制：注意力掩码上的两个区间";
// the window of the first chunk query starts at P - W + 1).  Keys below P come
// from the ring, the rest from the chunk.  false: the sequence cannot be served
// (negative values, or ring slots beyond the capacity would be read).
__device__ inline bool chunk_geom(const PrefillArgs& a, int32_t b, int32_t bm, int32_t bn, PrefillGeom& g) {
  const int32_t L = a.seq_prefix[b];
  const int64_t P = a.seq_start[b];
  if (L < 0 || P < 0) return false;
  const int64_t lw = (int64_t)L + a.window;
  if ((P < lw ? P : lw) > a.cg.slot_capacity) return false;
  const int64_t w0 = P - a.window + 1 > L ? P - a.window + 1 : (int64_t)L;
  g.T = a.num_q;
  g.Nk = (int32_t)(L + P + a.num_q - w0);  // <= slot_capacity + T <= nkp
  g.L = L;
  g.W = a.window;
  g.kv_start = w0;
  g.bm = bm;
  g.bn = bn;
  return true;
}

// Chunk prep: the same K / V^T copies as the prep kernel, gathered per key
// from the ring (keys below P: already rotated, copied as stored) or from the
// chunk (rotated here at the key's position), plus the chunk queries rotated at
// P + t and multiplied by scale * log2(e).  A ring page outside the pool gives
// NaN keys (so the rows that see them become NaN).
template <typename T, int D>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrefillArgs a) {
  constexpr int TK = 64;
  constexpr int HALF = D / 2;
  constexpr int PQ = HALF / 4;   // rotation pairs per thread
  constexpr int DQ = D / 4;      // V dims per thread
  __shared__ float cs_lds[TK][HALF][2];
  __shared__ T vt_lds[D][TK + 8];
  const int32_t nkp = a.nkp;
  const int32_t nkt = nkp / TK;
  const int tid = threadIdx.x;
  const int j = tid >> 2, qq = tid & 3;   // key row of the tile, quarter of the row
  const T* kn = static_cast<const T*>(a.k);
  const T* vn = static_cast<const T*>(a.v);
  const T* kc = static_cast<const T*>(a.k_cache);
  const T* vc = static_cast<const T*>(a.v_cache);
  T* kr = static_cast<T*>(a.k_rot);
  T* vt = kr + (int64_t)a.batch * a.hkv * nkp * D;

  for (int64_t blk = blockIdx.x; blk < (int64_t)a.batch * nkt; blk += gridDim.x) {
    const int32_t kt = (int32_t)(blk % nkt);
    const int32_t b = (int32_t)(blk / nkt);
    PrefillGeom geo;
    const bool ok = chunk_geom(a, b, 64, 64, geo);
    const int64_t P = ok ? a.seq_start[b] : 0;
    __syncthreads();   // the previous tile's V^T reads of vt_lds / cs_lds are done
    for (int idx = tid; idx < TK * HALF; idx += 256) {
      const int jj = idx / HALF, i = idx % HALF;
      const int32_t key = kt * TK + jj;
      float c = 1.f, sn = 0.f;
      if (ok && a.rope.enabled && key < geo.Nk) {
        const int64_t pos = pf_key_pos(geo, key);
        if (pos >= P) rope_cos_sin(pos, a.rope.inv_freq[i], c, sn);
      }
      cs_lds[jj][i][0] = c;
      cs_lds[jj][i][1] = sn;
    }
    __syncthreads();
    const int32_t key = kt * TK + j;
    const bool live = ok && key < geo.Nk;
    const int64_t pos = live ? pf_key_pos(geo, key) : 0;
    for (int32_t h = 0; h < a.hkv; ++h) {
      const int64_t bh = (int64_t)b * a.hkv + h;
      float x1[PQ], x2[PQ], vv[DQ];
      if (live && pos < P) {   // from the ring: stored rotated
        const int32_t slot = ring_slot(pos, geo.L, a.window);
        const int64_t base = region_offset(a.cg, a.block_table, b, h, slot);
        if (base >= 0) {
          load_vec(kc + base + k_in_region(slot, PQ * qq, D), x1, PQ);
          load_vec(kc + base + k_in_region(slot, HALF + PQ * qq, D), x2, PQ);
#pragma unroll
          for (int e = 0; e < DQ; ++e) vv[e] = Elem<T>::load(vc + base + v_in_region(slot, DQ * qq + e, D));
        } else {
#pragma unroll
          for (int e = 0; e < PQ; ++e) x1[e] = x2[e] = __builtin_nanf("");
#pragma unroll
          for (int e = 0; e < DQ; ++e) vv[e] = __builtin_nanf("");
        }
      } else if (live) {       // from the chunk: rotate at the key's position
        const int64_t src = (((int64_t)b * a.num_q + (pos - P)) * a.hkv + h) * D;
        load_vec(kn + src + PQ * qq, x1, PQ);
        load_vec(kn + src + HALF + PQ * qq, x2, PQ);
        load_vec(vn + src + DQ * qq, vv, DQ);
#pragma unroll
        for (int e = 0; e < PQ; ++e) {
          const float c = cs_lds[j][PQ * qq + e][0], sn = cs_lds[j][PQ * qq + e][1];
          const float y1 = x1[e] * c - x2[e] * sn, y2 = x2[e] * c + x1[e] * sn;
          x1[e] = y1;
          x2[e] = y2;
        }
      } else {
#pragma unroll
        for (int e = 0; e < PQ; ++e) x1[e] = x2[e] = 0.f;
#pragma unroll
        for (int e = 0; e < DQ; ++e) vv[e] = 0.f;
      }
      T* krow = kr + (bh * nkp + key) * D;
      store_vec(krow + PQ * qq, x1, PQ);
      store_vec(krow + HALF + PQ * qq, x2, PQ);
      const int js = vt_slot(j);
#pragma unroll
      for (int e = 0; e < DQ; ++e) {
        T tv;
        if (sizeof(T) == 2)
          tv = (T)f32_to_bf16_bits(vv[e]);   // exact: vv holds bf16 values
        else
          tv = (T)vv[e];
        vt_lds[DQ * qq + e][js] = tv;
      }
      __syncthreads();
      constexpr int EP = 16 / sizeof(T);
      for (int idx = tid; idx < D * (TK / EP); idx += 256) {
        const int d = idx / (TK / EP), c = idx % (TK / EP);
        u32x4 w;
        if (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = (uint32_t)(uint16_t)vt_lds[d][c * EP + 2 * e] | ((uint32_t)(uint16_t)vt_lds[d][c * EP + 2 * e + 1] << 16);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = __float_as_uint((float)vt_lds[d][c * EP + e]);
        }
        *reinterpret_cast<u32x4*>(vt + (bh * D + d) * nkp + kt * TK + c * EP) = w;
      }
      __syncthreads();
    }
  }
  // cos/sin of every chunk query position P + t (one row per sequence and query)
  const int64_t pairs = (int64_t)a.batch * a.num_q * HALF;
  for (int64_t idx = blockIdx.x * 256ll + tid; idx < pairs; idx += (int64_t)gridDim.x * 256) {
    const int32_t i = (int32_t)(idx % HALF);
    const int64_t bt = idx / HALF;          // b * T + t
    const int64_t P = a.seq_start[bt / a.num_q];
    float c = 1.f, sn = 0.f;
    if (a.rope.enabled && P >= 0) rope_cos_sin(P + bt % a.num_q, a.rope.inv_freq[i], c, sn);
    a.rope_cs[idx * 2 + 0] = c;
    a.rope_cs[idx * 2 + 1] = sn;
  }
}

// ---------------------------------------------------------------------------
// 2a. fp32 debug kernel: one thread per query row, LDS-tiled, same schedule
// ---------------------------------------------------------------------------
template <int D, bool kPerSeq>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int BM = PfTraits<float>::BM, BN = PfTraits<float>::BN;
  __shared__ float qs[BM][D + 1];
  __shared__ float ks[BN][D + 1];
  __shared__ float vs[BN][D + 1];
  PrefillGeom geo{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, BM, BN};
  const int32_t n_qt = pf_num_qtiles(geo);
  const Item it = decode_item(a, n_qt);
  if (!it.valid) return;
  const int tid = threadIdx.x;
  const int32_t t = it.qt * BM + tid;
  const bool row_ok = t < a.num_q;
  if (kPerSeq && !chunk_geom(a, it.b, BM, BN, geo)) {   // sequence cannot be served: NaN rows
    if (!row_ok) return;
    float* o = static_cast<float*>(a.out) + (((int64_t)it.b * a.num_q + t) * a.hq + it.hq) * D;
    for (int d = 0; d < D; ++d) o[d] = __builtin_nanf("");
    if (a.lse) a.lse[((int64_t)it.b * a.hq + it.hq) * a.num_q + t] = __builtin_nanf("");
    return;
  }
  const int32_t u = geo.Nk - a.num_q + t;  // the query's key index
  const int32_t kvh = it.hq / a.group;
  const int32_t nkp = a.nkp;
  const float* q = static_cast<const float*>(a.q);
  const float* kr = static_cast<const float*>(a.k_rot) + ((int64_t)it.b * a.hkv + kvh) * nkp * D;
  const float* vt = static_cast<const float*>(a.k_rot) + (int64_t)a.batch * a.hkv * nkp * D +
                    ((int64_t)it.b * a.hkv + kvh) * D * nkp;
  if (row_ok) {
    const float* qrow = q + (((int64_t)it.b * a.num_q + t) * a.hq + it.hq) * D;
    const float* cs = a.rope_cs + ((kPerSeq ? (int64_t)it.b * a.num_q : 0) + t) * (D / 2) * 2;
    for (int i = 0; i < D / 2; ++i) {
      const float c = cs[2 * i], s = cs[2 * i + 1];
      const float x1 = qrow[i], x2 = qrow[i + D / 2];
      qs[tid][i] = (x1 * c - x2 * s) * a.scale_log2;
      qs[tid][i + D / 2] = (x2 * c + x1 * s) * a.scale_log2;
    }
  }
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const Walk walk = pf_walk(geo, it.qt);
  for (int32_t ci = 0; ci < walk.n_cand; ++ci) {
    const int32_t kt = pf_walk_tile(walk, ci);
    const int kind = pf_walk_kind(geo, it.qt, walk, ci);
    __syncthreads();
    for (int idx = tid; idx < BN * D; idx += 64) {
      const int j = idx / D, d = idx % D;
      ks[j][d] = kr[((int64_t)kt * BN + j) * D + d];
      vs[j][d] = vt[(int64_t)d * nkp + vt_slot(kt * BN + j)];
    }
    __syncthreads();
    if (!row_ok) continue;
    float sc[BN];
    float mx = -INFINITY;
    for (int j = 0; j < BN; ++j) {
      float s = 0.f;
      for (int d = 0; d < D; ++d) s += qs[tid][d] * ks[j][d];
      const int32_t key = kt * BN + j;
      const bool vis = key < geo.Nk && (kind == 1 || pf_visible(geo, u, key));
      sc[j] = vis ? s : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
    for (int d = 0; d < D; ++d) acc[d] *= alpha;
    for (int j = 0; j < BN; ++j) {
      const float p = __builtin_amdgcn_exp2f(sc[j] - m_use);
      l_run += p;
      for (int d = 0; d < D; ++d) acc[d] += p * vs[j][d];
    }
  }
  if (!row_ok) return;
  float* o = static_cast<float*>(a.out) + (((int64_t)it.b * a.num_q + t) * a.hq + it.hq) * D;
  for (int d = 0; d < D; ++d) o[d] = acc[d] / l_run;
  if (a.lse) a.lse[((int64_t)it.b * a.hq + it.hq) * a.num_q + t] = (m_run + __log2f(l_run)) * kLn2;
}

// ---------------------------------------------------------------------------
// 2b. bf16 MFMA kernel
// ---------------------------------------------------------------------------
// Workgroup: 4 waves x 32 query rows = BM 128; key tiles of BN 64.
// 32x32x16 MFMA lane layout used throughout (lane l, half hf = l/32, col = l%32):
//   A[m][k]: lane (m + 32*(k/8)) element k%8        B[k][n]: lane (n + 32*(k/8)) element k%8
//   D[m][n]: lane (n + 32*((m/4)%2)) register 4*(m/8) + m%4
// The dim <-> k-slot map of QK is shared by both operands (dim 16*ks + 8*hf + e),
// so it never matters which physical k the hardware pairs.
//
// Softmax bookkeeping per query column: `ref` is the reference max (log2
// units); the S accumulator starts at -ref, so the MFMA itself yields s - ref
// and the fast path is just max / exp2 / sum / convert.
//
// Software pipeline: while tile j's probabilities are formed (VALU) and
// multiplied into O (MFMA), the scores of tile j+1 are computed (MFMA), so each
// wave always has independent matrix work to issue next to its vector work.
// K and V^T tiles go global -> LDS directly (global_load_lds_dwordx4, no
// staging registers) into a three-deep K ring and a two-deep V^T ring: step j
// requests K(j+3) and V(j+1) and ends once K(j+2) and V(j+1) have landed, so a
// K tile has two steps to arrive and a V^T tile one.  Inside a tile the
// 16-byte chunks of a row are XOR-swizzled by row so that the operand reads
// (16 consecutive rows, one chunk column) fall in distinct LDS banks.  The
// loads are issued as inline assembly with explicit waits: the compiler,
// seeing a direct-to-LDS load in flight, would make the next read of any
// buffer it may alias wait for every outstanding load.
template <int D, bool kPerSeq>
__global__ __launch_bounds__(256, PS_PREFILL_MIN_BLOCKS) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D / 16;        // QK k-steps
  constexpr int MT = D / 32;        // PV output d-tiles
  constexpr int KCH = D / 8;        // 16-byte chunks per K row
  constexpr int VCH = BN / 8;       // 16-byte chunks per V^T row
  constexpr int DMA = BN * D / 8 / 256;   // 1 KB wave loads per wave per tile (same for K and V^T)
  constexpr int SLOT = BN * D * 2;   // bytes of one K or V^T tile
  // K ring of three tiles, V^T ring of two (80 KB at D = 128: two workgroups fill a CU's LDS)
  __shared__ __attribute__((aligned(1024))) uint16_t k_ring[3 * BN * D];
  __shared__ __attribute__((aligned(1024))) uint16_t v_ring[2 * D * BN];

  PrefillGeom geo{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, BM, BN};
  const int32_t n_qt = pf_num_qtiles(geo);
  const Item it = decode_item(a, n_qt);
  if (!it.valid) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hf = lane >> 5;
  if (kPerSeq && !chunk_geom(a, it.b, BM, BN, geo)) {   // sequence cannot be served: NaN rows
    const int32_t tn = it.qt * BM + wave * 32 + col;
    if (tn >= a.num_q) return;
    uint16_t* orow = static_cast<uint16_t*>(a.out) + (((int64_t)it.b * a.num_q + tn) * a.hq + it.hq) * D;
    for (int d = hf * (D / 2); d < (hf + 1) * (D / 2); ++d) orow[d] = 0x7fc0;
    if (a.lse && hf == 0) a.lse[((int64_t)it.b * a.hq + it.hq) * a.num_q + tn] = __builtin_nanf("");
    return;
  }
  const int32_t num_k = geo.Nk, prefix_len = geo.L;
  const int32_t kvh = it.hq / a.group;
  const int32_t nkp = a.nkp;
  const uint16_t* kr = static_cast<const uint16_t*>(a.k_rot) + ((int64_t)it.b * a.hkv + kvh) * nkp * D;
  const uint16_t* vt = static_cast<const uint16_t*>(a.k_rot) + (int64_t)a.batch * a.hkv * nkp * D +
                       ((int64_t)it.b * a.hkv + kvh) * D * nkp;

  // Wave load p of wave w fills LDS chunks (4p + w)*64 + lane, i.e. rows
  // (4p + w)*64/CH + lane/CH; the row's swizzle depends on (w, lane) only (the
  // rows of one load step by a multiple of the swizzle period), so one source
  // offset per lane serves every p.
  const uint32_t koff = (uint32_t)((wave * (64 / KCH) + lane / KCH) * D +
                                   ((lane % KCH) ^ chunk_swizzle<KCH>(wave * (64 / KCH) + lane / KCH)) * 8);
  const uint32_t voff = (uint32_t)(lane / VCH) * (uint32_t)nkp +
                        (uint32_t)(((lane % VCH) ^ chunk_swizzle<VCH>(wave * (64 / VCH) + lane / VCH)) * 8);
  // tile kt -> ring slot `slot`: wave load p of this wave fills 1 KB chunk 4p + wave
  const uint32_t k_lds = lds_address(k_ring) + wave * 1024, v_lds = lds_address(v_ring) + wave * 1024;
  auto load_k = [&](int32_t kt, int32_t slot) {
    const uint16_t* src = kr + (int64_t)kt * BN * D + koff;
#pragma unroll
    for (int p = 0; p < DMA; ++p) dma_to_lds(src + p * 4 * (64 / KCH) * D, k_lds + slot * SLOT + p * 4096);
  };
  auto load_v = [&](int32_t kt, int32_t slot) {
    const uint16_t* src = vt + (int64_t)kt * BN + voff;
#pragma unroll
    for (int p = 0; p < DMA; ++p)   // wave load p covers V^T rows (p*4 + wave) * 64/VCH + [0, 64/VCH)
      dma_to_lds(src + (int64_t)((p * 4 + wave) * (64 / VCH)) * nkp, v_lds + slot * SLOT + p * 4096);
  };

  // The query row and its cos/sin are loaded first, then the walk is formed
  // and the first key/value tiles are requested: every load of the prologue is
  // in flight before the first use, so they share one memory round trip.
  const int32_t t = it.qt * BM + wave * 32 + col;
  const bool row_ok = t < a.num_q;
  const int32_t u = num_k - a.num_q + t;  // key index of this lane's query
  u32x4 qw[KS], cw[KS / 2][4];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                           (((int64_t)it.b * a.num_q + (row_ok ? t : 0)) * a.hq + it.hq) * D;
    // cos/sin of the query position: one table row per query (uniform
    // geometry) or per (sequence, query) (chunks continuing a ring); pairs
    // 16 ks + 8 hf + [0, 8) as 4 x 16 bytes per ks
    const float* cs = a.rope_cs + ((kPerSeq ? (int64_t)it.b * a.num_q : 0) + (row_ok ? t : 0)) * (D / 2) * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qw[ks] = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * hf);
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) cw[ks][j] = *reinterpret_cast<const u32x4*>(cs + 2 * (16 * ks + 8 * hf) + 4 * j);
  }

  // the walk (ps_sched.h): prefix candidates, then band candidates, each with
  // at least one visible pair; band kinds come from one precomputed fully
  // visible range.  Loads past the last candidate repeat it.
  const Walk walk = pf_walk(geo, it.qt);
  const int32_t n_cand = walk.n_cand;
  auto cand_tile = [&](int32_t ci) { return pf_walk_tile(walk, ci); };
  auto kind_at = [&](int32_t ci) { return pf_walk_kind(geo, it.qt, walk, ci); };
  auto tile_at = [&](int32_t ci) { return cand_tile(ci < n_cand ? ci : n_cand - 1); };

  // K(0), V(0), K(1) load while the query prologue runs (the prologue waits
  // for them), K(2) after it (in flight into the first step)
  if (n_cand > 0) {
    load_k(tile_at(0), 0);
    load_v(tile_at(0), 0);
    load_k(tile_at(1), 1);
  }

  // ---- query operand (B of S^T = K Q^T): query row t, dims 16*ks + 8*hf + e ----
  bf16x8 qop[KS];
  {
    float qv[KS][8];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[ks][2 * e] = lo_bf16(qw[ks][e]);
        qv[ks][2 * e + 1] = hi_bf16(qw[ks][e]);
      }
#pragma unroll
    for (int ks = 0; ks < KS / 2; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = __uint_as_float(cw[ks][e / 2][2 * (e % 2)]);
        const float s = __uint_as_float(cw[ks][e / 2][2 * (e % 2) + 1]);
        const float x1 = qv[ks][e], x2 = qv[ks + KS / 2][e];
        qv[ks][e] = x1 * c - x2 * s;
        qv[ks + KS / 2][e] = x2 * c + x1 * s;
      }
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qop[ks][e] = (bf16)(row_ok ? qv[ks][e] * a.scale_log2 : 0.f);
  }
  // per-lane visible key ranges: pinned keys [0, pre_end), chunk keys band_lo + [0, band_w]
  const int32_t pre_end = row_ok ? pf_min(prefix_len, u + 1) : 0;
  int32_t band_lo = pf_max(prefix_len, u - a.window + 1);
  const int32_t band_hi = pf_min(u, num_k - 1);
  uint32_t band_w = (uint32_t)(band_hi - band_lo);
  if (!row_ok || band_hi < band_lo) {  // empty band: no key satisfies the unsigned range test
    band_lo = 0x7fffffff;
    band_w = 0;
  }

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  float ref = 0.f;     // reference max (log2 units)
  float l_run = 0.f;   // lane-local partial sum of exp2(s - ref)
  f32x16 negref;       // -ref in every register: initial value of the S accumulators
#pragma unroll
  for (int i = 0; i < 16; ++i) negref[i] = 0.f;

  // LDS operand addresses (elements): row 32*m + col, logical chunk c -> c ^ swizzle(col)
  // Byte offsets (inside a tile) of this lane's first K and V^T operand
  // chunks.  Logical chunk 2s + hf lives at physical chunk (2s + hf) ^ swizzle,
  // i.e. at byte offset off ^ 32s: the chunk bits sit below the row bits, so
  // one XOR per k-step addresses every operand; the 32-row M-tiles are
  // immediate offsets.
  const uint32_t k_off = (uint32_t)(col * D + (hf ^ chunk_swizzle<KCH>(col)) * 8) * 2;
  const uint32_t v_off = (uint32_t)(col * BN + (hf ^ chunk_swizzle<VCH>(col)) * 8) * 2;
  auto frag = [](const uint16_t* buf, uint32_t byte_off) {
    return *reinterpret_cast<const bf16x8*>(reinterpret_cast<const char*>(buf) + byte_off);
  };

  // S^T - ref = K Q^T + (-ref) for the K tile in `kb`: two 32-key M-tiles; the
  // operands of k-step ks+1 are read while the MFMAs of k-step ks run
  auto qk = [&](const uint16_t* kb, f32x16* st) {
    bf16x8 k0 = frag(kb, k_off);
    bf16x8 k1 = frag(kb, k_off + 64 * D);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 n0 = k0, n1 = k1;
      if (ks + 1 < KS) {
        const uint32_t c = k_off ^ (32 * (ks + 1));
        n0 = frag(kb, c);
        n1 = frag(kb, c + 64 * D);
      }
      st[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qop[ks], ks == 0 ? negref : st[0], 0, 0, 0);
      st[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qop[ks], ks == 0 ? negref : st[1], 0, 0, 0);
      k0 = n0;
      k1 = n1;
    }
  };
  // element masks of a partly visible tile; key of register i of M-tile m2:
  // kt*BN + 32*m2 + 8*(i/4) + 4*hf + i%4
  auto mask = [&](int32_t kt, f32x16* st) {
    const int32_t kbase = kt * BN + 4 * hf;
    if (kt * BN >= prefix_len && kt * BN + BN <= num_k) {
      // chunk keys only, all in range: visible iff 0 <= u - key < W, one unsigned compare
      const uint32_t rel = (uint32_t)(row_ok ? u - kbase : -1 - a.window);
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t off = 32 * m2 + 8 * (i >> 2) + (i & 3);
          if (rel - off >= (uint32_t)a.window) st[m2][i] = -INFINITY;
        }
    } else {
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int32_t key = kbase + 32 * m2 + 8 * (i >> 2) + (i & 3);
          const bool vis = key < pre_end || (uint32_t)(key - band_lo) <= band_w;
          if (!vis) st[m2][i] = -INFINITY;
        }
    }
  };
  // row max of a fresh S tile
  auto tile_max = [&](const f32x16* st) {
    float m0 = fmaxf(st[0][0], st[1][0]), m1 = fmaxf(st[0][1], st[1][1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      m0 = fmaxf(m0, fmaxf(st[0][i], st[1][i]));
      m1 = fmaxf(m1, fmaxf(st[0][i + 1], st[1][i + 1]));
    }
    return max_xor32(fmaxf(m0, m1));
  };
  // the reference moves for a fresh S tile with row max mx (one rare,
  // wave-uniform branch):
  //  * the tile's max exceeds the reference by more than kRebase: move the
  //    reference up to it and rescale what is accumulated;
  //  * nothing accumulated yet and every score far below the reference: move
  //    it down so the first probabilities do not underflow (no rescale needed)
  auto rebase = [&](f32x16* st, float mx) {
    // per-lane (divergent) branch: both halves of a query column see the same
    // mx and ltot, so they take the same decision
    const float ltot = sum_xor32(l_run);
    const bool up = mx > kRebase;
    const bool down = !up && mx < -kRebaseLow && ltot == 0.f && mx != -INFINITY;
    if (up || down) {
      const float shift = mx;
      const float alpha = up ? __builtin_amdgcn_exp2f(-shift) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) acc[mt] *= alpha;
      ref += shift;
      negref -= shift;
#pragma unroll
      for (int m2 = 0; m2 < 2; ++m2) st[m2] -= shift;
    }
  };

  if (n_cand > 0) load_k(tile_at(2), 2);
  // the query operand is formed (the compiler waited for the query loads);
  // K(0), V(0), K(1) are complete once at most K(2)'s loads are outstanding
  __builtin_amdgcn_s_waitcnt(vmcnt_only(DMA));
  lds_barrier();
  f32x16 sa[2], sb[2];   // scores of tiles c0 / c0 + 1, alternating between steps
  if (n_cand > 0) {
    qk(k_ring, sa);
    if (kind_at(0) == 2) mask(cand_tile(0), sa);
    rebase(sa, tile_max(sa));
  }
  lds_barrier();   // every wave's reads of K(0) are done before the first step refills its slot
  int32_t c0 = 0;
  // one step of the walk: tile c0 (scores in sc, V^T in slot vcur) and tile
  // c0 + 1 (K in slot knext, scores into sn); V(c0 + 1) is requested into slot
  // vnext (V(c0 - 1), read last step) and K(c0 + 3) into slot kfree (K(c0), read
  // last step)
  auto step = [&](int32_t kfree, int32_t knext, int32_t vcur, int32_t vnext, f32x16* sc, f32x16* sn) {
    load_v(tile_at(c0 + 1), vnext);
    load_k(tile_at(c0 + 3), kfree);

    // Straight-line sections, each fenced against the scheduler: one MFMA
    // step, the LDS operand reads of the next one, and a share of the vector
    // work.  QK sections: scores of the next tile (past the last tile its K
    // buffer holds stale data: computed and discarded) and this tile's
    // probabilities (bf16 B operand of PV).  PV sections: O^T += V^T P^T (PV
    // k-step j covers keys 16j + 8*(e/4) + 4*hf + e%4) and the next tile's
    // row max.
    constexpr int EPS = 32 / KS;   // probabilities formed per QK section
    bf16x8 pop[4];
    float ps[2] = {0.f, 0.f};
    // (the slot offsets are multiples of 16 KB: the chunk XORs below leave them intact)
    uint32_t ko = knext * SLOT + k_off, vo = vcur * SLOT + v_off;
    asm volatile("" : "+v"(ko), "+v"(vo));   // keep the per-step XORs from being hoisted into registers
    // K operands two k-steps ahead (ring of three), the first V^T operands
    // read in the second-to-last QK section
    bf16x8 kf[3][2];
    kf[0][0] = frag(k_ring, ko);
    kf[0][1] = frag(k_ring, ko + 64 * D);
    kf[1][0] = frag(k_ring, ko ^ 32);
    kf[1][1] = frag(k_ring, (ko ^ 32) + 64 * D);
    bf16x8 va[MT];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 2 < KS) {
        const uint32_t c = ko ^ (32 * (ks + 2));
        kf[(ks + 2) % 3][0] = frag(k_ring, c);
        kf[(ks + 2) % 3][1] = frag(k_ring, c + 64 * D);
      } else if (ks + 2 == KS) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) va[mt] = frag(v_ring, vo + 64 * BN * mt);
      }
      sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks % 3][0], qop[ks], ks == 0 ? negref : sn[0], 0, 0, 0);
      sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks % 3][1], qop[ks], ks == 0 ? negref : sn[1], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int idx = ks * EPS + e, m2 = idx >> 4, i = idx & 15;
        const float p = __builtin_amdgcn_exp2f(sc[m2][i]);
        ps[i & 1] += p;
        pop[2 * m2 + (i >> 3)][i & 7] = (bf16)p;
      }
      if (ks + 2 < KS)   // the operand reads first,
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      else if (ks + 2 == KS)
        __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // then this k-step's MFMAs,
      __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);  // then the vector work
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += ps[0] + ps[1];
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8 vn[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        vn[mt] = j + 1 < 4 ? frag(v_ring, (vo ^ (32 * (j + 1))) + 64 * BN * mt) : va[mt];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[mt], pop[j], acc[mt], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const int idx = 8 * j + e, m2 = idx >> 4, i = idx & 15;
        mx0 = fmaxf(mx0, sn[m2][i]);
        mx1 = fmaxf(mx1, sn[m2][i + 1]);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) va[mt] = vn[mt];
      __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    asm volatile("" ::"v"(mx0), "v"(mx1));   // the max is formed in the PV sections above
    if (c0 + 1 < n_cand) {
      if (kind_at(c0 + 1) == 2) {
        mask(cand_tile(c0 + 1), sn);
        rebase(sn, tile_max(sn));
      } else {
        rebase(sn, max_xor32(fmaxf(mx0, mx1)));
      }
    }
    // V(c0 + 1) and K(c0 + 2) have landed once at most K(c0 + 3)'s loads are
    // outstanding; the barrier makes every wave's part visible and ends this
    // step's reads of the slots the next step refills
    __builtin_amdgcn_s_waitcnt(vmcnt_only(DMA));
    lds_barrier();
    ++c0;
  };
  int32_t r3 = 0;   // c0 mod 3: the K slot of tile c0
  while (c0 < n_cand) {
    const int32_t r3n = r3 == 2 ? 0 : r3 + 1;
    step(r3, r3n, 0, 1, sa, sb);
    r3 = r3n;
    if (c0 >= n_cand) break;
    const int32_t r3m = r3 == 2 ? 0 : r3 + 1;
    step(r3, r3m, 1, 0, sb, sa);
    r3 = r3m;
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));   // no load into LDS outlives the loop

  // ---- epilogue: l across the two halves, normalise, store ----
  l_run = sum_xor32(l_run);
  if (!row_ok) return;
  const float inv = 1.f / l_run;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + (((int64_t)it.b * a.num_q + t) * a.hq + it.hq) * D;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d = 32 * mt + 8 * i4 + 4 * hf;
      const uint2 w = uint2{pack_bf16x2(acc[mt][4 * i4] * inv, acc[mt][4 * i4 + 1] * inv),
                            pack_bf16x2(acc[mt][4 * i4 + 2] * inv, acc[mt][4 * i4 + 3] * inv)};
      *reinterpret_cast<uint2*>(orow + d) = w;
    }
  if (a.lse && hf == 0) a.lse[((int64_t)it.b * a.hq + it.hq) * a.num_q + t] = (ref + __log2f(l_run)) * kLn2;
}

// ---------------------------------------------------------------------------
// plan export: one workgroup enumerates the walk the attention kernels execute
// ---------------------------------------------------------------------------
constexpr int kPlanThreads = 256;

__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillGeom geo, int32_t* tiles,
                                                                    int32_t max_tiles, int32_t* num_tiles) {
  __shared__ int32_t part[kPlanThreads];
  const int tid = threadIdx.x;
  const int32_t n_qt = pf_num_qtiles(geo);
  const int32_t per = (n_qt + kPlanThreads - 1) / kPlanThreads;
  const int32_t q0 = tid * per, q1 = q0 + per < n_qt ? q0 + per : n_qt;
  int32_t cnt = 0;
  for (int32_t qt = q0; qt < q1; ++qt) {
    cnt += pf_walk(geo, qt).n_cand;
  }
  part[tid] = cnt;
  __syncthreads();
  if (tid == 0) {
    int32_t run = 0;
    for (int i = 0; i < kPlanThreads; ++i) {
      const int32_t c = part[i];
      part[i] = run;
      run += c;
    }
    *num_tiles = run;
  }
  __syncthreads();
  int32_t o = part[tid];
  for (int32_t qt = q0; qt < q1; ++qt) {
    const Walk walk = pf_walk(geo, qt);
    for (int32_t ci = 0; ci < walk.n_cand; ++ci) {
      const int32_t kt = pf_walk_tile(walk, ci);
      const int kind = pf_walk_kind(geo, qt, walk, ci);
      if (o < max_tiles) {
        tiles[3 * (int64_t)o + 0] = qt;
        tiles[3 * (int64_t)o + 1] = kt;
        tiles[3 * (int64_t)o + 2] = kind;
      }
      ++o;
    }
  }
}

template <typename T, int D, bool kPerSeq>
hipError_t launch_attention_t(const PrefillArgs& a, hipStream_t stream) {
  const int32_t n_qt = (a.num_q + a.bm - 1) / a.bm;
  const int64_t total = (int64_t)a.batch * a.hq * n_qt;
  const dim3 grid((uint32_t)(((total + 7) / 8) * 8));
  if (sizeof(T) == 2)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, kPerSeq>), grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_f32_kernel<D, kPerSeq>), grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

int64_t prep_blocks(const PrefillArgs& a) {
  int64_t blocks = (int64_t)a.batch * (a.nkp / 64);
  return blocks < 1 ? 1 : (blocks > 16384 ? 16384 : blocks);
}

template <typename T, int D>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_prep_kernel<T, D>), dim3((uint32_t)prep_blocks(a)), dim3(256), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attention_t<T, D, false>(a, stream);
}

template <typename T, int D>
hipError_t launch_chunk_t(const PrefillArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_prep_kernel<T, D>), dim3((uint32_t)prep_blocks(a)), dim3(256), 0, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_attention_t<T, D, true>(a, stream);
}

}  // namespace

void prefill_tile_shape(int32_t dtype, int32_t head_dim, int32_t* bm, int32_t* bn) {
  (void)head_dim;
  if (dtype == PS_BF16) {
    *bm = PfTraits<uint16_t>::BM;
    *bn = PfTraits<uint16_t>::BN;
  } else {
    *bm = PfTraits<float>::BM;
    *bn = PfTraits<float>::BN;
  }
}

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.num_q == 0) return hipSuccess;
  if (a.dtype == PS_BF16)
    return a.head_dim == 64 ? launch_prefill_t<uint16_t, 64>(a, stream) : launch_prefill_t<uint16_t, 128>(a, stream);
  return a.head_dim == 64 ? launch_prefill_t<float, 64>(a, stream) : launch_prefill_t<float, 128>(a, stream);
}

hipError_t launch_chunk_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.num_q == 0) return hipSuccess;
  if (a.dtype == PS_BF16)
    return a.head_dim == 64 ? launch_chunk_t<uint16_t, 64>(a, stream) : launch_chunk_t<uint16_t, 128>(a, stream);
  return a.head_dim == 64 ? launch_chunk_t<float, 64>(a, stream) : launch_chunk_t<float, 128>(a, stream);
}

hipError_t launch_prefill_plan(int32_t num_q, int32_t num_k, int32_t prefix_len, int32_t window,
                               int64_t kv_start, int32_t bm, int32_t bn, int32_t* tiles, int32_t max_tiles,
                               int32_t* num_tiles, hipStream_t stream) {
  PrefillGeom geo{num_q, num_k, prefix_len, window, kv_start, bm, bn};
  hipLaunchKernelGGL(prefill_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, geo, tiles, max_tiles, num_tiles);
  return hipGetLastError();
}

}  // namespace ps
