// Backward of the masked prefill attention: dq, dk, dv for the raw inputs.
//
// Blog "Prefix Sliding 完全拆解" (pinghaoyang.com.cn): section
// "超长 rollouts 的反向传播：截断回传" (the trainer back-propagates through the
// masked attention of the last 4W tokens; its loss mask only zeroes rows of the
// upstream gradient) and section "Kernel 实现：两层级过滤" (only tiles holding a
// visible pair are visited; element masks only on partly visible tiles).
//
// Per query head h with KV head g, log2 units (Q'' = scale*log2(e) * Q'):
//   P = exp2(Q'' K'^T - lse2)   (the forward's LSE, so no running max)
//   dV_g += P^T dO,  dP = dO V^T,  dS = P (dP - Di),  Di = rowsum(dO * O)
//   dQ' = scale * dS K',   dK'_g += ln2 * dS^T Q''
// and dQ, dK are dQ', dK' rotated back by -position (the rotation is orthogonal).
//
// Pipeline of one call:
//   1. key prep: K' row-major and d-major (keys permuted per 16, vt_slot), V
//      row-major, zero padded to nkp keys; cos/sin of the key positions.
//   2. query prep: Q'' row-major, lse2 (+inf on padding rows so their P is 0),
//      Di; cos/sin of the query positions.
//   3. dk/dv kernel: one workgroup per (batch, KV head, 128-key tile), each wave
//      owning 32 keys whose K' and V stay in registers as MFMA B operands; it
//      walks the query heads of the group and the 64-query blocks that see the
//      tile.  S = Q'' K'^T and dP = dO V^T put queries on the M side, so each
//      lane owns one key and the S / dS registers are directly the B operands of
//      dV^T += dO^T P and dK^T += Q''^T dS, whose A operands (dO^T, Q''^T in the
//      matching query order) come from the row-major tiles by transposing LDS
//      reads.  No atomics: every dk / dv row has one writer.  With room in the
//      workspace it also stores each block's dS^T tile for step 4.
//   4. dq kernel, on the forward's key-tile schedule: from the kept dS^T tiles,
//      dQ^T += K'^T dS^T (one product); without them it forms S^T = K' Q''^T,
//      dP^T = V dO^T and dS^T again first.
// All arithmetic on MFMA is bf16 x bf16 -> fp32; P and dS are rounded to bf16
// as MFMA operands.  The fp32 kernels at the end are the debug path (plain
// loops, one thread per query or key row).
#include "ps_internal.h"
#include "ps_sched.h"
#include "ps_tiles.h"

namespace ps {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2f = 0.69314718055994531f;

// ---------------------------------------------------------------------------
// 1. key prep: one workgroup per (batch, 64-key tile); thread = quarter of a key row
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_key_prep_kernel(BackwardArgs a) {
  constexpr int TK = 64;
  constexpr int HALF = D / 2;
  constexpr int PQ = HALF / 4;   // rotation pairs per thread
  constexpr int DQ = D / 4;      // value dims per thread
  __shared__ float cs_lds[TK][HALF][2];
  __shared__ T t_lds[D][TK + 8];
  PrefillGeom geo{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, 64, 64};
  const int32_t nkt = a.nkp / TK;
  const int tid = threadIdx.x;
  const int j = tid >> 2, qq = tid & 3;
  const T* k = static_cast<const T*>(a.k);
  const T* v = static_cast<const T*>(a.v);
  T* kr = static_cast<T*>(a.kr);
  T* krt = static_cast<T*>(a.krt);
  T* vr = static_cast<T*>(a.vr);
  for (int64_t blk = blockIdx.x; blk < (int64_t)a.batch * nkt; blk += gridDim.x) {
    const int32_t kt = (int32_t)(blk % nkt);
    const int32_t b = (int32_t)(blk / nkt);
    __syncthreads();
    for (int idx = tid; idx < TK * HALF; idx += 256) {
      const int jj = idx / HALF, i = idx % HALF;
      const int32_t key = kt * TK + jj;
      float c = 1.f, sn = 0.f;
      if (a.rope.enabled && key < a.num_k) rope_cos_sin(pf_key_pos(geo, key), a.rope.inv_freq[i], c, sn);
      cs_lds[jj][i][0] = c;
      cs_lds[jj][i][1] = sn;
      if (b == 0) {
        a.cs_k[((int64_t)key * HALF + i) * 2 + 0] = c;
        a.cs_k[((int64_t)key * HALF + i) * 2 + 1] = sn;
      }
    }
    __syncthreads();
    const int32_t key = kt * TK + j;
    for (int32_t h = 0; h < a.hkv; ++h) {
      const int64_t bh = (int64_t)b * a.hkv + h;
      float x1[PQ], x2[PQ], vv[DQ];
      if (key < a.num_k) {
        const int64_t src = (((int64_t)b * a.num_k + key) * a.hkv + h) * D;
        load_vec(k + src + PQ * qq, x1, PQ);
        load_vec(k + src + HALF + PQ * qq, x2, PQ);
        load_vec(v + src + DQ * qq, vv, DQ);
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
      T* krow = kr + (bh * a.nkp + key) * D;
      store_vec(krow + PQ * qq, x1, PQ);
      store_vec(krow + HALF + PQ * qq, x2, PQ);
      store_vec(vr + (bh * a.nkp + key) * D + DQ * qq, vv, DQ);
      // K'^T through LDS (rounded exactly as the row-major copy)
      const int js = vt_slot(j);
#pragma unroll
      for (int e = 0; e < PQ; ++e) {
        Elem<T>::store(&t_lds[PQ * qq + e][js], x1[e]);
        Elem<T>::store(&t_lds[HALF + PQ * qq + e][js], x2[e]);
      }
      __syncthreads();
      constexpr int EP = 16 / sizeof(T);
      for (int idx = tid; idx < D * (TK / EP); idx += 256) {
        const int d = idx / (TK / EP), c = idx % (TK / EP);
        *reinterpret_cast<u32x4*>(krt + (bh * D + d) * a.nkp + kt * TK + c * EP) =
            *reinterpret_cast<const u32x4*>(&t_lds[d][c * EP]);
      }
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// 2a. cos/sin of every query position, once (the query prep of every batch and
//     head and the dq kernel's back-rotation read it)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_query_cs_kernel(BackwardArgs a) {
  constexpr int HALF = D / 2;
  PrefillGeom geo{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, 64, 64};
  const int64_t n = (int64_t)a.num_q * HALF;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * 256) {
    const int32_t t = (int32_t)(idx / HALF), i = (int32_t)(idx % HALF);
    float c = 1.f, sn = 0.f;
    if (a.rope.enabled) rope_cos_sin(pf_query_pos(geo, t), a.rope.inv_freq[i], c, sn);
    reinterpret_cast<float2*>(a.cs_q)[idx] = make_float2(c, sn);
  }
}

// ---------------------------------------------------------------------------
// 2b. query prep: one workgroup per (batch, query head, 64-query tile)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_query_prep_kernel(BackwardArgs a) {
  constexpr int TQ = 64;
  constexpr int HALF = D / 2;
  constexpr int PQ = HALF / 4;
  constexpr int DQ = D / 4;
  const int32_t nqt = a.tqp / TQ;
  const int tid = threadIdx.x;
  const int j = tid >> 2, qq = tid & 3;
  const T* q = static_cast<const T*>(a.q);
  const T* o = static_cast<const T*>(a.out);
  const T* dout = static_cast<const T*>(a.d_out);
  T* qs = static_cast<T*>(a.qs);
  for (int64_t blk = blockIdx.x; blk < (int64_t)a.batch * a.hq * nqt; blk += gridDim.x) {
    const int32_t qt = (int32_t)(blk % nqt);
    const int64_t rest = blk / nqt;
    const int32_t h = (int32_t)(rest % a.hq);
    const int32_t b = (int32_t)(rest / a.hq);
    const int32_t t = qt * TQ + j;
    const bool row_ok = t < a.num_q;
    const int64_t bh = (int64_t)b * a.hq + h;
    float x1[PQ], x2[PQ];
    float dsum = 0.f;
    if (row_ok) {
      const int64_t src = (((int64_t)b * a.num_q + t) * a.hq + h) * D;
      load_vec(q + src + PQ * qq, x1, PQ);
      load_vec(q + src + HALF + PQ * qq, x2, PQ);
      const float4* cs = reinterpret_cast<const float4*>(a.cs_q + ((int64_t)t * HALF + PQ * qq) * 2);
      float csv[2 * PQ];
#pragma unroll
      for (int e = 0; e < PQ / 2; ++e) {
        const float4 w = cs[e];
        csv[4 * e] = w.x;
        csv[4 * e + 1] = w.y;
        csv[4 * e + 2] = w.z;
        csv[4 * e + 3] = w.w;
      }
#pragma unroll
      for (int e = 0; e < PQ; ++e) {
        const float c = csv[2 * e], sn = csv[2 * e + 1];
        const float y1 = x1[e] * c - x2[e] * sn, y2 = x2[e] * c + x1[e] * sn;
        x1[e] = y1 * a.scale_log2;
        x2[e] = y2 * a.scale_log2;
      }
      float od[DQ], ov[DQ];
      load_vec(dout + src + DQ * qq, od, DQ);
      load_vec(o + src + DQ * qq, ov, DQ);
#pragma unroll
      for (int e = 0; e < DQ; ++e) dsum += od[e] * ov[e];
    } else {
#pragma unroll
      for (int e = 0; e < PQ; ++e) x1[e] = x2[e] = 0.f;
    }
    // the four quarter-rows of a query are four consecutive lanes
    dsum += __shfl_xor(dsum, 1);
    dsum += __shfl_xor(dsum, 2);
    T* qrow = qs + (bh * a.tqp + t) * D;
    store_vec(qrow + PQ * qq, x1, PQ);
    store_vec(qrow + HALF + PQ * qq, x2, PQ);
    if (qq == 0) {
      a.lse2[bh * a.tqp + t] = row_ok ? a.lse[bh * a.num_q + t] * kLog2e : INFINITY;
      a.di[bh * a.tqp + t] = dsum;
    }
  }
}

// 32x32x16 MFMA lane layout (lane l, half hf = l/32, col = l%32):
//   A[m][k]: lane (m + 32*(k/8)) element k%8        B[k][n]: lane (n + 32*(k/8)) element k%8
//   D[m][n]: lane (n + 32*((m/4)%2)) register 4*(m/8) + m%4
// so register r of a D tile holds row m = 8*(r/4) + 4*hf + r%4 of column col.

// dS^T tiles the dk/dv kernel can keep for the dq kernel: one [128 keys][64
// queries] bf16 tile per visited (64-query block qb, 128-key tile kt) pair, at
// tile index ((b * hq + h) * (tqp / 64) + qb) * ds_slots + slot, where slot is
// the position of kt in the block's walk (prefix tiles, then band tiles; the
// walk holds exactly the tiles with a visible pair).  A row holds one key's 64
// queries in the order of the P / dS registers: position 16 j + 8 hf + e <->
// query 16 j + 8 (e / 4) + 4 hf + e % 4 (vt_slot).
constexpr int kDsKeys = 128, kDsQueries = 64;
__device__ inline int32_t ds_slot(const PrefillGeom& g64x128, int32_t qb, int32_t kt) {
  const TileRange tr = pf_tile_range(g64x128, qb);
  return kt < tr.n_prefix ? kt : tr.n_prefix + (kt - tr.band_lo);
}
__device__ inline int64_t ds_tile(const BackwardArgs& a, int32_t b, int32_t h, int32_t qb, int32_t slot) {
  return ((((int64_t)b * a.hq + h) * (a.tqp / kDsQueries) + qb) * a.ds_slots + slot) * (kDsKeys * kDsQueries);
}

// ---------------------------------------------------------------------------
// 3. dk / dv (bf16 MFMA); kKeepDs: also store each block's dS^T tile
// ---------------------------------------------------------------------------
template <int D, bool kKeepDs>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(BackwardArgs a) {
  constexpr int BK = 128;          // keys per workgroup, 32 per wave
  constexpr int BQ = 64;           // queries per step
  constexpr int KS = D / 16;
  constexpr int MT = D / 32;
  constexpr int RCH = D / 8;       // 16-byte chunks per row-major query row
  constexpr int DMA = BQ * D / 8 / 256;   // 1 KB wave loads per wave per tile (each of the four)
  // query block tiles, two buffers each; 16-byte chunks XOR-swizzled by row
  // (conflict-free operand reads without padding, so whole tiles go global ->
  // LDS directly)
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds[2][BQ * D];    // Q'' rows
  __shared__ __attribute__((aligned(1024))) uint16_t o_lds[2][BQ * D];    // dO rows
  __shared__ __attribute__((aligned(1024))) float ld_lds[2][2 * BQ];      // lse2, then Di
  __shared__ __attribute__((aligned(1024))) uint16_t st_lds[kKeepDs ? 4 * 32 * kDsQueries : 1];   // dS^T staging, per wave

  const int32_t n_kt = (a.num_k + BK - 1) / BK;
  const int64_t pairs = (int64_t)a.batch * a.hkv;
  // key-tile-major order: the tiles holding pinned keys (seen by every query,
  // the longest) start first; tiles of one (batch, KV head) land on one XCD
  const int64_t lin = blockIdx.x;
  if (lin >= pairs * n_kt) return;
  const int32_t kt = (int32_t)(lin / pairs);
  const int32_t kvh = (int32_t)((lin % pairs) % a.hkv);
  const int32_t b = (int32_t)((lin % pairs) / a.hkv);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int32_t k0 = kt * BK;
  const int32_t kw = k0 + 32 * wave + col;     // this lane's key
  const int64_t bkv = (int64_t)b * a.hkv + kvh;
  const uint16_t* kr = static_cast<const uint16_t*>(a.kr) + bkv * a.nkp * D;
  const uint16_t* vr = static_cast<const uint16_t*>(a.vr) + bkv * a.nkp * D;

  // the wave's keys as B operands: B[k = dim][n = key]
  bf16x8 kop[KS], vop[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kop[ks] = *reinterpret_cast<const bf16x8*>(kr + (int64_t)kw * D + 16 * ks + 8 * hf);
    vop[ks] = *reinterpret_cast<const bf16x8*>(vr + (int64_t)kw * D + 16 * ks + 8 * hf);
    // keep them in registers: left as plain loads of read-only memory, the
    // compiler re-issues them inside the loop and waits on them every step
    asm volatile("" : "+v"(kop[ks]), "+v"(vop[ks]));
  }

  // query blocks that can see the tile: from the first query at or after k0 to
  // the last query (pinned keys) or to the end of the last key's window
  const int32_t k1 = pf_min(k0 + BK, a.num_k) - 1;
  const int32_t off = a.num_k - a.num_q;          // key index of query 0
  const int32_t t_lo = pf_max(0, k0 - off);
  const int32_t t_hi = k0 < a.prefix_len ? a.num_q - 1 : pf_min(a.num_q - 1, k1 + a.window - 1 - off);
  const int32_t qb_lo = t_lo / BQ, qb_hi = t_lo <= t_hi ? t_hi / BQ : -1;
  const int32_t n_qb = qb_hi - qb_lo + 1;
  const int32_t n_it = n_qb > 0 ? n_qb * a.group : 0;
  PrefillGeom cg{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, BQ, BK};

  // block (head h, query block qb) -> LDS buffer bf, straight from global
  // memory: wave load p of wave w fills chunks (4p + w) * 64 + lane of each
  // tile; the swizzle of a chunk's row depends on (w, lane) only
  const int rrow = wave * (64 / RCH) + lane / RCH;                 // + 4p * 64 / RCH
  const int rchunk = (lane % RCH) ^ chunk_swizzle<RCH>(rrow);
  auto load_block = [&](int32_t h, int32_t qb, int bf) {
    const int64_t bh = (int64_t)b * a.hq + h;
    const uint16_t* qsb = static_cast<const uint16_t*>(a.qs) + (bh * a.tqp + (int64_t)qb * BQ) * D;
    const uint32_t w_off = wave * 1024;
#pragma unroll
    for (int p = 0; p < DMA; ++p) {
      const int r = rrow + 4 * p * (64 / RCH);   // query row of the block
      dma_to_lds(qsb + (int64_t)r * D + rchunk * 8, lds_address(q_lds[bf]) + w_off + p * 4096);
      const int32_t tr = pf_min(qb * BQ + r, a.num_q - 1);
      dma_to_lds(static_cast<const uint16_t*>(a.d_out) + (((int64_t)b * a.num_q + tr) * a.hq + h) * D + rchunk * 8,
                 lds_address(o_lds[bf]) + w_off + p * 4096);
    }
    // lse2 and Di of the block's 64 queries: 2 x 256 bytes, lanes 0-31 of wave 0
    if (wave == 0 && lane < 32) {
      const float* src = (lane < 16 ? a.lse2 : a.di) + bh * a.tqp + (int64_t)qb * BQ + 4 * (lane & 15);
      dma_to_lds(src, lds_address(ld_lds[bf]));
    }
  };
  // operand addresses (elements) inside a tile: row-major row r, logical chunk c
  auto rm_at = [&](int r, int c) { return r * D + ((c ^ chunk_swizzle<RCH>(r)) * 8); };

  f32x16 dk[MT], dv[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) dk[mt][i] = dv[mt][i] = 0.f;
  f32x16 zero;
#pragma unroll
  for (int i = 0; i < 16; ++i) zero[i] = 0.f;

  // iteration it -> (head in group, query block); blocks with no visible pair are skipped
  int32_t it = 0;
  int kind = 0;
  while (it < n_it && (kind = pf_classify(cg, qb_lo + it % n_qb, kt)) == 0) ++it;
  if (it < n_it) load_block(kvh * a.group + it / n_qb, qb_lo + it % n_qb, 0);
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  __syncthreads();
  int buf = 0;
  // dS^T of a block goes through the wave's LDS staging rows (32 keys x 128
  // bytes, 16-byte chunks XOR-swizzled by row % 8) so that each global store
  // writes 8 whole rows (1 KB); the stores of a block are issued in the middle
  // of the next iteration (measured: at its start, ahead of or behind the next
  // block's loads, they cost 3-10 % more)
  int64_t keep_at = -1;
  uint16_t* stg = st_lds + wave * 32 * kDsQueries;
  auto stage = [&](int r, int c) { return r * kDsQueries + ((c ^ (r & 7)) * 8); };
  uint16_t* ds = kKeepDs ? static_cast<uint16_t*>(a.ds) + (32 * wave + lane / 8) * kDsQueries + (lane % 8) * 8 : nullptr;
  bf16x8 kept[4];
  auto read_kept = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) kept[i] = *reinterpret_cast<const bf16x8*>(&stg[stage(8 * i + lane / 8, lane % 8)]);
  };
  auto store_kept = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<bf16x8*>(ds + keep_at + 8 * i * kDsQueries) = kept[i];
  };
  while (it < n_it) {
    const int32_t h = kvh * a.group + it / n_qb;
    const int32_t qb = qb_lo + it % n_qb;
    const int cur_kind = kind;
    int32_t nx = it + 1;
    int nkind = 0;
    while (nx < n_it && (nkind = pf_classify(cg, qb_lo + nx % n_qb, kt)) == 0) ++nx;
    if (kKeepDs && keep_at >= 0) read_kept();
    if (nx < n_it) load_block(kvh * a.group + nx / n_qb, qb_lo + nx % n_qb, buf ^ 1);   // its buffer was read last iteration

    // S = Q'' K'^T and dP = dO V^T (two 32-query M-tiles), then
    // dV^T += dO^T P and dK^T += Q''^T dS over the block's 64 queries.  One
    // wave per SIMD, so the wave overlaps its own matrix and vector work:
    // M-tile 1's products run while M-tile 0's P and dS are formed, and the
    // first half of the dV / dK k-steps (queries of M-tile 0) runs while
    // M-tile 1's are formed.  Register r of tile m2 <-> query
    // 32*m2 + 8*(r/4) + 4*hf + r%4 of the block; PV k-step j covers queries
    // 16j + 8*(e/4) + 4*hf + e%4 (M-tile j/2).
    f32x16 s[2], dp[2];
    bf16x8 pb[4], sb[4];
    auto products = [&](int m2) {
      const int r = 32 * m2 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(&q_lds[buf][rm_at(r, 2 * ks + hf)]);
        const bf16x8 oa = *reinterpret_cast<const bf16x8*>(&o_lds[buf][rm_at(r, 2 * ks + hf)]);
        s[m2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kop[ks], ks == 0 ? zero : s[m2], 0, 0, 0);
        dp[m2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vop[ks], ks == 0 ? zero : dp[m2], 0, 0, 0);
      }
    };
    auto softmax_ds = [&](int m2) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int ql = 32 * m2 + 8 * r4 + 4 * hf;
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&ld_lds[buf][ql]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&ld_lds[buf][BQ + ql]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float p = __builtin_amdgcn_exp2f(s[m2][r] - l4[e]);
          const float ds = p * (dp[m2][r] - d4[e]);
          pb[2 * m2 + (r >> 3)][r & 7] = (bf16)p;
          sb[2 * m2 + (r >> 3)][r & 7] = (bf16)ds;
        }
      }
    };
    // a partly visible block: queries that do not see this lane's key get S = -inf
    auto mask = [&](int m2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int32_t uq = off + qb * BQ + 32 * m2 + 8 * (r >> 2) + 4 * hf + (r & 3);
        if (!pf_visible(cg, uq, kw) || kw >= a.num_k) s[m2][r] = -INFINITY;
      }
    };
    auto dvdk = [&](int j) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // dims 32 mt + m, queries in the k order of P / dS: gathered from the row-major tiles
        const bf16x8 oa = gather_cols<D>(o_lds[buf], mt, j, lane);
        const bf16x8 qa = gather_cols<D>(q_lds[buf], mt, j, lane);
        dv[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, pb[j], dv[mt], 0, 0, 0);
        dk[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, sb[j], dk[mt], 0, 0, 0);
      }
    };
    const bool partial = __builtin_expect(cur_kind == 2, 0);   // partly visible blocks are few
    products(0);
    if (partial) mask(0);
    __builtin_amdgcn_sched_barrier(0);
    if (kKeepDs && keep_at >= 0) store_kept();   // the previous block's dS^T
    __builtin_amdgcn_sched_barrier(0);
    products(1);
    softmax_ds(0);
#pragma unroll
    for (int i = 0; i < 2 * KS; ++i) {   // each MFMA with an operand read and a share of the vector work
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (partial) mask(1);
    __builtin_amdgcn_sched_barrier(0);
    dvdk(0);
    dvdk(1);
    softmax_ds(1);
#pragma unroll
    for (int i = 0; i < 4 * MT; ++i) {   // (two transposing reads per operand)
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    dvdk(2);
    dvdk(3);
    if (kKeepDs) {
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<bf16x8*>(&stg[stage(col, 2 * j + hf)]) = sb[j];
      keep_at = ds_tile(a, b, h, qb, ds_slot(cg, qb, kt));
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));   // the next block has landed (this wave's part)
    __syncthreads();
    buf ^= 1;
    it = nx;
    kind = nkind;
  }
  if (kKeepDs && keep_at >= 0) {
    read_kept();
    store_kept();
  }

  // ---- epilogue: register r of tile mt <-> dim 32*mt + 8*(r/4) + 4*hf + r%4 of key kw;
  // dK' = ln2 * acc, rotated back by -position (dims d and d + D/2 pair up: tiles mt, mt + MT/2)
  if (kw >= a.num_k) return;
  uint16_t* dkrow = static_cast<uint16_t*>(a.dk) + (((int64_t)b * a.num_k + kw) * a.hkv + kvh) * D;
  uint16_t* dvrow = static_cast<uint16_t*>(a.dv) + (((int64_t)b * a.num_k + kw) * a.hkv + kvh) * D;
  const float* cs = a.cs_k + (int64_t)kw * D;
#pragma unroll
  for (int mt = 0; mt < MT / 2; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * mt + 8 * r4 + 4 * hf;
      float g1[4], g2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = cs[2 * (d + e)], sn = cs[2 * (d + e) + 1];
        const float x1 = dk[mt][4 * r4 + e] * kLn2f, x2 = dk[mt + MT / 2][4 * r4 + e] * kLn2f;
        g1[e] = x1 * c + x2 * sn;
        g2[e] = x2 * c - x1 * sn;
      }
      *reinterpret_cast<uint2*>(dkrow + d) = uint2{pack_bf16x2(g1[0], g1[1]), pack_bf16x2(g1[2], g1[3])};
      *reinterpret_cast<uint2*>(dkrow + d + D / 2) = uint2{pack_bf16x2(g2[0], g2[1]), pack_bf16x2(g2[2], g2[3])};
    }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * mt + 8 * r4 + 4 * hf;
      *reinterpret_cast<uint2*>(dvrow + d) = uint2{pack_bf16x2(dv[mt][4 * r4], dv[mt][4 * r4 + 1]),
                                                   pack_bf16x2(dv[mt][4 * r4 + 2], dv[mt][4 * r4 + 3])};
    }
}

// ---------------------------------------------------------------------------
// 4. dq (bf16 MFMA): the forward's decomposition and key-tile schedule
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(BackwardArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int KS = D / 16;
  constexpr int MT = D / 32;
  constexpr int RCH = D / 8;       // 16-byte chunks per key row
  constexpr int TCH = BN / 8;      // 16-byte chunks per d-major row
  constexpr int DMA = BN * D / 8 / 256;   // 1 KB wave loads per wave per tile
  // key tiles, two buffers each, 16-byte chunks XOR-swizzled by row (loaded
  // global -> LDS directly)
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2][BN * D];   // K' rows
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[2][BN * D];   // V rows
  __shared__ __attribute__((aligned(1024))) uint16_t t_lds[2][D * BN];   // K' d-major

  PrefillGeom geo{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, BM, BN};
  const int32_t n_qt = pf_num_qtiles(geo);
  // items ordered (batch, KV head, q-tile, head-in-group), each XCD a contiguous run
  const int64_t total = (int64_t)a.batch * a.hq * n_qt;
  const int64_t per = (total + 7) / 8;
  const int64_t lin = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (lin >= total) return;
  const int32_t hg = (int32_t)(lin % a.group);
  int64_t rest = lin / a.group;
  const int32_t qt = (int32_t)(rest % n_qt);
  rest /= n_qt;
  const int32_t kvh = (int32_t)(rest % a.hkv);
  const int32_t b = (int32_t)(rest / a.hkv);
  const int32_t hq = kvh * a.group + hg;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int64_t bkv = (int64_t)b * a.hkv + kvh;
  const uint16_t* kr = static_cast<const uint16_t*>(a.kr) + bkv * a.nkp * D;
  const uint16_t* vr = static_cast<const uint16_t*>(a.vr) + bkv * a.nkp * D;
  const uint16_t* ktr = static_cast<const uint16_t*>(a.krt) + bkv * D * a.nkp;

  // tile kt -> LDS buffer, straight from global memory: wave load p of wave w
  // fills chunks (4p + w) * 64 + lane; the swizzle of a chunk's row depends on
  // (w, lane) only
  const int rrow = wave * (64 / RCH) + lane / RCH;
  const int rchunk = (lane % RCH) ^ chunk_swizzle<RCH>(rrow);
  const int trow_l = wave * (64 / TCH) + lane / TCH;
  const int tchunk = (lane % TCH) ^ chunk_swizzle<TCH>(trow_l);
  auto load_kv = [&](int32_t kt, int b_) {
#pragma unroll
    for (int p = 0; p < DMA; ++p) {
      const int64_t o = ((int64_t)kt * BN + rrow + 4 * p * (64 / RCH)) * D + rchunk * 8;
      dma_to_lds(kr + o, lds_address(k_lds[b_]) + wave * 1024 + p * 4096);
      dma_to_lds(vr + o, lds_address(v_lds[b_]) + wave * 1024 + p * 4096);
    }
  };
  auto load_t = [&](int32_t kt, int b_) {
#pragma unroll
    for (int p = 0; p < DMA; ++p)
      dma_to_lds(ktr + (int64_t)(trow_l + 4 * p * (64 / TCH)) * a.nkp + (int64_t)kt * BN + tchunk * 8,
                 lds_address(t_lds[b_]) + wave * 1024 + p * 4096);
  };
  // operand addresses (elements) inside a tile: row-major row r, logical chunk c
  auto rm_at = [&](int r, int c) { return r * D + ((c ^ chunk_swizzle<RCH>(r)) * 8); };
  auto dm_at = [&](int r, int c) { return r * BN + ((c ^ chunk_swizzle<TCH>(r)) * 8); };

  const TileRange tr = pf_tile_range(geo, qt);
  const int32_t n_cand = tr.n_prefix + (tr.band_hi >= tr.band_lo ? tr.band_hi - tr.band_lo + 1 : 0);
  auto cand_tile = [&](int32_t ci) { return ci < tr.n_prefix ? ci : tr.band_lo + (ci - tr.n_prefix); };
  auto next_live = [&](int32_t ci, int& kind) {   // first candidate >= ci that is not skipped
    kind = 0;
#pragma clang loop vectorize(disable) interleave(disable) unroll(disable)
    while (ci < n_cand && (kind = pf_classify(geo, qt, cand_tile(ci))) == 0) ++ci;
    return ci;
  };
  // tiles c0 (j) and c1 (j+1) of the walk
  int kind0 = 0, kind1 = 0;
  int32_t c0 = next_live(0, kind0);
  int32_t c1 = c0 < n_cand ? next_live(c0 + 1, kind1) : n_cand;
  if (c0 < n_cand) {
    load_kv(cand_tile(c0), 0);
    load_t(cand_tile(c0), 0);
  }
  if (c1 < n_cand) load_kv(cand_tile(c1), 1);

  // this lane's query: B operands of S^T = K' Q''^T and dP^T = V dO^T
  const int32_t t = qt * BM + wave * 32 + col;
  const bool row_ok = t < a.num_q;
  const int32_t tc = row_ok ? t : 0;
  const int32_t u = a.num_k - a.num_q + t;
  const int64_t bh = (int64_t)b * a.hq + hq;
  bf16x8 qop[KS], dop[KS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.qs) + (bh * a.tqp + tc) * D;
    const uint16_t* drow = static_cast<const uint16_t*>(a.d_out) + (((int64_t)b * a.num_q + tc) * a.hq + hq) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qop[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks + 8 * hf);
      dop[ks] = *reinterpret_cast<const bf16x8*>(drow + 16 * ks + 8 * hf);
      asm volatile("" : "+v"(qop[ks]), "+v"(dop[ks]));   // registers, not re-issued loads
    }
  }
  const float lse2 = row_ok ? a.lse2[bh * a.tqp + t] : INFINITY;
  const float di = row_ok ? a.di[bh * a.tqp + t] : 0.f;
  const int32_t pre_end = row_ok ? pf_min(a.prefix_len, u + 1) : 0;
  int32_t band_lo = pf_max(a.prefix_len, u - a.window + 1);
  const int32_t band_hi = pf_min(u, a.num_k - 1);
  uint32_t band_w = (uint32_t)(band_hi - band_lo);
  if (!row_ok || band_hi < band_lo) {
    band_lo = 0x7fffffff;
    band_w = 0;
  }
  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;
  // initial value of the S^T accumulators: the MFMAs then yield s - lse2
  f32x16 neg_lse2, zero;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    neg_lse2[i] = -lse2;
    zero[i] = 0.f;
  }

  // register i of tile m2 <-> key kt*BN + 32*m2 + 8*(i/4) + 4*hf + i%4; keys
  // a partly visible tile hides get S - lse2 = -inf, so their P and dS are zero
  auto mask = [&](int32_t kt, f32x16* st) {
    const int32_t kbase = kt * BN + 4 * hf;
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int32_t key = kbase + 32 * m2 + 8 * (i >> 2) + (i & 3);
        const bool vis = key < pre_end || (uint32_t)(key - band_lo) <= band_w;
        if (!vis) st[m2][i] = -INFINITY;
      }
  };
  // S^T and dP^T of the K'/V tile in buffer b_ (not pipelined: the first tile)
  auto sdp = [&](int b_, f32x16* st, f32x16* dpt) {
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2) {
      const int r = 32 * m2 + col;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&k_lds[b_][rm_at(r, 2 * ks + hf)]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&v_lds[b_][rm_at(r, 2 * ks + hf)]);
        st[m2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qop[ks], ks == 0 ? neg_lse2 : st[m2], 0, 0, 0);
        dpt[m2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, dop[ks], ks == 0 ? zero : dpt[m2], 0, 0, 0);
      }
    }
  };

  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));   // (lse2 / Di and the first tiles)
  __syncthreads();
  f32x16 sa[2], pa[2], sb_[2], pb[2];   // S^T, dP^T of tiles c0 / c1, alternating between steps
  if (c0 < n_cand) {
    sdp(0, sa, pa);
    if (kind0 == 2) mask(cand_tile(c0), sa);
  }
  // One step, software-pipelined inside the wave (one wave per SIMD, so the
  // wave's own matrix and vector work must overlap): the S^T / dP^T products
  // of tile c1 run while tile c0's dS is formed, then dQ^T += K'^T dS^T for
  // tile c0.  K'/V of c1 sit in kv buffer kvb ^ 1, K'^T of c0 in t buffer tb;
  // the next tiles go straight to LDS: K'/V of c2 into kvb (c0's, read last
  // step) and K'^T of c1 into tb ^ 1 (read the step before).
  int kvb = 0, tb = 0;
  auto step = [&](f32x16* sc, f32x16* pc, f32x16* sn, f32x16* pn) {
    int kind2 = 0;
    const int32_t c2 = c1 < n_cand ? next_live(c1 + 1, kind2) : n_cand;
    if (c2 < n_cand) load_kv(cand_tile(c2), kvb);
    if (c1 < n_cand) load_t(cand_tile(c1), tb ^ 1);

    // sections: one k-step of the four S^T / dP^T products of tile c1 (its
    // operands read one k-step ahead) and a quarter-eighth of tile c0's dS
    constexpr int EPS = 32 / KS;
    bf16x8 sbv[4];
    const uint16_t* kb = k_lds[kvb ^ 1];
    const uint16_t* vb = v_lds[kvb ^ 1];
    auto kfrag = [&](const uint16_t* t_, int r, int ks) { return *reinterpret_cast<const bf16x8*>(&t_[rm_at(r, 2 * ks + hf)]); };
    bf16x8 k0 = kfrag(kb, col, 0), k1 = kfrag(kb, col + 32, 0);
    bf16x8 v0 = kfrag(vb, col, 0), v1 = kfrag(vb, col + 32, 0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 nk0 = k0, nk1 = k1, nv0 = v0, nv1 = v1;
      if (ks + 1 < KS) {
        nk0 = kfrag(kb, col, ks + 1);
        nk1 = kfrag(kb, col + 32, ks + 1);
        nv0 = kfrag(vb, col, ks + 1);
        nv1 = kfrag(vb, col + 32, ks + 1);
      }
      sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qop[ks], ks == 0 ? neg_lse2 : sn[0], 0, 0, 0);
      sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1, qop[ks], ks == 0 ? neg_lse2 : sn[1], 0, 0, 0);
      pn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v0, dop[ks], ks == 0 ? zero : pn[0], 0, 0, 0);
      pn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v1, dop[ks], ks == 0 ? zero : pn[1], 0, 0, 0);
#pragma unroll
      for (int e = 0; e < EPS; ++e) {
        const int idx = ks * EPS + e, m2 = idx >> 4, i = idx & 15;
        sbv[2 * m2 + (i >> 3)][i & 7] = (bf16)(__builtin_amdgcn_exp2f(sc[m2][i]) * (pc[m2][i] - di));
      }
      k0 = nk0;
      k1 = nk1;
      v0 = nv0;
      v1 = nv1;
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // the next k-step's operand reads,
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // this k-step's MFMAs,
      __builtin_amdgcn_sched_group_barrier(0x002, 32, 0);  // the vector work
      __builtin_amdgcn_sched_barrier(0);
    }
    // dQ''^T += K'^T dS^T for tile c0: k-step j covers keys 16j + 8*(e/4) + 4*hf + e%4
    {
      const uint16_t* tt = t_lds[tb];
      bf16x8 ta[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) ta[mt] = *reinterpret_cast<const bf16x8*>(&tt[dm_at(32 * mt + col, hf)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 tn[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          tn[mt] = j + 1 < 4 ? *reinterpret_cast<const bf16x8*>(&tt[dm_at(32 * mt + col, 2 * (j + 1) + hf)]) : ta[mt];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[mt], sbv[j], acc[mt], 0, 0, 0);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) ta[mt] = tn[mt];
        __builtin_amdgcn_sched_group_barrier(0x100, MT, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (__builtin_expect(c1 < n_cand && kind1 == 2, 0)) mask(cand_tile(c1), sn);   // partial tiles are few
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));   // this wave's part of the next tiles has landed
    __syncthreads();
    kvb ^= 1;
    tb ^= 1;
    c0 = c1;
    c1 = c2;
    kind1 = kind2;
  };
  while (c0 < n_cand) {
    step(sa, pa, sb_, pb);
    if (c0 >= n_cand) break;
    step(sb_, pb, sa, pa);
  }

  if (!row_ok) return;
  // dQ' = scale * acc, rotated back by -position
  uint16_t* dqrow = static_cast<uint16_t*>(a.dq) + (((int64_t)b * a.num_q + t) * a.hq + hq) * D;
  const float* cs = a.cs_q + (int64_t)t * D;
#pragma unroll
  for (int mt = 0; mt < MT / 2; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * mt + 8 * r4 + 4 * hf;
      float g1[4], g2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = cs[2 * (d + e)], sn = cs[2 * (d + e) + 1];
        const float x1 = acc[mt][4 * r4 + e] * a.scale, x2 = acc[mt + MT / 2][4 * r4 + e] * a.scale;
        g1[e] = x1 * c + x2 * sn;
        g2[e] = x2 * c - x1 * sn;
      }
      *reinterpret_cast<uint2*>(dqrow + d) = uint2{pack_bf16x2(g1[0], g1[1]), pack_bf16x2(g1[2], g1[3])};
      *reinterpret_cast<uint2*>(dqrow + d + D / 2) = uint2{pack_bf16x2(g2[0], g2[1]), pack_bf16x2(g2[2], g2[3])};
    }
}

// ---------------------------------------------------------------------------
// 4b. dq from the kept dS^T tiles (bf16 MFMA): dQ''^T += K'^T dS^T, one product
//     instead of three.  One workgroup per (batch, query head, 128-query tile),
//     walking the 64-key tiles of the forward's schedule.  Per tile the two
//     64-query halves' dS^T rows (keys of the tile, from the dk/dv kernel's
//     128-key tile) and the d-major K' tile go global -> LDS directly; a wave's
//     B operand (32 queries, 8 keys per lane) is gathered from the dS^T rows by
//     transposing LDS reads.  A half whose 64x128 block held no visible pair
//     has no tile: its waves skip the tile (its dS is zero).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 2) void bwd_dq_ds_kernel(BackwardArgs a) {
  constexpr int BM = 128, BN = 64;
  constexpr int MT = D / 32;
  constexpr int TCH = BN / 8;      // 16-byte chunks per d-major K' row
  constexpr int SCH = BM / 8;      // 16-byte chunks per dS^T row of the tile (two 64-query halves)
  __shared__ __attribute__((aligned(1024))) uint16_t s_lds[2][BN * BM];   // dS^T: [64 keys][128 queries]
  __shared__ __attribute__((aligned(1024))) uint16_t t_lds[2][D * BN];    // K' d-major: [D][64 keys]

  PrefillGeom geo{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, BM, BN};
  PrefillGeom g64{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, kDsQueries, kDsKeys};
  const int32_t n_qt = pf_num_qtiles(geo);
  // items ordered (batch, KV head, q-tile, head-in-group), each XCD a contiguous run
  const int64_t total = (int64_t)a.batch * a.hq * n_qt;
  const int64_t per = (total + 7) / 8;
  const int64_t lin = (int64_t)(blockIdx.x % 8) * per + blockIdx.x / 8;
  if (lin >= total) return;
  const int32_t hg = (int32_t)(lin % a.group);
  int64_t rest = lin / a.group;
  const int32_t qt = (int32_t)(rest % n_qt);
  rest /= n_qt;
  const int32_t kvh = (int32_t)(rest % a.hkv);
  const int32_t b = (int32_t)(rest / a.hkv);
  const int32_t hq = kvh * a.group + hg;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hf = lane >> 5;
  const int64_t bkv = (int64_t)b * a.hkv + kvh;
  const uint16_t* ktr = static_cast<const uint16_t*>(a.krt) + bkv * D * a.nkp;
  const uint16_t* dsb = static_cast<const uint16_t*>(a.ds);

  const TileRange tr = pf_tile_range(geo, qt);
  const int32_t n_cand = tr.n_prefix + (tr.band_hi >= tr.band_lo ? tr.band_hi - tr.band_lo + 1 : 0);
  auto cand_tile = [&](int32_t ci) { return ci < tr.n_prefix ? ci : tr.band_lo + (ci - tr.n_prefix); };
  // the kept tile of half qh (query block 2 qt + qh) for 64-key tile kt, or -1
  auto half_tile = [&](int32_t kt, int qh) -> int64_t {
    const int32_t qb = 2 * qt + qh;
    if (qb * kDsQueries >= a.num_q || pf_classify(g64, qb, kt >> 1) == 0) return -1;
    return ds_tile(a, b, hq, qb, ds_slot(g64, qb, kt >> 1)) + (int64_t)(kt & 1) * BN * kDsQueries;
  };

  // tile -> LDS buffer: wave load p of wave w fills chunks (4p + w) * 64 + lane;
  // the swizzle of a chunk's row depends on (w, lane) only
  const int srow = wave * (64 / SCH) + lane / SCH;                 // + 4p * 64 / SCH: key row
  const int schunk = (lane % SCH) ^ chunk_swizzle<SCH>(srow);      // logical chunk: half, 8 queries
  const int trow = wave * (64 / TCH) + lane / TCH;
  const int tchunk = (lane % TCH) ^ chunk_swizzle<TCH>(trow);
  auto load_tile = [&](int32_t kt, int b_, int64_t t0, int64_t t1) {
    // a missing half reads tile 0 of the region (in bounds; its waves skip it)
    const int64_t src = (schunk < SCH / 2 ? t0 : t1);
    const int64_t base = src >= 0 ? src : 0;
#pragma unroll
    for (int p = 0; p < BN * BM / 8 / 256; ++p)
      dma_to_lds(dsb + base + (int64_t)(srow + 4 * p * (64 / SCH)) * kDsQueries + (schunk % (SCH / 2)) * 8,
                 lds_address(s_lds[b_]) + wave * 1024 + p * 4096);
#pragma unroll
    for (int p = 0; p < D * BN / 8 / 256; ++p)
      dma_to_lds(ktr + (int64_t)(trow + 4 * p * (64 / TCH)) * a.nkp + (int64_t)kt * BN + tchunk * 8,
                 lds_address(t_lds[b_]) + wave * 1024 + p * 4096);
  };
  auto dm_at = [&](int r, int c) { return r * BN + ((c ^ chunk_swizzle<TCH>(r)) * 8); };

  f32x16 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;

  int32_t ci = 0;
  int64_t h0 = -1, h1 = -1;
  if (n_cand > 0) {
    h0 = half_tile(cand_tile(0), 0);
    h1 = half_tile(cand_tile(0), 1);
    load_tile(cand_tile(0), 0, h0, h1);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_only(0));
  __syncthreads();
  int buf = 0;
  const int qh = wave >> 1;   // this wave's half: queries 32 wave .. + 31 of the tile
  while (ci < n_cand) {
    const bool mine = (qh == 0 ? h0 : h1) >= 0;
    int64_t n0 = -1, n1 = -1;
    if (ci + 1 < n_cand) {
      n0 = half_tile(cand_tile(ci + 1), 0);
      n1 = half_tile(cand_tile(ci + 1), 1);
      load_tile(cand_tile(ci + 1), buf ^ 1, n0, n1);   // its buffer was read last step
    }
    if (mine) {
      // k-step j covers keys 16 j + 8 (e / 4) + 4 hf + e % 4: the d-major K' rows
      // (keys permuted per 16) and the gathered dS^T columns agree on that order
      const uint16_t* tt = t_lds[buf];
      const uint16_t* st = s_lds[buf];
      bf16x8 ta[MT], sbv = gather_cols<BM>(st, wave, 0, lane);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) ta[mt] = *reinterpret_cast<const bf16x8*>(&tt[dm_at(32 * mt + col, hf)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8 tn[MT], sn = sbv;
        if (j + 1 < 4) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            tn[mt] = *reinterpret_cast<const bf16x8*>(&tt[dm_at(32 * mt + col, 2 * (j + 1) + hf)]);
          sn = gather_cols<BM>(st, wave, j + 1, lane);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[mt], sbv, acc[mt], 0, 0, 0);
        if (j + 1 < 4) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) ta[mt] = tn[mt];
          sbv = sn;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(vmcnt_only(0));   // this wave's part of the next tiles has landed
    __syncthreads();
    buf ^= 1;
    h0 = n0;
    h1 = n1;
    ++ci;
  }

  // dQ' = scale * acc, rotated back by -position; column col of the accumulator
  // is tile column 32 wave + col, i.e. query vt_slot(32 wave + col) of the tile
  const int32_t t = qt * BM + vt_slot(32 * wave + col);
  if (t >= a.num_q) return;
  uint16_t* dqrow = static_cast<uint16_t*>(a.dq) + (((int64_t)b * a.num_q + t) * a.hq + hq) * D;
  const float* cs = a.cs_q + (int64_t)t * D;
#pragma unroll
  for (int mt = 0; mt < MT / 2; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * mt + 8 * r4 + 4 * hf;
      float g1[4], g2[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float c = cs[2 * (d + e)], sn = cs[2 * (d + e) + 1];
        const float x1 = acc[mt][4 * r4 + e] * a.scale, x2 = acc[mt + MT / 2][4 * r4 + e] * a.scale;
        g1[e] = x1 * c + x2 * sn;
        g2[e] = x2 * c - x1 * sn;
      }
      *reinterpret_cast<uint2*>(dqrow + d) = uint2{pack_bf16x2(g1[0], g1[1]), pack_bf16x2(g1[2], g1[3])};
      *reinterpret_cast<uint2*>(dqrow + d + D / 2) = uint2{pack_bf16x2(g2[0], g2[1]), pack_bf16x2(g2[2], g2[3])};
    }
}

// ---------------------------------------------------------------------------
// fp32 debug path: one thread per query row (dq) / key row (dk, dv)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void bwd_dq_f32_kernel(BackwardArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (int64_t)a.batch * a.hq * a.num_q) return;
  const int32_t t = (int32_t)(idx % a.num_q);
  const int32_t hq = (int32_t)((idx / a.num_q) % a.hq);
  const int32_t b = (int32_t)(idx / ((int64_t)a.num_q * a.hq));
  const int32_t kvh = hq / a.group;
  PrefillGeom geo{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, 64, 64};
  const int32_t u = a.num_k - a.num_q + t;
  const int64_t bh = (int64_t)b * a.hq + hq;
  const int64_t bkv = (int64_t)b * a.hkv + kvh;
  const float* qrow = static_cast<const float*>(a.qs) + (bh * a.tqp + t) * D;
  const float* drow = static_cast<const float*>(a.d_out) + (((int64_t)b * a.num_q + t) * a.hq + hq) * D;
  const float* kr = static_cast<const float*>(a.kr) + bkv * a.nkp * D;
  const float* vr = static_cast<const float*>(a.vr) + bkv * a.nkp * D;
  const float lse2 = a.lse2[bh * a.tqp + t], di = a.di[bh * a.tqp + t];
  float acc[D];
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  for (int32_t key = 0; key <= pf_min(u, a.num_k - 1); ++key) {
    if (!pf_visible(geo, u, key)) continue;
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < D; ++d) {
      s += qrow[d] * kr[(int64_t)key * D + d];
      dp += drow[d] * vr[(int64_t)key * D + d];
    }
    const float ds = __builtin_amdgcn_exp2f(s - lse2) * (dp - di);
    for (int d = 0; d < D; ++d) acc[d] += ds * kr[(int64_t)key * D + d];
  }
  float* dq = static_cast<float*>(a.dq) + (((int64_t)b * a.num_q + t) * a.hq + hq) * D;
  const float* cs = a.cs_q + (int64_t)t * D;
  for (int i = 0; i < D / 2; ++i) {
    const float c = cs[2 * i], sn = cs[2 * i + 1];
    const float x1 = acc[i] * a.scale, x2 = acc[i + D / 2] * a.scale;
    dq[i] = x1 * c + x2 * sn;
    dq[i + D / 2] = x2 * c - x1 * sn;
  }
}

template <int D>
__global__ __launch_bounds__(64) void bwd_dkdv_f32_kernel(BackwardArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 64 + threadIdx.x;
  if (idx >= (int64_t)a.batch * a.hkv * a.num_k) return;
  const int32_t key = (int32_t)(idx % a.num_k);
  const int32_t kvh = (int32_t)((idx / a.num_k) % a.hkv);
  const int32_t b = (int32_t)(idx / ((int64_t)a.num_k * a.hkv));
  PrefillGeom geo{a.num_q, a.num_k, a.prefix_len, a.window, a.kv_start, 64, 64};
  const int64_t bkv = (int64_t)b * a.hkv + kvh;
  const float* krow = static_cast<const float*>(a.kr) + (bkv * a.nkp + key) * D;
  const float* vrow = static_cast<const float*>(a.vr) + (bkv * a.nkp + key) * D;
  const int32_t off = a.num_k - a.num_q;
  float dk[D], dv[D];
  for (int d = 0; d < D; ++d) dk[d] = dv[d] = 0.f;
  for (int32_t g = 0; g < a.group; ++g) {
    const int32_t hq = kvh * a.group + g;
    const int64_t bh = (int64_t)b * a.hq + hq;
    for (int32_t t = pf_max(0, key - off); t < a.num_q; ++t) {
      if (!pf_visible(geo, off + t, key)) continue;
      const float* qrow = static_cast<const float*>(a.qs) + (bh * a.tqp + t) * D;
      const float* drow = static_cast<const float*>(a.d_out) + (((int64_t)b * a.num_q + t) * a.hq + hq) * D;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s += qrow[d] * krow[d];
        dp += drow[d] * vrow[d];
      }
      const float p = __builtin_amdgcn_exp2f(s - a.lse2[bh * a.tqp + t]);
      const float ds = p * (dp - a.di[bh * a.tqp + t]);
      for (int d = 0; d < D; ++d) {
        dk[d] += ds * qrow[d];
        dv[d] += p * drow[d];
      }
    }
  }
  float* dkr = static_cast<float*>(a.dk) + (((int64_t)b * a.num_k + key) * a.hkv + kvh) * D;
  float* dvr = static_cast<float*>(a.dv) + (((int64_t)b * a.num_k + key) * a.hkv + kvh) * D;
  const float* cs = a.cs_k + (int64_t)key * D;
  for (int i = 0; i < D / 2; ++i) {
    const float c = cs[2 * i], sn = cs[2 * i + 1];
    const float x1 = dk[i] * kLn2f, x2 = dk[i + D / 2] * kLn2f;
    dkr[i] = x1 * c + x2 * sn;
    dkr[i + D / 2] = x2 * c - x1 * sn;
  }
  for (int d = 0; d < D; ++d) dvr[d] = dv[d];
}

template <typename T, int D>
hipError_t launch_backward_t(const BackwardArgs& a, hipStream_t stream) {
  auto clamp = [](int64_t x) { return (uint32_t)(x < 1 ? 1 : (x > 16384 ? 16384 : x)); };
  hipLaunchKernelGGL((bwd_key_prep_kernel<T, D>), dim3(clamp((int64_t)a.batch * (a.nkp / 64))), dim3(256), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_query_cs_kernel<D>), dim3(clamp(((int64_t)a.num_q * (D / 2) + 255) / 256)), dim3(256), 0,
                     stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_query_prep_kernel<T, D>), dim3(clamp((int64_t)a.batch * a.hq * (a.tqp / 64))), dim3(256),
                     0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (sizeof(T) == 2) {
    const int64_t kv_items = (int64_t)a.batch * a.hkv * ((a.num_k + 127) / 128);
    const int64_t q_items = (int64_t)a.batch * a.hq * ((a.num_q + 127) / 128);
    const dim3 q_grid((uint32_t)(((q_items + 7) / 8) * 8));
    if (a.ds) {
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, true>), dim3((uint32_t)kv_items), dim3(256), 0, stream, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL((bwd_dq_ds_kernel<D>), q_grid, dim3(256), 0, stream, a);
    } else {
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, false>), dim3((uint32_t)kv_items), dim3(256), 0, stream, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
      hipLaunchKernelGGL((bwd_dq_kernel<D>), q_grid, dim3(256), 0, stream, a);
    }
  } else {
    const int64_t kv_rows = (int64_t)a.batch * a.hkv * a.num_k;
    hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D>), dim3((uint32_t)((kv_rows + 63) / 64)), dim3(64), 0, stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t q_rows = (int64_t)a.batch * a.hq * a.num_q;
    hipLaunchKernelGGL((bwd_dq_f32_kernel<D>), dim3((uint32_t)((q_rows + 63) / 64)), dim3(64), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
  if (a.batch == 0 || a.num_q == 0) return hipSuccess;
  if (a.dtype == PS_BF16)
    return a.head_dim == 64 ? launch_backward_t<uint16_t, 64>(a, stream) : launch_backward_t<uint16_t, 128>(a, stream);
  return a.head_dim == 64 ? launch_backward_t<float, 64>(a, stream) : launch_backward_t<float, 128>(a, stream);
}

}  // namespace ps
