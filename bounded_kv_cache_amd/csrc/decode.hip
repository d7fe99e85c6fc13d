// Split-KV decode attention over the bounded ring cache.
//
// Blog "Prefix Sliding 完全拆解" (pinghaoyang.com.cn): section
// "核心机制：注意力掩码上的两个区间" -- a query at position p sees the prefix and
// the last W tokens, so it reads min(p+1, L+W) keys whatever the trace length --
// and section "Kernel 实现：两层级过滤" (only prefix and window are read).  Since
// the ring's first min(p+1, L+W) slots hold exactly that set (keys stored
// pre-rotated), decode needs no element mask, only a length.
//
// Work item: (sequence, KV head, key split).  The G = Hq/Hkv query heads of the
// KV head are handled together so every K/V byte is read once per item.
//
// bf16 path (MFMA).  With G = 8 a key costs 8*D*2*2 flops per 4*D bytes, i.e.
// 8 flop/byte; fp32 VALU FMAs at the ~5.6 TB/s target would take ~57% of the
// non-packed vector peak before softmax, conversions and addressing.  The
// product is a genuine (skinny) contraction, so it goes to the matrix cores:
//   S^T[16 keys x 16 heads] = K[16 x 32] * Q^T[32 x 16]    (v_mfma_f32_16x16x32_bf16)
//   O^T[16 dims x 16 heads] += V^T[16 x 32 keys] * P^T[32 keys x 16 heads]
// Heads are padded to 16 (MFMA headroom is >10x).  Key rows of the two QK tiles
// of a 32-key chunk are permuted (row m of tile t is key 8*(m/4) + 4t + m%4) so
// that the S output registers of a lane ARE its P operand for the PV MFMA: lane
// (g = lane/16, n = lane%16) ends up holding keys 8g..8g+7 of head n, and no
// cross-lane shuffle is needed between the two products.  The V cache stores
// each run of 8 slots d-major, so the V^T operand (8 consecutive keys of one
// dim) is a single 16-byte load.  K operands are 16-byte loads of a key row.
// Everything goes HBM -> VGPR directly (no reuse to stage through LDS); chunks
// are double-buffered in registers.  The running max needs a 4-lane max per
// chunk; running sums stay lane-local until the end.
#include "ps_internal.h"

// Launch shape of the bf16 kernel: waves per workgroup and the minimum number
// of resident workgroups per CU the register allocation must allow.  A launch
// with no more workgroups than CUs (few sequences: 64 sequences x 2 KV heads x
// 2 splits fill 256 CUs once) runs eight waves per workgroup instead, one
// workgroup per CU, so each CU keeps as many loads in flight as two 4-wave
// workgroups would.
#ifndef PS_DECODE_WAVES
#define PS_DECODE_WAVES 4
#endif
#ifndef PS_DECODE_MIN_BLOCKS
#define PS_DECODE_MIN_BLOCKS 2
#endif
// 1: stream K/V with non-temporal loads (each byte is read exactly once)
#ifndef PS_DECODE_NT
#define PS_DECODE_NT 1
#endif

namespace ps {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

__device__ inline u32x4 stream_load(const uint16_t* p) {
#if PS_DECODE_NT
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
  return *reinterpret_cast<const u32x4*>(p);
#endif
}

// ---------------------------------------------------------------------------
// bf16 MFMA partial kernel
// ---------------------------------------------------------------------------
// kStats (heavy-hitter mode): 0 off; 1 per-slot statistics to HBM for the
// accumulate kernel; 2 statistics kept in LDS and the scores accumulated here
// (one workgroup per CU, the whole sequence in one split).
// kAppend: the step's token (k_new / v_new at pos) is appended by this kernel
// (one launch per decode step instead of an append launch and a decode launch).
template <int D, int NW, bool kReset, int kStats, bool kAppend = false>
__global__ __launch_bounds__(NW * 64, NW == 8 ? 1 : PS_DECODE_MIN_BLOCKS) void decode_bf16_kernel(
    DecodeArgs a) {
  constexpr int NC = D / 32;   // QK k-steps (32 dims each)
  constexpr int NDT = D / 16;  // PV d-tiles (16 dims each)
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;   // MFMA row/column index
  const int g = lane >> 4;   // MFMA lane group (k-slot group)

  int bid = blockIdx.x;
  const int split = bid % a.num_splits;
  bid /= a.num_splits;
  const int h = bid % a.geom.hkv;
  const int s = bid / a.geom.hkv;
  const CacheGeom& geo = a.geom;

  const int32_t L = a.prefix_len[s];
  const int64_t pos = a.pos[s];
  // visible keys = ring slots [0, min(p+1, L+W)) (+ the occupied heavy slots
  // right after the window); every one must exist
  int64_t nvis64 = pos + 1 < (int64_t)L + geo.window ? pos + 1 : (int64_t)L + geo.window;
  bool bad = L < 0 || pos < 0;
  if (kStats) {
    const int32_t hc = a.heavy_count[(int64_t)s * geo.hkv + h];
    nvis64 += hc;
    bad = bad || hc < 0 || hc > a.heavy_slots || (int64_t)L + geo.window + a.heavy_slots > geo.slot_capacity;
  }
  bad = bad || nvis64 > geo.slot_capacity;
  const int nvis = bad ? 0 : (int)nvis64;
  const int kb = split * a.split_keys;
  const int ke = kb + a.split_keys < nvis ? kb + a.split_keys : nvis;
  bf16x8 qop[NC];   // query operand, filled after the first chunk's loads are issued
  // Reset PE: prefix slots [0, L) are scored with the query rotated at its
  // renumbered position min(p, L+W-1); window keys keep their offsets to the
  // query (the whole window shifts by one amount), so they use qop
  bf16x8 qop_b[kReset ? NC : 1];

  // ---- per-lane load offsets inside a 32-key chunk (elements) ----
  // K tile t, row r -> key 8*(r/4) + 4t + r%4; k-step c covers dims 32c + 8g .. +8
  int koff[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) koff[t] = (8 * (r >> 2) + 4 * t + (r & 3)) * D + 8 * g;
  // V block g (keys 8g..8g+7), d-tile dt, dim 16*dt + r: 8 contiguous bf16
  const int voff = g * 8 * D + r * 8;

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
  const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
  // heavy-hitter statistics of this (sequence, KV head), chunk-major so that a
  // chunk's rows land as whole cache lines: [chunk][head of the group][32 keys]
  // fp16 s - m, and [chunk][head] fp32 m, the running max after that chunk
  const int nch = geo.slot_capacity / 32;
  const __amdgpu_buffer_rsrc_t stat_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      kStats == 1 ? static_cast<uint16_t*>(a.stat_scores) + ((int64_t)s * geo.hkv + h) * a.group * geo.slot_capacity
             : nullptr,
      (short)0, kStats == 1 ? a.group * geo.slot_capacity * 2 : 0, 0x00020000);
  const __amdgpu_buffer_rsrc_t max_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      kStats == 1 ? a.stat_max + ((int64_t)s * geo.hkv + h) * a.group * nch : nullptr, (short)0,
      kStats == 1 ? a.group * nch * 4 : 0, 0x00020000);
  // kStats 2: the same two arrays in LDS (the wave merge reuses the space later)
  __shared__ __attribute__((aligned(16)))
  uint8_t fused_lds[kStats == 2 ? (NW == kFusedStatsWaves ? kFusedStatsLds : kFusedStatsLdsSmall) : 16];
  uint16_t* const lds_x = reinterpret_cast<uint16_t*>(fused_lds);
  float* const lds_m = reinterpret_cast<float*>(fused_lds + nch * a.group * 64);

  // chunk index list of this wave: first chunk kb/32 + wave, stride NW
  const int c_end = (ke + 31) >> 5;   // chunks touching [kb, ke)
  int c = (kb >> 5) + wave;

  u32x4 kA[2][NC], vA[NDT], kB[2][NC], vB[NDT];

  // Paged cache: the page ids of this split's first 128 segments are fetched
  // once (one coalesced load per 64 pages) and picked per chunk with a lane
  // read, so a chunk's K/V loads never wait on a block-table load.
  const int seg0 = kb >> 6;
  int32_t page_cache[2] = {-1, -1};
  if (geo.paged) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int seg = seg0 + 64 * j + lane;
      if (seg < geo.max_pages) page_cache[j] = a.block_table[(int64_t)s * geo.max_pages + seg];
    }
  }
  auto chunk_base = [&](int key0) -> int64_t {
    if (!geo.paged) return region_offset(geo, a.block_table, s, h, key0);
    const int rel = (key0 >> 6) - seg0;
    int32_t page;
    if (rel < 64)
      page = __builtin_amdgcn_readlane(page_cache[0], rel);
    else if (rel < 128)
      page = __builtin_amdgcn_readlane(page_cache[1], rel - 64);
    else
      page = a.block_table[(int64_t)s * geo.max_pages + (key0 >> 6)];
    if (page < 0 || (int64_t)page >= geo.num_pages) return -1;
    return ((int64_t)page * geo.hkv + h) * (int64_t)(kRegionSlots * D);
  };

  auto load_chunk = [&](int ci, u32x4 (&kr)[2][NC], u32x4 (&vr)[NDT]) {
    const int key0 = ci << 5;
    const int64_t base = chunk_base(key0);
    if (base < 0) {
      bad = true;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) kr[t][cc] = u32x4{0, 0, 0, 0};
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vr[dt] = u32x4{0, 0, 0, 0};
      return;
    }
    const int in_reg = (key0 & 63) * D;
    const uint16_t* kp = kc + base + in_reg;
    const uint16_t* vp = vc + base + in_reg;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int cc = 0; cc < NC; ++cc) kr[t][cc] = stream_load(kp + koff[t] + 32 * cc);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vr[dt] = stream_load(vp + voff + dt * 16 * 8);
  };

  auto qk = [&](const bf16x8* qo, u32x4 (&kr)[2][NC], f32x4& st0, f32x4& st1) {
    st0 = f32x4{0.f, 0.f, 0.f, 0.f};
    st1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cc = 0; cc < NC; ++cc) {
      st0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[0][cc]), qo[cc], st0, 0, 0, 0);
      st1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[1][cc]), qo[cc], st1, 0, 0, 0);
    }
  };

  // kStats 2: this thread's first 8 scores, loaded now so that the update at
  // the end does not wait a memory round trip
  float4 sc_pre0 = make_float4(0.f, 0.f, 0.f, 0.f), sc_pre1 = sc_pre0;
  const int j_first = (L & ~7) + 8 * (int)threadIdx.x;
  if (kStats == 2 && !bad && j_first < nvis) {
    const float4* sp = reinterpret_cast<const float4*>(a.heavy_score +
                                                       ((int64_t)s * geo.hkv + h) * geo.slot_capacity + j_first);
    sc_pre0 = sp[0];
    sc_pre1 = sp[1];
  }
  // statistics of the last computed chunk, awaiting their store
  u32x4 st_x = {0u, 0u, 0u, 0u};
  float st_m = 0.f;
  int st_ci = -1;
  auto store_stats = [&]() {
    // every lane issues the same two stores (no branch, so the load pipeline's
    // wait counts stay exact); lanes of padding heads, for the max all but lane
    // group 0, and everything before the first chunk aim past the buffer range
    // and the hardware drops them.  Chunks never cross a split boundary, so the
    // -inf of a final partial chunk only lands in slots past the visible range.
    const bool live = st_ci >= 0 && r < a.group;
    const int xoff = (live ? (st_ci * a.group + r) * 32 + 8 * g : a.group * geo.slot_capacity) * 2;
    __builtin_amdgcn_raw_buffer_store_b128(st_x, stat_rsrc, xoff, 0, 0);
    const int moff = (live && g == 0 ? st_ci * a.group + r : a.group * nch) * 4;
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, st_m), max_rsrc, moff, 0, 0);
  };

  auto compute_chunk = [&](int ci, u32x4 (&kr)[2][NC], u32x4 (&vr)[NDT]) {
    f32x4 st0, st1;
    const int key0 = (ci << 5) + 8 * g;
    if (kReset && (ci << 5) < L) {
      qk(qop_b, kr, st0, st1);
      if (((ci + 1) << 5) > L) {   // the chunk holding the end of the prefix: window keys from qop
        f32x4 w0, w1;
        qk(qop, kr, w0, w1);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (key0 + i >= L) st0[i] = w0[i];
          if (key0 + 4 + i >= L) st1[i] = w1[i];
        }
      }
    } else {
      qk(qop, kr, st0, st1);
    }
    // lane holds head r, keys 8g + i (i<4 from tile 0, i>=4 from tile 1)
    float sv[8] = {st0[0], st0[1], st0[2], st0[3], st1[0], st1[1], st1[2], st1[3]};
    const bool tail = ((ci + 1) << 5) > ke || (ci << 5) < kb;
    if (tail) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int key = key0 + i;
        if (key >= ke || key < kb) sv[i] = -INFINITY;
      }
      // masked keys must contribute exactly zero: clear their V elements too
      // (slots past the visible length may hold anything, including NaN bits)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k0 = key0 + 2 * e;
          if (k0 >= ke || k0 < kb) vr[dt][e] &= 0xffff0000u;
          if (k0 + 1 >= ke || k0 + 1 < kb) vr[dt][e] &= 0x0000ffffu;
        }
      }
    }
    float mx = sv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, sv[i]);
    mx = max_xor16(mx);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float pv[8], xv[8];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      xv[i] = sv[i] - m_new;
      pv[i] = __builtin_amdgcn_exp2f(xv[i]);
      psum += pv[i];
    }
    if (kStats == 2) {
      if (r < a.group) {
        u32x4 xw;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xw[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(xv[2 * i], xv[2 * i + 1]));
        *reinterpret_cast<u32x4*>(lds_x + (ci * a.group + r) * 32 + 8 * g) = xw;
        if (g == 0) lds_m[ci * a.group + r] = m_new;
      }
    }
    if (kStats == 1) {
      // heavy-hitter statistics, stored with the next chunk's loads (a store
      // issued amid the math would hold the wave until the memory pipeline
      // takes it).  fp16 keeps s - m to 2^-11 near 0, where the mass is.
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st_x[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(xv[2 * i], xv[2 * i + 1]));
      st_m = m_new;
      st_ci = ci;
    }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) acc[dt] *= alpha;
    }
    bf16x8 pop;
#pragma unroll
    for (int i = 0; i < 8; ++i) pop[i] = (bf16)pv[i];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vr[dt]), pop, acc[dt], 0, 0, 0);
  };

  if (c < c_end) load_chunk(c, kA, vA);   // the first chunk is in flight during the query prologue
  // ---- query operand: rotate at pos, fold in scale*log2(e), round to bf16 ----
  // cos/sin of the query position: each lane forms one rotation pair (pair
  // lane % (D/2): the angle needs double precision, and the lanes of the
  // other query heads would form the same values), and every lane fetches the
  // pairs it rotates from the lane that formed them.
  float cs_l = 1.f, sn_l = 0.f, csb_l = 1.f, snb_l = 0.f;
  if (a.rope.enabled) {
    rope_cos_sin(pos, a.rope.inv_freq[lane % (D / 2)], cs_l, sn_l);
    if (kReset) {
      const int64_t lw1 = (int64_t)L + geo.window - 1;
      rope_cos_sin(pos < lw1 ? pos : lw1, a.rope.inv_freq[lane % (D / 2)], csb_l, snb_l);
    }
  }
  {
    const int G = a.group;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + ((int64_t)s * a.hq + h * G + (r < G ? r : 0)) * D;
    float qv[NC][8];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const uint4 w = *reinterpret_cast<const uint4*>(qrow + 32 * c + 8 * g);
      const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qv[c][2 * e] = (r < G) ? lo_bf16(ww[e]) : 0.f;
        qv[c][2 * e + 1] = (r < G) ? hi_bf16(ww[e]) : 0.f;
      }
    }
    if (kReset) {   // the query at its renumbered position min(p, L + W - 1), for prefix slots
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float cs = __shfl(csb_l, 32 * c + 8 * g + i), sn = __shfl(snb_l, 32 * c + 8 * g + i);
          const float x1 = qv[c][i], x2 = qv[c + NC / 2][i];
          qop_b[c][i] = (bf16)((x1 * cs - x2 * sn) * a.scale_log2);
          qop_b[c + NC / 2][i] = (bf16)((x2 * cs + x1 * sn) * a.scale_log2);
        }
      }
    }
    if (a.rope.enabled) {
#pragma unroll
      for (int c = 0; c < NC / 2; ++c) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float cs = __shfl(cs_l, 32 * c + 8 * g + i), sn = __shfl(sn_l, 32 * c + 8 * g + i);
          const float x1 = qv[c][i], x2 = qv[c + NC / 2][i];
          qv[c][i] = x1 * cs - x2 * sn;
          qv[c + NC / 2][i] = x2 * cs + x1 * sn;
        }
      }
    }
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 8; ++i) qop[c][i] = (bf16)(qv[c][i] * a.scale_log2);
  }

  // ---- kAppend: the token at pos goes to its ring slot (the append rule:
  // dropped for an invalid sequence or a slot beyond the capacity), written by
  // the wave that will read that slot's chunk, while its first chunk's loads
  // are in flight.  The wave loads that chunk only after the stores have
  // completed: if it is the first chunk (already loaded) the stores are waited
  // for and the chunk is loaded again; if it is the second (loaded at the top
  // of the loop) the stores are waited for first; any later chunk is loaded
  // after the wait for the first chunk's data, and the vector memory counter
  // retires a wave's loads and stores in issue order, so that wait has also
  // seen the stores (issued between the first chunk's loads and the second's)
  // complete.  The key is rotated with the append kernel's expression. ----
  if (kAppend && L >= 0 && pos >= 0) {
    const int32_t sn = ring_slot(pos, L, geo.window);
    const int ci_new = sn >> 5;
    if (sn < geo.slot_capacity && sn / a.split_keys == split && ci_new >= c && (ci_new - c) % NW == 0) {
      const int64_t base = region_offset(geo, a.block_table, s, h, sn);
      if (base >= 0) {
        const uint16_t* kn = static_cast<const uint16_t*>(a.k_new) + ((int64_t)s * geo.hkv + h) * D;
        const uint16_t* vn = static_cast<const uint16_t*>(a.v_new) + ((int64_t)s * geo.hkv + h) * D;
        uint16_t* kw = const_cast<uint16_t*>(kc) + base;
        uint16_t* vw = const_cast<uint16_t*>(vc) + base;
        if (lane < D / 2) {   // rotate-half pair (lane, lane + D/2) at pos: this lane's cos/sin, as the append kernel
          const int i = lane;
          const float x1 = bf16_to_f32(kn[i]), x2 = bf16_to_f32(kn[i + D / 2]);
          float y1, y2;
          rotate_pair(x1, x2, cs_l, sn_l, y1, y2);
          kw[k_in_region(sn, i, D)] = f32_to_bf16_bits(y1);
          kw[k_in_region(sn, i + D / 2, D)] = f32_to_bf16_bits(y2);
          vw[v_in_region(sn, i, D)] = vn[i];
          vw[v_in_region(sn, i + D / 2, D)] = vn[i + D / 2];
        }
        if (ci_new - c < 2 * NW) {
          __builtin_amdgcn_s_waitcnt(0);   // the stores (and the first chunk's loads) are complete
          if (ci_new == c) load_chunk(c, kA, vA);
        }
      }
    }
  }

  while (c < c_end) {
    if (kStats == 1) store_stats();
    if (c + NW < c_end) load_chunk(c + NW, kB, vB);
    compute_chunk(c, kA, vA);
    c += NW;
    if (c >= c_end) break;
    if (kStats == 1) store_stats();
    if (c + NW < c_end) load_chunk(c + NW, kA, vA);
    compute_chunk(c, kB, vB);
    c += NW;
  }
  if (kStats == 1) store_stats();

  // ---- finish the wave: sum the lane-local partial sums of each head ----
  l_run = sum_xor16(l_run);
  l_run = sum_xor32(l_run);

  // ---- merge the NW waves through LDS ----
  __shared__ float sm_o_own[kStats == 2 ? 1 : NW][D][17];
  float (*const sm_o)[D][17] = kStats == 2 ? reinterpret_cast<float (*)[D][17]>(fused_lds) : sm_o_own;
  __shared__ float sm_m[NW][16];
  __shared__ float sm_l[NW][16];
  __shared__ int sm_bad;
  if (threadIdx.x == 0) sm_bad = 0;
  __syncthreads();
  if (kStats != 2) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[wave][16 * dt + 4 * g + i][r] = acc[dt][i];
  }
  if (g == 0) {
    sm_m[wave][r] = m_run;
    sm_l[wave][r] = l_run;
  }
  if (bad) sm_bad = 1;
  __syncthreads();

  const int G = a.group;
  const bool any_bad = sm_bad != 0;
  if (kStats == 2) {
    // each row's log2-sum-exp2, then score[j] += sum over the group's heads of
    // exp2(s_j - lse2) for the visible non-prefix slots, 8 per thread (the
    // capacity is a multiple of 64, so a group never crosses a chunk)
    __shared__ float sm_lse2[16];
    if (threadIdx.x < G) {
      const int n = threadIdx.x;
      float M = -INFINITY;
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][n]);
      float l = 0.f;
      if (M != -INFINITY)
        for (int w = 0; w < NW; ++w) l += __builtin_amdgcn_exp2f(sm_m[w][n] - M) * sm_l[w][n];
      sm_lse2[n] = M + __log2f(l);
    }
    __syncthreads();
    float* score = a.heavy_score + ((int64_t)s * geo.hkv + h) * geo.slot_capacity;
    if (!any_bad) {
      for (int j0 = (L & ~7) + 8 * (int)threadIdx.x; j0 < nvis; j0 += 8 * NW * 64) {
        const int cj = j0 >> 5;
        float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int n = 0; n < G; ++n) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(lds_x + (cj * G + n) * 32 + (j0 & 31));
          const float off = lds_m[cj * G + n] - sm_lse2[n];
          // (the element goes through a named scalar: a bit cast straight from a
          // vector element read element 0 every time)
          const uint32_t ww[4] = {w[0], w[1], w[2], w[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const auto x = __builtin_bit_cast(_Float16 __attribute__((ext_vector_type(2))), ww[e]);
            m[2 * e] += __builtin_amdgcn_exp2f((float)x[0] + off);
            m[2 * e + 1] += __builtin_amdgcn_exp2f((float)x[1] + off);
          }
        }
        float4* sp = reinterpret_cast<float4*>(score + j0);
        const bool first = j0 == j_first;
        const float4 s0 = first ? sc_pre0 : sp[0], s1 = first ? sc_pre1 : sp[1];
        float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (j0 + i >= L && j0 + i < nvis) sv[i] += m[i];
        sp[0] = make_float4(sv[0], sv[1], sv[2], sv[3]);
        sp[1] = make_float4(sv[4], sv[5], sv[6], sv[7]);
      }
    }
    __syncthreads();   // the statistics are consumed: their space takes the wave merge
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[wave][16 * dt + 4 * g + i][r] = acc[dt][i];
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int n = idx / D;
    const int d = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][n]);
    float o = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm_m[w][n] - M);
        o += f * sm_o[w][d][n];
        l += f * sm_l[w][n];
      }
    }
    const int64_t row = (int64_t)s * a.hq + h * G + n;
    if (a.num_splits == 1) {
      const float val = any_bad ? __builtin_nanf("") : o / l;
      static_cast<uint16_t*>(a.out)[row * D + d] = f32_to_bf16_bits(val);
      if (kStats == 1 && d == 0) a.stat_lse2[row] = any_bad ? __builtin_nanf("") : M + __log2f(l);
    } else {
      const int64_t prow = row * a.num_splits + split;
      a.part_o[prow * D + d] = any_bad ? __builtin_nanf("") : o;
      if (d == 0) {
        a.part_ml[prow * 2 + 0] = any_bad ? __builtin_nanf("") : M;
        a.part_ml[prow * 2 + 1] = any_bad ? __builtin_nanf("") : l;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 debug partial kernel (plain VALU, LDS-tiled; correctness path)
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeArgs a) {
  constexpr int TK = 32;  // keys per tile
  __shared__ float qs[kMaxGroup][D];
  __shared__ float qs_b[kMaxGroup][D];   // Reset PE: the query for prefix slots
  __shared__ float ks[TK][D + 1];
  __shared__ float vs[TK][D + 1];
  __shared__ float ps_[kMaxGroup][TK];
  __shared__ float m_s[kMaxGroup], l_s[kMaxGroup], alpha_s[kMaxGroup];
  __shared__ int bad_s;

  int bid = blockIdx.x;
  const int split = bid % a.num_splits;
  bid /= a.num_splits;
  const int h = bid % a.geom.hkv;
  const int s = bid / a.geom.hkv;
  const CacheGeom& geo = a.geom;
  const int G = a.group;
  const int tid = threadIdx.x;

  const int32_t L = a.prefix_len[s];
  const int64_t pos = a.pos[s];
  int64_t nvis64 = pos + 1 < (int64_t)L + geo.window ? pos + 1 : (int64_t)L + geo.window;
  bool seq_bad = L < 0 || pos < 0;
  if (a.heavy_count) {
    const int32_t hc = a.heavy_count[(int64_t)s * geo.hkv + h];
    nvis64 += hc;
    seq_bad = seq_bad || hc < 0 || hc > a.heavy_slots ||
              (int64_t)L + geo.window + a.heavy_slots > geo.slot_capacity;
  }
  seq_bad = seq_bad || nvis64 > geo.slot_capacity;
  const int nvis = seq_bad ? 0 : (int)nvis64;
  const int kb = split * a.split_keys;
  const int ke = kb + a.split_keys < nvis ? kb + a.split_keys : nvis;

  const float* q = static_cast<const float*>(a.q);
  for (int idx = tid; idx < G * (D / 2); idx += 256) {
    const int n = idx / (D / 2), i = idx % (D / 2);
    const float* qr = q + ((int64_t)s * a.hq + h * G + n) * D;
    const float r1 = qr[i], r2 = qr[i + D / 2];
    float x1 = r1, x2 = r2;
    if (a.rope.enabled) {
      float c, sn;
      rope_cos_sin(pos, a.rope.inv_freq[i], c, sn);
      x1 = r1 * c - r2 * sn;
      x2 = r2 * c + r1 * sn;
    }
    qs[n][i] = x1 * a.scale_log2;
    qs[n][i + D / 2] = x2 * a.scale_log2;
    if (a.reset_pe) {
      const int64_t lw1 = (int64_t)L + geo.window - 1;
      float c = 1.f, sn = 0.f;
      if (a.rope.enabled) rope_cos_sin(pos < lw1 ? pos : lw1, a.rope.inv_freq[i], c, sn);
      qs_b[n][i] = (r1 * c - r2 * sn) * a.scale_log2;
      qs_b[n][i + D / 2] = (r2 * c + r1 * sn) * a.scale_log2;
    }
  }
  if (tid < kMaxGroup) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  if (tid == 0) bad_s = seq_bad ? 1 : 0;
  constexpr int NOUT = (kMaxGroup * D + 255) / 256;
  float acc[NOUT];
#pragma unroll
  for (int k = 0; k < NOUT; ++k) acc[k] = 0.f;
  const float* kc = static_cast<const float*>(a.k_cache);
  const float* vc = static_cast<const float*>(a.v_cache);
  __syncthreads();

  for (int t0 = kb; t0 < ke; t0 += TK) {
    const int64_t base = region_offset(geo, a.block_table, s, h, t0);
    if (base < 0) {
      if (tid == 0) bad_s = 1;
      break;
    }
    // tiles start at multiples of 32, so a tile never crosses a 64-slot region
    for (int idx = tid; idx < TK * D; idx += 256) {
      const int j = idx / D, d = idx % D;
      const int key = t0 + j;
      const bool ok = key < ke;
      ks[j][d] = ok ? kc[base + k_in_region(key, d, D)] : 0.f;
      vs[j][d] = ok ? vc[base + v_in_region(key, d, D)] : 0.f;
    }
    __syncthreads();
    for (int idx = tid; idx < G * TK; idx += 256) {
      const int n = idx / TK, j = idx % TK;
      const float* qv = (a.reset_pe && t0 + j < L) ? qs_b[n] : qs[n];
      float sc = 0.f;
      for (int d = 0; d < D; ++d) sc += qv[d] * ks[j][d];
      ps_[n][j] = (t0 + j < ke) ? sc : -INFINITY;
      if (a.stat_scores && t0 + j < ke)
        static_cast<float*>(a.stat_scores)[(((int64_t)s * geo.hkv + h) * G + n) * geo.slot_capacity + t0 + j] = sc;
    }
    __syncthreads();
    if (tid < G) {
      float mx = -INFINITY;
      for (int j = 0; j < TK; ++j) mx = fmaxf(mx, ps_[tid][j]);
      const float mn = fmaxf(m_s[tid], mx);
      const float al = __builtin_amdgcn_exp2f(m_s[tid] - mn);
      float sum = 0.f;
      for (int j = 0; j < TK; ++j) {
        const float e = __builtin_amdgcn_exp2f(ps_[tid][j] - mn);
        ps_[tid][j] = e;
        sum += e;
      }
      l_s[tid] = l_s[tid] * al + sum;
      m_s[tid] = mn;
      alpha_s[tid] = al;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NOUT; ++k) {
      const int idx = tid + 256 * k;
      if (idx < G * D) {
        const int n = idx / D, d = idx % D;
        float o = acc[k] * alpha_s[n];
        for (int j = 0; j < TK; ++j) o += ps_[n][j] * vs[j][d];
        acc[k] = o;
      }
    }
    __syncthreads();
  }
  __syncthreads();
  const bool any_bad = bad_s != 0;
#pragma unroll
  for (int k = 0; k < NOUT; ++k) {
    const int idx = tid + 256 * k;
    if (idx >= G * D) continue;
    const int n = idx / D, d = idx % D;
    const int64_t row = (int64_t)s * a.hq + h * G + n;
    if (a.num_splits == 1) {
      static_cast<float*>(a.out)[row * D + d] = any_bad ? __builtin_nanf("") : acc[k] / l_s[n];
      if (a.stat_lse2 && d == 0) a.stat_lse2[row] = any_bad ? __builtin_nanf("") : m_s[n] + __log2f(l_s[n]);
    } else {
      const int64_t prow = row * a.num_splits + split;
      a.part_o[prow * D + d] = any_bad ? __builtin_nanf("") : acc[k];
      if (d == 0) {
        a.part_ml[prow * 2 + 0] = any_bad ? __builtin_nanf("") : m_s[n];
        a.part_ml[prow * 2 + 1] = any_bad ? __builtin_nanf("") : l_s[n];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// combine: merge the split partials of each (sequence, query head) in split order
// ---------------------------------------------------------------------------
template <typename OutT, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
  const int64_t row = blockIdx.x;  // s * hq + head
  const int d = threadIdx.x;
  const int S = a.num_splits;
  const float* ml = a.part_ml + row * S * 2;
  float M = -INFINITY;
  bool nan = false;
  for (int i = 0; i < S; ++i) {
    const float m = ml[2 * i];
    nan |= (m != m);
    M = fmaxf(M, m);
  }
  float o = 0.f, l = 0.f;
  for (int i = 0; i < S; ++i) {
    const float m = ml[2 * i];
    if (m == -INFINITY) continue;  // empty split
    const float f = __builtin_amdgcn_exp2f(m - M);
    o += f * a.part_o[(row * S + i) * D + d];
    l += f * ml[2 * i + 1];
  }
  const float val = nan ? __builtin_nanf("") : o / l;
  Elem<OutT>::store(static_cast<OutT*>(a.out) + row * D + d, val);
  if (a.stat_lse2 && d == 0) a.stat_lse2[row] = nan ? __builtin_nanf("") : M + __log2f(l);
}

template <int D>
hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t stream) {
  const dim3 grid((uint32_t)((int64_t)a.num_seqs * a.geom.hkv * a.num_splits));
  if (a.dtype == PS_BF16) {
    constexpr int NW = PS_DECODE_WAVES;
    if (a.heavy_score && fused_stats_bytes(a.geom.slot_capacity, a.group) <= (size_t)kFusedStatsLdsSmall)
      hipLaunchKernelGGL((decode_bf16_kernel<D, NW, false, 2>), grid, dim3(NW * 64), 0, stream, a);
    else if (a.heavy_score)
      hipLaunchKernelGGL((decode_bf16_kernel<D, kFusedStatsWaves, false, 2>), grid, dim3(kFusedStatsWaves * 64), 0,
                         stream, a);
    else if (a.k_new && a.wide)
      hipLaunchKernelGGL((decode_bf16_kernel<D, 8, false, 0, true>), grid, dim3(8 * 64), 0, stream, a);
    else if (a.k_new)
      hipLaunchKernelGGL((decode_bf16_kernel<D, NW, false, 0, true>), grid, dim3(NW * 64), 0, stream, a);
    else if (a.heavy_count)
      hipLaunchKernelGGL((decode_bf16_kernel<D, NW, false, 1>), grid, dim3(NW * 64), 0, stream, a);
    else if (a.reset_pe)
      hipLaunchKernelGGL((decode_bf16_kernel<D, NW, true, 0>), grid, dim3(NW * 64), 0, stream, a);
    else if (a.wide)
      hipLaunchKernelGGL((decode_bf16_kernel<D, 8, false, 0>), grid, dim3(8 * 64), 0, stream, a);
    else
      hipLaunchKernelGGL((decode_bf16_kernel<D, NW, false, 0>), grid, dim3(NW * 64), 0, stream, a);
  } else {
    hipLaunchKernelGGL((decode_f32_kernel<D>), grid, dim3(256), 0, stream, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1) return e;
  const dim3 cgrid((uint32_t)((int64_t)a.num_seqs * a.hq));
  if (a.dtype == PS_BF16)
    hipLaunchKernelGGL((decode_combine_kernel<uint16_t, D>), cgrid, dim3(D), 0, stream, a);
  else
    hipLaunchKernelGGL((decode_combine_kernel<float, D>), cgrid, dim3(D), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.num_seqs == 0) return hipSuccess;
  return a.geom.head_dim == 64 ? launch_decode_d<64>(a, stream) : launch_decode_d<128>(a, stream);
}

}  // namespace ps
