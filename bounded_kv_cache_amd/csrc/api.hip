// C-ABI entry points: host-side validation, workspace sizing and launches.
// Every check the host can make happens before anything is enqueued.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <initializer_list>
#include <mutex>
#include <string>
#include <utility>

#include "ps_internal.h"
#include "ps_reset.h"
#include "ps_sched.h"

namespace {

thread_local std::string g_last_error;

// the bf16 attention kernel addresses eight V^T rows of one load with 32-bit
// byte offsets: 7 * padded keys * 2 bytes must stay below 2^32
constexpr size_t kMaxBf16PrefillKeys = (size_t)1 << 28;

ps_status fail(ps_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ps_status fail(ps_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

ps_status ok() {
  g_last_error.clear();
  return PS_OK;
}

// Element tensors are read and written with 16-byte vector accesses: every
// such pointer must be 16-byte aligned (a contiguous view at an odd storage
// offset is rejected here instead of being accessed misaligned).
ps_status check_aligned(std::initializer_list<std::pair<const void*, const char*>> ptrs, size_t align = 16) {
  for (const auto& p : ptrs)
    if (p.first && reinterpret_cast<uintptr_t>(p.first) % align != 0)
      return fail(PS_INVALID_ARGUMENT, "%s is not %zu-byte aligned", p.second, align);
  return PS_OK;
}

ps_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PS_HIP_ERROR, "%s: %s", what, hipGetErrorString(e));
}

ps_status check_attn(const ps_attn_desc* a) {
  if (!a) return fail(PS_INVALID_ARGUMENT, "attention descriptor is NULL");
  if (a->num_q_heads <= 0 || a->num_kv_heads <= 0)
    return fail(PS_INVALID_ARGUMENT, "head counts must be positive (Hq=%d, Hkv=%d)", a->num_q_heads, a->num_kv_heads);
  if (a->num_q_heads % a->num_kv_heads != 0)
    return fail(PS_INVALID_ARGUMENT, "Hq=%d is not a multiple of Hkv=%d", a->num_q_heads, a->num_kv_heads);
  if (a->num_q_heads / a->num_kv_heads > ps::kMaxGroup)
    return fail(PS_UNSUPPORTED, "query heads per KV head %d exceeds %d", a->num_q_heads / a->num_kv_heads,
                ps::kMaxGroup);
  if (a->head_dim != 64 && a->head_dim != 128) return fail(PS_UNSUPPORTED, "head_dim %d (64 or 128)", a->head_dim);
  if (a->dtype != PS_BF16 && a->dtype != PS_F32) return fail(PS_UNSUPPORTED, "dtype %d", a->dtype);
  if (!(a->softmax_scale > 0.f) || !isfinite(a->softmax_scale))
    return fail(PS_INVALID_ARGUMENT, "softmax_scale must be positive and finite");
  if (!(a->rope_theta >= 0.0) || !isfinite(a->rope_theta))
    return fail(PS_INVALID_ARGUMENT, "rope_theta must be >= 0 and finite");
  if (a->rope_theta > 0.0 && a->rope_theta <= 1.0) return fail(PS_INVALID_ARGUMENT, "rope_theta must exceed 1");
  if (a->pe_mode != PS_PE_CONTINUE && a->pe_mode != PS_PE_RESET && a->pe_mode != PS_PE_RESET_RECOMPUTE)
    return fail(PS_INVALID_ARGUMENT, "pe_mode %d (0 Continue PE, 1 Reset PE, 2 Reset PE re-rotating keys)",
                a->pe_mode);
  return PS_OK;
}

// Reset PE is a decode-only scoring mode.
ps_status continue_pe_only(const ps_attn_desc* a, const char* entry) {
  if (a->pe_mode != PS_PE_CONTINUE) return fail(PS_UNSUPPORTED, "%s supports Continue PE only (pe_mode 0)", entry);
  return PS_OK;
}

ps_status check_cache(const ps_cache_desc* c, const int32_t* block_table) {
  if (!c) return fail(PS_INVALID_ARGUMENT, "cache descriptor is NULL");
  if (c->window < 1) return fail(PS_INVALID_ARGUMENT, "window W=%d must be >= 1", c->window);
  if (c->page_size != 0 && c->page_size != 64)
    return fail(PS_UNSUPPORTED, "page_size %d (0 = contiguous or 64)", c->page_size);
  if (c->slot_capacity <= 0 || c->slot_capacity % 64 != 0)
    return fail(PS_INVALID_ARGUMENT, "slot_capacity %d must be a positive multiple of 64", c->slot_capacity);
  if (c->page_size == 64) {
    if (!block_table) return fail(PS_INVALID_ARGUMENT, "paged cache needs a block table");
    if (c->max_pages_per_seq * 64 != c->slot_capacity)
      return fail(PS_INVALID_ARGUMENT, "max_pages_per_seq*64 (%d) != slot_capacity (%d)", c->max_pages_per_seq * 64,
                  c->slot_capacity);
    if (c->num_pages <= 0) return fail(PS_INVALID_ARGUMENT, "paged cache needs num_pages > 0");
  }
  return PS_OK;
}

ps::CacheGeom make_geom(const ps_attn_desc* a, const ps_cache_desc* c) {
  ps::CacheGeom g;
  g.paged = c->page_size == 64 ? 1 : 0;
  g.hkv = a->num_kv_heads;
  g.head_dim = a->head_dim;
  g.window = c->window;
  g.slot_capacity = c->slot_capacity;
  g.max_pages = c->page_size == 64 ? c->max_pages_per_seq : 0;
  g.num_pages = c->page_size == 64 ? c->num_pages : 0;
  return g;
}

ps::RopeFreq make_rope(const ps_attn_desc* a) {
  ps::RopeFreq r;
  r.enabled = a->rope_theta > 0.0 ? 1 : 0;
  const int half = a->head_dim / 2;
  for (int i = 0; i < ps::kMaxHalfDim; ++i)
    r.inv_freq[i] = (r.enabled && i < half) ? pow(a->rope_theta, -2.0 * (double)i / (double)a->head_dim) : 0.0;
  return r;
}

int32_t device_cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 256;
  }
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  return cus;
}

// Split count.  A decode workgroup streams its keys at about the same rate
// whether one or two share a CU, so the time of s splits goes as the number
// of waves of one workgroup per CU, ceil(streams * s / CUs), times the 1/s of
// the keys each covers: the s minimising ceil(streams * s / CUs) / s is taken,
// the smallest on ties (each split adds a partial to merge), and splits never
// get shorter than 4 chunks per wave.  (Measured at 131072 with W = 4096 this
// picks the fastest or within 2 % of it for 8 to 1024 sequences.)
int32_t auto_splits(const ps_attn_desc* a, const ps_cache_desc* c, int32_t num_seqs, int32_t cus) {
  const int64_t streams = (int64_t)num_seqs * a->num_kv_heads;
  if (streams <= 0 || cus <= 0) return 1;
  int64_t max_s = c->slot_capacity / (32 * 4 * 4);
  if (max_s > 64) max_s = 64;
  int64_t best_s = 1, best_rounds = (streams + cus - 1) / cus;
  for (int64_t s = 2; s <= max_s; ++s) {
    const int64_t rounds = (streams * s + cus - 1) / cus;
    if (rounds * best_s < best_rounds * s) {   // rounds / s < best_rounds / best_s
      best_s = s;
      best_rounds = rounds;
    }
  }
  return (int32_t)best_s;
}

int32_t split_keys_for(const ps_cache_desc* c, int32_t splits) {
  const int32_t per = (c->slot_capacity + splits - 1) / splits;
  return (per + 31) / 32 * 32;
}

size_t decode_ws_bytes(const ps_attn_desc* a, int32_t num_seqs, int32_t splits) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)num_seqs * a->num_q_heads * splits;
  return rows * a->head_dim * sizeof(float) + rows * 2 * sizeof(float);
}

// Heavy-hitter step in bf16 with one split: when a sequence's statistics fit
// in LDS the decode kernel keeps them there and accumulates the scores itself.
bool heavy_fused(const ps_attn_desc* a, const ps_cache_desc* c, int32_t splits) {
  return a->dtype == PS_BF16 && splits == 1 &&
         ps::fused_stats_bytes(c->slot_capacity, a->num_q_heads / a->num_kv_heads) <= (size_t)ps::kFusedStatsLds;
}

// Heavy-hitter step: after the split partials (256-aligned), the per-slot
// statistics (fp16 s - m for bf16, fp32 s for fp32), the bf16 path's per-chunk
// maxima and each row's log2-sum-exp2; nothing for the fused step.
struct HeavyLayout {
  size_t scores, max, lse2, total;
};
HeavyLayout heavy_layout(const ps_attn_desc* a, const ps_cache_desc* c, int32_t num_seqs, int32_t splits) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const bool bf16 = a->dtype == PS_BF16;
  HeavyLayout l;
  l.scores = al(decode_ws_bytes(a, num_seqs, splits));
  if (heavy_fused(a, c, splits)) {
    l.max = l.lse2 = l.total = l.scores;
    return l;
  }
  l.max = l.scores + al((size_t)num_seqs * a->num_q_heads * c->slot_capacity * (bf16 ? 2 : 4));
  l.lse2 = l.max + (bf16 ? al((size_t)num_seqs * a->num_q_heads * (c->slot_capacity / 32) * sizeof(float)) : 0);
  l.total = l.lse2 + al((size_t)num_seqs * a->num_q_heads * sizeof(float));
  return l;
}

// Reset PE re-rotating keys: after the split partials (256-aligned), the
// renumbered query positions, the cos/sin table and the rotated key copy.
struct RecomputeLayout {
  size_t pos, table, keys, total;
};
RecomputeLayout recompute_layout(const ps_attn_desc* a, const ps_cache_desc* c, int32_t num_seqs, int32_t splits) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  RecomputeLayout l;
  l.pos = al(decode_ws_bytes(a, num_seqs, splits));
  l.table = l.pos + al((size_t)num_seqs * sizeof(int64_t));
  const size_t elem = a->dtype == PS_BF16 ? 2 : 4;
  l.keys = l.table + al((size_t)c->slot_capacity * (a->head_dim / 2) * 2 * elem);   // fp16 / fp32 (cos, sin)
  l.total = l.keys + al((size_t)num_seqs * a->num_kv_heads * c->slot_capacity * a->head_dim * elem);
  return l;
}

ps_status check_prefill_geom(int32_t window, int32_t prefix_len, int64_t kv_start, int32_t batch, int32_t num_q,
                             int32_t num_k) {
  if (window < 1) return fail(PS_INVALID_ARGUMENT, "window W=%d must be >= 1", window);
  if (prefix_len < 0) return fail(PS_INVALID_ARGUMENT, "prefix_len %d must be >= 0", prefix_len);
  if (batch < 0 || num_q < 0 || num_k < 0) return fail(PS_INVALID_ARGUMENT, "negative batch/query/key count");
  if (prefix_len > num_k) return fail(PS_INVALID_ARGUMENT, "prefix_len %d exceeds num_keys %d", prefix_len, num_k);
  if (kv_start < prefix_len) return fail(PS_INVALID_ARGUMENT, "kv_start %lld < prefix_len %d", (long long)kv_start, prefix_len);
  if (num_q > num_k) return fail(PS_INVALID_ARGUMENT, "num_queries %d exceeds num_keys %d", num_q, num_k);
  if (num_q > num_k - prefix_len && kv_start != prefix_len)
    return fail(PS_INVALID_ARGUMENT, "queries reach into the prefix, so kv_start must equal prefix_len");
  return PS_OK;
}

size_t prefill_ws_bytes(const ps_attn_desc* a, int32_t batch, int32_t num_q, int32_t num_k) {
  int32_t bm, bn;
  ps::prefill_tile_shape(a->dtype, a->head_dim, &bm, &bn);
  const size_t elem = a->dtype == PS_BF16 ? 2 : 4;
  const size_t nkp = ((size_t)num_k + bn - 1) / bn * bn;
  const size_t kv = 2 * (size_t)batch * a->num_kv_heads * nkp * a->head_dim * elem;
  const size_t table = (size_t)num_q * (a->head_dim / 2) * 2 * sizeof(float);
  return ((kv + 255) / 256) * 256 + table;
}

// Chunk prefill workspace: K / V^T copies of every sequence's key array (keys
// padded to pad64(slot_capacity + T)) and the rotated queries.
size_t chunk_nkp(const ps_cache_desc* c, int32_t chunk_len) {
  return ((size_t)c->slot_capacity + chunk_len + 63) / 64 * 64;
}

size_t chunk_ws_bytes(const ps_attn_desc* a, const ps_cache_desc* c, int32_t num_seqs, int32_t chunk_len) {
  const size_t elem = a->dtype == PS_BF16 ? 2 : 4;
  const size_t kv = 2 * (size_t)num_seqs * a->num_kv_heads * chunk_nkp(c, chunk_len) * a->head_dim * elem;
  const size_t cs = (size_t)num_seqs * chunk_len * (a->head_dim / 2) * 2 * sizeof(float);   // query cos/sin
  return ((kv + 255) / 256) * 256 + ((cs + 255) / 256) * 256;
}

// Backward workspace layout (each piece 256-byte aligned).
struct BwdLayout {
  size_t kr, krt, vr, qs, lse2, di, cs_q, cs_k, total;
  int32_t nkp, tqp;
};

BwdLayout bwd_layout(const ps_attn_desc* a, int32_t batch, int32_t num_q, int32_t num_k) {
  BwdLayout l;
  l.nkp = (num_k + 127) / 128 * 128;
  l.tqp = (num_q + 63) / 64 * 64;
  const size_t elem = a->dtype == PS_BF16 ? 2 : 4;
  const size_t d = a->head_dim;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t kv = al((size_t)batch * a->num_kv_heads * l.nkp * d * elem);
  const size_t qv = al((size_t)batch * a->num_q_heads * l.tqp * d * elem);
  const size_t rows = al((size_t)batch * a->num_q_heads * l.tqp * sizeof(float));
  size_t o = 0;
  l.kr = o; o += kv;
  l.krt = o; o += kv;
  l.vr = o; o += kv;
  l.qs = o; o += qv;
  l.lse2 = o; o += rows;
  l.di = o; o += rows;
  l.cs_q = o; o += al((size_t)num_q * d * sizeof(float));
  l.cs_k = o; o += al((size_t)l.nkp * d * sizeof(float));
  l.total = o;
  return l;
}

// dS^T tiles the bf16 backward can keep for its dq pass (one 128-key x
// 64-query bf16 tile per visited pair, ds_slots per 64-query block): bytes and
// slots; zero for fp32 or an empty call.
struct DsLayout {
  size_t bytes;
  int32_t slots;
};

DsLayout ds_layout(const ps_attn_desc* a, int32_t window, int32_t prefix_len, int64_t kv_start, int32_t batch,
                   int32_t num_q, int32_t num_k) {
  DsLayout d{0, 0};
  if (a->dtype != PS_BF16 || batch <= 0 || num_q <= 0 || num_k <= 0) return d;
  const ps::PrefillGeom g{num_q, num_k, prefix_len, window, kv_start, 64, 128};
  const int32_t nqb = (num_q + 63) / 64;
  for (int32_t qb = 0; qb < nqb; ++qb) {
    const int32_t n = ps::pf_walk(g, qb).n_cand;
    d.slots = n > d.slots ? n : d.slots;
  }
  d.bytes = (size_t)batch * a->num_q_heads * nqb * d.slots * (128 * 64 * 2);
  return d;
}

}  // namespace

extern "C" {

const char* ps_last_error(void) { return g_last_error.c_str(); }

int32_t ps_abi_version(void) { return PS_ABI_VERSION; }

const char* ps_status_string(ps_status st) {
  switch (st) {
    case PS_OK: return "ok";
    case PS_INVALID_ARGUMENT: return "invalid argument";
    case PS_UNSUPPORTED: return "unsupported";
    case PS_WORKSPACE_TOO_SMALL: return "workspace too small";
    case PS_HIP_ERROR: return "HIP error";
  }
  return "unknown status";
}

ps_status ps_kv_append(const ps_attn_desc* attn, const ps_cache_desc* cache, void* k_cache, void* v_cache,
                       const int32_t* block_table, const int32_t* prefix_len, const int64_t* start_pos,
                       const int32_t* seq_tokens, int32_t tokens_per_seq, const void* k_new, const void* v_new,
                       int32_t num_seqs, int32_t* slot_pos, hipStream_t stream) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if ((st = check_cache(cache, block_table)) != PS_OK) return st;
  if (num_seqs < 0 || tokens_per_seq < 0) return fail(PS_INVALID_ARGUMENT, "negative num_seqs or tokens_per_seq");
  if (num_seqs == 0 || tokens_per_seq == 0) return ok();
  if ((int64_t)num_seqs * tokens_per_seq > (int64_t)1 << 26)
    return fail(PS_INVALID_ARGUMENT, "num_seqs*tokens_per_seq exceeds 2^26 per call");
  if (!k_cache || !v_cache || !prefix_len || !start_pos || !k_new || !v_new)
    return fail(PS_INVALID_ARGUMENT, "NULL device pointer");
  if ((st = check_aligned({{k_cache, "k_cache"}, {v_cache, "v_cache"}, {k_new, "k_new"}, {v_new, "v_new"}})) != PS_OK)
    return st;
  ps::AppendArgs a{};
  a.geom = make_geom(attn, cache);
  a.dtype = attn->dtype;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.prefix_len = prefix_len;
  a.start_pos = start_pos;
  a.seq_tokens = seq_tokens;
  a.tokens_per_seq = tokens_per_seq;
  a.k_new = k_new;
  a.v_new = v_new;
  a.num_seqs = num_seqs;
  a.slot_pos = slot_pos;
  a.rope = make_rope(attn);
  if (attn->pe_mode == PS_PE_RESET_RECOMPUTE) a.rope.enabled = 0;   // keys are rotated at every read
  return from_hip(ps::launch_append(a, stream), "ps_kv_append launch");
}

int32_t ps_decode_num_splits(const ps_attn_desc* attn, const ps_cache_desc* cache, int32_t num_seqs) {
  if (check_attn(attn) != PS_OK || !cache || cache->slot_capacity <= 0 || num_seqs < 0) return 0;
  return auto_splits(attn, cache, num_seqs, device_cu_count());
}

size_t ps_decode_workspace_size(const ps_attn_desc* attn, const ps_cache_desc* cache, int32_t num_seqs,
                                int32_t num_splits) {
  if (check_attn(attn) != PS_OK || !cache || cache->slot_capacity <= 0 || num_seqs < 0 || num_splits < 0) return 0;
  const int32_t s = num_splits > 0 ? num_splits : auto_splits(attn, cache, num_seqs, device_cu_count());
  if (attn->pe_mode == PS_PE_RESET_RECOMPUTE) return recompute_layout(attn, cache, num_seqs, s).total;
  return decode_ws_bytes(attn, num_seqs, s);
}

namespace {
// ps_decode_attn, and with k_new / v_new the fused append of ps_decode_step
ps_status decode_call(const ps_attn_desc* attn, const ps_cache_desc* cache, const void* k_cache, const void* v_cache,
                      const int32_t* block_table, const int32_t* prefix_len, const int64_t* pos, const void* q,
                      void* out, int32_t num_seqs, int32_t num_splits, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, const void* k_new, const void* v_new, bool dry = false) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if ((st = check_cache(cache, block_table)) != PS_OK) return st;
  if (num_seqs < 0) return fail(PS_INVALID_ARGUMENT, "negative num_seqs");
  if (num_splits < 0) return fail(PS_INVALID_ARGUMENT, "negative num_splits");
  if (num_seqs == 0) return ok();
  if (!k_cache || !v_cache || !prefix_len || !pos || !q || !out) return fail(PS_INVALID_ARGUMENT, "NULL device pointer");
  if ((st = check_aligned({{k_cache, "k_cache"}, {v_cache, "v_cache"}, {q, "q"}, {out, "out"}, {k_new, "k_new"},
                           {v_new, "v_new"}, {workspace, "workspace"}})) != PS_OK)
    return st;
  if ((int64_t)num_seqs * attn->num_kv_heads * 64 > (int64_t)1 << 31)
    return fail(PS_INVALID_ARGUMENT, "num_seqs too large for one launch");
  const int32_t splits = num_splits > 0 ? num_splits : auto_splits(attn, cache, num_seqs, device_cu_count());
  if (splits > 1024 || splits > cache->slot_capacity / 32)
    return fail(PS_INVALID_ARGUMENT, "num_splits %d too large for slot_capacity %d", splits, cache->slot_capacity);
  const bool recompute = attn->pe_mode == PS_PE_RESET_RECOMPUTE;
  if (recompute && cache->page_size != 0)
    return fail(PS_UNSUPPORTED, "pe_mode 2 (Reset PE re-rotating keys) needs a contiguous cache");
  const size_t need = recompute ? recompute_layout(attn, cache, num_seqs, splits).total
                                : decode_ws_bytes(attn, num_seqs, splits);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PS_WORKSPACE_TOO_SMALL, "decode needs %zu workspace bytes, got %zu", need, workspace_bytes);
  if (dry) return ok();   // validation only
  ps::DecodeArgs a{};
  a.geom = make_geom(attn, cache);
  a.dtype = attn->dtype;
  a.hq = attn->num_q_heads;
  a.group = attn->num_q_heads / attn->num_kv_heads;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.prefix_len = prefix_len;
  a.pos = pos;
  a.q = q;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_splits = splits;
  a.split_keys = split_keys_for(cache, splits);
  float* ws = static_cast<float*>(workspace);
  const size_t rows = (size_t)num_seqs * attn->num_q_heads * splits;
  a.part_o = splits > 1 ? ws : nullptr;
  a.part_ml = splits > 1 ? ws + rows * attn->head_dim : nullptr;
  a.scale_log2 = attn->softmax_scale * 1.4426950408889634f;
  a.rope = make_rope(attn);
  a.reset_pe = attn->pe_mode == PS_PE_RESET ? 1 : 0;
  a.wide = (int64_t)num_seqs * attn->num_kv_heads * splits <= device_cu_count() ? 1 : 0;
  a.heavy_count = nullptr;
  a.heavy_score = nullptr;
  a.heavy_slots = 0;
  a.stat_scores = nullptr;
  a.stat_max = nullptr;
  a.stat_lse2 = nullptr;
  a.k_new = k_new;
  a.v_new = v_new;
  if (recompute) {   // rotate the visible keys at their renumbered positions, then decode the copy
    const RecomputeLayout l = recompute_layout(attn, cache, num_seqs, splits);
    char* w = static_cast<char*>(workspace);
    ps::ResetArgs r{};
    r.geom = a.geom;
    r.dtype = attn->dtype;
    r.num_seqs = num_seqs;
    r.k_cache = k_cache;
    r.prefix_len = prefix_len;
    r.pos = pos;
    r.rope = a.rope;
    r.table = w + l.table;
    r.k_out = w + l.keys;
    r.pos_out = reinterpret_cast<int64_t*>(w + l.pos);
    const ps_status rs = from_hip(ps::launch_reset_rerotate(r, stream), "ps_decode_attn key rotation launch");
    if (rs != PS_OK) return rs;
    a.k_cache = r.k_out;
    a.pos = r.pos_out;
    a.reset_pe = 0;
  }
  return from_hip(ps::launch_decode(a, stream), "ps_decode_attn launch");
}
}  // namespace

ps_status ps_decode_attn(const ps_attn_desc* attn, const ps_cache_desc* cache, const void* k_cache,
                         const void* v_cache, const int32_t* block_table, const int32_t* prefix_len, const int64_t* pos,
                         const void* q, void* out, int32_t num_seqs, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return decode_call(attn, cache, k_cache, v_cache, block_table, prefix_len, pos, q, out, num_seqs, num_splits,
                     workspace, workspace_bytes, stream, nullptr, nullptr);
}

ps_status ps_decode_step(const ps_attn_desc* attn, const ps_cache_desc* cache, void* k_cache, void* v_cache,
                         const int32_t* block_table, const int32_t* prefix_len, const int64_t* pos, const void* q,
                         const void* k_new, const void* v_new, void* out, int32_t num_seqs, int32_t num_splits,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if (num_seqs > 0 && (!k_new || !v_new)) return fail(PS_INVALID_ARGUMENT, "NULL device pointer");
  if (attn->dtype == PS_BF16 && attn->pe_mode == PS_PE_CONTINUE)   // one launch: append inside the decode kernel
    return decode_call(attn, cache, k_cache, v_cache, block_table, prefix_len, pos, q, out, num_seqs, num_splits,
                       workspace, workspace_bytes, stream, k_new, v_new);
  // other dtypes and PE modes: the append, then the decode, as two launches
  // everything the decode checks is checked before the append runs
  if ((st = decode_call(attn, cache, k_cache, v_cache, block_table, prefix_len, pos, q, out, num_seqs, num_splits,
                        workspace, workspace_bytes, stream, nullptr, nullptr, true)) != PS_OK)
    return st;
  if ((st = ps_kv_append(attn, cache, k_cache, v_cache, block_table, prefix_len, pos, nullptr, 1, k_new, v_new,
                         num_seqs, nullptr, stream)) != PS_OK)
    return st;
  return decode_call(attn, cache, k_cache, v_cache, block_table, prefix_len, pos, q, out, num_seqs, num_splits,
                     workspace, workspace_bytes, stream, nullptr, nullptr);
}

}  // extern "C"

namespace {
// Device scratch of ps_decode_step_noalloc: the split partials live in this
// file-scope device array (one copy per GPU, resident until the process ends)
// instead of a caller workspace.  Host code never passes the array's name to a
// kernel or a copy (on the host it is only a stand-in); it uses the device
// address hipGetSymbolAddress returns, looked up once per device with that
// device current.  Every call on a GPU shares that GPU's copy; the decode
// kernels overwrite every partial they later read, so nothing needs clearing.
constexpr size_t kScratchBytes = (size_t)8 << 20;
constexpr int kScratchDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices] = {};

ps_status scratch_for_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "ps_decode_step_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices) return fail(PS_UNSUPPORTED, "device index %d beyond %d", dev, kScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return from_hip(e != hipSuccess ? e : hipErrorInvalidSymbol,
                                               "ps_decode_step_noalloc: hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PS_OK;
}
}  // namespace

extern "C" {

size_t ps_decode_noalloc_scratch_bytes(void) { return kScratchBytes; }

ps_status ps_decode_step_noalloc(const ps_attn_desc* attn, const ps_cache_desc* cache, void* k_cache, void* v_cache,
                                 const int32_t* block_table, const int32_t* prefix_len, const int64_t* pos,
                                 const void* q, const void* k_new, const void* v_new, void* out, int32_t num_seqs,
                                 int32_t num_splits, hipStream_t stream) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if (!cache || cache->slot_capacity <= 0 || num_seqs < 0 || num_splits < 0)
    return fail(PS_INVALID_ARGUMENT, "invalid cache descriptor, num_seqs or num_splits");
  const size_t need = ps_decode_workspace_size(attn, cache, num_seqs, num_splits);
  if (need > kScratchBytes)
    return fail(PS_WORKSPACE_TOO_SMALL,
                "ps_decode_step_noalloc: this call needs %zu scratch bytes, beyond the library's static %zu "
                "(fewer splits or sequences per call, or ps_decode_step with a workspace)",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0 && (st = scratch_for_current_device(&ws)) != PS_OK) return st;
  return ps_decode_step(attn, cache, k_cache, v_cache, block_table, prefix_len, pos, q, k_new, v_new, out, num_seqs,
                        num_splits, ws, need > 0 ? kScratchBytes : 0, stream);
}

size_t ps_heavy_workspace_size(const ps_attn_desc* attn, const ps_cache_desc* cache, int32_t num_seqs,
                               int32_t num_splits) {
  if (check_attn(attn) != PS_OK || !cache || cache->slot_capacity <= 0 || num_seqs < 0 || num_splits < 0) return 0;
  const int32_t sp = num_splits > 0 ? num_splits : auto_splits(attn, cache, num_seqs, device_cu_count());
  return heavy_layout(attn, cache, num_seqs, sp).total;
}

ps_status ps_heavy_decode_step(const ps_attn_desc* attn, const ps_cache_desc* cache, int32_t heavy_slots,
                               void* k_cache, void* v_cache, const int32_t* block_table, const int32_t* prefix_len,
                               const int64_t* pos, const void* q, const void* k_new, const void* v_new, void* out,
                               int32_t num_seqs, float* score, int32_t* heavy_count, int64_t* heavy_pos,
                               int32_t num_splits, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if ((st = continue_pe_only(attn, "ps_heavy_decode_step")) != PS_OK) return st;
  if ((st = check_cache(cache, block_table)) != PS_OK) return st;
  if (num_seqs < 0 || num_splits < 0 || heavy_slots < 0)
    return fail(PS_INVALID_ARGUMENT, "negative num_seqs, num_splits or heavy_slots");
  if ((int64_t)cache->window + heavy_slots > cache->slot_capacity)
    return fail(PS_INVALID_ARGUMENT, "W + heavy_slots exceeds slot_capacity");
  if ((int64_t)(attn->num_q_heads / attn->num_kv_heads) * cache->slot_capacity * 4 >= ((int64_t)1 << 31))
    return fail(PS_INVALID_ARGUMENT, "slot_capacity too large for heavy-hitter statistics");
  if (num_seqs == 0) return ok();
  if (!k_cache || !v_cache || !prefix_len || !pos || !q || !k_new || !v_new || !out || !score || !heavy_count ||
      (heavy_slots > 0 && !heavy_pos))
    return fail(PS_INVALID_ARGUMENT, "NULL device pointer");
  if ((st = check_aligned({{k_cache, "k_cache"}, {v_cache, "v_cache"}, {q, "q"}, {out, "out"}, {k_new, "k_new"},
                           {v_new, "v_new"}, {score, "score"}, {workspace, "workspace"}})) != PS_OK)
    return st;
  if ((int64_t)num_seqs * attn->num_kv_heads * 64 > (int64_t)1 << 31)
    return fail(PS_INVALID_ARGUMENT, "num_seqs too large for one launch");
  const int32_t splits = num_splits > 0 ? num_splits : auto_splits(attn, cache, num_seqs, device_cu_count());
  if (splits > 1024 || splits > cache->slot_capacity / 32)
    return fail(PS_INVALID_ARGUMENT, "num_splits %d too large for slot_capacity %d", splits, cache->slot_capacity);
  const size_t need = ps_heavy_workspace_size(attn, cache, num_seqs, splits);
  if ((need > 0 && !workspace) || workspace_bytes < need)
    return fail(PS_WORKSPACE_TOO_SMALL, "heavy decode needs %zu workspace bytes, got %zu", need, workspace_bytes);
  char* w = static_cast<char*>(workspace);
  const HeavyLayout hl = heavy_layout(attn, cache, num_seqs, splits);
  void* stat_scores = w + hl.scores;
  float* stat_max = attn->dtype == PS_BF16 ? reinterpret_cast<float*>(w + hl.max) : nullptr;
  float* stat_lse2 = reinterpret_cast<float*>(w + hl.lse2);
  const ps::CacheGeom geom = make_geom(attn, cache);
  const ps::RopeFreq rope = make_rope(attn);
  ps::HeavyArgs h{};
  h.geom = geom;
  h.dtype = attn->dtype;
  h.hq = attn->num_q_heads;
  h.group = attn->num_q_heads / attn->num_kv_heads;
  h.heavy_slots = heavy_slots;
  h.k_cache = k_cache;
  h.v_cache = v_cache;
  h.block_table = block_table;
  h.prefix_len = prefix_len;
  h.pos = pos;
  h.num_seqs = num_seqs;
  h.score = score;
  h.heavy_count = heavy_count;
  h.heavy_pos = heavy_pos;
  h.stat_scores = stat_scores;
  h.stat_max = stat_max;
  h.stat_lse2 = stat_lse2;
  h.k_new = k_new;
  h.v_new = v_new;
  h.rope = rope;
  // 1-2. the token leaving the window (admission), then the new token into the ring
  hipError_t e = ps::launch_heavy_retire(h, stream);
  if (e != hipSuccess) return from_hip(e, "ps_heavy_decode_step retire launch");
  ps::DecodeArgs a{};   // 3. attention over prefix + window + heavy slots
  a.geom = geom;
  a.dtype = attn->dtype;
  a.hq = attn->num_q_heads;
  a.group = attn->num_q_heads / attn->num_kv_heads;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.prefix_len = prefix_len;
  a.pos = pos;
  a.q = q;
  a.out = out;
  a.num_seqs = num_seqs;
  a.num_splits = splits;
  a.split_keys = split_keys_for(cache, splits);
  const size_t rows = (size_t)num_seqs * attn->num_q_heads * splits;
  a.part_o = splits > 1 ? reinterpret_cast<float*>(w) : nullptr;
  a.part_ml = splits > 1 ? reinterpret_cast<float*>(w) + rows * attn->head_dim : nullptr;
  a.scale_log2 = attn->softmax_scale * 1.4426950408889634f;
  a.rope = rope;
  a.reset_pe = 0;
  a.heavy_count = heavy_count;
  a.heavy_slots = heavy_slots;
  const bool fused = heavy_fused(attn, cache, splits);
  a.stat_scores = fused ? nullptr : stat_scores;
  a.stat_max = fused ? nullptr : stat_max;
  a.stat_lse2 = fused ? nullptr : stat_lse2;
  a.heavy_score = fused ? score : nullptr;   // fused: the decode kernel also does step 4
  a.k_new = nullptr;   // the token is appended by the retire kernel above
  a.v_new = nullptr;
  if ((e = ps::launch_decode(a, stream)) != hipSuccess) return from_hip(e, "ps_heavy_decode_step decode launch");
  if (fused) return ok();
  return from_hip(ps::launch_heavy_accumulate(h, stream), "ps_heavy_decode_step accumulate launch");  // 4.
}

size_t ps_prefill_workspace_size(const ps_attn_desc* attn, int32_t batch, int32_t num_queries, int32_t num_keys) {
  if (check_attn(attn) != PS_OK || batch < 0 || num_queries < 0 || num_keys < 0) return 0;
  return prefill_ws_bytes(attn, batch, num_queries, num_keys);
}

ps_status ps_read_probe(const void* src, size_t bytes, uint32_t* checksum, hipStream_t stream) {
  if (!checksum || (bytes > 0 && !src)) return fail(PS_INVALID_ARGUMENT, "NULL pointer");
  if (bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return fail(PS_INVALID_ARGUMENT, "src and bytes must be 16-byte aligned");
  if (bytes > ((size_t)1 << 40)) return fail(PS_INVALID_ARGUMENT, "bytes %zu beyond 2^40", bytes);
  return from_hip(ps::launch_read_probe(src, (int64_t)bytes, checksum, device_cu_count(), stream), "ps_read_probe");
}

ps_status ps_prefill_tile_shape(const ps_attn_desc* attn, int32_t* block_m, int32_t* block_n) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if (!block_m || !block_n) return fail(PS_INVALID_ARGUMENT, "NULL output pointer");
  ps::prefill_tile_shape(attn->dtype, attn->head_dim, block_m, block_n);
  return ok();
}

ps_status ps_prefill_attn(const ps_attn_desc* attn, int32_t window, int32_t prefix_len, int64_t kv_start,
                          const void* q, const void* k, const void* v, int32_t batch, int32_t num_queries,
                          int32_t num_keys, void* out, float* lse, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if ((st = continue_pe_only(attn, "ps_prefill_attn")) != PS_OK) return st;
  if ((st = check_prefill_geom(window, prefix_len, kv_start, batch, num_queries, num_keys)) != PS_OK) return st;
  if (batch == 0 || num_queries == 0) return ok();
  if (!q || !k || !v || !out) return fail(PS_INVALID_ARGUMENT, "NULL device pointer");
  if ((st = check_aligned({{q, "q"}, {k, "k"}, {v, "v"}, {out, "out"}, {workspace, "workspace"}})) != PS_OK ||
      (st = check_aligned({{lse, "lse"}}, 4)) != PS_OK)
    return st;
  const size_t need = prefill_ws_bytes(attn, batch, num_queries, num_keys);
  if (!workspace || workspace_bytes < need)
    return fail(PS_WORKSPACE_TOO_SMALL, "prefill needs %zu workspace bytes, got %zu", need, workspace_bytes);
  int32_t bm, bn;
  ps::prefill_tile_shape(attn->dtype, attn->head_dim, &bm, &bn);
  if ((int64_t)batch * attn->num_q_heads * ((num_queries + bm - 1) / bm) + 8 > (int64_t)1 << 31)
    return fail(PS_INVALID_ARGUMENT, "prefill grid too large");
  ps::PrefillArgs a{};
  a.dtype = attn->dtype;
  a.hq = attn->num_q_heads;
  a.hkv = attn->num_kv_heads;
  a.group = attn->num_q_heads / attn->num_kv_heads;
  a.head_dim = attn->head_dim;
  a.window = window;
  a.prefix_len = prefix_len;
  a.kv_start = kv_start;
  a.batch = batch;
  a.num_q = num_queries;
  a.num_k = num_keys;
  a.bm = bm;
  a.bn = bn;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  const size_t elem = attn->dtype == PS_BF16 ? 2 : 4;
  const size_t nkp = ((size_t)num_keys + bn - 1) / bn * bn;
  if (attn->dtype == PS_BF16 && nkp > kMaxBf16PrefillKeys)
    return fail(PS_INVALID_ARGUMENT, "bf16 prefill takes at most 2^28 keys, got %d", num_keys);
  const size_t kv = 2 * (size_t)batch * attn->num_kv_heads * nkp * attn->head_dim * elem;
  a.k_rot = workspace;
  a.rope_cs = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((kv + 255) / 256) * 256);
  a.scale_log2 = attn->softmax_scale * 1.4426950408889634f;
  a.rope = make_rope(attn);
  a.nkp = (int32_t)nkp;
  a.seq_prefix = nullptr;
  a.seq_start = nullptr;
  a.k_cache = nullptr;
  a.v_cache = nullptr;
  a.block_table = nullptr;
  a.cg = ps::CacheGeom{};
  return from_hip(ps::launch_prefill(a, stream), "ps_prefill_attn launch");
}

size_t ps_prefill_backward_workspace_size(const ps_attn_desc* attn, int32_t batch, int32_t num_queries,
                                          int32_t num_keys) {
  if (check_attn(attn) != PS_OK || batch < 0 || num_queries < 0 || num_keys < 0) return 0;
  return bwd_layout(attn, batch, num_queries, num_keys).total;
}

size_t ps_prefill_backward_ds_workspace_size(const ps_attn_desc* attn, int32_t window, int32_t prefix_len,
                                             int64_t kv_start, int32_t batch, int32_t num_queries,
                                             int32_t num_keys) {
  if (check_attn(attn) != PS_OK ||
      check_prefill_geom(window, prefix_len, kv_start, batch, num_queries, num_keys) != PS_OK)
    return 0;
  return ds_layout(attn, window, prefix_len, kv_start, batch, num_queries, num_keys).bytes;
}

ps_status ps_prefill_attn_backward(const ps_attn_desc* attn, int32_t window, int32_t prefix_len, int64_t kv_start,
                                   const void* q, const void* k, const void* v, const void* out, const void* d_out,
                                   const float* lse, int32_t batch, int32_t num_queries, int32_t num_keys, void* dq,
                                   void* dk, void* dv, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if ((st = continue_pe_only(attn, "ps_prefill_attn_backward")) != PS_OK) return st;
  if ((st = check_prefill_geom(window, prefix_len, kv_start, batch, num_queries, num_keys)) != PS_OK) return st;
  if (batch == 0 || num_queries == 0) return ok();
  if (!q || !k || !v || !out || !d_out || !lse || !dq || !dk || !dv)
    return fail(PS_INVALID_ARGUMENT, "NULL device pointer");
  if ((st = check_aligned({{q, "q"}, {k, "k"}, {v, "v"}, {out, "out"}, {d_out, "d_out"}, {dq, "dq"}, {dk, "dk"},
                           {dv, "dv"}, {workspace, "workspace"}})) != PS_OK ||
      (st = check_aligned({{lse, "lse"}}, 4)) != PS_OK)
    return st;
  if ((int64_t)batch * attn->num_q_heads * ((num_queries + 127) / 128) + 8 > (int64_t)1 << 31 ||
      (int64_t)batch * attn->num_q_heads * num_queries > (int64_t)1 << 31 ||
      (int64_t)batch * attn->num_kv_heads * num_keys > (int64_t)1 << 31)
    return fail(PS_INVALID_ARGUMENT, "backward grid too large");
  if (num_keys > ((int32_t)1 << 30)) return fail(PS_INVALID_ARGUMENT, "num_keys exceeds 2^30");
  const BwdLayout l = bwd_layout(attn, batch, num_queries, num_keys);
  if (!workspace || workspace_bytes < l.total)
    return fail(PS_WORKSPACE_TOO_SMALL, "backward needs %zu workspace bytes, got %zu", l.total, workspace_bytes);
  // with room for them after the base layout, the dk/dv pass keeps its dS tiles for dq
  const DsLayout dl = ds_layout(attn, window, prefix_len, kv_start, batch, num_queries, num_keys);
  const bool keep_ds = dl.bytes > 0 && workspace_bytes - l.total >= dl.bytes;
  char* w = static_cast<char*>(workspace);
  ps::BackwardArgs a{};
  a.dtype = attn->dtype;
  a.hq = attn->num_q_heads;
  a.hkv = attn->num_kv_heads;
  a.group = attn->num_q_heads / attn->num_kv_heads;
  a.head_dim = attn->head_dim;
  a.window = window;
  a.prefix_len = prefix_len;
  a.kv_start = kv_start;
  a.batch = batch;
  a.num_q = num_queries;
  a.num_k = num_keys;
  a.nkp = l.nkp;
  a.tqp = l.tqp;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.d_out = d_out;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.kr = w + l.kr;
  a.krt = w + l.krt;
  a.vr = w + l.vr;
  a.qs = w + l.qs;
  a.lse2 = reinterpret_cast<float*>(w + l.lse2);
  a.di = reinterpret_cast<float*>(w + l.di);
  a.cs_q = reinterpret_cast<float*>(w + l.cs_q);
  a.cs_k = reinterpret_cast<float*>(w + l.cs_k);
  a.ds = keep_ds ? w + l.total : nullptr;
  a.ds_slots = keep_ds ? dl.slots : 0;
  a.scale = attn->softmax_scale;
  a.scale_log2 = attn->softmax_scale * 1.4426950408889634f;
  a.rope = make_rope(attn);
  return from_hip(ps::launch_backward(a, stream), "ps_prefill_attn_backward launch");
}

size_t ps_chunk_prefill_workspace_size(const ps_attn_desc* attn, const ps_cache_desc* cache, int32_t num_seqs,
                                       int32_t chunk_len) {
  if (check_attn(attn) != PS_OK || !cache || cache->slot_capacity <= 0 || num_seqs < 0 || chunk_len < 0) return 0;
  return chunk_ws_bytes(attn, cache, num_seqs, chunk_len);
}

ps_status ps_chunk_prefill_attn(const ps_attn_desc* attn, const ps_cache_desc* cache, void* k_cache, void* v_cache,
                                const int32_t* block_table, const int32_t* prefix_len, const int64_t* start_pos,
                                int32_t chunk_len, const void* q, const void* k_new, const void* v_new,
                                int32_t num_seqs, void* out, float* lse, int32_t* slot_pos, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if ((st = continue_pe_only(attn, "ps_chunk_prefill_attn")) != PS_OK) return st;
  if ((st = check_cache(cache, block_table)) != PS_OK) return st;
  if (num_seqs < 0 || chunk_len < 0) return fail(PS_INVALID_ARGUMENT, "negative num_seqs or chunk_len");
  if (num_seqs == 0 || chunk_len == 0) return ok();
  if (!k_cache || !v_cache || !prefix_len || !start_pos || !q || !k_new || !v_new || !out)
    return fail(PS_INVALID_ARGUMENT, "NULL device pointer");
  if ((st = check_aligned({{k_cache, "k_cache"}, {v_cache, "v_cache"}, {q, "q"}, {k_new, "k_new"}, {v_new, "v_new"},
                           {out, "out"}, {workspace, "workspace"}})) != PS_OK ||
      (st = check_aligned({{lse, "lse"}}, 4)) != PS_OK)
    return st;
  if ((int64_t)cache->slot_capacity + chunk_len > ((int64_t)1 << 30))
    return fail(PS_INVALID_ARGUMENT, "slot_capacity + chunk_len exceeds 2^30");
  if ((int64_t)num_seqs * chunk_len > (int64_t)1 << 26)
    return fail(PS_INVALID_ARGUMENT, "num_seqs*chunk_len exceeds 2^26 per call");
  int32_t bm, bn;
  ps::prefill_tile_shape(attn->dtype, attn->head_dim, &bm, &bn);
  if ((int64_t)num_seqs * attn->num_q_heads * ((chunk_len + bm - 1) / bm) + 8 > (int64_t)1 << 31)
    return fail(PS_INVALID_ARGUMENT, "chunk prefill grid too large");
  const size_t need = chunk_ws_bytes(attn, cache, num_seqs, chunk_len);
  if (!workspace || workspace_bytes < need)
    return fail(PS_WORKSPACE_TOO_SMALL, "chunk prefill needs %zu workspace bytes, got %zu", need, workspace_bytes);
  const size_t elem = attn->dtype == PS_BF16 ? 2 : 4;
  const size_t nkp = chunk_nkp(cache, chunk_len);
  if (attn->dtype == PS_BF16 && nkp > kMaxBf16PrefillKeys)
    return fail(PS_INVALID_ARGUMENT, "bf16 chunk prefill takes at most 2^28 keys per sequence");
  const size_t kv = 2 * (size_t)num_seqs * attn->num_kv_heads * nkp * attn->head_dim * elem;
  ps::PrefillArgs a{};
  a.dtype = attn->dtype;
  a.hq = attn->num_q_heads;
  a.hkv = attn->num_kv_heads;
  a.group = attn->num_q_heads / attn->num_kv_heads;
  a.head_dim = attn->head_dim;
  a.window = cache->window;
  a.prefix_len = 0;   // per sequence
  a.kv_start = 0;     // per sequence
  a.batch = num_seqs;
  a.num_q = chunk_len;
  a.num_k = 0;        // per sequence
  a.bm = bm;
  a.bn = bn;
  a.q = q;
  a.k = k_new;
  a.v = v_new;
  a.out = out;
  a.lse = lse;
  a.k_rot = workspace;
  a.rope_cs = reinterpret_cast<float*>(static_cast<char*>(workspace) + ((kv + 255) / 256) * 256);
  a.scale_log2 = attn->softmax_scale * 1.4426950408889634f;
  a.rope = make_rope(attn);
  a.nkp = (int32_t)nkp;
  a.seq_prefix = prefix_len;
  a.seq_start = start_pos;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.cg = make_geom(attn, cache);
  hipError_t e = ps::launch_chunk_prefill(a, stream);
  if (e != hipSuccess) return from_hip(e, "ps_chunk_prefill_attn launch");
  // the chunk joins the ring only after every chunk query has read the ring
  ps::AppendArgs ap{};
  ap.geom = a.cg;
  ap.dtype = attn->dtype;
  ap.k_cache = k_cache;
  ap.v_cache = v_cache;
  ap.block_table = block_table;
  ap.prefix_len = prefix_len;
  ap.start_pos = start_pos;
  ap.seq_tokens = nullptr;
  ap.tokens_per_seq = chunk_len;
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.num_seqs = num_seqs;
  ap.slot_pos = slot_pos;
  ap.rope = a.rope;
  ap.rope_cs = a.rope_cs;   // the chunk's positions P + t: the query table formed by the prep
  return from_hip(ps::launch_append(ap, stream), "ps_chunk_prefill_attn append launch");
}

ps_status ps_prefill_plan(const ps_attn_desc* attn, int32_t window, int32_t prefix_len, int64_t kv_start,
                          int32_t num_queries, int32_t num_keys, int32_t* tiles, int32_t max_tiles,
                          int32_t* num_tiles, hipStream_t stream) {
  ps_status st = check_attn(attn);
  if (st != PS_OK) return st;
  if ((st = check_prefill_geom(window, prefix_len, kv_start, 1, num_queries, num_keys)) != PS_OK) return st;
  if (!num_tiles || (max_tiles > 0 && !tiles)) return fail(PS_INVALID_ARGUMENT, "NULL device pointer");
  if (max_tiles < 0) return fail(PS_INVALID_ARGUMENT, "negative max_tiles");
  int32_t bm, bn;
  ps::prefill_tile_shape(attn->dtype, attn->head_dim, &bm, &bn);
  return from_hip(ps::launch_prefill_plan(num_queries, num_keys, prefix_len, window, kv_start, bm, bn, tiles,
                                          max_tiles, num_tiles, stream),
                  "ps_prefill_plan launch");
}

}  // extern "C"
