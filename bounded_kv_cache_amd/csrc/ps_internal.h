// Internal launch interface between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ps_common.h"

namespace ps {

struct AppendArgs {
  CacheGeom geom;
  int32_t dtype;  // ps_dtype
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* prefix_len;
  const int64_t* start_pos;
  const int32_t* seq_tokens;
  int32_t tokens_per_seq;
  const void* k_new;
  const void* v_new;
  int32_t num_seqs;
  int32_t* slot_pos;
  RopeFreq rope;
  // optional cos/sin of token t of sequence s at row s * tokens_per_seq + t,
  // [rows][D/2][2] (the chunk prefill's query table holds exactly these
  // positions); NULL: formed from the position
  const float* rope_cs;
};

struct DecodeArgs {
  CacheGeom geom;
  int32_t dtype;
  int32_t hq;
  int32_t group;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* prefix_len;
  const int64_t* pos;
  const void* q;
  void* out;
  int32_t num_seqs;
  int32_t num_splits;
  int32_t split_keys;     // keys per split, multiple of 32
  float* part_o;          // [num_seqs][hq][num_splits][D] (unnormalised)
  float* part_ml;         // [num_seqs][hq][num_splits][2]  (running max in log2 units, sum)
  float scale_log2;       // softmax_scale * log2(e)
  RopeFreq rope;
  int32_t reset_pe;       // 1: Reset PE scoring (prefix slots use the renumbered query)
  // 1: the launch has at most one workgroup per compute unit; the plain and
  // append-fused bf16 kernels then run eight waves per workgroup (twice the
  // loads in flight per CU)
  int32_t wide;
  // heavy-hitter mode (NULL / 0 otherwise): visible slots are [0, min(p+1, L+W) + heavy_count)
  const int32_t* heavy_count;  // [num_seqs][hkv]
  int32_t heavy_slots;         // H: heavy slots after the window, L + W + H <= slot_capacity
  // per visible slot and head, in log2 units: bf16 path, [num_seqs][hkv][slot_capacity / 32][group][32]
  // fp16 s - m with m the running max after the slot's 32-key chunk (in stat_max); fp32 path,
  // [num_seqs][hkv][group][slot_capacity] the score s itself
  void* stat_scores;
  float* stat_max;             // bf16 path: [num_seqs][hkv][slot_capacity / 32][group]; else NULL
  float* stat_lse2;            // [num_seqs][hq] log2-sum-exp2 of each query row
  // bf16, one split, statistics fit kFusedStatsLds: the decode kernel keeps the statistics in LDS and
  // adds the step's attention mass to these scores itself ([num_seqs][hkv][slot_capacity]); else NULL
  float* heavy_score;
  // bf16, Continue PE: the step's token [num_seqs][1][hkv][D] at pos, appended by the decode kernel
  // itself (k_cache / v_cache are then written); NULL otherwise
  const void* k_new;
  const void* v_new;
};

// Heavy-hitter bookkeeping around a decode step.
struct HeavyArgs {
  CacheGeom geom;
  int32_t dtype;
  int32_t hq, group;
  int32_t heavy_slots;
  void* k_cache;
  void* v_cache;
  const int32_t* block_table;
  const int32_t* prefix_len;
  const int64_t* pos;
  int32_t num_seqs;
  float* score;                // [num_seqs][hkv][slot_capacity] accumulated attention per slot
  int32_t* heavy_count;        // [num_seqs][hkv]
  int64_t* heavy_pos;          // [num_seqs][hkv][heavy_slots]
  const void* stat_scores;     // as DecodeArgs
  const float* stat_max;
  const float* stat_lse2;
  const void* k_new;           // the step's token [num_seqs][1][hkv][D], appended by the retire kernel
  const void* v_new;
  RopeFreq rope;
};

struct PrefillArgs {
  int32_t dtype;
  int32_t hq, hkv, group, head_dim;
  int32_t window, prefix_len;
  int64_t kv_start;
  int32_t batch, num_q, num_k;
  int32_t bm, bn;
  const void* q;
  const void* k;          // raw keys
  const void* v;
  void* out;
  float* lse;
  void* k_rot;            // workspace: rotated keys [batch][num_k][hkv][D]
  float* rope_cs;         // workspace: [num_q][D/2][2] cos/sin of query positions (chunks: [batch][num_q][D/2][2])
  float scale_log2;
  RopeFreq rope;
  int32_t nkp;            // key stride of the K / V^T copies (multiple of 64)
  // chunk mode: per-sequence geometry, keys below start_pos read from the ring
  const int32_t* seq_prefix;   // [batch] L of each sequence
  const int64_t* seq_start;    // [batch] first chunk position P of each sequence
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  CacheGeom cg;
};

// Backward of the masked prefill (dq, dk, dv for the raw inputs).
struct BackwardArgs {
  int32_t dtype;
  int32_t hq, hkv, group, head_dim;
  int32_t window, prefix_len;
  int64_t kv_start;
  int32_t batch, num_q, num_k;
  int32_t nkp;            // keys padded to a multiple of 128
  int32_t tqp;            // queries padded to a multiple of 64
  const void* q;          // [batch][num_q][hq][D] raw
  const void* k;          // [batch][num_k][hkv][D] raw
  const void* v;
  const void* out;        // forward output [batch][num_q][hq][D]
  const void* d_out;      // upstream gradient, same layout
  const float* lse;       // forward LSE [batch][hq][num_q] (natural log)
  void* dq;
  void* dk;
  void* dv;
  // workspace
  void* kr;               // [batch][hkv][nkp][D] rotated keys
  void* krt;              // [batch][hkv][D][nkp] rotated keys, d-major, keys permuted per 16 (vt_slot)
  void* vr;               // [batch][hkv][nkp][D] values, zero padded
  void* qs;               // [batch][hq][tqp][D] rotated queries * scale * log2(e)
  float* lse2;            // [batch][hq][tqp] lse * log2(e); +inf on padding rows
  float* di;              // [batch][hq][tqp] rowsum(d_out * out)
  float* cs_q;            // [num_q][D/2][2] cos/sin of the query positions
  float* cs_k;            // [nkp][D/2][2] cos/sin of the key positions
  void* ds;               // optional dS^T tiles kept by the dk/dv kernel for the dq kernel (null: dq recomputes
                          // S and dP): [batch][hq][tqp/64][ds_slots][128 keys][64 queries]
  int32_t ds_slots;       // tiles per 64-query block: the longest walk of 128-key tiles of a block
  float scale;            // softmax scale
  float scale_log2;       // scale * log2(e)
  RopeFreq rope;
};

hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
// Heavy-hitter decode with the statistics in LDS; per 32-slot chunk and query
// head they take 32 fp16 values and one fp32 max.  Statistics up to
// kFusedStatsLdsSmall: 4 waves per workgroup, two workgroups per CU (as the
// plain decode); up to kFusedStatsLds: 8 waves, one workgroup per CU.
constexpr int kFusedStatsWaves = 8;
constexpr int kFusedStatsLds = 152 * 1024;
constexpr int kFusedStatsLdsSmall = 79 * 1024;
inline size_t fused_stats_bytes(int32_t slot_capacity, int32_t group) {
  return (size_t)(slot_capacity / 32) * group * (32 * 2 + 4);
}

hipError_t launch_read_probe(const void* src, int64_t bytes, uint32_t* checksum, int cu_count, hipStream_t stream);
hipError_t launch_heavy_retire(const HeavyArgs& a, hipStream_t stream);
hipError_t launch_heavy_accumulate(const HeavyArgs& a, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_chunk_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_plan(int32_t num_q, int32_t num_k, int32_t prefix_len, int32_t window,
                               int64_t kv_start, int32_t bm, int32_t bn, int32_t* tiles,
                               int32_t max_tiles, int32_t* num_tiles, hipStream_t stream);

// Tile shape of the prefill kernels for a dtype / head_dim.
void prefill_tile_shape(int32_t dtype, int32_t head_dim, int32_t* bm, int32_t* bn);

}  // namespace ps
