// Reset PE with the keys re-rotated on every step (see reset_pe.hip).
#pragma once

#include "ps_internal.h"

namespace ps {

struct ResetArgs {
  CacheGeom geom;            // contiguous cache
  int32_t dtype;
  int32_t num_seqs;
  const void* k_cache;       // un-rotated keys
  const int32_t* prefix_len;
  const int64_t* pos;
  RopeFreq rope;
  void* table;               // [slot_capacity][head_dim / 2] cos, sin of each renumbered position:
                             // an fp16 pair (bf16 keys) or an fp32 pair (fp32 keys)
  void* k_out;               // keys rotated at their renumbered positions, same layout as the cache
  int64_t* pos_out;          // [num_seqs] renumbered query position min(p, L + W - 1)
};

hipError_t launch_reset_rerotate(const ResetArgs& a, hipStream_t stream);

}  // namespace ps
