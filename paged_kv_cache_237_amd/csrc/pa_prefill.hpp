// Interface of the prefill kernels (prefill.hip) to the host layer: the
// launch arguments and the launcher.  Kept apart from the other kernels'
// interfaces so that the prefill's code depends on this header alone.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_common.hpp"

namespace pa {

struct PrefillArgs {
  const uint16_t* q;
  const uint4* k_cache;
  const uint4* v_cache;
  const int32_t* block_table;
  const int32_t* cu_q;
  const int32_t* ctx_lens;
  uint16_t* out;
  int64_t num_blocks;
  int batch;
  int hq;
  int hkv;
  int mbps;
  int max_q;
  float scale_log2;
  // context split (see prefill.hip): a query block of more than split_tiles
  // key tiles is cut into up to max_splits parts merged through the records
  int split_tiles;
  int max_splits;
  int64_t total_q;   // rows the records are sized for
  float* rec_ml;     // [max_splits][total_q][hq][2] (m, l)
  float* rec_o;      // [max_splits][total_q][hq][kDim] unnormalised outputs
  // Plan of a ragged launch (null: grid order, the host's split), written by
  // the plan kernel on the same stream: plan[0] = number of workgroup items
  // n, plan[1] = the part length in tiles (split_tiles is then its minimum),
  // plan[2] = number of cut blocks; plan[kPlanHeader + k], k < n, = the k-th
  // longest item as (b * nqb_max + jrev) * 16 + part (max_splits <= 16).
  // plan_rec[b * nqb_max + jrev] = first record slot of a cut block (a slot
  // holds kRowsPerWG rows per kv head; rec_ml / rec_o are then indexed by
  // (slot * hkv + g) * kRowsPerWG + row); plan_cnt[slot * hkv + g] = the
  // arrival counter of cut block (first slot, kv head g).
  int32_t* plan;
  int32_t* plan_rec;
  int32_t* plan_cnt;
  int plan_items;  // items the plan's grid has room for
  int slots;       // workgroup slots the part length is shared over
};

// Query rows per prefill workgroup.
constexpr int kPrefillRows = 128;
// int32 words before the plan's item list (the count, padded to 256 B).
constexpr int kPlanHeader = 64;
// A plan's part length is the launch's tiles per slot divided by this; its
// cut blocks then have fewer than 2 * kPlanShareDiv * slots / hkv parts.
// Half the share (2) was slower on every ragged batch measured (chunked
// prefill mixed with decode rows 268.7 -> 303.3 us): more, shorter parts
// and merges for no shorter critical path.
constexpr int kPlanShareDiv = 1;

hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t s);

}  // namespace pa
