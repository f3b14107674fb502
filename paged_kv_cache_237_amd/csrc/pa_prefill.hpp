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
  // Longest-first dispatch (null: grid order).  plan[0] = number of
  // workgroup items n; plan[kPlanHeader + k], k < n, = the k-th longest
  // (sequence, part, query block) as jrev * batch * max_splits + b *
  // max_splits + part.  Written by the plan kernel on the same stream.
  int32_t* plan;
};

// Query rows per prefill workgroup.
constexpr int kPrefillRows = 128;
// int32 words before the plan's item list (the count, padded to 256 B).
constexpr int kPlanHeader = 64;

hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t s);

}  // namespace pa
