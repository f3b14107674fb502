// Slot-mapped store of new keys/values into the paged cache (gfx950).
//
// What it computes: for each new token i with slot s = slot_mapping[i] >= 0,
// the bits of k_new[i][g][:] and v_new[i][g][:] go to row s % 256 of
// physical block s / 256, for every kv head g (nano-vllm hub page,
// "Attention + Triton Kernel": a slot mapping writes new K/V into
// preallocated blocks; "KV Cache block management": 256-token blocks).
//
// Mapping: one workgroup per (64 consecutive tokens, kv head).  K is stored
// as 16-byte chunks [chunk][row][8], so with lane = token the 64 lanes of a
// wave write one contiguous KiB per chunk whenever the slots are consecutive
// (the usual case when a prompt fills its blocks).  V rows are 256 contiguous
// bytes: 16 lanes copy one row, 4 rows per wave instruction.  A pure copy,
// bound by HBM bandwidth; slots outside the pool are skipped.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

__global__ __launch_bounds__(256) void store_kv_kernel(StoreArgs a) {
  const int g = blockIdx.y;
  const int64_t i0 = int64_t(blockIdx.x) * kTile;
  const int lane = lane_id();
  const int wv = threadIdx.x >> 6;

  // K: lane = token, this wave copies chunks 4*wv .. 4*wv+3 of every token.
  {
    const int64_t i = i0 + lane;
    const int slot = i < a.n ? a.slots[i] : -1;
    if (slot >= 0 && int64_t(slot) < a.num_slots) {
      const int64_t blk = slot / kBlock;
      const int row = slot % kBlock;
      const uint4* src = a.k_new + (i * a.hkv + g) * kChunks + wv * 4;
      uint4* dst = a.k_cache + ((blk * a.hkv + g) * kChunks + wv * 4) * kBlock + row;
      const uint4 c0 = src[0], c1 = src[1], c2 = src[2], c3 = src[3];
      dst[0 * kBlock] = c0;
      dst[1 * kBlock] = c1;
      dst[2 * kBlock] = c2;
      dst[3 * kBlock] = c3;
    }
  }
  // V: 16 lanes per token row; this wave copies tokens 16*wv .. 16*wv+15.
  uint4 vals[4];
  int64_t dsts[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = wv * 16 + j * 4 + (lane >> 4);
    const int64_t i = i0 + r;
    const int slot = i < a.n ? a.slots[i] : -1;
    dsts[j] = -1;
    if (slot >= 0 && int64_t(slot) < a.num_slots) {
      const int64_t blk = slot / kBlock;
      const int row = slot % kBlock;
      vals[j] = a.v_new[(i * a.hkv + g) * kChunks + (lane & 15)];
      dsts[j] = ((blk * a.hkv + g) * kBlock + row) * kChunks + (lane & 15);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (dsts[j] >= 0) a.v_cache[dsts[j]] = vals[j];
}

hipError_t launch_store_kv(const StoreArgs& a, hipStream_t s) {
  const dim3 grid(unsigned((a.n + kTile - 1) / kTile), unsigned(a.hkv));
  hipLaunchKernelGGL(store_kv_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
