// Whole-block copies inside the paged cache (gfx950).
//
// What it computes (CSDN essay comparing nanoVLLM and vLLM, first section:
// blocks are allocated and shared per sequence through the block table, and
// vLLM can preempt a sequence by moving its KV cache out of GPU memory and
// back): for every pair (src, dst), block dst of the K cache and of the V
// cache, all kv heads, receives a bit copy of block src.  This is the
// copy-on-write step when a shared block is about to be extended by one of
// its owners.
//
// Mapping: one workgroup per (pair, kv head, K or V): a block-head is one
// contiguous 64 KiB tile in both caches, copied as 16 loads of 16 bytes per
// thread, all issued before the stores, with the non-temporal cache policy.  Pairs with an index outside the pool
// (e.g. -1 padding) or with src == dst are skipped.  A pure copy, bound by
// HBM bandwidth (64 KiB read + 64 KiB written per workgroup).
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

// Copies read and write each byte once: non-temporal loads and stores (the NT
// cache policy) keep the copied blocks from displacing reusable lines;
// measured 512 block pairs 217.6 -> 208.2 us (one box, interleaved).  (The
// store of new tokens, whose lines a decode reads right after, stays on the
// default policy: NT made it slower, 26.5 -> 38.2 us for 16,384 tokens.)
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 nt_load(const uint4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_store(const uint4& v, uint4* p) {
  const nt_u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, reinterpret_cast<nt_u32x4*>(p));
}

constexpr int kTileChunks = kBlock * kChunks;  // 16-byte chunks of a block-head: 4096

__global__ __launch_bounds__(256) void copy_blocks_kernel(CopyBlocksArgs a) {
  const int64_t p = blockIdx.x;
  const int g = blockIdx.y;
  const int src = a.pairs[2 * p];
  const int dst = a.pairs[2 * p + 1];
  if (src < 0 || dst < 0 || int64_t(src) >= a.num_blocks || int64_t(dst) >= a.num_blocks ||
      src == dst)
    return;
  uint4* base = blockIdx.z == 0 ? a.k_cache : a.v_cache;
  const uint4* s = base + (int64_t(src) * a.hkv + g) * kTileChunks + threadIdx.x;
  uint4* d = base + (int64_t(dst) * a.hkv + g) * kTileChunks + threadIdx.x;
  uint4 c[kTileChunks / 256];
#pragma unroll
  for (int j = 0; j < kTileChunks / 256; ++j) c[j] = nt_load(s + 256 * j);
#pragma unroll
  for (int j = 0; j < kTileChunks / 256; ++j) nt_store(c[j], d + 256 * j);
}

hipError_t launch_copy_blocks(const CopyBlocksArgs& a, hipStream_t s) {
  const dim3 grid(unsigned(a.n_pairs), unsigned(a.hkv), 2u);
  hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
