// Pieces shared by the matrix-core decode kernels (decode_mfma.hip: 17..32
// rows per (sequence, kv head) on v_mfma_f32_32x32x16_bf16;
// decode_mfma16.hip: 5..16 rows on v_mfma_f32_16x16x32_bf16): a tile's
// buffer descriptors, the V loads and their LDS store, the transposing reads
// that gather a B operand from that store, and the walk of a wave's run over
// the flattened tile list.  Both kernels read K and V in 64-token tiles with
// the non-temporal policy and keep V in LDS as it arrives, one row per token.
#pragma once

#include "decode_common.hpp"

namespace pa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

constexpr float kMfLazy = 8.f;    // log2 headroom before O is rescaled
constexpr uint32_t kMfOnePair = 0x3F803F80u;  // (1.0, 1.0) in bf16

__device__ __forceinline__ bf16x8_t as_bf8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

// Compiler-level ordering of one wave's LDS accesses (the hardware keeps a
// wave's LDS operations in order; the V tile is written and read through
// differently typed pointers and builtins).
__device__ __forceinline__ void lds_order() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

struct MfTile {
  __amdgpu_buffer_rsrc_t rk, rv;
  int r0, valid;  // first row of the tile in its block; tokens inside the context
};

// Tile t of segment (sequence, kv head g) whose block-table entry is phys:
// buffer descriptors whose ranges end at the block-head tile (K) and after
// the last valid row (V), so rows past the context load zeros (the cache may
// hold NaN patterns there).  A bad entry (or the "next tile" past a run's
// end, phys = -1) gives no valid row.
__device__ __forceinline__ MfTile mf_tile(const DecodeArgs& a, int phys, int g, int t, int ctx) {
  MfTile tl;
  const bool ok = phys >= 0 && int64_t(phys) < a.num_blocks;
  tl.valid = ok ? min(kTile, ctx - t * kTile) : 0;
  tl.r0 = (t & 3) * kTile;
  const int64_t bh = (ok ? int64_t(phys) : 0) * a.hkv + g;
  tl.rk = make_rsrc(a.k_cache + bh * (kChunks * kBlock), 65536u);
  tl.rv = make_rsrc(a.v_cache + bh * (kBlock * kChunks), uint32_t(tl.r0 + tl.valid) * 256u);
  return tl;
}

// V rows of a tile: vr[4 j + i] = chunk (lane & 15) of token
// 16 j + 4 (lane >> 4) + i (16 lanes read one 256-byte row).
__device__ __forceinline__ void mf_issue_v(const MfTile& tl, uint4 (&vr)[16]) {
  const int lane = lane_id();
  const uint32_t base = (uint32_t(tl.r0 + 4 * (lane >> 4)) * kChunks + uint32_t(lane & 15)) * 16u;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[4 * j + i] = buf_load16_stream(tl.rv, base + uint32_t(16 * j + i) * 256u, 0u);
}

// The V rows of mf_issue_v into LDS as they are: token t at row t, Stride
// bf16 per row, one 16-byte store per chunk.
template <int Stride>
__device__ __forceinline__ void mf_store_v_rows(uint16_t* v, const uint4 (&vr)[16]) {
  const int lane = lane_id();
  const int ch = lane & 15;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(v + (16 * j + 4 * (lane >> 4) + i) * Stride + 8 * ch) = vr[4 * j + i];
}

// A B operand of 8 keys gathered from V rows in LDS by two transposing reads
// (ds_read_b64_tr_b16): in each 16-lane group, lane i receives element i % 4
// of the 4 bf16 that lanes i / 4, 4 + i / 4, 8 + i / 4 and 12 + i / 4 point
// at.  With lane s pointing at dims 4 (s % 4) .. + 3 (past a common base) of
// key s / 4, lane i receives dim i of keys 0 .. 3; the second read, `apart`
// bf16 further, gives keys 4 .. 7 of the operand.
__device__ __forceinline__ bf16x8_t tr_read_pair(const uint16_t* p, int apart) {
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(p + apart));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// A tile of the flattened list as a wave's stream sees it (wave-uniform):
// its segment (b, g), index t of nt in the segment, the context, the block
// holding it; live when it belongs to the run (and the batch).
struct MfCur {
  int b, g, t, nt, ctx, phys;
  bool live;
};

// The tile after c: the next one of its segment or the first of the next
// non-empty segment; live only when in_run (it is still inside the run).
__device__ __forceinline__ MfCur mf_next(const DecodeArgs& a, const MfCur& c, bool in_run) {
  MfCur n = c;
  n.live = false;
  n.phys = -1;
  if (!c.live || !in_run) return n;
  n.t = c.t + 1;
  if (n.t == c.nt) {
    n.t = 0;
    if (++n.g == a.hkv) {
      n.g = 0;
      do {
        n.b = __builtin_amdgcn_readfirstlane(n.b + 1);
        n.ctx = n.b < a.batch ? clamp_ctx(a, ld_uniform(a.ctx_lens, n.b)) : 0;
        n.nt = n.b < a.batch ? tiles_of(n.ctx) : 1;
      } while (n.nt == 0);
    }
  }
  n.live = n.b < a.batch;
  if (n.live) n.phys = ld_uniform(a.block_table, int64_t(n.b) * a.mbps + (n.t >> 2));
  return n;
}

}  // namespace
}  // namespace pa
