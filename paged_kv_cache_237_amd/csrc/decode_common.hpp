// Work-list machinery shared by the decode kernels (decode.hip: one or a few
// query rows per (sequence, kv head) on the vector ALUs; decode_mfma.hip:
// up to 32 rows on the matrix cores): context clamping, wave-uniform scalar
// loads, the flattened tile list and its cut into per-wave runs (weighted by
// XCD), the wave that owns a tile, query-row addressing of virtual heads,
// coherent accesses to the partial records, and the waves' progress hints.
#pragma once

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int n) {
  const int cap = a.mbps * kBlock;
  return n < 0 ? 0 : (n > cap ? cap : n);
}

__device__ __forceinline__ int tiles_of(int n) { return (n + kTile - 1) / kTile; }

// Positions streamed from the cache: all of them, or all but the appended one.
template <bool Append>
__device__ __forceinline__ int stream_ctx(const DecodeArgs& a, int n) {
  const int c = clamp_ctx(a, n);
  return Append ? (c > 0 ? c - 1 : 0) : c;
}

// Load of a value the kernel never writes (block table, context lengths) at a
// wave-uniform index, through the constant address space: it becomes a
// scalar load, which is counted apart from the vector loads of K and V, so
// waiting for it does not wait for the tile loads in flight.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int64_t i) {
  using cint = const __attribute__((address_space(4))) int32_t;
  return ((cint*)p)[i];
}

// Query/output row of virtual head v of segment (b, g), and whether it is a
// real query row (not padding).  Without the causal rows (one query row per
// sequence) the G heads of a kv head are simply contiguous.
template <int G, bool Causal>
__device__ __forceinline__ int64_t vrow(const DecodeArgs& a, int b, int g, int v) {
  if constexpr (!Causal) return (int64_t(b) * a.hkv + g) * G + v;
  return (int64_t(b) * a.ql + (v >> a.gr_shift)) * a.hq + int64_t(g) * a.gr + (v & (a.gr - 1));
}
template <bool Causal>
__device__ __forceinline__ bool vreal(const DecodeArgs& a, int v) {
  return !Causal || (v >> a.gr_shift) < a.ql;
}

// Progress counters of a workgroup's waves (LDS), read by the other waves of
// the workgroup as a scheduling hint: relaxed atomics at workgroup scope
// (plain LDS accesses in the generated code).
__device__ __forceinline__ void prog_set(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ int prog_get(int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Tiles per sequence of the first 64 sequences (lane = sequence), their
// inclusive scan, and the number of tiles of all segments (identical in every
// lane); `locate` reuses the first 64 from registers.
struct TileScan {
  int nt, incl, total;
};

template <bool Append>
__device__ TileScan scan_tiles(const DecodeArgs& a) {
  const int lane = lane_id();
  TileScan sc;
  sc.nt = lane < a.batch ? tiles_of(stream_ctx<Append>(a, a.ctx_lens[lane])) : 0;
  sc.incl = wave_incl_scan(sc.nt);
  int tot = __builtin_amdgcn_readlane(sc.incl, kWave - 1);
  for (int b0 = kWave; b0 < a.batch; b0 += kWave) {
    const int b = b0 + lane;
    const int nt = b < a.batch ? tiles_of(stream_ctx<Append>(a, a.ctx_lens[b])) : 0;
    tot += wave_sum_i(nt);
  }
  sc.total = tot * a.hkv;
  return sc;
}

// Sequence holding tile `pos` of the flattened list and the tiles of all
// sequences before it.
template <bool Append>
__device__ void locate(const DecodeArgs& a, const TileScan& sc, int pos, int& b_out, int& before_out) {
  const int lane = lane_id();
  int base = 0;
  for (int b0 = 0; b0 < a.batch; b0 += kWave) {
    const int b = b0 + lane;
    const int nt = b0 == 0 ? sc.nt : (b < a.batch ? tiles_of(stream_ctx<Append>(a, a.ctx_lens[b])) : 0);
    const int incl = b0 == 0 ? sc.incl : wave_incl_scan(nt);
    const int tot = __builtin_amdgcn_readlane(incl, kWave - 1);
    if (pos < (base + tot) * a.hkv) {
      const uint64_t hit = __ballot((base + incl) * a.hkv > pos);
      const int l = __ffsll((unsigned long long)hit) - 1;
      b_out = b0 + l;
      before_out = base + __builtin_amdgcn_readlane(incl - nt, l);
      return;
    }
    base += tot;
  }
  b_out = a.batch;
  before_out = base;
}

// The runs.  Waves are numbered block * NW + wave-in-block, and block b runs
// on XCD b % 8.  A wave on an even-numbered XCD weighs run_w_even, one on an
// odd-numbered XCD run_w_odd; with W(w) the summed weight of waves 0 .. w-1
// and S = W(n_waves), wave w streams tiles [total*W(w)/S, total*W(w+1)/S)
// (rounded down), so run lengths follow the weights to within one tile.
// That is used only when every run of waves 0 .. n_waves-1 holds at least one
// tile (total * min weight >= S): the merge expects an arrival from every
// wave between the first and the last run of a cut segment.  Otherwise (fewer
// tiles than waves, roughly) the tiles are cut into runs of `per` =
// ceil(total / n_waves), empty only at the end.
struct Runs {
  int64_t total;
  int64_t sum;  // S
  int n_waves, we, wo;
  int per;      // > 0: equal runs of per tiles
};

// W(w): blocks alternate even, odd XCD, so a pair of blocks weighs NW*(we+wo).
template <int NW>
__device__ __forceinline__ int64_t run_weight_before(const Runs& r, int w) {
  const int blk = w / NW, wv = w - blk * NW;
  const int64_t s = int64_t(blk >> 1) * NW * (r.we + r.wo);
  return (blk & 1) ? s + int64_t(NW) * r.we + int64_t(wv) * r.wo : s + int64_t(wv) * r.we;
}

template <int NW>
__device__ __forceinline__ Runs make_runs(const DecodeArgs& a, int total) {
  Runs r;
  r.total = total;
  r.n_waves = a.n_waves;
  r.we = a.run_w_even;
  r.wo = a.run_w_odd;
  r.sum = run_weight_before<NW>(r, a.n_waves);
  r.per = int64_t(total) * min(r.we, r.wo) >= r.sum ? 0 : (total + a.n_waves - 1) / a.n_waves;
  return r;
}

template <int NW>
__device__ __forceinline__ int run_start(const Runs& r, int w) {
  if (r.per > 0) return int(min(int64_t(w) * r.per, r.total));
  return w >= r.n_waves ? int(r.total) : int(r.total * run_weight_before<NW>(r, w) / r.sum);
}

// The wave whose run holds tile `tile` (< total).  Weighted runs: the largest
// w with total*W(w)/S <= tile, i.e. W(w) <= V = ((tile+1)*S - 1) / total,
// found by inverting W piecewise.
template <int NW>
__device__ __forceinline__ int wave_of(const Runs& r, int tile) {
  if (r.per > 0) return tile / r.per;
  const int64_t v = ((int64_t(tile) + 1) * r.sum - 1) / r.total;
  const int64_t pair = int64_t(NW) * (r.we + r.wo);
  const int64_t p = v / pair;
  const int64_t rest = v - p * pair;
  return int(rest < int64_t(NW) * r.we ? (2 * p) * NW + rest / r.we
                                       : (2 * p + 1) * NW + (rest - int64_t(NW) * r.we) / r.wo);
}

// Loads of K/V tiles, which a decode reads exactly once: with the
// non-temporal cache policy (the NT bit) the lines are not kept for reuse.
// Measured against the default policy (same kernels, bit-identical outputs,
// one box, interleaved): 8 x 131,072-token decode step 717.7 -> 638.6 us,
// Qwen3-0.6B shape 120.6 -> 106.7 us, Qwen3-4B shape 635.4 -> 561.7 us.  The
// prefill, whose query blocks reuse each tile from L2, keeps the default
// (the NT bit made it 17 % slower).
constexpr int kCpolStream = 2;  // NT in the buffer builtins' cache-policy operand

__device__ __forceinline__ uint4 buf_load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), kCpolStream);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Partial records cross XCDs (each XCD has its own L2), so they are written
// and read at agent scope, which the hardware keeps coherent by itself (no
// whole-L2 writeback or invalidate is needed, unlike a device-scope fence).
// On gfx950 an agent-scope access is an ordinary one with the SC1 cache-policy
// bit: single words go through relaxed agent-scope atomics, and the O vectors
// through 16- and 8-byte buffer accesses that carry the same bit (a record is
// padded to a multiple of 16 bytes), one transaction per chunk instead of one
// per word.
constexpr int kCpolAgent = 16;  // SC1 in the buffer builtins' cache-policy operand

__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Four floats at byte offset off of the record (16-byte aligned).
__device__ __forceinline__ void st_coherent4(__amdgpu_buffer_rsrc_t rec, uint32_t off, float x, float y,
                                             float z, float w) {
  const u32x4_t v = {__float_as_uint(x), __float_as_uint(y), __float_as_uint(z), __float_as_uint(w)};
  __builtin_amdgcn_raw_buffer_store_b128(v, rec, int(off), 0, kCpolAgent);
}
// Two floats at byte offset off of the record (8-byte aligned).
__device__ __forceinline__ void ld_coherent2(__amdgpu_buffer_rsrc_t rec, uint32_t off, float& x, float& y) {
  typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(rec, int(off), 0, kCpolAgent);
  const unsigned lo = v.x, hi = v.y;
  x = __uint_as_float(lo);
  y = __uint_as_float(hi);
}

}  // namespace pa
