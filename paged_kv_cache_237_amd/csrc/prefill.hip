// Causal varlen prefill attention over the paged cache, on gfx950 MFMA.
//
// What it computes (nano-vllm hub page, "Scheduler": prefill runs the prompt
// and fills the cache; CSDN essay comparing nanoVLLM and vLLM, third section:
// exact attention in on-chip tiles, and the vLLM reading section: prefill is
// the compute-bound phase with its own kernel): for query row i of sequence b,
// at position a = ctx_b - q_len_b + i, o = softmax(scale * q K[0..a]^T) V[0..a]
// per head, with K/V read through the sequence's block table.
//
// One workgroup = 4 waves = 128 query rows (G heads x 128/G positions) of one
// (sequence, kv head), so every K/V tile staged in LDS serves all G heads.
// Tiles of 64 keys never straddle a 256-token block (one table lookup each).
// A tile's K and V go straight from memory into LDS (buffer_load ... lds, no
// registers on the way), two LDS buffers deep: tile t+1 is in flight while
// tile t is computed.
// Per wave and tile (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   S^T = K Q^T : A = K rows from LDS (16 B per lane, the cache's 8-dim chunks),
//                 B = the wave's 32 query rows, held in registers for the whole
//                 loop.  The accumulator then holds one query row per lane
//                 (column) and 16 keys per register set, so row max and row
//                 sum are in-lane plus one exchange with lane^32.
//   O  = P V    : A = bf16(P) taken straight from the S^T accumulator -- the
//                 contraction runs over keys in the accumulator's register
//                 order (per 16 keys, lane half h holds keys 4h..4h+3 and
//                 8+4h..8+4h+3), so P never moves between lanes.  V is kept
//                 in LDS as it is in the cache ([key][dim], 256-byte rows
//                 whose 16-byte chunks are XOR-rotated by 4 (key mod 4)), and
//                 a lane's B operand -- its dim of those 8
//                 keys -- is gathered by two transposing LDS reads
//                 (ds_read_b64_tr_b16: in each 16-lane group, lane j points
//                 at 4 dims of key j / 4 and receives dim j % 4 of the
//                 group's 4 keys, so the group holds 16 dims x 4 keys).
// Query blocks of at most 16 rows (a sequence with q_len x G <= 16) take a
// separate path, described at prefill_short below.
//
// Online softmax in the log2 domain (scale*log2 e folded into one FMA) with a
// lazy rescale: the reference max only moves when a row's max grows by more
// than 2^8, so O is rescaled rarely.  Tiles entirely above a wave's diagonal
// are skipped; only tiles crossing it are masked.  Keys past the context are
// loaded as zeros through raw-buffer range checks (the cache may hold NaN
// patterns there).  Workgroups are dispatched longest-first: grid z counts
// query blocks from the end of each sequence.
//
// Context split: a query block whose keys span more than split_tiles tiles
// (a long cached prefix) is cut into nsplit = ceil(tiles / split_tiles) key
// ranges of near-equal length, one workgroup each, so that no workgroup
// streams a very long context alone (grid x = sequence * max_splits + part).
// Each part leaves its rows' unnormalised state (m, l, O) in the workspace
// records, and a second, small kernel on the same stream merges them:
// M = max m_i, L = sum 2^(m_i - M) l_i, o = sum 2^(m_i - M) O_i / L (the same
// split-context identity as decode), taken part by part with an online
// rescale.  The kernel boundary makes the records visible, so both sides use
// ordinary cached accesses.
#include <math.h>

#include "pa_device.hpp"
#include "pa_prefill.hpp"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef short v8i16_t __attribute__((ext_vector_type(8)));

constexpr int kRowsPerWG = kPrefillRows;  // query rows (head, position) per workgroup: 32 per wave
constexpr int kKeys = 64;        // keys per K/V tile
constexpr int kVStride = kDim;   // bf16 per V row (one key) in LDS
constexpr float kLazyRescale = 8.f;  // log2 headroom before O is rescaled
constexpr uint32_t kBf16OnePair = 0x3F803F80u;  // (1.0, 1.0) in bf16

// LDS: two K tiles and two V tiles; tile t is read from buffer t&1 while
// tile t+1 is written into the other.  V row `key` holds dims 8 c .. 8 c + 7
// in 16-byte chunk c ^ 4 (key & 3): the 4 keys that a 16-lane transposing
// read spans then sit on 4 different quarters of the banks.
struct __align__(16) PrefillLds {
  uint4 k[2][kChunks * kKeys];       // [buf][chunk][key] 16-byte chunks: 2 x 16 KiB
  uint16_t v[2][kKeys * kVStride];   // [buf][key][rotated chunk][8] bf16: 2 x 16 KiB
  float rowf[4][32];                 // per-wave row factors
};
static_assert(sizeof(PrefillLds) >= 4 * 32 * kDim * 2, "epilogue staging fits");

__device__ __forceinline__ bf16x8_t as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint4 zero4() { return make_uint4(0, 0, 0, 0); }

struct TileGeom {
  __amdgpu_buffer_rsrc_t rk, rv;
  int r0, valid;
};

__device__ __forceinline__ TileGeom tile_geom(const PrefillArgs& a, const int32_t* table, int g,
                                              int ctx, int t) {
  const int key0 = t * kKeys;
  // a scalar load (the LDS-DMA writes would otherwise keep the compiler
  // from proving the table unchanged, and it would use a vector load)
  const int phys = ((const __attribute__((address_space(4))) int32_t*)table)[key0 / kBlock];
  const bool ok = phys >= 0 && int64_t(phys) < a.num_blocks;
  TileGeom tg;
  tg.valid = ok ? min(kKeys, ctx - key0) : 0;
  tg.r0 = key0 % kBlock;
  const int64_t bh = (ok ? int64_t(phys) : 0) * a.hkv + g;
  tg.rk = make_rsrc(a.k_cache + bh * (kChunks * kBlock), 65536u);
  // keys past the context load zeros (the cache may hold NaN patterns there)
  tg.rv = make_rsrc(a.v_cache + bh * (kBlock * kChunks), uint32_t(tg.r0 + tg.valid) * 256u);
  return tg;
}

// Tile t straight into the LDS buffers kbuf / vbuf.  In buffer_load ... lds,
// lane l of an instruction writes its 16 bytes at the instruction's LDS base
// + 16 l, and lanes outside the buffer's range write zeros (keys past the
// context: the cache may hold NaN patterns there).  Wave w of 4 takes K
// chunks w + 4 j (lane = key: 1 KiB of [chunk][key] per instruction) and V
// rows 16 w + 4 i .. + 3 (16 lanes per 256-byte row, lane l reading the
// chunk that belongs at position l % 16 of its rotated row).  The waves
// wait for these with s_waitcnt vmcnt(0) and a barrier before reading.
__device__ __forceinline__ void dma_tile(const PrefillArgs& a, const int32_t* table, int g, int ctx, int t,
                                         int w, int lane, uint4* kbuf, uint16_t* vbuf) {
  const TileGeom tg = tile_geom(a, table, g, ctx, t);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ch = w + 4 * j;
    const uint32_t off = lane < tg.valid ? uint32_t(ch * kBlock + tg.r0 + lane) * 16u : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tg.rk, (__attribute__((address_space(3))) void*)(kbuf + ch * kKeys),
                                             16, off, 0, 0, 0);
  }
  const int c = (lane & 15) ^ (4 * (lane >> 4));  // row 16 w + 4 i + l / 16 has key & 3 = l / 16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row0 = 16 * w + 4 * i;
    const uint32_t off = uint32_t((tg.r0 + row0 + (lane >> 4)) * kChunks + c) * 16u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(tg.rv, (__attribute__((address_space(3))) void*)(vbuf + row0 * kVStride),
                                             16, off, 0, 0, 0);
  }
}

// Geometry of query block jrev (counted from the end) of sequence b, shared
// by the attention and merge kernels so that both agree on every split.
template <int G>
struct BlockGeom {
  int q0, qlen, ctx, nqb, p0, shift, ntiles, nsplit;

  // split_tiles: the launch's part length (the host's, or the plan's)
  __device__ __forceinline__ BlockGeom(const PrefillArgs& a, int b, int jrev, int split_tiles) {
    constexpr int QB = kRowsPerWG / G;
    q0 = a.cu_q[b];
    qlen = max(0, a.cu_q[b + 1] - q0);
    ctx = min(max(a.ctx_lens[b], 0), a.mbps * kBlock);
    nqb = (qlen + QB - 1) / QB;
    p0 = (nqb - 1 - jrev) * QB;
    shift = ctx - qlen;  // absolute position of query row 0
    // keys the whole block needs
    const int last_row = min(p0 + QB, qlen) - 1;
    const int kend = min(shift + last_row + 1, ctx);
    ntiles = kend > 0 ? (kend + kKeys - 1) / kKeys : 0;
    // records exist only when they are sized for every row
    nsplit = ntiles > split_tiles ? min((ntiles - 1) / split_tiles + 1, a.max_splits) : 1;
    if (nsplit > 1 && a.plan == nullptr && int64_t(a.cu_q[a.batch]) > a.total_q) nsplit = 1;
  }
};

template <int G>
__device__ __forceinline__ int nqb_max_of(const PrefillArgs& a) {
  constexpr int QB = kRowsPerWG / G;
  return (a.max_q + QB - 1) / QB;
}

// The launch's part length: the host's, or the one the plan chose on the
// device (wave-uniform).
__device__ __forceinline__ int split_tiles_of(const PrefillArgs& a) {
  return a.plan != nullptr ? __builtin_amdgcn_readfirstlane(a.plan[1]) : a.split_tiles;
}

// Record rows of query block (b, jrev) at kv head g, part `part`: in grid
// order, by query row and head, sized for max_splits parts of every row;
// with a plan, in the record slots the plan gave the block (plan_rec),
// kRowsPerWG rows per (slot, kv head).  rec_base is the wave-uniform row of
// the block's row 0 and rec_off the offset of its row R (head R / QB,
// position R % QB) from it, so that the records' buffer descriptors stay in
// scalar registers and the rows go into the per-lane offset.
template <int G>
__device__ __forceinline__ int64_t rec_base(const PrefillArgs& a, int b, int jrev, int g, int part, int q0,
                                            int p0) {
  if (a.plan != nullptr) {
    const int slot = a.plan_rec[b * nqb_max_of<G>(a) + jrev] + part;
    return (int64_t(slot) * a.hkv + g) * kRowsPerWG;
  }
  return (int64_t(part) * a.total_q + q0 + p0) * a.hq + g * G;
}
template <int G>
__device__ __forceinline__ int rec_off(const PrefillArgs& a, int R) {
  constexpr int QB = kRowsPerWG / G;
  return a.plan != nullptr ? R : (R % QB) * a.hq + R / QB;
}

// Records are written with the SC1 cache-policy bit (agent-coherent: not
// kept dirty in an XCD's private L2) and, where the last part of a block to
// finish merges them, read with it too.
constexpr int kCpolAgent = 16;
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Buffer descriptor of the records from p on (rows reached through the
// per-lane offset, a few MiB at most).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rec_rsrc(const float* p) {
  return make_rsrc(p, 0x7FFFFFF0u);
}

// One part of a split query block: its rows' (m, l, O) to the records.
template <int G>
__device__ void write_part(const PrefillArgs& a, int b, int jrev, int g, int part, int q0, int qlen, int p0,
                           const f32x16_t (&o)[4], float m, float ltot) {
  constexpr int QB = kRowsPerWG / G;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int col = lane & 31;
  const int half = lane >> 5;
  const int64_t base = rec_base<G>(a, b, jrev, g, part, q0, p0);
  const __amdgpu_buffer_rsrc_t rm = rec_rsrc(a.rec_ml + base * 2);
  const __amdgpu_buffer_rsrc_t ro = rec_rsrc(a.rec_o + base * kDim);
  const bool coherent = a.plan != nullptr;  // merged by the last part to finish
  // (m, l): lane (col, half 0) owns row w*32 + col
  {
    const int R = w * 32 + col;
    if (half == 0 && p0 + R % QB < qlen) {
      const u32x2_t v = {__float_as_uint(m), __float_as_uint(ltot)};
      const int off = rec_off<G>(a, R) * 8;
      if (coherent)
        __builtin_amdgcn_raw_buffer_store_b64(v, rm, off, 0, kCpolAgent);
      else
        __builtin_amdgcn_raw_buffer_store_b64(v, rm, off, 0, 0);
    }
  }
  // O: register 4*qd + i of o[n] is row 8*qd + 4*half + i of the wave, dim 32*n + col
#pragma unroll
  for (int qd = 0; qd < 4; ++qd)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int R = w * 32 + 8 * qd + 4 * half + i;
      if (p0 + R % QB < qlen) {
        const int off = rec_off<G>(a, R) * (kDim * 4) + 4 * col;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const unsigned v = __float_as_uint(o[n][4 * qd + i]);
          if (coherent)
            __builtin_amdgcn_raw_buffer_store_b32(v, ro, off + 128 * n, 0, kCpolAgent);
          else
            __builtin_amdgcn_raw_buffer_store_b32(v, ro, off + 128 * n, 0, 0);
        }
      }
    }
}

// Merge of 64 * H rows (from row 64 * r0) of split query block (b, jrev) at
// kv head g: thread (r8, d4) rows r0 * 64 + r8 + 8i (i < 8 H), dims 4*d4 ..
// +3.  The loads of one part for all the thread's rows are issued together,
// and those of part s + 1 before part s is folded in (online rescale, in
// part order).  Coherent: the records are read with SC1 loads (a merge by
// the last part to finish, in the same kernel as the other parts).
template <int G, int H, bool Coherent>
__device__ void merge_rows(const PrefillArgs& a, const BlockGeom<G>& bg, int b, int jrev, int g, int r0) {
  constexpr int QB = kRowsPerWG / G;
  constexpr int NR = 8 * H;  // rows per thread
  const int r8 = threadIdx.x >> 5, d4 = threadIdx.x & 31;
  int Rs[NR];
  bool ok[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    Rs[i] = 64 * r0 + r8 + 8 * i;
    ok[i] = bg.p0 + Rs[i] % QB < bg.qlen;
  }
  float M[NR], L[NR], acc[NR][4];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    M[i] = -INFINITY;
    L[i] = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[i][e] = 0.f;
  }
  struct Part {
    u32x2_t ml[NR];
    u32x4_t u[NR];
  };
  int offs[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) offs[i] = rec_off<G>(a, ok[i] ? Rs[i] : 0);
  auto load = [&](int s, Part& p) {
    const int64_t base = rec_base<G>(a, b, jrev, g, s, bg.q0, bg.p0);
    const __amdgpu_buffer_rsrc_t rm = rec_rsrc(a.rec_ml + base * 2);
    const __amdgpu_buffer_rsrc_t ro = rec_rsrc(a.rec_o + base * kDim);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      p.ml[i] = __builtin_amdgcn_raw_buffer_load_b64(rm, offs[i] * 8, 0, Coherent ? kCpolAgent : 0);
      p.u[i] = __builtin_amdgcn_raw_buffer_load_b128(ro, offs[i] * (kDim * 4) + 16 * d4, 0,
                                                     Coherent ? kCpolAgent : 0);
    }
  };
  Part cur, nxt;
  load(0, cur);
  for (int s = 0; s < bg.nsplit; ++s) {
    if (s + 1 < bg.nsplit) load(s + 1, nxt);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const unsigned m0 = cur.ml[i].x, l0 = cur.ml[i].y;
      const float pm = __uint_as_float(m0), pl = __uint_as_float(l0);
      const float mn = fmaxf(M[i], pm);
      if (mn == -INFINITY) continue;  // no visible key in any part so far
      const float fo = __builtin_amdgcn_exp2f(M[i] - mn);  // 0 while M is -inf
      const float fs = __builtin_amdgcn_exp2f(pm - mn);
      const unsigned x = cur.u[i].x, y = cur.u[i].y, z = cur.u[i].z, w = cur.u[i].w;
      L[i] = L[i] * fo + pl * fs;
      acc[i][0] = acc[i][0] * fo + __uint_as_float(x) * fs;
      acc[i][1] = acc[i][1] * fo + __uint_as_float(y) * fs;
      acc[i][2] = acc[i][2] * fo + __uint_as_float(z) * fs;
      acc[i][3] = acc[i][3] * fo + __uint_as_float(w) * fs;
      M[i] = mn;
    }
    if (s + 1 < bg.nsplit) cur = nxt;
  }
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    if (!ok[i]) continue;
    const int R = Rs[i];
    const float inv = L[i] > 0.f ? 1.f / L[i] : 0.f;
    // record row (q row, head) = output row
    const int64_t orow = (int64_t(bg.q0) + bg.p0 + R % QB) * a.hq + g * G + R / QB;
    uint2* dst = reinterpret_cast<uint2*>(a.out + orow * kDim + 4 * d4);
    *dst = make_uint2(pack_bf16x2(acc[i][0] * inv, acc[i][1] * inv),
                      pack_bf16x2(acc[i][2] * inv, acc[i][3] * inv));
  }
}

// Merge kernel of a launch in grid order (the host's split): workgroup
// (b, g, z) takes rows 64*(z&1) .. +63 of block z/2.  The kernel boundary
// makes the records visible.
template <int G>
__global__ __launch_bounds__(256) void prefill_merge_kernel(PrefillArgs a) {
  const int b = blockIdx.x, g = blockIdx.y;
  const int jrev = blockIdx.z >> 1, rhalf = blockIdx.z & 1;
  const BlockGeom<G> bg(a, b, jrev, a.split_tiles);
  if (jrev >= bg.nqb || bg.nsplit <= 1) return;
  merge_rows<G, 1, false>(a, bg, b, jrev, g, rhalf);
}

// With a plan, the parts of a cut block merge without a second kernel: each
// part, once its records are written, counts its arrival on the block's
// counter (zeroed by the plan kernel), and the last to arrive merges.  Why
// that part sees every record (the ordering the one-row decode relies on as
// well): every wave waits until its SC1 record stores are complete (s_waitcnt
// vmcnt(0)), the workgroup barrier follows, and only then is the arrival
// issued, an atomic performed at the memory side; the part that merges has
// seen every other arrival, hence every other part's completed stores, and
// it reads the records with SC1 loads, which do not hit a line another XCD's
// L2 may hold.
template <int G>
__device__ void arrive_and_merge(const PrefillArgs& a, const BlockGeom<G>& bg, int b, int jrev, int g) {
  __shared__ int last;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's record stores have completed
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0) {
    const int slot = a.plan_rec[b * nqb_max_of<G>(a) + jrev];
    const int prev = __hip_atomic_fetch_add(a.plan_cnt + slot * a.hkv + g, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
    last = prev == bg.nsplit - 1;
  }
  __syncthreads();
  if (!last) return;
  merge_rows<G, 1, true>(a, bg, b, jrev, g, 0);
  merge_rows<G, 1, true>(a, bg, b, jrev, g, 1);
}

// ---- short query blocks ----------------------------------------------------
// A sequence whose rows all fit 16 (q_len x G <= 16: decode rows and a few
// drafted tokens in a chunked-prefill batch) would leave most of a 128-row
// workgroup idle and stream its context one tile per workgroup round trip.
// Such a block takes its 16 rows (row v = token v / G, head v % G) as one
// 16-row block of v_mfma_f32_16x16x32_bf16 in every wave, and each wave
// streams a quarter of the part's key tiles on its own: K straight from
// memory into A operands (chunk 4 ks + j of token 16 ms + l % 16), V into
// the wave's own LDS rows and back through transposing reads in P's key
// order, the next tile's loads in flight while one is computed.  The four
// partial states (m, l, O) are then merged through LDS.  Such a block reads
// each tile once (its rows share one kv head), so its loads take the
// non-temporal policy, like the decode's.  Measured (one box, interleaved):
// chunked prefill mixed with 64 decode rows 273.3 -> 260.2 us, 64 x 4
// tokens 131.2 -> 115.9 us, 64 x 6 tokens 134.7 -> 122.0 us; the same path
// with the default policy gained 1 % or nothing (the rows were waiting on
// memory, not on the workgroup's bytes in flight).
constexpr int kShortRows = 16;
constexpr int kSVStride = 144;  // bf16 per V row in a wave's LDS (128 dims + pad, 288 B)
typedef float f32x4_t __attribute__((ext_vector_type(4)));
// A workgroup's dynamic LDS: the main path's buffers or the short path's
// four waves of V rows, whichever is larger.
constexpr size_t kShortLds = 4 * kKeys * kSVStride * 2 + 4 * 16 * 4;
constexpr size_t kPrefillLds = sizeof(PrefillLds) > kShortLds ? sizeof(PrefillLds) : kShortLds;
// A launch whose blocks are all short asks for more LDS than it uses, so
// that one workgroup runs per CU instead of two: its waves stream memory,
// and at that occupancy they did so faster (one box, interleaved: 64 x 4
// tokens 112.0 -> 110.6 us, 64 x 6 tokens 123.0 -> 120.6 us).
constexpr size_t kShortOnlyLds = 96 * 1024;
static_assert(kShortOnlyLds >= kPrefillLds && 2 * kShortOnlyLds > 160 * 1024, "one workgroup per CU");
static_assert(4 * (kShortRows * kDim + 2 * kShortRows) * 4 <= kPrefillLds, "short-path merge fits");

// A 16-byte load with the non-temporal cache policy (NT bit of the buffer
// builtins' cache-policy operand): the lines are not kept for reuse.
__device__ __forceinline__ uint4 ld16nt(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float xor16_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned a = r[0], b = r[1];
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

template <int G>
__device__ void prefill_short(const PrefillArgs& a, const BlockGeom<G>& bg, int b, int g, int part, int nsplit,
                              int t_begin, int t_end, unsigned char* lds_raw) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int q0 = bg.q0, qlen = bg.qlen, ctx = bg.ctx, shift = bg.shift;
  const int32_t* table = a.block_table + int64_t(b) * a.mbps;
  uint16_t* vbuf = reinterpret_cast<uint16_t*>(lds_raw) + w * (kKeys * kSVStride);
  float* rowf = reinterpret_cast<float*>(lds_raw + 4 * kKeys * kSVStride * 2) + 16 * w;
  const float c = fabsf(a.scale_log2);

  // this lane's score row (column of S^T): v = col
  const int tv = col / G, hv = col % G;
  const bool real = tv < qlen;
  const int lim = real ? min(shift + tv, ctx - 1) : -1;  // last visible key

  uint4 qop[4];
  {
    const uint4* src = reinterpret_cast<const uint4*>(
        a.q + (int64_t(q0) + (real ? tv : 0)) * (int64_t(a.hq) * kDim) + int64_t(g * G + hv) * kDim);
    const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 u = real ? src[4 * ks + grp] : zero4();
      u.x ^= flip;
      u.y ^= flip;
      u.z ^= flip;
      u.w ^= flip;
      qop[ks] = u;
    }
  }

  const int n = t_end - t_begin;
  const int w0 = t_begin + n * w / 4, w1 = t_begin + n * (w + 1) / 4;

  uint4 kr[16], vr[16];
  int valid = 0;
  auto issue = [&](int t) {
    const TileGeom tg = tile_geom(a, table, g, ctx, t);
#pragma unroll
    for (int ms = 0; ms < 4; ++ms) {
      const int key = 16 * ms + col;
      const uint32_t off = key < tg.valid ? uint32_t(tg.r0 + key) * 16u + uint32_t(grp) * 4096u : kOutOfRange;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kr[4 * ms + ks] = ld16nt(tg.rk, off + uint32_t(ks) * 16384u);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      vr[i] = ld16nt(tg.rv, uint32_t((tg.r0 + 4 * i + grp) * kChunks + col) * 16u);
    return tg.valid;
  };
  if (w0 < w1) valid = issue(w0);

  f32x4_t o[8];
#pragma unroll
  for (int nb = 0; nb < 8; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[nb][r] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int t = w0; t < w1; ++t) {
    const int key0 = t * kKeys;
    f32x4_t s[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[ms][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
        s[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kr[4 * ms + ks]), as_bf16x8(qop[ks]), s[ms], 0, 0, 0);
    // this tile's V into the wave's LDS rows, then the next tile's loads
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<uint4*>(vbuf + (4 * i + grp) * kSVStride + 8 * col) = vr[i];
    __builtin_amdgcn_wave_barrier();
    const int cur_valid = valid;
    if (t + 1 < w1) valid = issue(t + 1);

    // mask keys past the row's last visible key and past the context
    if (key0 + kKeys - 1 > lim || cur_valid < kKeys) {
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kk = 16 * ms + 4 * grp + r;
          s[ms][r] = (key0 + kk <= lim && kk < cur_valid) ? s[ms][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[ms][r]);
    mt = xor32_max(xor16_max(mt)) * c;
    const float mnew = fmaxf(m, mt);
    const bool need = mnew > m + kLazyRescale;
    if (__ballot(need) != 0) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;
      if (need) {
        l *= alpha;
        m = mnew;
      }
      if (grp == 0) rowf[col] = alpha;
      __builtin_amdgcn_wave_barrier();
      const float4 al = *reinterpret_cast<const float4*>(&rowf[4 * grp]);
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) {
        o[nb][0] *= al.x;
        o[nb][1] *= al.y;
        o[nb][2] *= al.z;
        o[nb][3] *= al.w;
      }
      __builtin_amdgcn_wave_barrier();
    }
    const float mref = m == -INFINITY ? 0.f : m;
    bf16x8_t pop[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float pf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = __builtin_amdgcn_exp2f(fmaf(s[2 * ks][e], c, -mref));
        pf[4 + e] = __builtin_amdgcn_exp2f(fmaf(s[2 * ks + 1][e], c, -mref));
      }
      const uint4 pb = pack8(pf);
      l = dot2_bf16(pb.x, kBf16OnePair, l);
      l = dot2_bf16(pb.y, kBf16OnePair, l);
      l = dot2_bf16(pb.z, kBf16OnePair, l);
      l = dot2_bf16(pb.w, kBf16OnePair, l);
      pop[ks] = as_bf16x8(pb);
    }
    // O += P V: lane (dim 16 nb + col, group grp) gathers keys 32 ks + 16 r +
    // 4 grp + {0..3} with transposing reads (lane col points at dims 4 (col &
    // 3) .. +3 of key 32 ks + 16 r + 4 grp + col / 4).  MFMA i = 8 ks + nb;
    // its operand is read kVAhead MFMAs ahead, in this fixed order (left to
    // itself, the compiler puts every operand in one register quad and waits
    // for each read right before its MFMA).
    const uint16_t* vsrc = vbuf + (4 * grp + (col >> 2)) * kSVStride + 4 * (col & 3);
    auto vop_of = [&](int i) {
      const int off0 = 32 * (i >> 3) * kSVStride + 16 * (i & 7);
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16_t*)(vsrc + off0));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16_t*)(vsrc + off0 + 16 * kSVStride));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    constexpr int kVAhead = 4;
    bf16x8_t vop[16];
#pragma unroll
    for (int i = 0; i < kVAhead; ++i) vop[i] = vop_of(i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + kVAhead < 16) vop[i + kVAhead] = vop_of(i + kVAhead);
      o[i & 7] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop[i >> 3], vop[i], o[i & 7], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_wave_barrier();
  }
  const float ltot = xor32_sum(xor16_sum(l));

  // ---- merge of the four waves' states through LDS ----
  __syncthreads();  // every wave is done with its V rows
  float* st = reinterpret_cast<float*>(lds_raw);
  constexpr int kSt = kShortRows * kDim + 2 * kShortRows;  // floats per wave: O, m, l
  {
    float* my = st + w * kSt;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb) my[(4 * grp + r) * kDim + 16 * nb + col] = o[nb][r];
    if (grp == 0) {
      my[kShortRows * kDim + col] = m;
      my[kShortRows * kDim + kShortRows + col] = ltot;
    }
  }
  __syncthreads();
  const int row = tid >> 4, d0 = 8 * (tid & 15);  // 16 rows x 16 groups of 8 dims
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < 4; ++k) M = fmaxf(M, st[k * kSt + kShortRows * kDim + row]);
  const float ref = M == -INFINITY ? 0.f : M;
  float L = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float f = __builtin_amdgcn_exp2f(st[k * kSt + kShortRows * kDim + row] - ref);
    L = fmaf(st[k * kSt + kShortRows * kDim + kShortRows + row], f, L);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(st[k * kSt + row * kDim + d0 + e], f, acc[e]);
  }
  const int rt = row / G, rh = row % G;
  if (nsplit > 1) {
    if (rt < qlen) {
      // the block's row R = head * QB + position, as the merge takes it
      const int64_t base = rec_base<G>(a, b, 0, g, part, q0, 0);
      const int off = rec_off<G>(a, rh * (kRowsPerWG / G) + rt);
      const __amdgpu_buffer_rsrc_t rm = rec_rsrc(a.rec_ml + base * 2);
      const __amdgpu_buffer_rsrc_t ro = rec_rsrc(a.rec_o + base * kDim);
      const int om = off * 8, oo = off * (kDim * 4) + 4 * d0;
      const u32x2_t v = {__float_as_uint(M), __float_as_uint(L)};
      const u32x4_t lo = {__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                          __float_as_uint(acc[3])};
      const u32x4_t hi = {__float_as_uint(acc[4]), __float_as_uint(acc[5]), __float_as_uint(acc[6]),
                          __float_as_uint(acc[7])};
      if (a.plan != nullptr) {  // merged by the last part to finish
        if ((tid & 15) == 0) __builtin_amdgcn_raw_buffer_store_b64(v, rm, om, 0, kCpolAgent);
        __builtin_amdgcn_raw_buffer_store_b128(lo, ro, oo, 0, kCpolAgent);
        __builtin_amdgcn_raw_buffer_store_b128(hi, ro, oo + 16, 0, kCpolAgent);
      } else {
        if ((tid & 15) == 0) __builtin_amdgcn_raw_buffer_store_b64(v, rm, om, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(lo, ro, oo, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(hi, ro, oo + 16, 0, 0);
      }
    }
    // every thread reaches the arrival's barriers
    if (a.plan != nullptr) arrive_and_merge<G>(a, bg, b, 0, g);
    return;
  }
  if (rt >= qlen) return;
  const int64_t orow = (int64_t(q0) + rt) * a.hq + g * G + rh;  // output row
  const float inv = L > 0.f ? 1.f / L : 0.f;
  uint4 val;
  val.x = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  val.y = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  val.z = pack_bf16x2(acc[4] * inv, acc[5] * inv);
  val.w = pack_bf16x2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(a.out + orow * kDim + d0) = val;
}

template <int G>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int QB = kRowsPerWG / G;  // positions per workgroup
  extern __shared__ __align__(16) unsigned char lds_raw[];
  PrefillLds& sm = *reinterpret_cast<PrefillLds*>(lds_raw);
  float (*rowf)[32] = sm.rowf;

  int b, part, g, jrev;
  if (a.plan != nullptr) {
    // 1-D grid: item k of the longest-first list, kv head fastest
    const int k = int(blockIdx.x) / a.hkv;
    g = int(blockIdx.x) - k * a.hkv;
    if (k >= a.plan[0]) return;
    const int id = a.plan[kPlanHeader + k];  // (b * nqb_max + jrev) * 16 + part
    const int c = id >> 4, nq = nqb_max_of<G>(a);
    part = id & 15;
    b = c / nq;
    jrev = c - b * nq;
  } else {
    b = int(blockIdx.x) / a.max_splits;
    part = int(blockIdx.x) - b * a.max_splits;
    g = blockIdx.y;
    jrev = blockIdx.z;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int half = lane >> 5;
  const int jl = lane & 15, dg = (lane >> 4) & 1;  // lane in its 16-lane group; dims 16 dg ..

  const BlockGeom<G> bg(a, b, jrev, split_tiles_of(a));
  if (jrev >= bg.nqb) return;
  const int q0 = bg.q0, qlen = bg.qlen, ctx = bg.ctx, p0 = bg.p0, shift = bg.shift;
  const int ntiles = bg.ntiles, nsplit = bg.nsplit;

  // This lane's query row (the S^T column it owns): head hl, position pos.
  const int R = w * 32 + col;
  const int hl = R / QB;
  const int pos = p0 + R % QB;
  const int head = g * G + hl;
  const bool row_ok = pos < qlen;
  const int a_pos = row_ok ? min(shift + pos, ctx - 1) : -1;  // last visible key

  // Wave-uniform key range of this wave's rows.
  int amax = a_pos, amin = a_pos;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    amax = max(amax, __shfl_xor(amax, d, 64));
    amin = min(amin, __shfl_xor(amin, d, 64));
  }
  amax = __builtin_amdgcn_readfirstlane(amax);
  amin = __builtin_amdgcn_readfirstlane(amin);

  const int32_t* table = a.block_table + int64_t(b) * a.mbps;

  // This part's key tiles [t_begin, t_end).
  if (part >= nsplit) return;
  const int t_begin = int(int64_t(ntiles) * part / nsplit);
  const int t_end = int(int64_t(ntiles) * (part + 1) / nsplit);
  if (qlen * G <= kShortRows) {
    prefill_short<G>(a, bg, b, g, part, nsplit, t_begin, t_end, lds_raw);
    return;
  }

  // Q^T operand: dims 16*ks + 8*half .. +7 of the lane's row, 8 k-steps.
  // With a negative scale the sign goes into q (exact in bf16), so scores are
  // scaled by a positive factor and a row's largest score is its largest
  // weight (the row max below relies on that).
  bf16x8_t qop[8];
  {
    const uint4* qrow = reinterpret_cast<const uint4*>(
        a.q + (int64_t(q0) + (row_ok ? pos : 0)) * (int64_t(a.hq) * kDim) + int64_t(head) * kDim);
    const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      uint4 u = row_ok ? qrow[2 * ks + half] : zero4();
      u.x ^= flip;
      u.y ^= flip;
      u.z ^= flip;
      u.w ^= flip;
      qop[ks] = as_bf16x8(u);
    }
  }

  // Tile t+1 is loaded into one LDS buffer while tile t is computed from
  // the other.
  if (t_begin < t_end) dma_tile(a, table, g, ctx, t_begin, w, lane, sm.k[t_begin & 1], sm.v[t_begin & 1]);

  const float c = fabsf(a.scale_log2);
  f32x16_t o[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[n][r] = 0.f;
  float m = -INFINITY;  // running reference max of the lane's row (log2 units)
  float l = 0.f;        // partial row sum over this lane's keys

  // S^T = K Q^T of the tile in K buffer kb: two independent 32-key chains.
  auto scores = [&](const uint4* __restrict__ kb, f32x16_t (&s)[2]) {
    const uint4* ksrc = kb + half * kKeys + col;  // chunk 2ks+half, key 32ms+col
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[ms][r] = 0.f;
    // K operands are read 8 ahead of the MFMAs that use them
    uint4 ka[8][2];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) ka[ks][ms] = ksrc[2 * ks * kKeys + 32 * ms];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int ms = 0; ms < 2; ++ms) {
        ka[ks + 4][ms] = ksrc[2 * (ks + 4) * kKeys + 32 * ms];
        s[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[ks][ms]), qop[ks], s[ms], 0, 0, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 4; ks < 8; ++ks) {
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
        s[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ka[ks][ms]), qop[ks], s[ms], 0, 0, 0);
    }
  };

  // Softmax of tile t's scores and O += P V with the tile in V buffer vb.
  auto softmax_pv = [&](int t, const uint16_t* __restrict__ vb, f32x16_t (&s)[2]) {
    const int key0 = t * kKeys;
    // V operand (k-step ks, dims 32 n + col) of the product below
    const uint16_t* vrow = vb + (4 * half + (jl >> 2)) * kVStride + 16 * dg + 4 * (jl & 3);
    auto vop_of = [&](int ks, int n) {
      const uint16_t* vsrc = vrow + 32 * (n ^ (jl >> 2)) + 16 * ks * kVStride;
      const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16_t*)(vsrc));
      const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4i16_t*)(vsrc + 8 * kVStride));
      return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // the first k-step's operands are read now, while the score MFMAs finish,
    // rather than right before the first product MFMA
    bf16x8_t v0[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) v0[n] = vop_of(0, n);
    __builtin_amdgcn_sched_barrier(0);
    // mask keys past the row's position (diagonal / tail tiles)
    if (key0 + kKeys - 1 > amin) {
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + 32 * ms + (r & 3) + 8 * (r >> 2) + 4 * half;
          s[ms][r] = key <= a_pos ? s[ms][r] : -INFINITY;
        }
    }
    // online softmax with lazy rescale
    float mt = -INFINITY;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[ms][r]);
    mt = xor32_max(mt) * c;
    const float mnew = fmaxf(m, mt);
    const bool need = mnew > m + kLazyRescale;  // also true for the first finite max
    if (__ballot(need) != 0) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;
      if (need) {
        l *= alpha;
        m = mnew;
      }
      if (half == 0) rowf[w][col] = alpha;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const float4 al = *reinterpret_cast<const float4*>(&rowf[w][8 * qd + 4 * half]);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          o[n][4 * qd + 0] *= al.x;
          o[n][4 * qd + 1] *= al.y;
          o[n][4 * qd + 2] *= al.z;
          o[n][4 * qd + 3] *= al.w;
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    const float mref = m == -INFINITY ? 0.f : m;

    // P = 2^(c s - m) as bf16 A operands; row sums of the rounded weights
    bf16x8_t pop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float pf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        pf[e] = __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][8 * (ks & 1) + e], c, -mref));
      const uint4 pb = pack8(pf);
      // sum of the bf16 weights the MFMA consumes (dot with (1, 1) pairs)
      l = dot2_bf16(pb.x, kBf16OnePair, l);
      l = dot2_bf16(pb.y, kBf16OnePair, l);
      l = dot2_bf16(pb.z, kBf16OnePair, l);
      l = dot2_bf16(pb.w, kBf16OnePair, l);
      pop[ks] = as_bf16x8(pb);
    }

    // O += P V.  The B operand of lane (dim 32 n + col, half) is V of keys
    // 16 ks + 4 half + {0..3} and 16 ks + 8 + 4 half + {0..3} (P's order),
    // two transposing LDS reads: in each 16-lane group, lane j points at dims
    // 4 (j & 3) .. +3 of key j >> 2 and receives its own dim of all 4 keys.
    // Those keys have key & 3 = j >> 2, so dims 32 n .. 32 n + 31 of the
    // lane's row sit 32 (n ^ (j >> 2)) bf16 into it.
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pop[ks], ks == 0 ? v0[n] : vop_of(ks, n), o[n], 0, 0, 0);
  };

  // One tile: the loads of tile t+1 into buffers (kn, vn), then tile t from
  // (kc, vc).  The restrict pointers tell the compiler that the LDS-DMA
  // writes and this tile's LDS reads are disjoint; otherwise it would make
  // every read wait for the writes just issued (the wait for a tile's own
  // loads is the explicit one at the top of the loop).
  auto step = [&](int t, const uint4* __restrict__ kc, const uint16_t* __restrict__ vc, uint4* __restrict__ kn,
                  uint16_t* __restrict__ vn) {
    if (t + 1 < t_end) dma_tile(a, table, g, ctx, t + 1, w, lane, kn, vn);
    if (t * kKeys > amax) return;  // every key of the tile is above this wave's diagonal
    f32x16_t s[2];
    scores(kc, s);
    // The softmax and P.V of a tile are one dependent chain (max, exponentials,
    // product); the other workgroup's wave on this SIMD fills the gaps with its
    // own work.  Issue priority over the chain (not over the scores, and not
    // dropped before the product) shortened every multi-tile workload: on
    // three boxes, interleaved, 8 x 2048 by 0.7-1.4 %, chunked prefill mixed
    // by 2.3-3.1 %, a chunk over a 65,536-token prefix by 5.4-6.0 %.
    __builtin_amdgcn_s_setprio(1);
    softmax_pv(t, vc, s);
    __builtin_amdgcn_s_setprio(0);
  };
  for (int t = t_begin; t < t_end; ++t) {
    __builtin_amdgcn_s_waitcnt(0xF70);  // vmcnt(0): this wave's part of tile t is in LDS
    // every wave's part; and every wave is past tile t-1, whose buffers the
    // loads of tile t+1 now overwrite
    __syncthreads();
    step(t, sm.k[t & 1], sm.v[t & 1], sm.k[(t + 1) & 1], sm.v[(t + 1) & 1]);
  }

  const float ltot = xor32_sum(l);
  if (nsplit > 1) {
    write_part<G>(a, b, jrev, g, part, q0, qlen, p0, o, m, ltot);
    if (a.plan != nullptr) arrive_and_merge<G>(a, bg, b, jrev, g);
    return;
  }

  // ---- epilogue: O / l -> bf16, staged through LDS for 16-byte stores -------
  __syncthreads();  // tile buffers are reused below
  if (half == 0) rowf[w][col] = ltot > 0.f ? 1.f / ltot : 0.f;
  __builtin_amdgcn_wave_barrier();
  uint16_t* stage = reinterpret_cast<uint16_t*>(lds_raw) + w * (32 * kDim);  // [32 rows][128]
#pragma unroll
  for (int qd = 0; qd < 4; ++qd) {
    const float4 inv = *reinterpret_cast<const float4*>(&rowf[w][8 * qd + 4 * half]);
    const float iv[4] = {inv.x, inv.y, inv.z, inv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 8 * qd + 4 * half + i;
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const __bf16 v = static_cast<__bf16>(o[n][4 * qd + i] * iv[i]);
        stage[row * kDim + 32 * n + col] = __builtin_bit_cast(uint16_t, v);
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  // 32 rows x 16 chunks = 512 chunks, 8 per lane
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int idx = lane + 64 * j;
    const int row = idx >> 4, ch = idx & 15;
    const int Rr = w * 32 + row;
    const int p = p0 + Rr % QB;
    if (p < qlen) {
      const int hh = g * G + Rr / QB;
      const uint4 val = reinterpret_cast<const uint4*>(stage)[row * kChunks + ch];
      uint4* dst = reinterpret_cast<uint4*>(a.out + (int64_t(q0) + p) * (int64_t(a.hq) * kDim) +
                                            int64_t(hh) * kDim);
      dst[ch] = val;
    }
  }
}

// Plan of a launch whose blocks differ in length on the device (ragged
// query lengths), in one workgroup:
// * the part length: the hardware dispatches workgroups in grid order as
//   slots free up, and one block streaming far more tiles than the launch's
//   share per slot ends the launch late.  With W the tiles of all query
//   blocks and kv heads, a block of more than L = max(split_tiles, ceil(W /
//   slots)) tiles is cut into ceil(tiles / L) parts (at most max_splits) of
//   near-equal length, merged afterwards; each cut block gets consecutive
//   record slots (plan_rec).
//   Every cut block has more than L tiles, so the cut blocks number fewer
//   than W / L <= slots / hkv and their parts fewer than 2 W / L <= 2 slots /
//   hkv: the records the host sizes for 2 slots x kRowsPerWG rows suffice.
//   The parts merge without a second kernel (arrive_and_merge); the plan
//   zeroes their arrival counters (plan_cnt, one per first slot and kv head).
// * the order: the items (query block, part) counted per length (the whole
//   block's tiles, 5/4 of them for a short block; kPlanBuckets - 1 and more
//   counted together), the counts turned
//   into offsets in order of decreasing length, every item written at its
//   offset; items of one length keep no particular order and record slots
//   go to cut blocks in no particular order (each item writes its own rows
//   or records, and the merge reads a block's parts in part order, so the
//   outputs do not depend on either).
constexpr int kPlanThreads = 1024;
constexpr int kPlanBuckets = 4096;

template <int G>
__global__ __launch_bounds__(kPlanThreads) void prefill_plan_kernel(PrefillArgs a) {
  __shared__ int cnt[kPlanBuckets];  // per key = kPlanBuckets - 1 - min(length, kPlanBuckets - 1)
  __shared__ int wsum[kPlanThreads / 64];
  __shared__ long long wtiles[kPlanThreads / 64];
  __shared__ int n_slots, n_cut, split_len;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kPlanBuckets; i += kPlanThreads) cnt[i] = 0;
  if (tid == 0) {
    n_slots = 0;
    n_cut = 0;
  }

  const int nqb_max = nqb_max_of<G>(a);
  const int64_t cands = int64_t(a.batch) * nqb_max;

  // W: tiles of every query block (one kv head)
  long long mine = 0;
  for (int64_t c = tid; c < cands; c += kPlanThreads) {
    const int b = int(c / nqb_max);
    const int jrev = int(c - int64_t(b) * nqb_max);
    const BlockGeom<G> bg(a, b, jrev, INT32_MAX);
    if (jrev < bg.nqb) mine += bg.ntiles;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) mine += __shfl_xor(mine, d, 64);
  if (lane == 0) wtiles[w] = mine;
  __syncthreads();
  if (tid == 0) {
    long long wt = 0;
    for (int i = 0; i < kPlanThreads / 64; ++i) wt += wtiles[i];
    const long long den = (long long)a.slots * kPlanShareDiv;
    long long share = (wt * a.hkv + den - 1) / den;
    share = share < a.split_tiles ? a.split_tiles : share;
    split_len = int(share > INT32_MAX ? INT32_MAX : share);
    a.plan[1] = split_len;
  }
  __syncthreads();
  const int L = split_len;

  // fn(item id, key) for every item of the launch; cut blocks get their
  // record slots and merge-list places on the way (first pass only)
  auto for_items = [&](bool first, auto&& fn) {
    for (int64_t c = tid; c < cands; c += kPlanThreads) {
      const int b = int(c / nqb_max);
      const int jrev = int(c - int64_t(b) * nqb_max);
      const BlockGeom<G> bg(a, b, jrev, L);
      if (jrev >= bg.nqb) continue;
      if (first && bg.nsplit > 1) {
        const int slot = atomicAdd(&n_slots, bg.nsplit);
        a.plan_rec[c] = slot;
        atomicAdd(&n_cut, 1);
        for (int g = 0; g < a.hkv; ++g) a.plan_cnt[slot * a.hkv + g] = 0;  // arrival counters
      }
      // the parts of a cut block go by the whole block's length, so that
      // they start in the first round rather than after every longer item;
      // a short block (the short-row path: memory-bound, so its tiles take
      // longer than a chunk's while the chip streams) counts 5/4 of its
      // tiles (chunked prefill mixed with decode rows 252.6 -> 245.8 us,
      // 248.3 -> 241.4 us; 4/3, 3/2 and 2 gained less, 2/3 lost)
      const int len = bg.qlen * G <= kShortRows ? bg.ntiles * 5 / 4 : bg.ntiles;
      for (int part = 0; part < bg.nsplit; ++part)
        fn(int(c) * 16 + part, kPlanBuckets - 1 - min(len, kPlanBuckets - 1));
    }
  };
  for_items(true, [&](int, int key) { atomicAdd(&cnt[key], 1); });
  __syncthreads();

  // exclusive scan of the counts in key order: thread t owns keys 4t .. 4t+3
  constexpr int kPer = kPlanBuckets / kPlanThreads;
  int c4[kPer], own = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    c4[i] = cnt[kPer * tid + i];
    own += c4[i];
  }
  int incl = own;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int before = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kPlanThreads / 64; ++i) {
    before += i < w ? wsum[i] : 0;
    total += wsum[i];
  }
  int off = before + incl - own;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    cnt[kPer * tid + i] = off;
    off += c4[i];
  }
  if (tid == 0) {
    a.plan[0] = total;
    a.plan[2] = n_cut;
  }
  __syncthreads();

  int32_t* order = a.plan + kPlanHeader;
  for_items(false, [&](int id, int key) { order[atomicAdd(&cnt[key], 1)] = id; });
}

template <int G>
static hipError_t launch_prefill_g(const PrefillArgs& a, hipStream_t s) {
  constexpr int QB = kRowsPerWG / G;
  // more than 64 KiB of LDS per workgroup must be opted into
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&prefill_kernel<G>), hipFuncAttributeMaxDynamicSharedMemorySize,
      int(kShortOnlyLds));
  if (attr != hipSuccess) return attr;
  const int nqb = (a.max_q + QB - 1) / QB;
  if (a.plan != nullptr) {
    hipLaunchKernelGGL(prefill_plan_kernel<G>, dim3(1), dim3(kPlanThreads), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // workgroups for every possible item (kv head fastest); those past the
    // plan's count exit at once
    hipLaunchKernelGGL(prefill_kernel<G>, dim3(unsigned(a.plan_items) * unsigned(a.hkv)), dim3(256),
                       kPrefillLds, s, a);
    return hipGetLastError();
  }
  const dim3 grid(unsigned(a.batch) * unsigned(a.max_splits), unsigned(a.hkv), unsigned(nqb));
  const size_t lds = int64_t(a.max_q) * G <= kShortRows ? kShortOnlyLds : kPrefillLds;
  hipLaunchKernelGGL(prefill_kernel<G>, grid, dim3(256), lds, s, a);
  if (a.max_splits > 1) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_merge_kernel<G>, dim3(unsigned(a.batch), unsigned(a.hkv), unsigned(2 * nqb)),
                       dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_prefill_g<1>(a, s);
    case 2: return launch_prefill_g<2>(a, s);
    case 4: return launch_prefill_g<4>(a, s);
    case 8: return launch_prefill_g<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
