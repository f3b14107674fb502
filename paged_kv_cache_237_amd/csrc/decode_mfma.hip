// Decode of several query rows per sequence on the matrix cores (gfx950).
//
// What it computes: pa_decode_multi -- q_per_seq new tokens per sequence,
// token i attending to the cached positions up to its own (ctx - q_per_seq + i),
// softmax(scale * q K^T) V per head (CSDN essay comparing nanoVLLM and vLLM,
// first and third sections: paged cache, exact attention in on-chip tiles;
// its section on speculative decoding: a draft model proposes a few tokens
// and the target model checks them in one pass) -- when the rows of one
// (sequence, kv head), q_per_seq tokens x G query heads, number 17 to 32: too
// many for the vector-ALU decode kernel (decode.hip), which keeps a row's
// accumulators per head in registers.
//
// Work decomposition: the one-row decode's.  Every (sequence, kv head) is a
// segment of 64-token tiles; all segments are laid end to end and cut into
// one run per wave, weighted by the XCD the wave runs on; a run covering a
// whole segment writes the output, a cut segment leaves one partial state
// (m, l, O) per run and the last wave to arrive merges them.  A workgroup is
// 4 waves, one per SIMD, so each wave may use the SIMD's whole register file:
// the K and V of the next tile stay in flight while the current one is
// computed.
//
// One tile, one wave, the segment's 32 rows (row v = query token v / G and
// head v % G; rows past q_per_seq * G are zero padding):
//   S^T = K Q^T : v_mfma_f32_32x32x16_bf16 with the K tile as the A operand
//                 loaded straight from memory -- the cache keeps 8 dims of a
//                 token in one 16-byte chunk, so a half-wave's load of one
//                 chunk of 32 tokens is one operand -- and Q^T as the B
//                 operand, held in registers for the segment.  The
//                 accumulator holds one row per lane column.
//   softmax    : keys past the context, and past each row's own position,
//                 are masked; row max in-lane plus one lane^32 exchange; log2
//                 domain with a lazy rescale (the reference max moves only
//                 when a row max grows by more than 2^8).
//   O += P V   : P rounded to bf16 straight from the S^T accumulator (A
//                 operand: lane half h holds keys 16 ks + 4 h + {0..3, 8..11}
//                 of k-step ks); V is kept in the wave's LDS as it arrives,
//                 one row per token, and a lane's B operand (its dim of those
//                 8 keys) is two transposing reads (ds_read_b64_tr_b16).
//                 Against a V tile transposed to [dim][key] on its way into
//                 LDS (permutes and 8-byte stores): 64 x 6 tokens with 32 q
//                 heads 133.1 -> 131.1 us, 131072-token contexts unchanged
//                 (one box, interleaved).
// The row sums add the bf16 weights the MFMA consumes.  Memory traffic is
// the K and V rows of each context read once; the matrix work of a tile is a
// small part of the time its 32 KiB take to arrive, so, like the one-row
// decode, the kernel is bound by HBM bandwidth.
#include <math.h>

#include "decode_mfma_common.hpp"

namespace pa {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMfRows = 32;       // rows per segment: one MFMA block
constexpr int kMfWaves = 4;       // waves per workgroup, one per SIMD
// Tiles whose K and V are in flight while one is computed: 1 (the next
// tile's loads go into the registers the current tile frees) or 2 (two
// register buffers, alternating).
constexpr int kMfDepth = 1;
static_assert(partial_floats(kMfRows) == kMfRows * (kDim + 2), "record layout");

constexpr int kMfVStride = 160;  // bf16 per V row in LDS (128 dims + pad: the transposing reads hit no bank twice)

// One wave's LDS: the V tile, one row per token (also the output staging at
// the end of a piece), and per-row factors exchanged between lanes.
struct MfLds {
  uint16_t vt[kTile * kMfVStride];
  float rowf[kMfRows];
};

// K as A operands: kr[8 ms + ks] = chunk 2 ks + half of token 32 ms + col.
__device__ __forceinline__ void mf_issue_k(const MfTile& tl, uint4 (&kr)[16]) {
  const int lane = lane_id();
  const int col = lane & 31, half = lane >> 5;
#pragma unroll
  for (int ms = 0; ms < 2; ++ms) {
    const int key = 32 * ms + col;
    const uint32_t off = key < tl.valid ? uint32_t(tl.r0 + key) * 16u + uint32_t(half) * 4096u : kOutOfRange;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kr[8 * ms + ks] = buf_load16_stream(tl.rk, off + uint32_t(ks) * 8192u, 0u);
  }
}

// Q^T of segment (b, g) as B operands: dims 16 ks + 8 half .. +7 of row
// col; padding rows are zero.  With a negative scale the sign is moved into
// q (exact in bf16), so the scores are always scaled by a positive factor
// and a row's largest score is its largest weight.
__device__ __forceinline__ void mf_load_q(const DecodeArgs& a, int b, int g, uint4 (&qop)[8]) {
  const int lane = lane_id();
  const int v = lane & 31, half = lane >> 5;
  const bool real = (v >> a.gr_shift) < a.ql;
  const uint4* src = reinterpret_cast<const uint4*>(a.q + vrow<kMfRows, true>(a, b, g, real ? v : 0) * kDim);
  const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) {
    uint4 u = real ? src[2 * ks + half] : make_uint4(0u, 0u, 0u, 0u);
    u.x ^= flip;
    u.y ^= flip;
    u.z ^= flip;
    u.w ^= flip;
    qop[ks] = u;
  }
}

// Merge of the partial records of segment seg written by waves w0..w1: for
// every real row, M = max m_i, L = sum 2^(m_i - M) l_i, o = sum 2^(m_i - M)
// O_i / L.  Lane = 4 dims (4 (lane % 32) ..) of 16 rows (16 (lane / 32) ..);
// a record is one round of loads (16-byte reads, each half-wave covering a
// row's 512 bytes), and the next record's loads are issued before the
// current one is folded in.
struct MfRecPart {
  float m[16], l[16];
  float4 u[16];
};

__device__ __forceinline__ void mf_load_rec(const DecodeArgs& a, int rec_idx, int rh, int d0, MfRecPart& p) {
  const float* rec = a.ws + int64_t(rec_idx) * partial_floats(kMfRows);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, uint32_t(partial_floats(kMfRows)) * 4u);
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p.m[r] = ld_coherent(rec + kMfRows * kDim + rh + r);
    p.l[r] = ld_coherent(rec + kMfRows * kDim + kMfRows + rh + r);
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rr, int(uint32_t((rh + r) * kDim + d0) * 4u), 0,
                                                             kCpolAgent);
    const unsigned x = v.x, y = v.y, z = v.z, w = v.w;
    p.u[r] = make_float4(__uint_as_float(x), __uint_as_float(y), __uint_as_float(z), __uint_as_float(w));
  }
}

__device__ void mf_merge(const DecodeArgs& a, int seg, int b, int g, int w0, int w1) {
  const int lane = lane_id();
  const int d0 = 4 * (lane & 31), rh = 16 * (lane >> 5);
  const int nreal = min(kMfRows, a.ql << a.gr_shift);
  float M[16], L[16];
  float4 U[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    M[r] = -INFINITY;
    L[r] = 0.f;
    U[r] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  MfRecPart cur;
  mf_load_rec(a, seg + w0, rh, d0, cur);
  for (int w = w0; w <= w1; ++w) {
    MfRecPart nxt;
    if (w < w1) mf_load_rec(a, seg + w + 1, rh, d0, nxt);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float mn = fmaxf(M[r], cur.m[r]);
      const float ref = mn == -INFINITY ? 0.f : mn;
      const float sa = __builtin_amdgcn_exp2f(M[r] - ref);
      const float sb = __builtin_amdgcn_exp2f(cur.m[r] - ref);
      L[r] = L[r] * sa + cur.l[r] * sb;
      U[r].x = U[r].x * sa + cur.u[r].x * sb;
      U[r].y = U[r].y * sa + cur.u[r].y * sb;
      U[r].z = U[r].z * sa + cur.u[r].z * sb;
      U[r].w = U[r].w * sa + cur.u[r].w * sb;
      M[r] = mn;
    }
    if (w < w1) cur = nxt;
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (rh + r >= nreal) break;
    const float inv = L[r] > 0.f ? 1.f / L[r] : 0.f;
    uint2* out = reinterpret_cast<uint2*>(a.out + vrow<kMfRows, true>(a, b, g, rh + r) * kDim + d0);
    *out = make_uint2(pack_bf16x2(U[r].x * inv, U[r].y * inv), pack_bf16x2(U[r].z * inv, U[r].w * inv));
  }
}

// Streams tiles [pos, end) of the flattened list (this wave's run) with
// kMfDepth tiles in flight: the loads of tile i + kMfDepth go into the
// registers tile i frees (K after its scores, V after its store to LDS) --
// also across segment boundaries (block-table entries are looked up ahead;
// the next segment's q is loaded when a piece ends).  Each piece (run ∩
// segment) ends with either the bf16 output (whole segment) or a partial
// record at seg + wave.  Returns the number of cut segments, whose (b, g,
// first run, last run) go to pend_*.
__device__ int mf_stream_run(const DecodeArgs& a, const TileScan& sc, int pos, int end, const Runs& runs,
                             int wave, MfLds& L, int* prog, int wv, int (&pend_b)[2], int (&pend_g)[2],
                             int (&pend_w0)[2], int (&pend_w1)[2]) {
  const int lane = lane_id();
  const int col = lane & 31, half = lane >> 5;
  const float c = fabsf(a.scale_log2);
  int done = 0;

  MfCur c0;
  {
    int b, before;
    locate<false>(a, sc, pos, b, before);
    if (b >= a.batch) return 0;
    int nt = tiles_of(clamp_ctx(a, a.ctx_lens[b]));
    const int off = pos - before * a.hkv;
    const int g = off / nt;
    c0.b = __builtin_amdgcn_readfirstlane(b);
    c0.g = __builtin_amdgcn_readfirstlane(g);
    c0.t = __builtin_amdgcn_readfirstlane(off - g * nt);
    c0.nt = __builtin_amdgcn_readfirstlane(nt);
    c0.ctx = __builtin_amdgcn_readfirstlane(clamp_ctx(a, a.ctx_lens[b]));
    c0.live = true;
    c0.phys = ld_uniform(a.block_table, int64_t(c0.b) * a.mbps + (c0.t >> 2));
  }
  MfCur c1 = mf_next(a, c0, pos + 1 < end);

  uint4 qop[8];
  mf_load_q(a, c0.b, c0.g, qop);
  uint4 kA[16], vA[16], kB[kMfDepth == 2 ? 16 : 1][16], vB[kMfDepth == 2 ? 16 : 1][16];
  MfTile tA = mf_tile(a, c0.phys, c0.g, c0.t, c0.ctx);
  MfTile tB = mf_tile(a, c1.phys, c1.g, c1.t, c1.ctx);
  mf_issue_k(tA, kA);
  mf_issue_v(tA, vA);
  if constexpr (kMfDepth == 2) {
    mf_issue_k(tB, kB[0]);
    mf_issue_v(tB, vB[0]);
  }

  f32x16_t o[4];
#pragma unroll
  for (int n = 0; n < 4; ++n)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[n][r] = 0.f;
  float m = -INFINITY;  // reference max of the lane's row (log2 units)
  float l = 0.f;        // partial row sum over this lane's keys
  int piece_t0 = c0.t;
  int npend = 0;
  int i = pos;  // index of tile c0 in the flattened list

  // One tile: c0 from (kr, vr) whose geometry is tl; c1 is in flight in the
  // other buffer.  Returns whether a next tile follows in this run.
  auto step = [&](uint4 (&kr)[16], uint4 (&vr)[16], MfTile& tl) -> bool {
    const MfCur c2 = kMfDepth == 2 ? mf_next(a, c1, i + 2 < end) : c1;  // the tile loaded into kr, vr next
    const bool seg_end = c0.t + 1 == c0.nt;
    const bool has_next = i + 1 < end;
    const bool next_ok = c1.live;

    // issue priority: a wave ahead of its slowest sibling yields
    {
      ++done;
      if (lane == 0) prog_set(&prog[wv], done);
      int slowest = done;
#pragma unroll
      for (int w = 0; w < kMfWaves; ++w) slowest = min(slowest, prog_get(&prog[w]));
      if (__builtin_amdgcn_readfirstlane(slowest) + 1 < done)
        __builtin_amdgcn_s_setprio(0);
      else
        __builtin_amdgcn_s_setprio(2);
    }

    // --- S^T = K Q^T (two independent 32-key chains)
    f32x16_t s[2];
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[ms][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
        s[ms] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf8(kr[8 * ms + ks]), as_bf8(qop[ks]), s[ms], 0, 0, 0);
    const MfTile t2 = mf_tile(a, c2.phys, c2.g, c2.t, c2.ctx);
    mf_issue_k(t2, kr);  // K of tile i + kMfDepth into the registers just read

    // --- V of this tile into LDS, then V of tile i + kMfDepth into its registers
    lds_order();
    mf_store_v_rows<kMfVStride>(L.vt, vr);
    mf_issue_v(t2, vr);
    lds_order();

    // --- online softmax (log2 domain, lazy rescale)
    const int key0 = c0.t * kTile;
    const int last0 = c0.ctx - a.ql;  // last key of query token 0
    if (key0 + kTile - 1 > last0 || tl.valid < kTile) {
      const int lim = min(last0 + (col >> a.gr_shift) - key0, tl.valid - 1);  // last visible key of the row
#pragma unroll
      for (int ms = 0; ms < 2; ++ms)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 32 * ms + (r & 3) + 8 * (r >> 2) + 4 * half;
          s[ms][r] = key <= lim ? s[ms][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int ms = 0; ms < 2; ++ms)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[ms][r]);
    mt = xor32_max(mt) * c;
    const float mnew = fmaxf(m, mt);
    const bool need = mnew > m + kMfLazy;  // also true for the first finite max
    if (__ballot(need) != 0) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;
      if (need) {
        l *= alpha;
        m = mnew;
      }
      if (half == 0) L.rowf[col] = alpha;
      lds_order();
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const float4 al = *reinterpret_cast<const float4*>(&L.rowf[8 * qd + 4 * half]);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          o[n][4 * qd + 0] *= al.x;
          o[n][4 * qd + 1] *= al.y;
          o[n][4 * qd + 2] *= al.z;
          o[n][4 * qd + 3] *= al.w;
        }
      }
      lds_order();
    }
    const float mref = m == -INFINITY ? 0.f : m;
    bf16x8_t pop[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      float pf[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = __builtin_amdgcn_exp2f(fmaf(s[ks >> 1][8 * (ks & 1) + e], c, -mref));
      const uint4 pb = pack8(pf);
      l = dot2_bf16(pb.x, kMfOnePair, l);
      l = dot2_bf16(pb.y, kMfOnePair, l);
      l = dot2_bf16(pb.z, kMfOnePair, l);
      l = dot2_bf16(pb.w, kMfOnePair, l);
      pop[ks] = as_bf8(pb);
    }

    // --- O += P V (dims 32 n + col, keys 16 ks + 4 half + {0..3, 8..11})
    // within each 16-lane group (its dims 32 n + 16 dg .. + 15), lane jl
    // points at dims 4 (jl & 3) .. + 3 of key 16 ks + 4 half + jl / 4; the
    // second read takes the keys 8 further
    const int jl = col & 15, dg = col >> 4;
    const uint16_t* vsrc = L.vt + (4 * half + (jl >> 2)) * kMfVStride + 16 * dg + 4 * (jl & 3);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const bf16x8_t vop = tr_read_pair(vsrc + 16 * ks * kMfVStride + 32 * n, 8 * kMfVStride);
        o[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pop[ks], vop, o[n], 0, 0, 0);
      }
    lds_order();

    // --- end of a piece: the output rows or a partial record
    if (seg_end || !has_next) {
      const float ltot = xor32_sum(l);
      if (piece_t0 == 0 && seg_end) {
        // O / l -> bf16, staged in LDS as [row][128] for 16-byte stores
        if (half == 0) L.rowf[col] = ltot > 0.f ? 1.f / ltot : 0.f;
        lds_order();
        uint16_t* stage = L.vt;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) {
          const float4 inv = *reinterpret_cast<const float4*>(&L.rowf[8 * qd + 4 * half]);
          const float iv[4] = {inv.x, inv.y, inv.z, inv.w};
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int row = 8 * qd + 4 * half + r4;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
              const __bf16 v = static_cast<__bf16>(o[n][4 * qd + r4] * iv[r4]);
              stage[row * kDim + 32 * n + col] = __builtin_bit_cast(uint16_t, v);
            }
          }
        }
        lds_order();
        const int nreal = min(kMfRows, a.ql << a.gr_shift);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int idx = lane + 64 * j;
          const int row = idx >> 4, ch = idx & 15;
          if (row < nreal) {
            const uint4 val = reinterpret_cast<const uint4*>(stage)[row * kChunks + ch];
            reinterpret_cast<uint4*>(a.out + vrow<kMfRows, true>(a, c0.b, c0.g, row) * kDim)[ch] = val;
          }
        }
        lds_order();
      } else {
        const int seg = c0.b * a.hkv + c0.g;
        float* rec = a.ws + int64_t(seg + wave) * partial_floats(kMfRows);
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, uint32_t(partial_floats(kMfRows)) * 4u);
#pragma unroll
        for (int qd = 0; qd < 4; ++qd)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int row = 8 * qd + 4 * half + r4;
#pragma unroll
            for (int n = 0; n < 4; ++n)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[n][4 * qd + r4]), rr,
                                                    int(uint32_t(row * kDim + 32 * n + col) * 4u), 0, kCpolAgent);
          }
        if (half == 0) {
          st_coherent(rec + kMfRows * kDim + col, m);
          st_coherent(rec + kMfRows * kDim + kMfRows + col, ltot);
        }
        const int start = i - c0.t;  // first tile of the segment in the flattened list
        pend_b[npend] = c0.b;
        pend_g[npend] = c0.g;
        pend_w0[npend] = wave_of<kMfWaves>(runs, start);
        pend_w1[npend] = wave_of<kMfWaves>(runs, start + c0.nt - 1);
        ++npend;
      }
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[n][r] = 0.f;
      m = -INFINITY;
      l = 0.f;
      piece_t0 = c1.t;
      // q of the next segment (its loads are waited for by the next scores)
      if (next_ok) mf_load_q(a, c1.b, c1.g, qop);
    }
    tl = t2;  // this buffer now holds tile i + kMfDepth
    c0 = c1;
    c1 = kMfDepth == 2 ? c2 : mf_next(a, c1, i + 2 < end);
    ++i;
    return next_ok;
  };

  if constexpr (kMfDepth == 2) {
    while (step(kA, vA, tA) && step(kB[0], vB[0], tB)) {
    }
  } else {
    while (step(kA, vA, tA)) {
    }
  }
  return npend;
}

__global__ __launch_bounds__(kMfWaves * kWave, 1) void decode_mfma_kernel(DecodeArgs a) {
  __shared__ MfLds lds[kMfWaves];
  __shared__ int prog[kMfWaves];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = blockIdx.x * kMfWaves + wv;
  if (lane_id() == 0) prog[wv] = 0;
  __syncthreads();

  // Empty contexts have no tiles: all their rows are zero.  Written on the
  // way out, so that no wave waits for it before streaming.
  auto zero_empty_rows = [&]() {
    if (wave >= a.n_waves) return;
    for (int bb = wave; bb < a.batch; bb += a.n_waves) {
      if (clamp_ctx(a, ld_uniform(a.ctx_lens, bb)) != 0) continue;
      uint32_t* o = reinterpret_cast<uint32_t*>(a.out + int64_t(bb) * a.ql * a.hq * kDim);
      for (int i = lane_id(); i < a.ql * a.hq * (kDim / 2); i += kWave) o[i] = 0u;
    }
  };

  const TileScan sc = scan_tiles<false>(a);
  const Runs runs = make_runs<kMfWaves>(a, sc.total);
  const int pos = run_start<kMfWaves>(runs, wave);
  const int end = run_start<kMfWaves>(runs, wave + 1);
  if (pos >= end) {
    if (lane_id() == 0) prog_set(&prog[wv], 1 << 30);
    zero_empty_rows();
    return;
  }

  int pend_b[2], pend_g[2], pend_w0[2], pend_w1[2];
  const int npend = mf_stream_run(a, sc, pos, end, runs, wave, lds[wv], prog, wv, pend_b, pend_g, pend_w0, pend_w1);
  if (lane_id() == 0) prog_set(&prog[wv], 1 << 30);
  __builtin_amdgcn_s_setprio(0);

  // Arrivals, ordered as in the one-row decode: SC1 record stores, a wait
  // for their completion, then the memory-side atomic; the last arriver
  // merges and resets the counter.
  if (npend > 0) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    for (int i = 0; i < npend; ++i) {
      const int seg = pend_b[i] * a.hkv + pend_g[i];
      int prev = 0;
      if (lane_id() == 0)
        prev = __hip_atomic_fetch_add(a.counters + seg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev == pend_w1[i] - pend_w0[i]) {
        mf_merge(a, seg, pend_b[i], pend_g[i], pend_w0[i], pend_w1[i]);
        if (lane_id() == 0) __hip_atomic_store(a.counters + seg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  zero_empty_rows();
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
  if (a.k_new != nullptr) return hipErrorInvalidValue;  // several rows: no appended token
  const unsigned blocks = unsigned((a.n_waves + kMfWaves - 1) / kMfWaves);
  hipLaunchKernelGGL(decode_mfma_kernel, dim3(blocks), dim3(kMfWaves * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
