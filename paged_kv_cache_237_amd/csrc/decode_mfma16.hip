// Decode of 5 to 16 query rows per (sequence, kv head) on the matrix cores
// (gfx950): pa_decode_multi for, e.g., 5 drafted tokens + the next one at 2 q
// heads per kv head (12 rows), or 4 new tokens at 2 (8 rows; up to 8 rows of
// several tokens the vector-ALU decode measured 16-20 % slower).
//
// What it computes is decode_mfma.hip's (CSDN essay comparing nanoVLLM and
// vLLM, first and third sections: paged cache, exact attention in on-chip
// tiles; its section on speculative decoding: the drafted tokens are checked
// in one pass): token i of q_per_seq attends to the cached positions up to
// its own (ctx - q_per_seq + i), softmax(scale * q K^T) V per head.  The work
// decomposition (flattened tile list, weighted runs, partial records, last
// arriver's merge) is the same too, with one 4-wave workgroup per CU.  What
// differs is the block size: the rows fit one 16-row block of
// v_mfma_f32_16x16x32_bf16, so the matrix work per tile, the score, output
// and q registers and the partial records (8.3 KB instead of 16.6 KB) are
// half those of the 32-row kernel.  Measured against the 32-row kernel on
// the same rows (one box, interleaved): 64 sequences x 6 tokens at 16 q / 8
// kv heads over U{512..4096} 142.1 -> 128.5 us, 8 x 131,072 tokens x 6 rows
// 654.0 -> 632.7 us.  Two workgroups per CU (256 registers a wave, a few
// spilled) were slower on both (134.3 and 656.3 us): short contexts then
// cut each segment across twice the waves, and long ones gained nothing
// from the extra bytes in flight.
//
// One tile, one wave, the segment's 16 rows (row v = query token v / G and
// head v % G; rows past q_per_seq * G are zero padding).  Operand layouts of
// v_mfma_f32_16x16x32_bf16 (lane l, group j = l / 16): A holds row l % 16,
// k = 8 j .. 8 j + 7; B holds column l % 16, the same k; the accumulator
// holds column l % 16, rows 4 j .. 4 j + 3.
//   S^T = K Q^T : A = 16 keys x 32 dims of K straight from memory (the
//                 cache's 8-dim chunk 4 ks + j of token 16 ms + l % 16),
//                 B = Q^T, 32 dims x 16 rows, held in registers for the
//                 segment.  The accumulator of key block ms holds row
//                 l % 16 and keys 16 ms + 4 j .. +3.
//   softmax    : masks, row max in-lane plus the lane^16 and lane^32
//                 exchanges, log2 domain with the lazy rescale.
//   O += P V   : per 32 keys, A = bf16(P) straight from the accumulators of
//                 key blocks 2 ks and 2 ks + 1 (lane group j holds keys 4 j ..
//                 4 j + 3 and 16 + 4 j .. 16 + 4 j + 3, taken as k = 8 j ..
//                 8 j + 7); V is kept in the wave's LDS as it arrives (one row
//                 per token), and a lane's B operand (its dim l % 16 of those
//                 8 keys) is two transposing reads (ds_read_b64_tr_b16), as in
//                 the prefill.  Against a transposed V tile (permutes and
//                 8-byte stores): 64 x 6 tokens 129.1 -> 127.5 us, long
//                 contexts unchanged (one box, interleaved).  The
//                 accumulator of dim block n holds dims 16 n + l % 16, rows
//                 4 j .. 4 j + 3.
#include <math.h>

#include "decode_mfma_common.hpp"

namespace pa {
namespace {

typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kM16Rows = 16;   // rows per segment: one 16-row MFMA block
constexpr int kM16Waves = 4;   // waves per workgroup, one per SIMD
static_assert(partial_floats(kM16Rows) == kM16Rows * (kDim + 2), "record layout");

constexpr int kM16VStride = 144;  // bf16 per V row in LDS (128 dims + pad: the transposing reads hit no bank twice)

// One wave's LDS: the V tile, one row per token (also the output staging at
// the end of a piece), and per-row factors exchanged between lanes.
struct M16Lds {
  uint16_t vt[kTile * kM16VStride];
  float rowf[kM16Rows];
};

__device__ __forceinline__ float xor16_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned a = r[0], b = r[1];
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}

// K as A operands: kr[4 ms + ks] = chunk 4 ks + j of token 16 ms + l % 16.
__device__ __forceinline__ void m16_issue_k(const MfTile& tl, uint4 (&kr)[16]) {
  const int lane = lane_id();
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) {
    const int key = 16 * ms + col;
    const uint32_t off = key < tl.valid ? uint32_t(tl.r0 + key) * 16u + uint32_t(grp) * 4096u : kOutOfRange;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kr[4 * ms + ks] = buf_load16_stream(tl.rk, off + uint32_t(ks) * 16384u, 0u);
  }
}


// Q^T of segment (b, g) as B operands: dims 32 ks + 8 j .. +7 of row l % 16;
// padding rows are zero.  A negative scale's sign goes into q (exact in
// bf16), so the scores are scaled by a positive factor and a row's largest
// score is its largest weight.
__device__ __forceinline__ void m16_load_q(const DecodeArgs& a, int b, int g, uint4 (&qop)[4]) {
  const int lane = lane_id();
  const int v = lane & 15, grp = lane >> 4;
  const bool real = (v >> a.gr_shift) < a.ql;
  const uint4* src = reinterpret_cast<const uint4*>(a.q + vrow<kM16Rows, true>(a, b, g, real ? v : 0) * kDim);
  const uint32_t flip = a.scale_log2 < 0.f ? 0x80008000u : 0u;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    uint4 u = real ? src[4 * ks + grp] : make_uint4(0u, 0u, 0u, 0u);
    u.x ^= flip;
    u.y ^= flip;
    u.z ^= flip;
    u.w ^= flip;
    qop[ks] = u;
  }
}

// Merge of the partial records of segment seg written by waves w0..w1 (the
// split-context identity: M = max m_i, L = sum 2^(m_i - M) l_i, o = sum
// 2^(m_i - M) O_i / L).  Lane = 4 dims (4 (lane % 32) ..) of 8 rows (8 (lane
// / 32) ..); one record is one round of loads, and the next record's loads
// are issued before the current one is folded in.
struct M16RecPart {
  float m[8], l[8];
  float4 u[8];
};

__device__ __forceinline__ void m16_load_rec(const DecodeArgs& a, int rec_idx, int rh, int d0, M16RecPart& p) {
  const float* rec = a.ws + int64_t(rec_idx) * partial_floats(kM16Rows);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, uint32_t(partial_floats(kM16Rows)) * 4u);
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    p.m[r] = ld_coherent(rec + kM16Rows * kDim + rh + r);
    p.l[r] = ld_coherent(rec + kM16Rows * kDim + kM16Rows + rh + r);
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rr, int(uint32_t((rh + r) * kDim + d0) * 4u), 0,
                                                             kCpolAgent);
    const unsigned x = v.x, y = v.y, z = v.z, w = v.w;
    p.u[r] = make_float4(__uint_as_float(x), __uint_as_float(y), __uint_as_float(z), __uint_as_float(w));
  }
}

__device__ void m16_merge(const DecodeArgs& a, int seg, int b, int g, int w0, int w1) {
  const int lane = lane_id();
  const int d0 = 4 * (lane & 31), rh = 8 * (lane >> 5);
  const int nreal = min(kM16Rows, a.ql << a.gr_shift);
  float M[8], L[8];
  float4 U[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    M[r] = -INFINITY;
    L[r] = 0.f;
    U[r] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  M16RecPart cur;
  m16_load_rec(a, seg + w0, rh, d0, cur);
  for (int w = w0; w <= w1; ++w) {
    M16RecPart nxt;
    if (w < w1) m16_load_rec(a, seg + w + 1, rh, d0, nxt);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
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
  for (int r = 0; r < 8; ++r) {
    if (rh + r >= nreal) break;
    const float inv = L[r] > 0.f ? 1.f / L[r] : 0.f;
    uint2* out = reinterpret_cast<uint2*>(a.out + vrow<kM16Rows, true>(a, b, g, rh + r) * kDim + d0);
    *out = make_uint2(pack_bf16x2(U[r].x * inv, U[r].y * inv), pack_bf16x2(U[r].z * inv, U[r].w * inv));
  }
}

// Streams tiles [pos, end) of the flattened list (this wave's run): the K
// and V of tile i + 1 are loaded into the registers tile i frees (K after
// its scores, V after its store to LDS), so one tile is in flight while
// one is computed -- also across segment boundaries (block-table entries are
// looked up a tile ahead; the next segment's q is loaded when a piece ends).
// Each piece (run ∩ segment) ends with either the bf16 output (whole
// segment) or a partial record at seg + wave.  Returns the number of cut
// segments, whose (b, g, first run, last run) go to pend_*.
__device__ int m16_stream_run(const DecodeArgs& a, const TileScan& sc, int pos, int end, const Runs& runs,
                              int wave, M16Lds& L, int* prog, int wv, int (&pend_b)[2], int (&pend_g)[2],
                              int (&pend_w0)[2], int (&pend_w1)[2]) {
  const int lane = lane_id();
  const int col = lane & 15, grp = lane >> 4;
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

  uint4 qop[4];
  m16_load_q(a, c0.b, c0.g, qop);
  uint4 kr[16], vr[16];
  MfTile tl = mf_tile(a, c0.phys, c0.g, c0.t, c0.ctx);
  m16_issue_k(tl, kr);
  mf_issue_v(tl, vr);

  f32x4_t o[8];
#pragma unroll
  for (int n = 0; n < 8; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) o[n][r] = 0.f;
  float m = -INFINITY;  // reference max of the lane's row (log2 units)
  float l = 0.f;        // partial row sum over this lane's keys
  int piece_t0 = c0.t;
  int npend = 0;
  int i = pos;  // index of tile c0 in the flattened list

  while (true) {
    const bool seg_end = c0.t + 1 == c0.nt;
    const bool has_next = i + 1 < end;
    const bool next_ok = c1.live;

    // issue priority: a wave ahead of its slowest sibling yields
    {
      ++done;
      if (lane == 0) prog_set(&prog[wv], done);
      int slowest = done;
#pragma unroll
      for (int w = 0; w < kM16Waves; ++w) slowest = min(slowest, prog_get(&prog[w]));
      if (__builtin_amdgcn_readfirstlane(slowest) + 1 < done)
        __builtin_amdgcn_s_setprio(0);
      else
        __builtin_amdgcn_s_setprio(2);
    }

    // --- S^T = K Q^T (four independent 16-key chains)
    f32x4_t s[4];
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[ms][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
        s[ms] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf8(kr[4 * ms + ks]), as_bf8(qop[ks]), s[ms], 0, 0, 0);
    const MfTile t1 = mf_tile(a, c1.phys, c1.g, c1.t, c1.ctx);
    m16_issue_k(t1, kr);  // K of tile i + 1 into the registers just read

    // --- V of this tile into LDS, then V of tile i + 1 into its registers
    lds_order();
    mf_store_v_rows<kM16VStride>(L.vt, vr);
    mf_issue_v(t1, vr);
    lds_order();

    // --- online softmax (log2 domain, lazy rescale)
    const int key0 = c0.t * kTile;
    const int last0 = c0.ctx - a.ql;  // last key of query token 0
    if (key0 + kTile - 1 > last0 || tl.valid < kTile) {
      const int lim = min(last0 + (col >> a.gr_shift) - key0, tl.valid - 1);  // last visible key of the row
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * ms + 4 * grp + r;
          s[ms][r] = key <= lim ? s[ms][r] : -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[ms][r]);
    mt = xor32_max(xor16_max(mt)) * c;
    const float mnew = fmaxf(m, mt);
    const bool need = mnew > m + kMfLazy;  // also true for the first finite max
    if (__ballot(need) != 0) {
      const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;
      if (need) {
        l *= alpha;
        m = mnew;
      }
      if (grp == 0) L.rowf[col] = alpha;
      lds_order();
      const float4 al = *reinterpret_cast<const float4*>(&L.rowf[4 * grp]);
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        o[n][0] *= al.x;
        o[n][1] *= al.y;
        o[n][2] *= al.z;
        o[n][3] *= al.w;
      }
      lds_order();
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
      l = dot2_bf16(pb.x, kMfOnePair, l);
      l = dot2_bf16(pb.y, kMfOnePair, l);
      l = dot2_bf16(pb.z, kMfOnePair, l);
      l = dot2_bf16(pb.w, kMfOnePair, l);
      pop[ks] = as_bf8(pb);
    }

    // --- O += P V (dims 16 n + col, P's keys of k-step ks in LDS order)
    // lane (dim 16 n + col, group grp) gathers keys 32 ks + 16 r + 4 grp +
    // {0..3} with transposing reads: lane col points at dims 4 (col & 3) ..
    // +3 of key 32 ks + 16 r + 4 grp + col / 4 and receives its own dim
    const uint16_t* vsrc = L.vt + (4 * grp + (col >> 2)) * kM16VStride + 4 * (col & 3);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int n = 0; n < 8; ++n) {
        const bf16x8_t vop = tr_read_pair(vsrc + 32 * ks * kM16VStride + 16 * n, 16 * kM16VStride);
        o[n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pop[ks], vop, o[n], 0, 0, 0);
      }
    lds_order();

    // --- end of a piece: the output rows or a partial record
    if (seg_end || !has_next) {
      const float ltot = xor32_sum(xor16_sum(l));
      if (piece_t0 == 0 && seg_end) {
        // O / l -> bf16, staged in LDS as [row][128] for 16-byte stores
        if (grp == 0) L.rowf[col] = ltot > 0.f ? 1.f / ltot : 0.f;
        lds_order();
        uint16_t* stage = L.vt;
        const float4 inv = *reinterpret_cast<const float4*>(&L.rowf[4 * grp]);
        const float iv[4] = {inv.x, inv.y, inv.z, inv.w};
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int row = 4 * grp + r4;
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const __bf16 v = static_cast<__bf16>(o[n][r4] * iv[r4]);
            stage[row * kDim + 16 * n + col] = __builtin_bit_cast(uint16_t, v);
          }
        }
        lds_order();
        const int nreal = min(kM16Rows, a.ql << a.gr_shift);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int idx = lane + 64 * j;
          const int row = idx >> 4, ch = idx & 15;
          if (row < nreal) {
            const uint4 val = reinterpret_cast<const uint4*>(stage)[row * kChunks + ch];
            reinterpret_cast<uint4*>(a.out + vrow<kM16Rows, true>(a, c0.b, c0.g, row) * kDim)[ch] = val;
          }
        }
        lds_order();
      } else {
        const int seg = c0.b * a.hkv + c0.g;
        float* rec = a.ws + int64_t(seg + wave) * partial_floats(kM16Rows);
        const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, uint32_t(partial_floats(kM16Rows)) * 4u);
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int row = 4 * grp + r4;
#pragma unroll
          for (int n = 0; n < 8; ++n)
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[n][r4]), rr,
                                                  int(uint32_t(row * kDim + 16 * n + col) * 4u), 0, kCpolAgent);
        }
        if (grp == 0) {
          st_coherent(rec + kM16Rows * kDim + col, m);
          st_coherent(rec + kM16Rows * kDim + kM16Rows + col, ltot);
        }
        const int start = i - c0.t;  // first tile of the segment in the flattened list
        pend_b[npend] = c0.b;
        pend_g[npend] = c0.g;
        pend_w0[npend] = wave_of<kM16Waves>(runs, start);
        pend_w1[npend] = wave_of<kM16Waves>(runs, start + c0.nt - 1);
        ++npend;
      }
#pragma unroll
      for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[n][r] = 0.f;
      m = -INFINITY;
      l = 0.f;
      piece_t0 = c1.t;
      // q of the next segment (its loads are waited for by the next scores)
      if (next_ok) m16_load_q(a, c1.b, c1.g, qop);
    }
    if (!next_ok) break;
    tl = t1;
    c0 = c1;
    c1 = mf_next(a, c1, i + 2 < end);
    ++i;
  }
  return npend;
}

__global__ __launch_bounds__(kM16Waves * kWave, 1) void decode_mfma16_kernel(DecodeArgs a) {
  __shared__ M16Lds lds[kM16Waves];
  __shared__ int prog[kM16Waves];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = blockIdx.x * kM16Waves + wv;
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
  const Runs runs = make_runs<kM16Waves>(a, sc.total);
  const int pos = run_start<kM16Waves>(runs, wave);
  const int end = run_start<kM16Waves>(runs, wave + 1);
  if (pos >= end) {
    if (lane_id() == 0) prog_set(&prog[wv], 1 << 30);
    zero_empty_rows();
    return;
  }

  int pend_b[2], pend_g[2], pend_w0[2], pend_w1[2];
  const int npend =
      m16_stream_run(a, sc, pos, end, runs, wave, lds[wv], prog, wv, pend_b, pend_g, pend_w0, pend_w1);
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
        m16_merge(a, seg, pend_b[i], pend_g[i], pend_w0[i], pend_w1[i]);
        if (lane_id() == 0) __hip_atomic_store(a.counters + seg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  zero_empty_rows();
}

}  // namespace

hipError_t launch_decode_mfma16(const DecodeArgs& a, hipStream_t s) {
  if (a.k_new != nullptr) return hipErrorInvalidValue;  // several rows: no appended token
  const unsigned blocks = unsigned((a.n_waves + kM16Waves - 1) / kM16Waves);
  hipLaunchKernelGGL(decode_mfma16_kernel, dim3(blocks), dim3(kM16Waves * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
