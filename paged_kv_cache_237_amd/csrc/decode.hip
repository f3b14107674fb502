// Paged decode attention with a split-context merge (gfx950).
//
// What it computes (CSDN essay comparing nanoVLLM and vLLM, first and third
// sections; the vLLM decode-kernel description in the same essay): for each
// sequence b and query head h, softmax(scale * q K^T) V over the
// context_lens[b] cached tokens of kv head h / G, read through the sequence's
// block table.
//
// Work decomposition.  Every (sequence, kv head) pair is a "segment" of
// ceil(ctx/64) tiles of 64 tokens.  All segments are laid end to end and the
// resulting list of tiles is cut into n_waves runs, one per wave, whose
// lengths are set by the XCD the wave runs on (shorter on the slower,
// odd-numbered XCDs), whatever the length mix.  A workgroup holds the waves
// of one CU; the CU's waves share its bandwidth but are not served evenly, so
// a wave that gets ahead of its slowest sibling yields issue priority
// (s_setprio) and the CU's runs end together.
//
// Several query rows per sequence (the causal decode of a few new tokens at
// once): the ql rows x G heads of one (sequence, kv head) are the kernel's
// "virtual heads" (G template = their count rounded up to a power of two);
// virtual head v is query row v / G_real and sees the keys up to
// ctx - ql + v / G_real, an additive mask per head.  With one row per
// sequence (Causal = false) the mask and the general row addressing
// compile away.
//
// Appending the step's token (pa_decode_append): the newest position of each
// sequence is not read from the cache.  The positions before it are streamed
// as above; whichever wave finalises a (sequence, kv head) -- the one that
// streamed it whole, the last one to arrive at its merge, or, for a context
// of one token, the wave that writes its empty rows -- folds the new token in
// as one more partial state (score q.k_new, weight 2^(score - M), value
// v_new) and writes k_new / v_new into the cache at that position.  No wave
// reads that position during the call, so the store needs no ordering; it
// replaces the separate store launch of a decode step.
//
// A run streams its tiles as one software pipeline: the K loads of the next
// tile are issued as soon as the current tile's scores are computed and its V
// loads as soon as the current PV is done, also across segment boundaries
// (the next segment's q and block-table entry are fetched a tile ahead, the
// block table and context lengths with scalar loads), so the wave always has
// a tile's worth of loads in flight.
//
// A run that covers a whole segment writes the bf16 output at once.  A
// segment cut between runs leaves one partial state (m, l, u) per run in the
// workspace; each contributing wave then bumps the segment's counter
// (agent-scope atomic once its record stores have completed) and the last one
// to arrive merges them:
// M = max m_i,  L = sum 2^(m_i-M) l_i,  o = sum 2^(m_i-M) u_i / L  (the
// split-context form of the online softmax), and resets the counter to zero,
// so the workspace counters are zero again after every call.
// The partial of segment s written by wave w goes to record s + w: segments
// and runs are both contiguous intervals of the tile list, so two distinct
// non-empty (segment, run) intersections never share s + w.
//
// One tile, one wave (G query heads of one kv head):
//   * K of the tile is 16 loads of 16 B per lane, lane = token: the cache
//     stores K as [chunk][row][8], so each load is one contiguous KiB.
//   * V of the tile is 16 loads of 16 B, 16 lanes per token row, 4 rows per
//     load (again one contiguous KiB).
//   * QK: lane t computes the G scores of its token with v_dot2c_f32_bf16
//     against q held in LDS (broadcast reads) -- no cross-lane reduction.
//   * softmax: one wave max per head per tile (DPP rows + 4 lane reads);
//     scores are kept in the log2 domain (scale * log2 e folded in).
//   * PV: p goes through LDS to the (row, chunk) layout of V; fp32 FMAs;
//     the 4 row-partials are folded once per piece.
// Memory traffic is the K and V rows of the context read once, plus q and
// out; the kernel is bound by HBM bandwidth.
#include <math.h>

#include <mutex>
#include <vector>

#include "decode_common.hpp"
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

template <int G>
struct GroupShape {
  static constexpr int kWaves = decode_group_waves(G);  // one workgroup per CU
  static constexpr int kThreads = kWaves * kWave;
};

// The appended token of (sequence b, kv head g), position ctx-1: every lane
// holds 16-byte chunk (lane & 15) of its K and V rows.  ok is false when the
// sequence is empty or the position's block-table entry lies outside the
// pool: the token then neither counts nor is stored (a block outside the pool
// is masked in pa_decode too).  new_token_load only issues the loads (their
// addresses depend on b and g alone), so callers start it early and use the
// rows later; new_token_store writes them into the cache (lanes 0..15).
struct NewToken {
  bool ok;
  int phys, row;
  uint4 kc, vc;
};

__device__ __forceinline__ NewToken new_token_load(const DecodeArgs& a, int b, int g) {
  const int j = lane_id() & 15;
  const int64_t src = (int64_t(b) * a.hkv + g) * kChunks + j;
  NewToken tk;
  tk.kc = a.k_new[src];
  tk.vc = a.v_new[src];
  const int c = clamp_ctx(a, ld_uniform(a.ctx_lens, b));
  const int p = c - 1;
  tk.phys = c >= 1 ? ld_uniform(a.block_table, int64_t(b) * a.mbps + p / kBlock) : -1;
  tk.row = p % kBlock;
  tk.ok = tk.phys >= 0 && int64_t(tk.phys) < a.num_blocks;
  return tk;
}

__device__ __forceinline__ void new_token_store(const DecodeArgs& a, const NewToken& tk, int g) {
  const int lane = lane_id();
  if (tk.ok && lane < 16) {
    const int64_t bh = int64_t(tk.phys) * a.hkv + g;
    a.k_store[(bh * kChunks + lane) * kBlock + tk.row] = tk.kc;
    a.v_store[(bh * kBlock + tk.row) * kChunks + lane] = tk.vc;
  }
}

__device__ __forceinline__ NewToken new_token(const DecodeArgs& a, int b, int g) {
  const NewToken tk = new_token_load(a, b, g);
  new_token_store(a, tk, g);
  return tk;
}

// Score (log2 units) of a query against the appended key, given the lane's
// chunk (lane & 15) of each: every 16-lane row of the wave sums the 16 chunk
// products, so every lane gets the score.
__device__ __forceinline__ float new_token_score(const DecodeArgs& a, const uint4& qc, const uint4& kc) {
  return row16_sum(dot8_bf16(qc, kc, 0.f)) * a.scale_log2;
}

// Merge the partial records of segment `seg` written by waves w0..w1 into
// its G output rows (lane = 2 dims).  One pass with an online rescale; the
// loads of four records are issued together.  With Append, the new token is
// folded in last.
template <int G, bool Causal, bool Append>
__device__ void merge_segment(const DecodeArgs& a, int seg, int b, int g, int w0, int w1) {
  const int lane = lane_id();
  float M[G], L[G], U0[G], U1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = -INFINITY;
    L[h] = U0[h] = U1[h] = 0.f;
  }
  // the appended token's rows and the queries' chunks, loaded under the records
  NewToken tk;
  uint4 qc[G];
  uint32_t vw = 0u;
  if constexpr (Append) {
    tk = new_token_load(a, b, g);
    vw = reinterpret_cast<const uint32_t*>(a.v_new + (int64_t(b) * a.hkv + g) * kChunks)[lane];
#pragma unroll
    for (int h = 0; h < G; ++h)
      qc[h] = reinterpret_cast<const uint4*>(a.q + vrow<G, Causal>(a, b, g, h) * kDim)[lane & 15];
  }
  for (int w = w0; w <= w1; w += 4) {
    float mm[4][G], ll[4][G], ua[4][G], ub[4][G];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool have = w + j <= w1;
      const float* rec = a.ws + int64_t(seg + (have ? w + j : w0)) * partial_floats(G);
      const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, uint32_t(partial_floats(G)) * 4u);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mm[j][h] = have ? ld_coherent(rec + G * kDim + h) : -INFINITY;
        ll[j][h] = have ? ld_coherent(rec + G * kDim + G + h) : 0.f;
        ld_coherent2(rr, uint32_t(h * kDim + 2 * lane) * 4u, ua[j][h], ub[j][h]);
        if (!have) ua[j][h] = ub[j][h] = 0.f;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mn = fmaxf(M[h], mm[j][h]);
        const float ref = mn == -INFINITY ? 0.f : mn;
        const float sa = __builtin_amdgcn_exp2f(M[h] - ref);
        const float sb = __builtin_amdgcn_exp2f(mm[j][h] - ref);
        L[h] = L[h] * sa + ll[j][h] * sb;
        U0[h] = U0[h] * sa + ua[j][h] * sb;
        U1[h] = U1[h] * sa + ub[j][h] * sb;
        M[h] = mn;
      }
  }
  if constexpr (Append) {
    new_token_store(a, tk, g);
    if (tk.ok) {
      const float v0 = bf16_lo(vw), v1 = bf16_hi(vw);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float sn = new_token_score(a, qc[h], tk.kc);
        const float mn = fmaxf(M[h], sn);
        const float sa = __builtin_amdgcn_exp2f(M[h] - mn);
        const float sb = __builtin_amdgcn_exp2f(sn - mn);
        L[h] = L[h] * sa + sb;
        U0[h] = U0[h] * sa + v0 * sb;
        U1[h] = U1[h] * sa + v1 * sb;
        M[h] = mn;
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (!vreal<Causal>(a, h)) continue;
    const float inv = L[h] > 0.f ? 1.f / L[h] : 0.f;
    uint32_t* out = reinterpret_cast<uint32_t*>(a.out + vrow<G, Causal>(a, b, g, h) * kDim);
    out[lane] = pack_bf16x2(U0[h] * inv, U1[h] * inv);
  }
}

// Buffer descriptors and offsets of one tile's K and V loads.
//   K: lane = token; rows past the context get an out-of-range offset and
//      load zeros (their scores are masked).
//   V: the buffer ends after the last valid row, so rows past the context
//      load zeros too (they may hold NaN patterns in memory, which must not
//      reach p * v).
struct TileLoads {
  __amdgpu_buffer_rsrc_t rk, rv;
  uint32_t koff, voff;
  int valid;  // tokens of the tile inside the context (0 for a bad block entry)
};

__device__ __forceinline__ TileLoads tile_loads(const DecodeArgs& a, int phys, int g, int t, int ctx) {
  const int lane = lane_id();
  TileLoads tl;
  const bool ok = phys >= 0 && int64_t(phys) < a.num_blocks;
  tl.valid = ok ? min(kTile, ctx - t * kTile) : 0;
  const int r0 = (t & 3) * kTile;
  const int64_t bh = (ok ? int64_t(phys) : 0) * a.hkv + g;  // block-head tile index
  tl.rk = make_rsrc(a.k_cache + bh * (kChunks * kBlock), 65536u);
  tl.rv = make_rsrc(a.v_cache + bh * (kBlock * kChunks), uint32_t(r0 + tl.valid) * 256u);
  tl.koff = lane < tl.valid ? uint32_t(r0 + lane) * 16u : kOutOfRange;
  tl.voff = uint32_t((r0 + (lane >> 4)) * kChunks + (lane & 15)) * 16u;
  return tl;
}

__device__ __forceinline__ void issue_k(const TileLoads& tl, uint4 (&kr)[kChunks]) {
#pragma unroll
  for (int c = 0; c < kChunks; ++c) kr[c] = buf_load16_stream(tl.rk, tl.koff, uint32_t(c) * 4096u);
}

__device__ __forceinline__ void issue_v(const TileLoads& tl, uint4 (&vr)[16]) {
#pragma unroll
  for (int k = 0; k < 16; ++k) vr[k] = buf_load16_stream(tl.rv, tl.voff + uint32_t(k) * 1024u, 0u);
}

// Streams tiles [pos, end) of the flattened list (this wave's run) as one
// software pipeline: the K loads of the next tile are issued as soon as the
// current tile's scores are computed and its V loads as soon as the current
// PV is done, also across segment boundaries (the next segment's q and
// block-table entry are fetched a tile ahead), so the wave always has a
// tile's worth of loads in flight.  Each piece (run ∩ segment) ends with a
// fold of the row partials and either the bf16 output (whole segment) or a
// partial record at seg + wave.  Returns the number of cut segments, whose
// (b, g, first run, last run) are stored in pend_*.
template <int G, bool Causal, bool Append>
__device__ int stream_run(const DecodeArgs& a, const TileScan& sc, int pos, int end, const Runs& runs, int wave, uint4* q_lds,
                          float* p_lds, int* prog, int wv, int (&pend_b)[2], int (&pend_g)[2],
                          int (&pend_w0)[2], int (&pend_w1)[2]) {
  constexpr int NW = GroupShape<G>::kWaves;
  int done = 0;  // tiles streamed by this wave
  const int lane = lane_id();
  constexpr int kQPerLane = (G * kChunks + kWave - 1) / kWave;

  int b, before;
  locate<Append>(a, sc, pos, b, before);
  if (b >= a.batch) return 0;
  int nt = tiles_of(stream_ctx<Append>(a, a.ctx_lens[b]));
  const int off = pos - before * a.hkv;
  int g = off / nt;
  int t = off - g * nt;
  int ctx = stream_ctx<Append>(a, a.ctx_lens[b]);
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  t = __builtin_amdgcn_readfirstlane(t);
  nt = __builtin_amdgcn_readfirstlane(nt);
  ctx = __builtin_amdgcn_readfirstlane(ctx);

  // prologue: q of the first segment, loads of the first tile
  if constexpr (!Causal) {
    // one query row per sequence: the G heads are contiguous
    const uint4* qsrc = reinterpret_cast<const uint4*>(a.q + vrow<G, Causal>(a, b, g, 0) * kDim);
    for (int i = lane; i < G * kChunks; i += kWave) q_lds[i] = qsrc[i];
  } else {
    for (int i = lane; i < G * kChunks; i += kWave) {
      const int v = i / kChunks;
      q_lds[i] = vreal<Causal>(a, v) ? reinterpret_cast<const uint4*>(a.q + vrow<G, Causal>(a, b, g, v) * kDim)[i % kChunks]
                             : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  TileLoads cur = tile_loads(a, ld_uniform(a.block_table, int64_t(b) * a.mbps + (t >> 2)), g, t, ctx);
  uint4 kr[kChunks], vr[16];
  issue_k(cur, kr);
  issue_v(cur, vr);
  __builtin_amdgcn_wave_barrier();

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  const int vrow4 = lane >> 4;  // row within a 4-row V load
  int piece_t0 = t;            // first tile of the current piece
  int npend = 0;

  for (; pos < end; ++pos) {
    // --- where the next tile is (same segment, or the next non-empty one)
    const bool has_next = pos + 1 < end;
    int nb = b, ng = g, ntt = t + 1, nnt = nt, nctx = ctx;
    const bool seg_end = t + 1 == nt;
    if (seg_end && has_next) {
      ntt = 0;
      if (++ng == a.hkv) {
        ng = 0;
        nctx = 0;
        do {
          nb = __builtin_amdgcn_readfirstlane(nb + 1);
          nctx = nb < a.batch ? stream_ctx<Append>(a, ld_uniform(a.ctx_lens, nb)) : 0;
          nnt = nb < a.batch ? tiles_of(nctx) : 1;
        } while (nnt == 0);
      }
    }
    const bool next_ok = has_next && nb < a.batch;
    // the appended token of a segment this wave streams whole: its rows (and
    // its slot) are loaded under the segment's last tile, for the fold at the
    // end of the piece
    NewToken tk_next;
    tk_next.ok = false;
    if constexpr (Append) {
      if (seg_end && piece_t0 == 0) tk_next = new_token_load(a, b, g);
    }
    // the next segment's q, loaded under this segment's last tile
    uint4 qn[kQPerLane];
    if (seg_end && next_ok) {
      if constexpr (!Causal) {
        const uint4* qsrc = reinterpret_cast<const uint4*>(a.q + vrow<G, Causal>(a, nb, ng, 0) * kDim);
#pragma unroll
        for (int j = 0; j < kQPerLane; ++j) {
          const int i = lane + j * kWave;
          qn[j] = i < G * kChunks ? qsrc[i] : make_uint4(0u, 0u, 0u, 0u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < kQPerLane; ++j) {
          const int i = lane + j * kWave;
          const int v = i / kChunks;
          qn[j] = i < G * kChunks && vreal<Causal>(a, v)
                      ? reinterpret_cast<const uint4*>(a.q + vrow<G, Causal>(a, nb, ng, v) * kDim)[i % kChunks]
                      : make_uint4(0u, 0u, 0u, 0u);
        }
      }
    }
    // past the end of the run the "next tile" has no block: its loads are
    // all out of range and return zeros without touching memory (issuing
    // them unconditionally lets the registers be reused in place)
    const int nphys = next_ok ? ld_uniform(a.block_table, int64_t(nb) * a.mbps + (ntt >> 2)) : -1;

    // The waves of a CU share its bandwidth but are not served evenly; a
    // wave ahead of its slowest sibling yields issue priority, so that they
    // progress together and the CU finishes its runs at once.
    {
      ++done;
      if (lane == 0) prog_set(&prog[wv], done);
      int slowest = done;
#pragma unroll
      for (int w = 0; w < NW; ++w) slowest = min(slowest, prog_get(&prog[w]));
      if (__builtin_amdgcn_readfirstlane(slowest) + 1 < done)
        __builtin_amdgcn_s_setprio(0);
      else
        __builtin_amdgcn_s_setprio(2);
    }

    // --- scores of the current tile (q from LDS, broadcast reads)
    asm volatile("" ::: "memory");
    const bool kval = lane < cur.valid;
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
    // Two chunks of q per step; the scheduling barrier keeps the compiler
    // from pulling all G*64 dwords of q into registers at once.
#pragma unroll
    for (int c = 0; c < kChunks; c += 2) {
      uint4 qa[G], qb[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        qa[h] = q_lds[h * kChunks + c];
        qb[h] = q_lds[h * kChunks + c + 1];
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = dot8_bf16(qb[h], kr[c + 1], dot8_bf16(qa[h], kr[c], s[h]));
      __builtin_amdgcn_sched_barrier(0);
    }
    // K of the next tile into the registers just freed
    const TileLoads nxt = tile_loads(a, nphys, ng, ntt, nctx);
    issue_k(nxt, kr);
    __builtin_amdgcn_sched_barrier(0);

    // --- online softmax (log2 domain)
    const int key = t * kTile + lane;
    const int last0 = ctx - a.ql;  // last key of query row 0 of the sequence
#pragma unroll
    for (int h = 0; h < G; ++h) {
      // additive mask: keeps the dot products unconditional (a select on
      // kval would let the compiler sink them into a branch); with several
      // query rows per sequence, row h >> gr_shift sees keys up to
      // last0 + that row
      const bool vis = Causal ? kval && key <= last0 + (h >> a.gr_shift) : kval;
      const float sh = fmaf(s[h], a.scale_log2, vis ? 0.f : -INFINITY);
      const float mn = fmaxf(m[h], wave_max(sh));
      const float ref = mn == -INFINITY ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m[h] - ref);
      const float p = __builtin_amdgcn_exp2f(sh - ref);
      l[h] = l[h] * alpha + p;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      m[h] = mn;
      p_lds[lane * G + h] = p;
    }
    __builtin_amdgcn_wave_barrier();

    // --- PV of the current tile
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float* pp = p_lds + (4 * k + vrow4) * G;
      float pv[G];
#pragma unroll
      for (int h = 0; h < G; ++h) pv[h] = pp[h];
      float v[8];
      unpack8(vr[k], v);
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(pv[h], v[e], acc[h][e]);
      }
      if (k & 1) __builtin_amdgcn_sched_barrier(0);
    }
    // V of the next tile into the registers just freed
    issue_v(nxt, vr);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_wave_barrier();

    // --- end of a piece: fold, then the output row or a partial record
    if (seg_end || !has_next) {
      float lsum[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        // the 4 row-partials (lanes l, l^16, l^32, l^48 hold the same dims)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          float x = acc[h][e];
          x = xor16_sum(x);
          acc[h][e] = xor32_sum(x);
        }
        lsum[h] = wave_sum(l[h]);
      }
      if (piece_t0 == 0 && seg_end) {
        if constexpr (Append) {
          // lane holds dims 8*(lane & 15) .. +7 of every head; q is still
          // this segment's in LDS
          const NewToken tk = tk_next;
          new_token_store(a, tk, g);
          if (tk.ok) {
            float vn[8];
            unpack8(tk.vc, vn);
#pragma unroll
            for (int h = 0; h < G; ++h) {
              const float sn = new_token_score(a, q_lds[h * kChunks + (lane & 15)], tk.kc);
              const float mn = fmaxf(m[h], sn);
              const float sa = __builtin_amdgcn_exp2f(m[h] - mn);
              const float sb = __builtin_amdgcn_exp2f(sn - mn);
              lsum[h] = lsum[h] * sa + sb;
#pragma unroll
              for (int e = 0; e < 8; ++e) acc[h][e] = acc[h][e] * sa + vn[e] * sb;
            }
          }
        }
        if (lane < 16) {
#pragma unroll
          for (int h = 0; h < G; ++h) {
            if (!vreal<Causal>(a, h)) continue;
            const float inv = lsum[h] > 0.f ? 1.f / lsum[h] : 0.f;
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = acc[h][e] * inv;
            uint4* dst = reinterpret_cast<uint4*>(a.out + vrow<G, Causal>(a, b, g, h) * kDim);
            dst[lane] = pack8(o);
          }
        }
      } else {
        const int seg = b * a.hkv + g;
        float* rec = a.ws + int64_t(seg + wave) * partial_floats(G);
        if (lane < 16) {
          const __amdgpu_buffer_rsrc_t rr = make_rsrc(rec, uint32_t(partial_floats(G)) * 4u);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const uint32_t off = uint32_t(h * kDim + lane * 8) * 4u;
            st_coherent4(rr, off, acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
            st_coherent4(rr, off + 16u, acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
          }
        }
        if (lane < G) {
          float mv = m[0], lv = lsum[0];
#pragma unroll
          for (int h = 1; h < G; ++h)
            if (lane == h) { mv = m[h]; lv = lsum[h]; }
          st_coherent(rec + G * kDim + lane, mv);
          st_coherent(rec + G * kDim + G + lane, lv);
        }
        const int start = pos - t;  // first tile of the segment in the flattened list
        pend_b[npend] = b;
        pend_g[npend] = g;
        pend_w0[npend] = wave_of<NW>(runs, start);
        pend_w1[npend] = wave_of<NW>(runs, start + nt - 1);
        ++npend;
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
      }
      piece_t0 = ntt;
      if (next_ok) {
        // q of the next segment (loaded a tile ago)
#pragma unroll
        for (int j = 0; j < kQPerLane; ++j) {
          const int i = lane + j * kWave;
          if (i < G * kChunks) q_lds[i] = qn[j];
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
    if (!next_ok) break;
    b = nb;
    g = ng;
    t = ntt;
    nt = nnt;
    ctx = nctx;
    cur = nxt;
  }
  return npend;
}

template <int G, bool Causal, bool Append>
__global__ __launch_bounds__(GroupShape<G>::kThreads) void decode_split_kernel(DecodeArgs a) {
  constexpr int NW = GroupShape<G>::kWaves;
  __shared__ uint4 q_lds[NW][G * kChunks];
  __shared__ float p_lds[NW][kTile * G];
  __shared__ int prog[NW];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = blockIdx.x * NW + wv;
  if (lane_id() == 0) prog[wv] = 0;
  __syncthreads();

  // Empty contexts have no tiles: their output rows are zero.  With Append,
  // a context of one token streams nothing either: its rows are that token's
  // V (the softmax of a single score is 1), and the token is stored here.
  // Written on the way out, so that no wave waits for it before streaming.
  auto zero_empty_rows = [&]() {
    if (wave >= a.n_waves) return;
    for (int bb = wave; bb < a.batch; bb += a.n_waves) {
      const int c = clamp_ctx(a, ld_uniform(a.ctx_lens, bb));
      if (Append && c == 1) {
        for (int gg = 0; gg < a.hkv; ++gg) {
          const NewToken tk = new_token(a, bb, gg);
          if (lane_id() < 16) {
            uint4* o = reinterpret_cast<uint4*>(a.out + (int64_t(bb) * a.hq + int64_t(gg) * a.gr) * kDim);
            for (int hh = 0; hh < a.gr; ++hh) o[hh * kChunks + lane_id()] = tk.ok ? tk.vc : make_uint4(0u, 0u, 0u, 0u);
          }
        }
        continue;
      }
      if (c != 0) continue;
      uint32_t* o = reinterpret_cast<uint32_t*>(a.out + int64_t(bb) * a.ql * a.hq * kDim);
      for (int i = lane_id(); i < a.ql * a.hq * (kDim / 2); i += kWave) o[i] = 0u;
    }
  };

  const TileScan sc = scan_tiles<Append>(a);
  const Runs runs = make_runs<NW>(a, sc.total);
  const int pos = run_start<NW>(runs, wave);
  const int end = run_start<NW>(runs, wave + 1);
  if (pos >= end) {
    if (lane_id() == 0) prog_set(&prog[wv], 1 << 30);
    zero_empty_rows();
    return;
  }

  // A run cuts at most two segments (its first and its last); their arrivals
  // are counted once the whole run has been streamed, so the record stores
  // never stall the loads.
  int pend_b[2], pend_g[2], pend_w0[2], pend_w1[2];
  const int npend = stream_run<G, Causal, Append>(a, sc, pos, end, runs, wave, q_lds[wv], p_lds[wv], prog, wv, pend_b,
                                  pend_g, pend_w0, pend_w1);
  // a finished wave no longer holds its siblings back
  if (lane_id() == 0) prog_set(&prog[wv], 1 << 30);
  __builtin_amdgcn_s_setprio(0);

  // Arrivals, and why the last arriver sees every record.  The records are
  // written with SC1 stores and read with SC1 loads: on gfx950 these are
  // coherent across the XCDs' private L2s (an SC1 store is not kept dirty in
  // the L2, an SC1 load does not hit a line another XCD may have written).
  // s_waitcnt vmcnt(0) waits until this wave's record stores are complete
  // (acknowledged by the memory side) before the arrival is issued; the
  // arrival is an atomic performed at the memory side, and a wave merges
  // only after its own atomic returned the count of every other arrival, so
  // every contributing wave's records were complete before the merging wave
  // issues its first record load.  In the language memory model this needs a
  // release by the writers and an acquire by the merger at agent scope,
  // which the compiler implements as a write-back and an invalidate of the
  // whole L2 of an XCD; measured on 8 x 131,072 tokens that made the launch
  // 1.8x slower (720 -> 1,270 us) even with the acquire only in the merging
  // waves, so the ordering rests on the ISA's guarantees above.
  if (npend > 0) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's record stores have completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    for (int i = 0; i < npend; ++i) {
      const int seg = pend_b[i] * a.hkv + pend_g[i];
      int prev = 0;
      if (lane_id() == 0)
        prev = __hip_atomic_fetch_add(a.counters + seg, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      prev = __builtin_amdgcn_readfirstlane(prev);
      if (prev == pend_w1[i] - pend_w0[i]) {
        merge_segment<G, Causal, Append>(a, seg, pend_b[i], pend_g[i], pend_w0[i], pend_w1[i]);
        if (lane_id() == 0)
          __hip_atomic_store(a.counters + seg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  zero_empty_rows();
}

template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
  constexpr int NW = GroupShape<G>::kWaves;
  const unsigned split_blocks = unsigned((a.n_waves + NW - 1) / NW);
  // one query row per sequence needs no causal mask inside the context; the
  // appended token is supported with one query row only
  if (a.k_new != nullptr) {
    if (a.ql != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((decode_split_kernel<G, false, true>), dim3(split_blocks), dim3(GroupShape<G>::kThreads), 0,
                       s, a);
  } else if (a.ql == 1) {
    hipLaunchKernelGGL((decode_split_kernel<G, false, false>), dim3(split_blocks), dim3(GroupShape<G>::kThreads), 0,
                       s, a);
  } else {
    hipLaunchKernelGGL((decode_split_kernel<G, true, false>), dim3(split_blocks), dim3(GroupShape<G>::kThreads), 0,
                       s, a);
  }
  return hipGetLastError();
}

// Workspace of the allocation-free decode step (pa_decode_append_noalloc),
// for callers that cannot allocate device memory: the same partial records
// and arrival counters as a caller's workspace, in an array of fixed size
// that each device holds from the library's load until the process ends.
// Host code never passes the array's name to a kernel (on the host it only
// names the symbol); it uses the device address that hipGetSymbolAddress
// returns, found once per device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

__global__ __launch_bounds__(256) void zero16_kernel(uint4* p, int64_t n16) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n16; i += int64_t(gridDim.x) * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t noalloc_scratch(hipStream_t s, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::vector<void*> addr;  // per device; null until looked up
  std::lock_guard<std::mutex> lock(mu);
  if (dev >= 0 && size_t(dev) < addr.size() && addr[dev] != nullptr) {
    *ptr = addr[dev];
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return e;
  if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
  // The counters must start at zero: the whole array is cleared once, by a
  // kernel on the caller's stream (no memset node, in case the stream is
  // being captured); every call leaves its counters at zero again.
  hipLaunchKernelGGL(zero16_kernel, dim3(1024), dim3(256), 0, s, static_cast<uint4*>(p),
                     int64_t(kNoAllocScratchBytes / 16));
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (size_t(dev) >= addr.size()) addr.resize(size_t(dev) + 1, nullptr);
  addr[dev] = p;
  *ptr = p;
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int group, hipStream_t s) {
  switch (group) {
    case 1: return launch_decode_g<1>(a, s);
    case 2: return launch_decode_g<2>(a, s);
    case 4: return launch_decode_g<4>(a, s);
    case 8: return launch_decode_g<8>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
