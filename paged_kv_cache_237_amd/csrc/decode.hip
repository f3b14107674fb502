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
// resulting list of tiles is cut into n_waves equal runs, one per wave, so
// every wave streams the same number of bytes whatever the length mix.  A run
// that covers a whole segment writes the bf16 output at once.  A segment cut
// between runs leaves one partial state (m, l, u) per run in the workspace;
// each contributing wave then bumps the segment's counter (agent-scope
// atomic after a release fence) and the last one to arrive merges them:
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
//     the 4 row-partials are folded once per run.
// Memory traffic is the K and V rows of the context read once, plus q and
// out; the kernel is bound by HBM bandwidth.
#include <math.h>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

constexpr int kWavesPerWG = 4;

__device__ __forceinline__ int clamp_ctx(const DecodeArgs& a, int n) {
  const int cap = a.mbps * kBlock;
  return n < 0 ? 0 : (n > cap ? cap : n);
}

__device__ __forceinline__ int tiles_of(int n) { return (n + kTile - 1) / kTile; }

// Number of tiles of all segments (identical in every lane).
__device__ int total_tiles(const DecodeArgs& a) {
  const int lane = lane_id();
  int tot = 0;
  for (int b0 = 0; b0 < a.batch; b0 += kWave) {
    const int b = b0 + lane;
    const int nt = b < a.batch ? tiles_of(clamp_ctx(a, a.ctx_lens[b])) : 0;
    tot += wave_sum_i(nt);
  }
  return tot * a.hkv;
}

// Sequence holding tile `pos` of the flattened list and the tiles of all
// sequences before it.
__device__ void locate(const DecodeArgs& a, int pos, int& b_out, int& before_out) {
  const int lane = lane_id();
  int base = 0;
  for (int b0 = 0; b0 < a.batch; b0 += kWave) {
    const int b = b0 + lane;
    const int nt = b < a.batch ? tiles_of(clamp_ctx(a, a.ctx_lens[b])) : 0;
    const int incl = wave_incl_scan(nt);
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

// Partial records cross XCDs (each XCD has its own L2), so they are written
// and read with agent-scope atomic accesses, which the hardware keeps coherent
// by themselves (no whole-L2 writeback or invalidate is needed, unlike a
// device-scope fence).
__device__ __forceinline__ void st_coherent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_coherent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the partial records of segment `seg` written by waves w0..w1 into
// its G output rows (lane = 2 dims).  One pass with an online rescale; the
// loads of four records are issued together.
template <int G>
__device__ void merge_segment(const DecodeArgs& a, int seg, int b, int g, int w0, int w1) {
  const int lane = lane_id();
  const int hq = a.hkv * G;
  float M[G], L[G], U0[G], U1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    M[h] = -INFINITY;
    L[h] = U0[h] = U1[h] = 0.f;
  }
  for (int w = w0; w <= w1; w += 4) {
    float mm[4][G], ll[4][G], ua[4][G], ub[4][G];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool have = w + j <= w1;
      const float* rec = a.ws + int64_t(seg + (have ? w + j : w0)) * partial_floats(G);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        mm[j][h] = have ? ld_coherent(rec + G * kDim + h) : -INFINITY;
        ll[j][h] = have ? ld_coherent(rec + G * kDim + G + h) : 0.f;
        ua[j][h] = have ? ld_coherent(rec + h * kDim + 2 * lane) : 0.f;
        ub[j][h] = have ? ld_coherent(rec + h * kDim + 2 * lane + 1) : 0.f;
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
  uint32_t* out = reinterpret_cast<uint32_t*>(a.out + (int64_t(b) * hq + g * G) * kDim);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float inv = L[h] > 0.f ? 1.f / L[h] : 0.f;
    out[h * (kDim / 2) + lane] = pack_bf16x2(U0[h] * inv, U1[h] * inv);
  }
}

template <int G>
__device__ void decode_run(const DecodeArgs& a, int b, int g, int t_lo, int t_hi, int nt, int wave,
                           uint4* q_lds, float* p_lds) {
  const int lane = lane_id();
  b = __builtin_amdgcn_readfirstlane(b);
  g = __builtin_amdgcn_readfirstlane(g);
  t_lo = __builtin_amdgcn_readfirstlane(t_lo);
  t_hi = __builtin_amdgcn_readfirstlane(t_hi);
  const int hq = a.hkv * G;
  const int ctx = __builtin_amdgcn_readfirstlane(clamp_ctx(a, a.ctx_lens[b]));

  // q of the G heads of this kv head: G*256 bytes, staged once per run.
  const uint4* qsrc = reinterpret_cast<const uint4*>(a.q + (int64_t(b) * hq + g * G) * kDim);
  for (int i = lane; i < G * kChunks; i += kWave) q_lds[i] = qsrc[i];
  __builtin_amdgcn_wave_barrier();

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  const int vrow = lane >> 4;   // row within a 4-row V load
  const int vchunk = lane & 15; // 16-byte chunk within a V row

  for (int t = t_lo; t < t_hi; ++t) {
    // q stays in LDS: re-read it every tile (broadcast reads) instead of
    // letting the compiler hoist G*64 registers of it out of the loop.
    asm volatile("" ::: "memory");
    const int phys = a.block_table[int64_t(b) * a.mbps + (t >> 2)];
    const bool ok = phys >= 0 && int64_t(phys) < a.num_blocks;
    const int valid = ok ? min(kTile, ctx - t * kTile) : 0;
    const int r0 = (t & 3) * kTile;
    const int64_t bh = (ok ? int64_t(phys) : 0) * a.hkv + g;  // block-head tile index
    // K: lane = token; rows past the context get an out-of-range offset and
    // load zeros (their scores are masked below).  V: the buffer ends after
    // the last valid row, so rows past the context load zeros too (they may
    // hold NaN patterns in memory, which must not reach p * v).
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_cache + bh * (kChunks * kBlock), 65536u);
    const __amdgpu_buffer_rsrc_t rv =
        make_rsrc(a.v_cache + bh * (kBlock * kChunks), uint32_t(r0 + valid) * 256u);
    const bool kval = lane < valid;
    const uint32_t koff = kval ? uint32_t(r0 + lane) * 16u : kOutOfRange;
    const uint32_t voff = uint32_t((r0 + vrow) * kChunks + vchunk) * 16u;
    uint4 kr[kChunks], vr[16];
#pragma unroll
    for (int c = 0; c < kChunks; ++c) kr[c] = buf_load16(rk, koff, uint32_t(c) * 4096u);
#pragma unroll
    for (int k = 0; k < 16; ++k) vr[k] = buf_load16(rv, voff + uint32_t(k) * 1024u, 0u);

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

#pragma unroll
    for (int h = 0; h < G; ++h) {
      // additive mask: keeps the dot products unconditional (a select on
      // kval would let the compiler sink them into a branch)
      const float sh = fmaf(s[h], a.scale_log2, kval ? 0.f : -INFINITY);
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

#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float* pp = p_lds + (4 * k + vrow) * G;
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
    __builtin_amdgcn_wave_barrier();
  }

  // Fold the 4 row-partials (lanes l, l^16, l^32, l^48 hold the same dims).
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = acc[h][e];
      x += __shfl_xor(x, 16, kWave);
      x += __shfl_xor(x, 32, kWave);
      acc[h][e] = x;
    }
    l[h] = wave_sum(l[h]);
  }

  if (t_lo == 0 && t_hi == nt) {
    if (lane < 16) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float inv = l[h] > 0.f ? 1.f / l[h] : 0.f;
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = acc[h][e] * inv;
        uint4* dst = reinterpret_cast<uint4*>(a.out + (int64_t(b) * hq + g * G + h) * kDim);
        dst[lane] = pack8(o);
      }
    }
  } else {
    const int seg = b * a.hkv + g;
    float* rec = a.ws + int64_t(seg + wave) * partial_floats(G);
    if (lane < 16) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) st_coherent(rec + h * kDim + lane * 8 + e, acc[h][e]);
    }
    if (lane < G) {
      float mv = m[0], lv = l[0];
#pragma unroll
      for (int h = 1; h < G; ++h)
        if (lane == h) { mv = m[h]; lv = l[h]; }
      st_coherent(rec + G * kDim + lane, mv);
      st_coherent(rec + G * kDim + G + lane, lv);
    }
  }
}

template <int G>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  __shared__ uint4 q_lds[kWavesPerWG][G * kChunks];
  __shared__ float p_lds[kWavesPerWG][kTile * G];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = blockIdx.x * kWavesPerWG + wv;

  // Empty contexts have no tiles: their output rows are zero.
  if (wave < a.n_waves) {
    const int hq = a.hkv * G;
    for (int bb = wave; bb < a.batch; bb += a.n_waves) {
      if (clamp_ctx(a, a.ctx_lens[bb]) != 0) continue;
      uint32_t* o = reinterpret_cast<uint32_t*>(a.out + int64_t(bb) * hq * kDim);
      for (int i = lane_id(); i < hq * (kDim / 2); i += kWave) o[i] = 0u;
    }
  }

  const int total = total_tiles(a);
  const int per = (total + a.n_waves - 1) / a.n_waves;
  int pos = wave * per;
  const int end = min(pos + per, total);
  if (pos >= end) return;

  int b, before;
  locate(a, pos, b, before);
  if (b >= a.batch) return;
  int nt = tiles_of(clamp_ctx(a, a.ctx_lens[b]));
  int off = pos - before * a.hkv;
  int g = off / nt;
  int t = off - g * nt;
  // A run cuts at most two segments (its first and its last); their arrivals
  // are counted once the whole run has been streamed, so the record stores
  // never stall the loads.
  int pend_b[2], pend_g[2], pend_w0[2], pend_w1[2];
  int npend = 0;
  while (true) {
    const int take = min(nt - t, end - pos);
    decode_run<G>(a, b, g, t, t + take, nt, wave, q_lds[wv], p_lds[wv]);
    if (!(t == 0 && take == nt)) {
      const int start = pos - t;  // first tile of the segment in the flattened list
      pend_b[npend] = b;
      pend_g[npend] = g;
      pend_w0[npend] = start / per;
      pend_w1[npend] = (start + nt - 1) / per;
      ++npend;
    }
    pos += take;
    if (pos >= end) break;
    t = 0;
    if (++g == a.hkv) {
      g = 0;
      do {
        ++b;
        nt = b < a.batch ? tiles_of(clamp_ctx(a, a.ctx_lens[b])) : 1;
      } while (nt == 0);
      if (b >= a.batch) break;
    }
  }

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
        merge_segment<G>(a, seg, pend_b[i], pend_g[i], pend_w0[i], pend_w1[i]);
        if (lane_id() == 0)
          __hip_atomic_store(a.counters + seg, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
  const unsigned split_blocks = unsigned((a.n_waves + kWavesPerWG - 1) / kWavesPerWG);
  hipLaunchKernelGGL(decode_split_kernel<G>, dim3(split_blocks), dim3(256), 0, s, a);
  return hipGetLastError();
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
