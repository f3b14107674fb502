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
// that covers a whole segment writes the bf16 output at once; a segment cut
// between runs leaves one partial state (m, l, u) per run in the workspace,
// and a second kernel merges those:  M = max m_i,  L = sum 2^(m_i-M) l_i,
// o = sum 2^(m_i-M) u_i / L  (the split-context form of the online softmax).
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

// Tiles of the sequences before b (identical in every lane).
__device__ int tiles_before(const DecodeArgs& a, int b) {
  const int lane = lane_id();
  int tot = 0;
  for (int b0 = 0; b0 < b; b0 += kWave) {
    const int bb = b0 + lane;
    const int nt = bb < b ? tiles_of(clamp_ctx(a, a.ctx_lens[bb])) : 0;
    tot += wave_sum_i(nt);
  }
  return tot;
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
    float* rec = a.ws + int64_t(b * a.hkv + g + wave) * partial_floats(G);
    if (lane < 16) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float4* dst = reinterpret_cast<float4*>(rec + h * kDim + lane * 8);
        dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      }
    }
    if (lane < G) {
      float mv = m[0], lv = l[0];
#pragma unroll
      for (int h = 1; h < G; ++h)
        if (lane == h) { mv = m[h]; lv = l[h]; }
      rec[G * kDim + lane] = mv;
      rec[G * kDim + G + lane] = lv;
    }
  }
}

template <int G>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  __shared__ uint4 q_lds[kWavesPerWG][G * kChunks];
  __shared__ float p_lds[kWavesPerWG][kTile * G];
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wave = blockIdx.x * kWavesPerWG + wv;

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
  while (true) {
    const int take = min(nt - t, end - pos);
    decode_run<G>(a, b, g, t, t + take, nt, wave, q_lds[wv], p_lds[wv]);
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
}

// One wave per segment: merge its partial states, or write zeros for an empty
// context.  Segments finished by a single run were written by the split kernel.
template <int G>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
  const int lane = lane_id();
  const int seg = blockIdx.x * kWavesPerWG + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (seg >= a.batch * a.hkv) return;
  const int b = seg / a.hkv;
  const int g = seg - b * a.hkv;
  const int hq = a.hkv * G;
  const int nt = tiles_of(clamp_ctx(a, a.ctx_lens[b]));
  uint32_t* out = reinterpret_cast<uint32_t*>(a.out + (int64_t(b) * hq + g * G) * kDim);
  if (nt == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) out[h * (kDim / 2) + lane] = 0u;
    return;
  }
  const int total = total_tiles(a);
  const int per = (total + a.n_waves - 1) / a.n_waves;
  const int start = tiles_before(a, b) * a.hkv + g * nt;
  const int w0 = start / per;
  const int w1 = (start + nt - 1) / per;
  if (w0 == w1) return;

  for (int h = 0; h < G; ++h) {
    float big = -INFINITY;
    for (int w = w0; w <= w1; ++w) {
      const float* rec = a.ws + int64_t(seg + w) * partial_floats(G);
      big = fmaxf(big, rec[G * kDim + h]);
    }
    const float ref = big == -INFINITY ? 0.f : big;
    float sum = 0.f, u0 = 0.f, u1 = 0.f;
    for (int w = w0; w <= w1; ++w) {
      const float* rec = a.ws + int64_t(seg + w) * partial_floats(G);
      const float f = __builtin_amdgcn_exp2f(rec[G * kDim + h] - ref);
      sum = fmaf(f, rec[G * kDim + G + h], sum);
      const float2 u = reinterpret_cast<const float2*>(rec + h * kDim)[lane];
      u0 = fmaf(f, u.x, u0);
      u1 = fmaf(f, u.y, u1);
    }
    const float inv = sum > 0.f ? 1.f / sum : 0.f;
    out[h * (kDim / 2) + lane] = pack_bf16x2(u0 * inv, u1 * inv);
  }
}

template <int G>
static hipError_t launch_decode_g(const DecodeArgs& a, hipStream_t s) {
  const unsigned split_blocks = unsigned((a.n_waves + kWavesPerWG - 1) / kWavesPerWG);
  hipLaunchKernelGGL(decode_split_kernel<G>, dim3(split_blocks), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned merge_blocks = unsigned((a.batch * a.hkv + kWavesPerWG - 1) / kWavesPerWG);
  hipLaunchKernelGGL(decode_merge_kernel<G>, dim3(merge_blocks), dim3(256), 0, s, a);
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
