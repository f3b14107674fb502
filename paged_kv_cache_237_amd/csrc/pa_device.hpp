// Device helpers shared by the gfx950 kernels of libpa: bf16 bit handling,
// the bf16 dot-product instruction, and wave64 reductions built on DPP row
// operations plus lane reads.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight bf16 (one 16-byte chunk) widened to fp32, in memory order.
__device__ __forceinline__ void unpack8(const uint4& u, float (&f)[8]) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x);
  f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z);
  f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair with round-to-nearest-even (one
// v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint4 pack8(const float (&f)[8]) {
  uint4 u;
  u.x = pack_bf16x2(f[0], f[1]);
  u.y = pack_bf16x2(f[2], f[3]);
  u.z = pack_bf16x2(f[4], f[5]);
  u.w = pack_bf16x2(f[6], f[7]);
  return u;
}

// acc + a.lo*b.lo + a.hi*b.hi for two packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

__device__ __forceinline__ float dot8_bf16(const uint4& a, const uint4& b, float acc) {
  acc = dot2_bf16(a.x, b.x, acc);
  acc = dot2_bf16(a.y, b.y, acc);
  acc = dot2_bf16(a.z, b.z, acc);
  return dot2_bf16(a.w, b.w, acc);
}

// DPP controls (GCN/CDNA encoding).
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16

template <int Ctrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
}
template <int Ctrl>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, Ctrl, 0xF, 0xF, false);
}

__device__ __forceinline__ float readlane_f(float x, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Max over the 16 lanes of each DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  return fmaxf(x, dpp_f<kDppMirror>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x + dpp_f<kDppMirror>(x);
}
__device__ __forceinline__ int row16_sum_i(int x) {
  x += dpp_i<kDppXor1>(x);
  x += dpp_i<kDppXor2>(x);
  x += dpp_i<kDppHalfMirror>(x);
  return x + dpp_i<kDppMirror>(x);
}

// x combined with the value of lane l^32 (or l^16) in VALU, with no LDS
// round trip.  v_permlane32_swap exchanges lanes 32..63 of its first operand
// with lanes 0..31 of its second; given x twice, the two results hold, in
// every lane, x of lanes l%32 and l%32 + 32 -- the lane's own value and its
// partner's, so a commutative combine of the two equals x_l op x_(l^32)
// bit for bit.  v_permlane16_swap does the same for 16-lane rows 1, 3 against
// rows 0, 2.  The results are copied to plain integers before use.
__device__ __forceinline__ float xor32_max(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned a = r[0], b = r[1];
  return fmaxf(__uint_as_float(a), __uint_as_float(b));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const unsigned a = r[0], b = r[1];
  return __uint_as_float(a) + __uint_as_float(b);
}
__device__ __forceinline__ float xor16_sum(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const unsigned a = r[0], b = r[1];
  return __uint_as_float(a) + __uint_as_float(b);
}

// Wave-uniform max / sum of one value per lane.
__device__ __forceinline__ float wave_max(float x) {
  x = row16_max(x);
  return fmaxf(fmaxf(readlane_f(x, 0), readlane_f(x, 16)), fmaxf(readlane_f(x, 32), readlane_f(x, 48)));
}
__device__ __forceinline__ float wave_sum(float x) {
  x = row16_sum(x);
  return (readlane_f(x, 0) + readlane_f(x, 16)) + (readlane_f(x, 32) + readlane_f(x, 48));
}
__device__ __forceinline__ int wave_sum_i(int x) {
  x = row16_sum_i(x);
  return (__builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16)) +
         (__builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48));
}

__device__ __forceinline__ int wave_max_i(int x) {
  x = max(x, dpp_i<kDppXor1>(x));
  x = max(x, dpp_i<kDppXor2>(x));
  x = max(x, dpp_i<kDppHalfMirror>(x));
  x = max(x, dpp_i<kDppMirror>(x));
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Inclusive prefix sum across the 64 lanes (lane i gets x_0 + ... + x_i),
// in DPP: shifts by 1, 2, 4, 8 within each 16-lane row (lanes shifted in from
// outside the row read 0), then the last lane of row 0 / row 2 is added to
// rows 1 / 3 (row_bcast:15) and the last lane of row 1 to rows 2 and 3
// (row_bcast:31).  Disabled rows keep the `old` operand, 0.
constexpr int kDppRowShr1 = 0x111;
constexpr int kDppRowBcast15 = 0x142;
constexpr int kDppRowBcast31 = 0x143;

__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1 + 1, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1 + 3, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1 + 7, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xC, 0xF, false);
  return x;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Raw buffer access.  A load whose offset (VGPR offset plus immediate) is at
// or past num_records bytes returns zeros and touches no memory, which gives
// branch-free masking of rows past the end of a context.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kBufferWord3 = 0x00020000;  // gfx9 family: 32-bit data format, raw

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kBufferWord3);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// An offset no buffer here reaches: loads at it return zeros.
constexpr uint32_t kOutOfRange = 0x40000000u;

}  // namespace pa
