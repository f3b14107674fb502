// Measurement helper, not part of the pa_* interface: a load-only kernel that
// streams a device buffer the way the decode kernel streams a KV cache, so
// the benchmark can report the HBM read rate a launch of that shape and size
// reaches on the machine at hand, beside the vendor peak.
//
// Shape: one 512-thread workgroup (8 waves) per compute unit, as the decode
// launch has.  The buffer is cut into 32 KiB pieces (the bytes of one 64-token
// K/V tile); wave w of n streams pieces [P*w/n, P*(w+1)/n), each lane loading
// 32 x 16 bytes per piece, and folds what it loads into one word, written out
// so that no load is dead.  The loads use the default cache policy, or the
// non-temporal one (NT bit) that the decode kernels use for K/V tiles.
//
// int pa_probe_stream_read(const void* buf, int64_t bytes, int32_t n_workgroups,
//                          int32_t nontemporal, void* sink, void* stream)
//   buf    device buffer, 16-byte aligned, `bytes` a positive multiple of 32 KiB
//   sink   device buffer of n_workgroups * 512 floats (overwritten)
//   stream hipStream_t; the call is asynchronous on it
// Returns 0, -1 (null pointer), -2 (bad size) or -6 (launch error).
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

constexpr int kPieceUint4 = 32768 / 16;  // 16-byte words per 32 KiB piece

typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16(const uint4* p, bool nt) {
  if (!nt) return *p;
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool Nt>
__global__ __launch_bounds__(512) void stream_read_kernel(const uint4* __restrict__ buf, int64_t pieces,
                                                          float* __restrict__ sink) {
  const int64_t n_waves = int64_t(gridDim.x) * 8;
  const int64_t w = int64_t(blockIdx.x) * 8 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t p0 = pieces * w / n_waves, p1 = pieces * (w + 1) / n_waves;
  uint32_t acc = 0;
  for (int64_t p = p0; p < p1; ++p) {
    const uint4* src = buf + p * kPieceUint4 + lane;
    uint4 r[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) r[i] = load16(src + 64 * i, Nt);
#pragma unroll
    for (int i = 0; i < 32; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
  }
  sink[int64_t(blockIdx.x) * 512 + threadIdx.x] = float(acc & 0xFFFF);
}

}  // namespace

extern "C" int pa_probe_stream_read(const void* buf, int64_t bytes, int32_t n_workgroups,
                                    int32_t nontemporal, void* sink, void* stream) {
  if (buf == nullptr || sink == nullptr) return -1;
  if (bytes <= 0 || bytes % 32768 != 0 || n_workgroups <= 0 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return -2;
  if (nontemporal)
    hipLaunchKernelGGL(stream_read_kernel<true>, dim3(unsigned(n_workgroups)), dim3(512), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 32768,
                       static_cast<float*>(sink));
  else
    hipLaunchKernelGGL(stream_read_kernel<false>, dim3(unsigned(n_workgroups)), dim3(512), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint4*>(buf), bytes / 32768,
                       static_cast<float*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
