// Device-side checks of the data-dependent preconditions of the calls (the
// debug mode of the library): slots inside the pool, context lengths inside
// [0, min(max_context_len, max_blocks_per_seq * 256)], every block-table
// entry a sequence uses inside the pool, and for varlen calls a well-formed
// cu_seqlens_q with q_len <= context length.  The kernels only read the
// arrays, inside their stated sizes whatever their contents, and OR the
// violated conditions into one device word that the host resets (with a
// one-thread kernel, so that no memset is ever recorded) and reads back.
#include <algorithm>

#include "pa_internal.hpp"

namespace pa {

__device__ int g_check_flags;

__global__ void reset_check_flags_kernel() { g_check_flags = 0; }

__global__ __launch_bounds__(256) void check_slots_kernel(const int32_t* slots, int64_t n,
                                                           int64_t num_slots) {
  int found = 0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256)
    if (slots[i] >= num_slots) found = kCheckSlot;
  if (found) atomicOr(&g_check_flags, found);
}

__global__ __launch_bounds__(256) void check_seqs_kernel(SeqCheckArgs a) {
  const int b = blockIdx.x * 256 + threadIdx.x;
  if (b >= a.batch) return;
  int found = 0;
  const int64_t cap = min(int64_t(a.max_context_len), int64_t(a.mbps) * 256);
  const int ctx = a.ctx_lens[b];
  if (ctx < 0 || ctx > cap) found |= kCheckCtx;
  // entries of the blocks the sequence uses (never past its table row)
  const int64_t used = min((int64_t(max(ctx, 0)) + 255) / 256, int64_t(a.mbps));
  const int32_t* row = a.block_table + int64_t(b) * a.mbps;
  for (int64_t j = 0; j < used; ++j) {
    const int32_t e = row[j];
    if (e < 0 || e >= a.num_blocks) found |= kCheckTable;
  }
  if (a.cu_q != nullptr) {
    const int q = a.cu_q[b + 1] - a.cu_q[b];
    if (q < 0 || q > max(ctx, 0) || q > a.max_q) found |= kCheckRows;
    if (b == 0 && a.cu_q[0] != 0) found |= kCheckRows;
    if (b == a.batch - 1 && int64_t(a.cu_q[a.batch]) != a.total_q) found |= kCheckRows;
  } else if (a.rows_per_seq > 1 && ctx < a.rows_per_seq) {
    found |= kCheckRows;
  }
  if (found) atomicOr(&g_check_flags, found);
}

static hipError_t read_flags(hipStream_t s, int* flags) {
  hipError_t e = hipMemcpyFromSymbolAsync(flags, HIP_SYMBOL(g_check_flags), sizeof(int), 0,
                                          hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

hipError_t check_slots(const int32_t* slots, int64_t n, int64_t num_slots, hipStream_t s, int* flags) {
  hipLaunchKernelGGL(reset_check_flags_kernel, dim3(1), dim3(1), 0, s);
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(check_slots_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, slots, n, num_slots);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return read_flags(s, flags);
}

hipError_t check_seqs(const SeqCheckArgs& a, hipStream_t s, int* flags) {
  hipLaunchKernelGGL(reset_check_flags_kernel, dim3(1), dim3(1), 0, s);
  hipLaunchKernelGGL(check_seqs_kernel, dim3(unsigned((a.batch + 255) / 256)), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return read_flags(s, flags);
}

}  // namespace pa
