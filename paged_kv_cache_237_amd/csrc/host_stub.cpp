// Device-side stand-in for the sanitizer build of the host layer.  api.cpp and
// block_manager.cpp are compiled with the host compiler's address and
// undefined-behaviour sanitizers and linked with this file instead of the
// kernels and the HIP runtime, so that every host path -- argument checks,
// workspace sizing, error strings, the block manager -- runs under the
// sanitizers on a machine without a GPU.  Every device operation reports
// that no device is present, as the HIP runtime does on such a machine.
#include <hip/hip_runtime_api.h>

#include "pa_internal.hpp"
#include "pa_prefill.hpp"

namespace pa {

hipError_t check_slots(const int32_t*, int64_t, int64_t, hipStream_t, int*) { return hipErrorNoDevice; }
hipError_t check_seqs(const SeqCheckArgs&, hipStream_t, int*) { return hipErrorNoDevice; }
hipError_t launch_store_kv(const StoreArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_copy_blocks(const CopyBlocksArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_mfma(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode_mfma16(const DecodeArgs&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill(const PrefillArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t noalloc_scratch(hipStream_t, void**) { return hipErrorNoDevice; }

}  // namespace pa

extern "C" {

hipError_t hipGetDevice(int*) { return hipErrorNoDevice; }
hipError_t hipDeviceGetAttribute(int*, hipDeviceAttribute_t, int) { return hipErrorNoDevice; }
const char* hipGetErrorName(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "hipErrorNoDevice"; }
const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "no error" : "no device (host-only build)"; }
hipError_t hipMemcpyAsync(void*, const void*, size_t, hipMemcpyKind, hipStream_t) { return hipErrorNoDevice; }

}  // extern "C"
