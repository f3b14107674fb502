// Causal varlen prefill over the paged cache (gfx950): placeholder until the
// MFMA kernel lands; reports "not supported".
#include "pa_internal.hpp"

namespace pa {

hipError_t launch_prefill(const PrefillArgs&, int, hipStream_t) { return hipErrorNotSupported; }

}  // namespace pa
