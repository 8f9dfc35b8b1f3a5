// Tiled bf16 prefill kernels (matrix cores).  Placeholder until implemented.
#include "common.h"

namespace attn {
bool prefill_mfma_supported(const FwdArgs&) { return false; }
hipError_t launch_prefill_mfma(const FwdArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
