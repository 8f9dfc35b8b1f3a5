// Paged split-KV decode kernels.  Placeholder until implemented.
#include "common.h"

namespace attn {
bool decode_supported(const FwdArgs&) { return false; }
size_t decode_workspace_bytes(const FwdArgs&) { return 0; }
hipError_t launch_decode(const FwdArgs&, void*, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attn
