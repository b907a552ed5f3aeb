// Chunked forward (placeholder until the fused kernel lands).
#include "ckda_internal.h"

namespace ckda {
bool fwd_supported(int32_t, int32_t, int32_t, int32_t) { return false; }
launch_result launch_fwd(const FwdArgs&, int32_t, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace ckda
