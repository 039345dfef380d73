// Internal declaration of the output epilogue (gdn_epilogue.hip).
// Not part of the C-ABI; include/gdn.h is.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

// Gated RMSNorm of `rows` rows of dv values; y may be o (in place).
hipError_t launch_gated_rmsnorm(const void* o, const void* g, const float* w, void* y, long long rows, int dv,
                                float eps, int dtype, hipStream_t stream);

}  // namespace gdn
