// Internal declarations of the prefill backward (gdn_backward.hip).
// Not part of the C-ABI; include/gdn.h is.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace gdn {

// Arguments of one backward launch.  Layouts as the prefill's: q, k [B, T, H, dk];
// v, do [B, T, H, dv]; alpha [B, T, H] or [B, T, H, dk]; beta [B, T, H];
// S0, dS_final [B, H, dv, dk] (either may be null: zeros).  Outputs dq, dk
// [B, T, H, dk] and dv [B, T, H, dv] in the operand dtype; dalpha fp32 in
// alpha's shape; dbeta fp32 [B, T, H]; dS0 fp32 [B, H, dv, dk] (may be null).
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const float* beta;
  const float* S0;
  const void* dout;
  const float* dS_final;
  void* dq;
  void* dk;
  void* dv;
  float* dalpha;
  float* dbeta;
  float* dS0;
  int B, T, H, dk_, dv_;
  int dtype;   // 0 fp32, 1 bf16
  int mode;    // 0 none, 1 scalar, 2 channel
};

size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv, int dtype, int mode);
hipError_t launch_backward(const BackwardArgs& a, void* workspace, hipStream_t stream);

// The chunk-level backward (gdn_bwd_chunk.hip): bf16, no, scalar or
// per-channel decay, T > 0.  The token-level kernels take every other case.
bool chunk_backward_applies(int T, int dk, int dv, int dtype, int mode);
size_t chunk_backward_workspace_bytes(int B, int T, int H, int dk, int dv, int mode);
hipError_t launch_chunk_backward(const BackwardArgs& a, void* workspace, hipStream_t stream);

}  // namespace gdn
