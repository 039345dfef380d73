// Internal declarations shared by the translation units of libgdn.so.
// Not part of the C-ABI; include/gdn.h is.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

// Per-token prologue of the mixer layers, applied inside the kernels (all off
// by default).
struct Prologue {
  int qk_norm = 0;                  // q, k <- x / sqrt(|x|^2 + norm_eps) per (token, head)
  float norm_eps = 0.f;
  int beta_logits = 0;              // beta <- sigmoid(beta)
  int alpha_logits = 0;             // log alpha <- -A[h] softplus(alpha + dt_bias)
  const float* A = nullptr;         // [H]
  const float* dt_bias = nullptr;   // [H] (scalar decay) or [H, dk] (per channel); may be null
};

// log(1 + e^y) without overflow, and the logistic function (fp32).
__device__ inline float softplus_f(float y) { return fmaxf(y, 0.f) + log1pf(__expf(-fabsf(y))); }
__device__ inline float sigmoid_f(float x) { return 1.f / (1.f + __expf(-x)); }

// Arguments of one prefill launch.  Pointers are device pointers; layouts are
// the C-ABI's: q, k [B, T, H, dk]; v, o [B, T, H, dv]; alpha [B, T, H] or
// [B, T, H, dk]; beta [B, T, H]; S0, S_final [B, H, dv, dk].
struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const float* beta;
  const float* S0;   // may be null (zeros)
  void* o;
  float* S_final;    // may be null
  int B, T, H, dk, dv;
  int dtype;         // 0 fp32, 1 bf16
  int mode;          // 0 none, 1 scalar, 2 channel, 3 Gated DeltaNet-2 (channel decay,
                     // erase gate [B, T, H, dk] and write gate [B, T, H, dv] in place of beta)
  const void* erase = nullptr;   // mode 3, operand dtype
  const void* write = nullptr;   // mode 3, operand dtype
  // Packed batch of sequences of varying length: B sequences back to back on
  // a token axis of length T (the layouts above with a leading batch of 1),
  // sequence b holding tokens cu_seqlens[b] .. cu_seqlens[b + 1] - 1 (device
  // int32 [B + 1]).  Null for B rows of T tokens each.
  const int* cu_seqlens = nullptr;
  int nslots = 0;    // packed batch: chunk records per head, T / 64 + B
  Prologue pro;
  // Per-channel decay, backward only: the per-channel prep kernel also writes
  // each chunk's At[r][s] = sum_c k_r[c] k_s[c] exp(G_r[c] - G_s[c]) (s < r,
  // else 0), fp32 [C][C] per record slot.  Null in the forward.
  float* a_tilde = nullptr;
  // Scalar decay, bf16: one fp32 per chunk record (same index), the log of a
  // bound on the norm of the chunk's state transition (written by the prep
  // kernel, read by the state kernel to place the lead-ins of split slices).
  // Null: not written, and every lead-in starts at chunk 0.
  float* horizon = nullptr;
};

// Arguments of one decode launch: q, k [B, H, dk]; v, o [B, H, dv];
// alpha [B, H] or [B, H, dk]; beta [B, H]; S [B, H, dv, dk] in/out.
struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* alpha;
  const float* beta;
  float* S;
  void* o;
  int B, H, dk, dv;
  int dtype;
  int mode;
  Prologue pro;
  const void* erase = nullptr;   // mode 3: [B, H, dk]
  const void* write = nullptr;   // mode 3: [B, H, dv]
};

// Device workspace the prefill needs, per chunk of every head.  Scalar or no
// decay: T = (I + A)^-1 diag(beta) (64 x 64 elements of the operand dtype),
// in fp32 also the masked intra-chunk attention P (64 x 64), and the chunk's
// decay factors (3 x 64 fp32).  Per-channel decay: T and P, the decay-scaled
// K, Q and K (64 x dk each, operand dtype) and the chunk's per-channel decay
// (dk fp32).
size_t prefill_workspace_bytes(int B, int T, int H, int dk, int dtype, int mode);
// The same for a packed batch of N sequences with T tokens in all.
size_t prefill_varlen_workspace_bytes(int N, int T, int H, int dk, int dtype, int mode);
// Chunk records per head of a packed batch (an upper bound of the chunks of
// any N sequences with T tokens in all: sequence b's chunk n takes record
// slot cu_seqlens[b] / 64 + b + n).
int varlen_slots(int N, int T);
// Enqueue the prefill kernels; returns the launch status.
hipError_t launch_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream);
// Bytes of one chunk record of the prefill workspace.  bf16 with scalar or no
// decay, unnormalised q and k: T [64][64] bf16 (row-major), then five fp32
// rows of 64: G_r (the running sum of log alpha inside the chunk, the same
// past the sequence end), exp(G_r), exp(G_C - G_r), exp(G_r) again and ones.
size_t prefill_record_bytes(int dk, int dtype, int mode);
// Enqueue only the first prefill kernel, which writes the chunk records.
hipError_t launch_prefill_prep(const PrefillArgs& a, void* workspace, hipStream_t stream);
// Bytes of the per-device scratch array of the prefill entry point that
// allocates nothing (the same value as GDN_NOALLOC_SCRATCH_BYTES).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
// Device address of that array on the current device (looked up once per
// device, then cached).
hipError_t noalloc_scratch(void** ptr);
// Enqueue one decode step; returns the launch status.
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace gdn
