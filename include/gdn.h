/*
 * gdn.h — C-ABI of the MI355X (gfx950) gated delta-rule library (libgdn.so).
 *
 * The library computes the gated delta-rule linear-attention recurrence, per
 * batch entry b and head h, with a state S of shape d_v x d_k:
 *
 *     S_t = S_{t-1} D_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,   o_t = S_t q_t
 *
 * where D_t is
 *   GDN_DECAY_NONE     I                   (DeltaNet: "Linear Attention
 *                                           Architectures" notes, section 2.3,
 *                                           Eqs. 9-10 and 14; "On State Reduction
 *                                           in Linear Attention" notes, section
 *                                           2.1, Eq. 2)
 *   GDN_DECAY_SCALAR   alpha_t I           (Gated DeltaNet: linear-attention
 *                                           notes, section 2.4, Eqs. 15-17)
 *   GDN_DECAY_CHANNEL  Diag(alpha_t)       (Kimi Delta Attention: same notes,
 *                                           section 2.5, Eqs. 18-20; the diagonal
 *                                           acts on the key channels, from the right)
 *
 * The decay is applied before the write error is formed, and the output reads
 * the updated state (linear-attention notes, section 2.1, Eq. 8).  No scale
 * is applied to q (NextTransformer "method sources" page, backend section:
 * scale = 1); q and k are used as given (a layer normalises them beforehand).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers to contiguous row-major tensors in
 *    the layouts stated per argument.  The caller owns every buffer; the library
 *    allocates nothing, keeps no global state and is re-entrant.
 *  - Work is enqueued on `stream` (NULL = the default stream) and the call
 *    returns without synchronising.
 *  - Arguments are validated before anything is enqueued.  On any error the
 *    call returns a negative gdn_status, writes nothing and enqueues nothing.
 *    A failed kernel launch returns GDN_ERR_LAUNCH.  No exception crosses the ABI.
 *  - Gates may take their boundary values: beta in [0, 1], alpha in [0, 1].
 *  - Supported sizes: d_k in {64, 128}, d_v in {64, 128}, chunk = 64.
 *    Other sizes return GDN_ERR_UNSUPPORTED.
 *  - Decay numerics: log alpha is floored at -100 (alpha below e^-100 acts as
 *    e^-100, about 3.7e-44: an fp32 subnormal, so a state or key term scaled by
 *    it is some 1e-43 of the unit-size terms it is summed with, below fp32
 *    resolution; exact zeros are accepted).  Per-channel decay: inside a
 *    chunk the kernels split decay ratios at anchor tokens at most 16 tokens
 *    away; a channel whose decay over such a span exceeds e^64 is handled by
 *    an exact element-wise path instead (slower, same results), so any alpha
 *    in [0, 1] is accepted, including exact zeros.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_NULL = -1,         /* a required pointer is NULL                      */
  GDN_ERR_SHAPE = -2,        /* a size is negative, zero where it must not be,  */
                             /* or the element count overflows                  */
  GDN_ERR_DTYPE = -3,        /* unknown gdn_dtype or gdn_decay value            */
  GDN_ERR_UNSUPPORTED = -4,  /* d_k, d_v or chunk outside the supported set     */
  GDN_ERR_WORKSPACE = -5,    /* workspace smaller than the size queried         */
  GDN_ERR_LAUNCH = -6,       /* the HIP runtime refused a launch or a copy      */
  GDN_ERR_ALIAS = -7,        /* forbidden aliasing between inputs and outputs   */
  GDN_ERR_VALUE = -8         /* a scalar argument is out of range               */
} gdn_status;

/* Element type of q, k, v and o (and of a per-channel alpha). */
typedef enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 } gdn_dtype;

/* Decay family; see the header comment. */
typedef enum gdn_decay {
  GDN_DECAY_NONE = 0,     /* alpha unused, may be NULL                          */
  GDN_DECAY_SCALAR = 1,   /* alpha fp32, one value per (b, t, h)                */
  GDN_DECAY_CHANNEL = 2   /* alpha in `dtype`, one value per (b, t, h, key chan)*/
} gdn_decay;

/*
 * Per-token prologue of the mixer layers, fused into the kernels by the
 * *_fused entry points (a NULL prologue there means none of it).
 *
 *   l2norm_qk     nonzero: q_t <- q_t / sqrt(|q_t|^2 + eps) and k_t likewise,
 *                 per (token, head), in fp32 on the values as loaded (the layers
 *                 normalise queries and keys per head: "Don't Read Everything"
 *                 notes, section 2.1; residual-learning notes, section 2.2;
 *                 NextTransformer "method sources" page, baseline section).
 *                 With eps = 0 a zero vector gives NaN.
 *   eps           >= 0 and finite (GDN_ERR_VALUE otherwise); the pages leave it open.
 *   beta_logits   nonzero: `beta` holds logits x and the recurrence uses
 *                 sigmoid(x) (NextTransformer page, DeltaNet entry).
 *   alpha_logits  nonzero, decay modes only (ignored for GDN_DECAY_NONE):
 *                 `alpha` holds x and log alpha = -A[h] softplus(x + dt_bias),
 *                 a Mamba2-style decay (residual-learning notes, section 2.2);
 *                 floored at -100 like every log alpha here.
 *   A             DEVICE fp32 [H], the per-head rates (positive); required when
 *                 alpha_logits is set and the call reads gates (GDN_ERR_NULL).
 *   dt_bias       DEVICE fp32 [H] for a scalar decay, [H, dk] for a per-channel
 *                 decay; NULL means zero.
 * A and dt_bias must not alias any output or the workspace.
 */
typedef struct gdn_prologue {
  int l2norm_qk;
  float eps;
  int beta_logits;
  int alpha_logits;
  const float* A;
  const float* dt_bias;
} gdn_prologue;

/*
 * Bytes of device workspace gdn_chunk_fwd needs for these sizes (0 means the
 * workspace pointer may be NULL).  Returns 0 for arguments gdn_chunk_fwd would
 * reject.
 */
size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                     gdn_dtype dtype, gdn_decay mode);

/*
 * Chunked prefill over T tokens (any T >= 0; the last chunk may be partial).
 *
 *   q, k      [B, T, H, dk]   `dtype`
 *   v         [B, T, H, dv]   `dtype`
 *   alpha     mode SCALAR: fp32 [B, T, H]; mode CHANNEL: `dtype` [B, T, H, dk];
 *             mode NONE: ignored (may be NULL)
 *   beta      fp32 [B, T, H]
 *   S0        fp32 [B, H, dv, dk], the state before token 0; NULL means zeros
 *             ("On State Reduction" notes, section 2.1: S_0 = 0)
 *   o         [B, T, H, dv]   `dtype`, written: o_t = S_t q_t, rounded to
 *             nearest-even from fp32 when `dtype` is bf16
 *   S_final   fp32 [B, H, dv, dk], written: the state after the last token; may
 *             be NULL when the caller does not need it.  S_final == S0 (in-place
 *             hand-off) is allowed; no other output may alias an input.
 *   workspace device memory of at least gdn_chunk_fwd_workspace_bytes(...)
 *             bytes (may be NULL when that is 0); its contents on entry do not
 *             matter and on return are unspecified.
 *
 * The chunkwise form (decay-weighted beta K K^T, a unit-lower-triangular
 * solve, then a sequential pass over chunks carrying the fp32 state) is an
 * exact rewrite of the token recurrence; the NextTransformer page's numerics
 * section describes the same precision split used here: fp32 carried state
 * and accumulation, bf16 operands when the inputs are bf16.
 * T = 0 copies S0 (or zeros) to S_final and writes no o.
 */
gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v,
                         const void* alpha, const float* beta, const float* S0,
                         void* o, float* S_final,
                         void* workspace, size_t workspace_bytes,
                         int B, int T, int H, int dk, int dv, int chunk,
                         gdn_dtype dtype, gdn_decay mode, hipStream_t stream);

/*
 * gdn_chunk_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The chunk records live in a scratch array
 * inside the library's device code, GDN_NOALLOC_SCRATCH_BYTES bytes per GPU,
 * held by every GPU the library runs on until the process ends.  This call
 * allocates nothing (no hipMalloc, no allocating library routine); the caller
 * still passes every input and output, with the layouts, semantics and
 * errors of gdn_chunk_fwd.
 *
 *   - A call whose gdn_chunk_fwd_workspace_bytes(...) exceeds
 *     GDN_NOALLOC_SCRATCH_BYTES returns GDN_ERR_WORKSPACE before anything is
 *     enqueued (for bf16 scalar decay at d_k = 128: up to 7081 chunk-heads,
 *     B * H * ceil(T / 64); per-channel decay: 1016).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap on
 *     one GPU (concurrent streams, or host threads sharing a device) race
 *     and give unspecified results.  Calls in order on one stream are safe.
 *     The array keeps the last call's contents; nothing in it needs to start
 *     at zero.
 *   - The current device must be the device of `stream` (the array of the
 *     current device is used).  The first call on a device looks the array's
 *     address up once (GDN_ERR_LAUNCH if the runtime refuses).
 */
#define GDN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v,
                                 const void* alpha, const float* beta, const float* S0,
                                 void* o, float* S_final,
                                 int B, int T, int H, int dk, int dv, int chunk,
                                 gdn_dtype dtype, gdn_decay mode, hipStream_t stream);

/*
 * Bytes of device workspace gdn_chunk_fwd_varlen needs for N sequences with T
 * tokens in all (0 means the workspace pointer may be NULL).  It depends only
 * on N and T, not on how the tokens are split.  Returns 0 for arguments
 * gdn_chunk_fwd_varlen would reject.
 */
size_t gdn_chunk_fwd_varlen_workspace_bytes(int N, int T, int H, int dk, int dv, int chunk,
                                            gdn_dtype dtype, gdn_decay mode);

/*
 * Chunked prefill of a packed batch: N sequences of varying length lie back to
 * back on one token axis of length T, and the state starts again from S0[s]
 * at the first token of sequence s (and nowhere else; the NextTransformer
 * "method sources" page, baseline section, resets the recurrent state at the
 * start of every packed row).  Each sequence is cut into chunks of 64 from its
 * own first token; every sequence may end in a partial chunk.
 *
 *   q, k        [T, H, dk]   `dtype`   (the gdn_chunk_fwd layouts with B = 1)
 *   v           [T, H, dv]   `dtype`
 *   alpha       mode SCALAR: fp32 [T, H]; mode CHANNEL: `dtype` [T, H, dk];
 *               mode NONE: ignored (may be NULL)
 *   beta        fp32 [T, H]
 *   S0          fp32 [N, H, dv, dk], sequence s's initial state; NULL means zeros
 *   o           [T, H, dv]   `dtype`, written
 *   S_final     fp32 [N, H, dv, dk], written: each sequence's state after its
 *               last token (S0[s], or zeros, for an empty sequence); may be NULL.
 *               S_final == S0 is allowed; no other output may alias an input.
 *   cu_seqlens  DEVICE int32 [N + 1]: sequence s holds tokens cu_seqlens[s] ..
 *               cu_seqlens[s + 1] - 1.  The caller guarantees cu_seqlens[0] = 0,
 *               cu_seqlens[N] = T and no decrease (empty sequences are allowed).
 *               The offsets are read only on the device, so they are not
 *               validated; the kernels clamp them into [0, T], so malformed
 *               offsets give unspecified results but no access outside the
 *               buffers.  Must not alias o, S_final or the workspace.
 *   workspace   at least gdn_chunk_fwd_varlen_workspace_bytes(...) bytes.
 *
 * N = 0 requires T = 0 (GDN_ERR_SHAPE otherwise) and does nothing.  Errors,
 * asynchrony and numerics are those of gdn_chunk_fwd.
 */
gdn_status gdn_chunk_fwd_varlen(const void* q, const void* k, const void* v,
                                const void* alpha, const float* beta, const float* S0,
                                void* o, float* S_final, const int* cu_seqlens,
                                void* workspace, size_t workspace_bytes,
                                int N, int T, int H, int dk, int dv, int chunk,
                                gdn_dtype dtype, gdn_decay mode, hipStream_t stream);

/*
 * Chunked prefill with the prologue fused in: gdn_chunk_fwd when cu_seqlens is
 * NULL (B rows of T tokens), gdn_chunk_fwd_varlen when it is not (B packed
 * sequences with T tokens in all); arguments, layouts, workspace size and
 * errors are those of that entry point, plus the prologue's (see
 * gdn_prologue).  Normalised q and k are never materialised: the kernels fold
 * the inverse norms into the per-row factors they already apply (the decay
 * weights of K K^T, Q K^T and the chunk's state products), so no extra pass
 * over q or k is made.
 */
gdn_status gdn_chunk_fwd_fused(const void* q, const void* k, const void* v,
                               const void* alpha, const float* beta, const float* S0,
                               void* o, float* S_final, const int* cu_seqlens,
                               const gdn_prologue* prologue,
                               void* workspace, size_t workspace_bytes,
                               int B, int T, int H, int dk, int dv, int chunk,
                               gdn_dtype dtype, gdn_decay mode, hipStream_t stream);

/*
 * One decode step (the recurrence body for a single token), S updated in place.
 *
 *   q, k      [B, H, dk]   `dtype`
 *   v         [B, H, dv]   `dtype`
 *   alpha     mode SCALAR: fp32 [B, H]; mode CHANNEL: `dtype` [B, H, dk];
 *             mode NONE: ignored (may be NULL)
 *   beta      fp32 [B, H]
 *   S         fp32 [B, H, dv, dk], read and overwritten with the new state
 *   o         [B, H, dv]   `dtype`, written
 *
 * Per state row i the step needs S_i D k and S_i D q (one pass over the row),
 * then u_i = beta (v_i - S_i D k), o_i = S_i D q + u_i (k . q) and
 * S_i <- S_i D + u_i k^T — the predict/correct reading of the Gated DeltaNet
 * output ("Enhancing Linear Attention with Residual Learning" notes, section
 * 1.2, Table 1) — so the fp32 state is read once and written once.
 * o must not alias S, q, k or v.
 */
gdn_status gdn_decode_step(const void* q, const void* k, const void* v,
                           const void* alpha, const float* beta, float* S, void* o,
                           int B, int H, int dk, int dv,
                           gdn_dtype dtype, gdn_decay mode, hipStream_t stream);

/*
 * gdn_decode_step with the prologue fused in (q and k normalised in fp32,
 * beta and alpha from logits); alpha logits are [B, H] (scalar) or [B, H, dk]
 * (per channel), dt_bias [H] or [H, dk].  A NULL prologue is gdn_decode_step.
 */
gdn_status gdn_decode_step_fused(const void* q, const void* k, const void* v,
                                 const void* alpha, const float* beta, float* S, void* o,
                                 const gdn_prologue* prologue,
                                 int B, int H, int dk, int dv,
                                 gdn_dtype dtype, gdn_decay mode, hipStream_t stream);

/*
 * Gated DeltaNet-2 ("Linear Attention Architectures" notes, section 2.6,
 * Eqs. 21-24): the delta rule with its erase and write controls split into a
 * key-side vector b_t and a value-side vector w_t, and a per-key-channel decay:
 *
 *     S~ = S_{t-1} Diag(alpha_t),  e_t = b_t * k_t,  z_t = w_t * v_t,
 *     S_t = S~ + (z_t - S~ e_t) k_t^T,              o_t = S_t q_t
 *
 * (the outer product takes k_t itself).  b_t = w_t = beta_t 1 gives the
 * per-channel rule of gdn_chunk_fwd.  Prefill, batched (cu_seqlens NULL, the
 * gdn_chunk_fwd layouts) or packed (the gdn_chunk_fwd_varlen layouts):
 *
 *   alpha     `dtype` [.., T, H, dk]   per-channel decay in [0, 1]
 *   erase     `dtype` [.., T, H, dk]   b_t
 *   write     `dtype` [.., T, H, dv]   w_t
 * and q, k, v, S0, o, S_final, workspace as for GDN_DECAY_CHANNEL (the
 * workspace size is gdn_chunk_fwd(_varlen)_workspace_bytes with that mode).
 * Errors as for gdn_chunk_fwd; erase and write are required when T > 0.
 */
gdn_status gdn2_chunk_fwd(const void* q, const void* k, const void* v, const void* alpha,
                          const void* erase, const void* write, const float* S0, void* o,
                          float* S_final, const int* cu_seqlens, void* workspace,
                          size_t workspace_bytes, int B, int T, int H, int dk, int dv, int chunk,
                          gdn_dtype dtype, hipStream_t stream);

/*
 * One Gated DeltaNet-2 decode step, S updated in place: q, k, alpha, erase
 * [B, H, dk]; v, write, o [B, H, dv]; S fp32 [B, H, dv, dk].  Per state row i:
 * s_e = S_i D e, s_q = S_i D q, u_i = w_i v_i - s_e, o_i = s_q + u_i (k . q),
 * S_i <- S_i D + u_i k^T.
 */
gdn_status gdn2_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                            const void* erase, const void* write, float* S, void* o,
                            int B, int H, int dk, int dv, gdn_dtype dtype, hipStream_t stream);

/*
 * Bytes of device workspace gdn_chunk_bwd needs (0: the pointer may be NULL).
 * bf16 (the chunk-level kernels): per chunk of 64 tokens of every head, the
 * forward's chunk record (no or scalar decay: T and five gate rows, 9,472
 * bytes; per-channel: the per-channel record), the bf16 entry state and the
 * bf16 end-of-chunk state gradient (2 d_v d_k bytes each); per-channel decay
 * also At (16 KB) and the intermediate products of the gradient kernels
 * (fp32: 2 C^2 + 3 C d_k + d_k values).  fp32 (the token-level kernels): state
 * checkpoints (d_v x d_k fp32 per 8 tokens of every head) and one partial of
 * the row sums per 32-row value slice.  0 for rejected arguments.
 */
size_t gdn_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                     gdn_dtype dtype, gdn_decay mode);

/*
 * Backward of gdn_chunk_fwd: the gradients of
 *     L = sum(dout * o) + sum(dS_final * S_T)
 * with respect to every input (the pages' KDA training keeps a custom
 * first-order backward: NextTransformer "method sources" page, KDA entry).
 *
 *   q, k, v, alpha, beta, S0   as given to gdn_chunk_fwd (S0 may be NULL)
 *   dout      [B, T, H, dv] `dtype`: dL/do
 *   dS_final  fp32 [B, H, dv, dk] or NULL (zeros): dL/dS_T
 *   dq, dk    [B, T, H, dk] `dtype`, written
 *   dv        [B, T, H, dv] `dtype`, written
 *   dalpha    fp32 in alpha's shape ([B, T, H] or [B, T, H, dk]), written;
 *             ignored for GDN_DECAY_NONE
 *   dbeta     fp32 [B, T, H], written
 *   dS0       fp32 [B, H, dv, dk], written (also when S0 is NULL: the
 *             gradient at the zero state); may be NULL
 *   workspace gdn_chunk_bwd_workspace_bytes(...) bytes
 * No output may alias an input, another output or the workspace.  The
 * computation is deterministic (no atomics).  Gradients are accumulated in
 * fp32 and rounded once to `dtype`.  bf16 runs the reverse mode of the chunk
 * form (MFMA products; X and dU as bf16 hi + lo pairs where dbeta needs them;
 * with per-channel decay the channel-weighted C x C contractions run on the
 * vector ALUs, every weight exp(G_r - G_s) at most 1); fp32 runs the token
 * recurrence in reverse from state checkpoints.  Errors as for gdn_chunk_fwd.
 */
gdn_status gdn_chunk_bwd(const void* q, const void* k, const void* v, const void* alpha,
                         const float* beta, const float* S0, const void* dout,
                         const float* dS_final, void* dq, void* dk, void* dv, float* dalpha,
                         float* dbeta, float* dS0, void* workspace, size_t workspace_bytes,
                         int B, int T, int H, int dk_, int dv_, int chunk, gdn_dtype dtype,
                         gdn_decay mode, hipStream_t stream);

/*
 * Output epilogue of the Gated DeltaNet mixer (NextTransformer "method
 * sources" page, baseline section, Gated DeltaNet entry: the output passes an
 * RMSNorm, a gain and a SiLU gate; backend section: the output-gated
 * RMSNorm).  For each of `rows` rows of d_v values:
 *
 *     out = o / sqrt(mean(o^2) + eps) * weight * silu(gate),   silu(g) = g / (1 + e^-g)
 *
 *   o, gate   [rows, dv] `dtype` (rows = B * T * H for a prefill's output
 *             [B, T, H, dv], B * H for a decode step's [B, H, dv])
 *   weight    fp32 [dv], the gain, shared by all rows
 *   out       [rows, dv] `dtype`, written; may be o itself (in place), must
 *             not otherwise overlap o, gate or weight (GDN_ERR_ALIAS)
 *   eps       >= 0 and finite (GDN_ERR_VALUE); the pages leave it open
 * Arithmetic in fp32, one rounding to `dtype`.  dv in {64, 128}.  rows = 0
 * does nothing.  The state kernels split d_v over workgroups, so this runs as
 * its own pass over the finished output.
 */
gdn_status gdn_gated_rmsnorm(const void* o, const void* gate, const float* weight, void* out, long long rows,
                             int dv, float eps, gdn_dtype dtype, hipStream_t stream);

/* Static, human-readable name of a status code (never NULL). */
const char* gdn_status_string(gdn_status s);

/* Library ABI version: major * 10000 + minor * 100 + patch. */
int gdn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
