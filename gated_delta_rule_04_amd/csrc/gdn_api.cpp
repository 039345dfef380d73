// C-ABI of libgdn.so: argument validation, then the launches.
// The declarations, layouts and error semantics are in include/gdn.h.
#include "gdn.h"

#include <stdint.h>

#include <cmath>

#include "gdn_backward.h"
#include "gdn_epilogue.h"
#include "gdn_internal.h"

static_assert(gdn::kNoAllocScratchBytes == GDN_NOALLOC_SCRATCH_BYTES,
              "the scratch size of the header and of the kernels agree");

namespace {

constexpr int kChunk = 64;

bool supported_dim(int d) { return d == 64 || d == 128; }

size_t elem_size(gdn_dtype dt) { return dt == GDN_BF16 ? 2 : 4; }

// Byte range [lo, hi) of a buffer; an empty range never overlaps.
struct Range {
  uintptr_t lo, hi;
};

Range range_of(const void* p, size_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, p ? lo + bytes : lo};
}

bool overlaps(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

// n = a * b * c * d with an overflow check against 2^62 elements.
bool count4(long long a, long long b, long long c, long long d, long long* n) {
  const long long lim = 1LL << 62;
  long long x = 1;
  for (long long f : {a, b, c, d}) {
    if (f < 0) return false;
    if (f != 0 && x > lim / f) return false;
    x *= f;
  }
  *n = x;
  return true;
}

gdn_status check_common(int B, int H, int dk, int dv, gdn_dtype dtype, gdn_decay mode) {
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
  if (mode != GDN_DECAY_NONE && mode != GDN_DECAY_SCALAR && mode != GDN_DECAY_CHANNEL)
    return GDN_ERR_DTYPE;
  if (B < 0 || H < 0 || dk <= 0 || dv <= 0) return GDN_ERR_SHAPE;
  if (!supported_dim(dk) || !supported_dim(dv)) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_version(void) { return 300; }

const char* gdn_status_string(gdn_status s) {
  switch (s) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: invalid or overflowing size";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unknown dtype or decay mode";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: d_k, d_v or chunk not supported";
    case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace too small";
    case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH: the HIP runtime refused the launch";
    case GDN_ERR_ALIAS: return "GDN_ERR_ALIAS: forbidden aliasing between arguments";
    case GDN_ERR_VALUE: return "GDN_ERR_VALUE: a scalar argument is out of range";
  }
  return "unknown gdn_status";
}

size_t gdn_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                     gdn_dtype dtype, gdn_decay mode) {
  if (check_common(B, H, dk, dv, dtype, mode) != GDN_OK || T < 0 || chunk != kChunk) return 0;
  long long n;
  if (!count4(B, T, H, 1, &n)) return 0;
  return gdn::prefill_workspace_bytes(B, T, H, dk, (int)dtype, (int)mode);
}

size_t gdn_chunk_fwd_varlen_workspace_bytes(int N, int T, int H, int dk, int dv, int chunk,
                                            gdn_dtype dtype, gdn_decay mode) {
  if (check_common(N, H, dk, dv, dtype, mode) != GDN_OK || T < 0 || chunk != kChunk) return 0;
  long long n;
  if (!count4((long long)T / kChunk + N, H, 1, 1, &n) || (long long)T / kChunk + N > 0x7fffffffLL)
    return 0;
  return gdn::prefill_varlen_workspace_bytes(N, T, H, dk, (int)dtype, (int)mode);
}

}  // extern "C"

namespace {

// The prologue's arguments, checked; `reads_gates` says whether the kernels
// will read the gates (A is then required when alpha comes from logits).
gdn_status take_prologue(const gdn_prologue* pro, gdn_decay mode, bool reads_gates, int H, int dk,
                         gdn::Prologue* out, Range* ra, Range* rb) {
  *out = gdn::Prologue{};
  *ra = Range{0, 0};
  *rb = Range{0, 0};
  if (!pro) return GDN_OK;
  if (!(pro->eps >= 0.f) || !std::isfinite(pro->eps)) return GDN_ERR_VALUE;
  out->qk_norm = pro->l2norm_qk != 0;
  out->norm_eps = pro->eps;
  out->beta_logits = pro->beta_logits != 0;
  out->alpha_logits = pro->alpha_logits != 0 && mode != GDN_DECAY_NONE;
  if (out->alpha_logits) {
    if (reads_gates && !pro->A) return GDN_ERR_NULL;
    out->A = pro->A;
    out->dt_bias = pro->dt_bias;
    *ra = range_of(pro->A, (size_t)H * 4);
    *rb = range_of(pro->dt_bias, (size_t)H * (mode == GDN_DECAY_CHANNEL ? dk : 1) * 4);
  }
  return GDN_OK;
}

// Prefill over B rows of T tokens (cu_seqlens NULL and packed false) or over a
// packed batch of B sequences with T tokens in all.
// Gated DeltaNet-2 (erase and write gates given): mode is GDN_DECAY_CHANNEL
// for every check and 3 for the kernels, and beta is not read.
gdn_status prefill(const void* q, const void* k, const void* v, const void* alpha,
                   const float* beta, const float* S0, void* o, float* S_final,
                   const int* cu_seqlens, bool packed, const gdn_prologue* pro, void* workspace,
                   size_t workspace_bytes, int B, int T, int H, int dk, int dv, int chunk,
                   gdn_dtype dtype, gdn_decay mode, hipStream_t stream,
                   const void* erase = nullptr, const void* write = nullptr, bool gdn2 = false,
                   bool noalloc = false) {
  gdn_status st = check_common(B, H, dk, dv, dtype, mode);
  if (st != GDN_OK) return st;
  if (T < 0) return GDN_ERR_SHAPE;
  if (chunk != kChunk) return GDN_ERR_UNSUPPORTED;
  if (packed && B == 0 && T > 0) return GDN_ERR_SHAPE;   // tokens outside every sequence
  const int rows = packed ? 1 : B;   // leading axis of the token tensors
  long long nqk, nv, ntok, nS;
  if (!count4(rows, T, H, dk, &nqk) || !count4(rows, T, H, dv, &nv) ||
      !count4(rows, T, H, 1, &ntok) || !count4(B, H, dv, dk, &nS))
    return GDN_ERR_SHAPE;
  if ((long long)B * H * (dv / 32) > 0x7fffffffLL) return GDN_ERR_SHAPE;
  if (packed && ((long long)T / kChunk + B > 0x7fffffffLL ||
                 ((long long)T / kChunk + B) * H > 0x7fffffffLL))
    return GDN_ERR_SHAPE;
  const size_t ws_need = packed
                             ? gdn_chunk_fwd_varlen_workspace_bytes(B, T, H, dk, dv, chunk, dtype, mode)
                             : gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, chunk, dtype, mode);
  if (noalloc ? ws_need > gdn::kNoAllocScratchBytes : workspace_bytes < ws_need)
    return GDN_ERR_WORKSPACE;
  const bool has_tokens = T > 0;
  gdn::Prologue pa;
  Range rA, rbias;
  st = take_prologue(pro, mode, has_tokens, H, dk, &pa, &rA, &rbias);
  if (st != GDN_OK) return st;
  if (B == 0 || H == 0) return GDN_OK;
  if (packed && !cu_seqlens) return GDN_ERR_NULL;
  if (ws_need > 0 && !workspace && !noalloc) return GDN_ERR_NULL;
  if (has_tokens) {
    if (!q || !k || !v || !o) return GDN_ERR_NULL;
    if (gdn2 ? (!erase || !write) : !beta) return GDN_ERR_NULL;
    if (mode != GDN_DECAY_NONE && !alpha) return GDN_ERR_NULL;
  }
  if (!has_tokens && !S_final) return GDN_OK;  // nothing to write

  const size_t es = elem_size(dtype);
  const size_t a_bytes = mode == GDN_DECAY_SCALAR ? (size_t)ntok * 4
                         : mode == GDN_DECAY_CHANNEL ? (size_t)nqk * es : 0;
  Range rq = range_of(has_tokens ? q : nullptr, (size_t)nqk * es);
  Range rk = range_of(has_tokens ? k : nullptr, (size_t)nqk * es);
  Range rv = range_of(has_tokens ? v : nullptr, (size_t)nv * es);
  Range ra = range_of(has_tokens && mode != GDN_DECAY_NONE ? alpha : nullptr, a_bytes);
  Range rb = range_of(has_tokens && !gdn2 ? beta : nullptr, (size_t)ntok * 4);
  Range re = range_of(has_tokens && gdn2 ? erase : nullptr, (size_t)nqk * es);
  Range rwg = range_of(has_tokens && gdn2 ? write : nullptr, (size_t)nv * es);
  Range rs0 = range_of(S0, (size_t)nS * 4);
  Range rcu = range_of(packed ? cu_seqlens : nullptr, ((size_t)B + 1) * 4);
  Range ro = range_of(has_tokens ? o : nullptr, (size_t)nv * es);
  Range rsf = range_of(S_final, (size_t)nS * 4);
  if (!has_tokens) rA = rbias = Range{0, 0};
  for (Range in : {rq, rk, rv, ra, rb, re, rwg, rs0, rcu, rA, rbias})
    if (overlaps(ro, in)) return GDN_ERR_ALIAS;
  for (Range in : {rq, rk, rv, ra, rb, re, rwg, ro, rcu, rA, rbias})
    if (overlaps(rsf, in)) return GDN_ERR_ALIAS;
  if (overlaps(rsf, rs0) && (const void*)S_final != (const void*)S0) return GDN_ERR_ALIAS;
  // (the library's own scratch array cannot alias a caller's buffer)
  Range rw = range_of(ws_need > 0 && !noalloc ? workspace : nullptr, ws_need);
  for (Range in : {rq, rk, rv, ra, rb, re, rwg, rs0, rcu, ro, rsf, rA, rbias})
    if (overlaps(rw, in)) return GDN_ERR_ALIAS;
  if (noalloc && ws_need > 0 && gdn::noalloc_scratch(&workspace) != hipSuccess)
    return GDN_ERR_LAUNCH;

  gdn::PrefillArgs a{q, k, v, alpha, gdn2 ? nullptr : beta, S0, o, S_final, B, T, H, dk, dv,
                     (int)dtype, gdn2 ? 3 : (int)mode};
  a.erase = erase;
  a.write = write;
  if (packed) {
    a.cu_seqlens = cu_seqlens;
    a.nslots = gdn::varlen_slots(B, T);
  }
  a.pro = pa;
  return gdn::launch_prefill(a, workspace, stream) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status decode(const void* q, const void* k, const void* v, const void* alpha,
                  const float* beta, float* S, void* o, const gdn_prologue* pro, int B, int H,
                  int dk, int dv, gdn_dtype dtype, gdn_decay mode, hipStream_t stream,
                  const void* erase = nullptr, const void* write = nullptr, bool gdn2 = false) {
  gdn_status st = check_common(B, H, dk, dv, dtype, mode);
  if (st != GDN_OK) return st;
  long long nqk, nv, nh, nS;
  if (!count4(B, H, dk, 1, &nqk) || !count4(B, H, dv, 1, &nv) || !count4(B, H, 1, 1, &nh) ||
      !count4(B, H, dv, dk, &nS))
    return GDN_ERR_SHAPE;
  if ((long long)B * H > 0x7fffffffLL) return GDN_ERR_SHAPE;
  gdn::Prologue pa;
  Range rA, rbias;
  st = take_prologue(pro, mode, B > 0 && H > 0, H, dk, &pa, &rA, &rbias);
  if (st != GDN_OK) return st;
  if (B == 0 || H == 0) return GDN_OK;
  if (!q || !k || !v || !S || !o) return GDN_ERR_NULL;
  if (gdn2 ? (!erase || !write) : !beta) return GDN_ERR_NULL;
  if (mode != GDN_DECAY_NONE && !alpha) return GDN_ERR_NULL;

  const size_t es = elem_size(dtype);
  const size_t a_bytes = mode == GDN_DECAY_SCALAR ? (size_t)nh * 4
                         : mode == GDN_DECAY_CHANNEL ? (size_t)nqk * es : 0;
  Range rq = range_of(q, (size_t)nqk * es), rk = range_of(k, (size_t)nqk * es);
  Range rv = range_of(v, (size_t)nv * es);
  Range ra = range_of(mode != GDN_DECAY_NONE ? alpha : nullptr, a_bytes);
  Range rb = range_of(gdn2 ? nullptr : beta, (size_t)nh * 4);
  Range re = range_of(gdn2 ? erase : nullptr, (size_t)nqk * es);
  Range rwg = range_of(gdn2 ? write : nullptr, (size_t)nv * es);
  Range rs = range_of(S, (size_t)nS * 4), ro = range_of(o, (size_t)nv * es);
  for (Range in : {rq, rk, rv, ra, rb, re, rwg, rs, rA, rbias})
    if (overlaps(ro, in)) return GDN_ERR_ALIAS;
  for (Range in : {rq, rk, rv, ra, rb, re, rwg, rA, rbias})
    if (overlaps(rs, in)) return GDN_ERR_ALIAS;

  gdn::DecodeArgs a{q, k, v, alpha, gdn2 ? nullptr : beta, S, o, B, H, dk, dv, (int)dtype,
                    gdn2 ? 3 : (int)mode};
  a.pro = pa;
  a.erase = erase;
  a.write = write;
  return gdn::launch_decode(a, stream) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

gdn_status gdn_chunk_fwd(const void* q, const void* k, const void* v, const void* alpha,
                         const float* beta, const float* S0, void* o, float* S_final,
                         void* workspace, size_t workspace_bytes, int B, int T, int H, int dk,
                         int dv, int chunk, gdn_dtype dtype, gdn_decay mode,
                         hipStream_t stream) {
  return prefill(q, k, v, alpha, beta, S0, o, S_final, nullptr, false, nullptr, workspace,
                 workspace_bytes, B, T, H, dk, dv, chunk, dtype, mode, stream);
}

gdn_status gdn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* alpha,
                                 const float* beta, const float* S0, void* o, float* S_final,
                                 int B, int T, int H, int dk, int dv, int chunk, gdn_dtype dtype,
                                 gdn_decay mode, hipStream_t stream) {
  return prefill(q, k, v, alpha, beta, S0, o, S_final, nullptr, false, nullptr, nullptr, 0, B, T,
                 H, dk, dv, chunk, dtype, mode, stream, nullptr, nullptr, false, true);
}

gdn_status gdn_chunk_fwd_varlen(const void* q, const void* k, const void* v, const void* alpha,
                                const float* beta, const float* S0, void* o, float* S_final,
                                const int* cu_seqlens, void* workspace, size_t workspace_bytes,
                                int N, int T, int H, int dk, int dv, int chunk, gdn_dtype dtype,
                                gdn_decay mode, hipStream_t stream) {
  return prefill(q, k, v, alpha, beta, S0, o, S_final, cu_seqlens, true, nullptr, workspace,
                 workspace_bytes, N, T, H, dk, dv, chunk, dtype, mode, stream);
}

gdn_status gdn_chunk_fwd_fused(const void* q, const void* k, const void* v, const void* alpha,
                               const float* beta, const float* S0, void* o, float* S_final,
                               const int* cu_seqlens, const gdn_prologue* prologue,
                               void* workspace, size_t workspace_bytes, int B, int T, int H,
                               int dk, int dv, int chunk, gdn_dtype dtype, gdn_decay mode,
                               hipStream_t stream) {
  return prefill(q, k, v, alpha, beta, S0, o, S_final, cu_seqlens, cu_seqlens != nullptr,
                 prologue, workspace, workspace_bytes, B, T, H, dk, dv, chunk, dtype, mode, stream);
}

gdn_status gdn_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                           const float* beta, float* S, void* o, int B, int H, int dk, int dv,
                           gdn_dtype dtype, gdn_decay mode, hipStream_t stream) {
  return decode(q, k, v, alpha, beta, S, o, nullptr, B, H, dk, dv, dtype, mode, stream);
}

gdn_status gdn_decode_step_fused(const void* q, const void* k, const void* v, const void* alpha,
                                 const float* beta, float* S, void* o,
                                 const gdn_prologue* prologue, int B, int H, int dk, int dv,
                                 gdn_dtype dtype, gdn_decay mode, hipStream_t stream) {
  return decode(q, k, v, alpha, beta, S, o, prologue, B, H, dk, dv, dtype, mode, stream);
}

gdn_status gdn2_chunk_fwd(const void* q, const void* k, const void* v, const void* alpha,
                          const void* erase, const void* write, const float* S0, void* o,
                          float* S_final, const int* cu_seqlens, void* workspace,
                          size_t workspace_bytes, int B, int T, int H, int dk, int dv, int chunk,
                          gdn_dtype dtype, hipStream_t stream) {
  return prefill(q, k, v, alpha, nullptr, S0, o, S_final, cu_seqlens, cu_seqlens != nullptr,
                 nullptr, workspace, workspace_bytes, B, T, H, dk, dv, chunk, dtype,
                 GDN_DECAY_CHANNEL, stream, erase, write, true);
}

gdn_status gdn2_decode_step(const void* q, const void* k, const void* v, const void* alpha,
                            const void* erase, const void* write, float* S, void* o, int B,
                            int H, int dk, int dv, gdn_dtype dtype, hipStream_t stream) {
  return decode(q, k, v, alpha, nullptr, S, o, nullptr, B, H, dk, dv, dtype, GDN_DECAY_CHANNEL,
                stream, erase, write, true);
}

gdn_status gdn_gated_rmsnorm(const void* o, const void* gate, const float* weight, void* out, long long rows,
                             int dv, float eps, gdn_dtype dtype, hipStream_t stream) {
  if (dtype != GDN_F32 && dtype != GDN_BF16) return GDN_ERR_DTYPE;
  if (rows < 0 || dv <= 0) return GDN_ERR_SHAPE;
  if (!supported_dim(dv)) return GDN_ERR_UNSUPPORTED;
  long long n;
  if (!count4(rows, dv, 1, 1, &n)) return GDN_ERR_SHAPE;
  if (!(eps >= 0.f) || !std::isfinite(eps)) return GDN_ERR_VALUE;
  if (rows == 0) return GDN_OK;
  if (!o || !gate || !weight || !out) return GDN_ERR_NULL;
  const size_t bytes = (size_t)n * elem_size(dtype);
  const Range ro = range_of(out, bytes);
  if (overlaps(ro, range_of(gate, bytes)) || overlaps(ro, range_of(weight, (size_t)dv * 4)))
    return GDN_ERR_ALIAS;
  if (out != o && overlaps(ro, range_of(o, bytes))) return GDN_ERR_ALIAS;
  return gdn::launch_gated_rmsnorm(o, gate, weight, out, rows, dv, eps, (int)dtype, stream) == hipSuccess
             ? GDN_OK
             : GDN_ERR_LAUNCH;
}

size_t gdn_chunk_bwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk,
                                     gdn_dtype dtype, gdn_decay mode) {
  if (check_common(B, H, dk, dv, dtype, mode) != GDN_OK || T < 0 || chunk != kChunk) return 0;
  long long n;
  if (!count4(B, T, H, dk, &n) || !count4(B, H, dv, dk, &n)) return 0;
  return gdn::backward_workspace_bytes(B, T, H, dk, dv, (int)dtype, (int)mode);
}

gdn_status gdn_chunk_bwd(const void* q, const void* k, const void* v, const void* alpha,
                         const float* beta, const float* S0, const void* dout,
                         const float* dS_final, void* dq, void* dk, void* dv, float* dalpha,
                         float* dbeta, float* dS0, void* workspace, size_t workspace_bytes,
                         int B, int T, int H, int dk_, int dv_, int chunk, gdn_dtype dtype,
                         gdn_decay mode, hipStream_t stream) {
  gdn_status st = check_common(B, H, dk_, dv_, dtype, mode);
  if (st != GDN_OK) return st;
  if (T < 0) return GDN_ERR_SHAPE;
  if (chunk != kChunk) return GDN_ERR_UNSUPPORTED;
  long long nqk, nv, ntok, nS;
  if (!count4(B, T, H, dk_, &nqk) || !count4(B, T, H, dv_, &nv) || !count4(B, T, H, 1, &ntok) ||
      !count4(B, H, dv_, dk_, &nS))
    return GDN_ERR_SHAPE;
  if ((long long)B * H * (dv_ / 32) > 0x7fffffffLL || nqk / 4 / 256 > 0x7fffffffLL)
    return GDN_ERR_SHAPE;
  const size_t ws_need = gdn_chunk_bwd_workspace_bytes(B, T, H, dk_, dv_, chunk, dtype, mode);
  if (workspace_bytes < ws_need) return GDN_ERR_WORKSPACE;
  if (B == 0 || H == 0) return GDN_OK;
  if (ws_need > 0 && !workspace) return GDN_ERR_NULL;
  const bool has_tokens = T > 0;
  if (has_tokens) {
    if (!q || !k || !v || !beta || !dout || !dq || !dk || !dv || !dbeta) return GDN_ERR_NULL;
    if (mode != GDN_DECAY_NONE && (!alpha || !dalpha)) return GDN_ERR_NULL;
  }
  if (!has_tokens && !dS0) return GDN_OK;   // nothing to write

  const size_t es = elem_size(dtype);
  const size_t a_bytes = mode == GDN_DECAY_SCALAR ? (size_t)ntok * 4
                         : mode == GDN_DECAY_CHANNEL ? (size_t)nqk * es : 0;
  const size_t da_bytes = mode == GDN_DECAY_SCALAR ? (size_t)ntok * 4
                          : mode == GDN_DECAY_CHANNEL ? (size_t)nqk * 4 : 0;
  const bool t = has_tokens;
  const Range ins[] = {range_of(t ? q : nullptr, (size_t)nqk * es),
                       range_of(t ? k : nullptr, (size_t)nqk * es),
                       range_of(t ? v : nullptr, (size_t)nv * es),
                       range_of(t && mode != GDN_DECAY_NONE ? alpha : nullptr, a_bytes),
                       range_of(t ? beta : nullptr, (size_t)ntok * 4),
                       range_of(S0, (size_t)nS * 4),
                       range_of(t ? dout : nullptr, (size_t)nv * es),
                       range_of(dS_final, (size_t)nS * 4)};
  const Range outs[] = {range_of(t ? dq : nullptr, (size_t)nqk * es),
                        range_of(t ? dk : nullptr, (size_t)nqk * es),
                        range_of(t ? dv : nullptr, (size_t)nv * es),
                        range_of(t && mode != GDN_DECAY_NONE ? (void*)dalpha : nullptr, da_bytes),
                        range_of(t ? (void*)dbeta : nullptr, (size_t)ntok * 4),
                        range_of(dS0, (size_t)nS * 4),
                        range_of(ws_need > 0 ? workspace : nullptr, ws_need)};
  for (const Range& o : outs) {
    for (const Range& in : ins)
      if (overlaps(o, in)) return GDN_ERR_ALIAS;
    for (const Range& o2 : outs)
      if (&o2 != &o && overlaps(o, o2)) return GDN_ERR_ALIAS;
  }

  gdn::BackwardArgs a{q, k, v, alpha, beta, S0, dout, dS_final, dq, dk, dv, dalpha, dbeta, dS0,
                      B, T, H, dk_, dv_, (int)dtype, (int)mode};
  return gdn::launch_backward(a, workspace, stream) == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // extern "C"
