/*
 * Plain fp64 CPU oracle of the gated delta-rule recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (per batch b and head h, state S of shape d_v x d_k):
 *
 *   S <- S0 (zeros when S0 is NULL: "On State Reduction in Linear Attention"
 *         notes, section 2.1, initial state S_0 = 0)
 *   for t = 0 .. T-1:
 *     S <- S D_t        decay first.  DeltaNet: D_t = I.  Gated DeltaNet:
 *                       D_t = alpha_t I (scalar).  Kimi Delta Attention:
 *                       D_t = Diag(alpha_t) on the key channels, i.e. column c
 *                       of S is scaled by alpha_t[c].
 *                       ("Linear Attention Architectures" notes, sections 2.4
 *                       and 2.5, Eqs. 15-17 and 18-20: the old state is decayed
 *                       before the error is formed; KDA's Diag multiplies S
 *                       from the right.)
 *     p <- S k_t        prediction of the decayed memory for the current key
 *     u <- beta_t (v_t - p)      scaled write error ("pseudo-value" u_t of the
 *                       state-reduction notes, section 2.2)
 *     S <- S + u k_t^T  delta write (DeltaNet, Eqs. 9-10 / 14 of the
 *                       linear-attention notes, section 2.3)
 *     o_t <- S q_t      the query reads the UPDATED state (Eq. 8, section 2.1
 *                       of the linear-attention notes)
 *   S_final <- S
 *
 * No scale is applied to q (the NextTransformer "method sources" page, backend
 * section, registers scale = 1).  q and k are used exactly as given.
 *
 * The decode step is the loop body run once with S in/out.
 *
 * Mode 3 (Gated DeltaNet-2, see oracle_step_gdn2) replaces beta by an erase
 * gate b [.., dk] on the key side and a write gate w [.., dv] on the value
 * side; its alpha is per key channel.
 *
 * Layouts (row-major, contiguous):
 *   q, k   [B, T, H, dk]      v, o [B, T, H, dv]
 *   alpha  mode 0: unused (may be NULL); mode 1: [B, T, H]; mode 2: [B, T, H, dk]
 *   beta   [B, T, H]
 *   S0, S_final [B, H, dv, dk]
 *
 * Built with plain -O2 (no fast-math, no BLAS): every sum runs in index order.
 * OpenMP only distributes independent (b, h) heads over threads.
 */
#include <stdlib.h>
#include <string.h>

#define MODE_NONE 0
#define MODE_SCALAR 1
#define MODE_CHANNEL 2
#define MODE_GDN2 3

/* One recurrence step on the state S (dv x dk) of one head. */
static void oracle_step(double* S, const double* q, const double* k,
                        const double* v, const double* alpha, double beta,
                        double* o, int dk, int dv, int mode, double* p) {
  int i, c;
  /* decay first */
  if (mode == MODE_SCALAR) {
    for (i = 0; i < dv * dk; ++i) S[i] *= alpha[0];
  } else if (mode == MODE_CHANNEL) {
    for (i = 0; i < dv; ++i)
      for (c = 0; c < dk; ++c) S[i * dk + c] *= alpha[c];
  }
  /* prediction from the decayed state */
  for (i = 0; i < dv; ++i) {
    double acc = 0.0;
    for (c = 0; c < dk; ++c) acc += S[i * dk + c] * k[c];
    p[i] = acc;
  }
  /* delta write with the pseudo-value u_i = beta (v_i - p_i) */
  for (i = 0; i < dv; ++i) {
    double u = beta * (v[i] - p[i]);
    for (c = 0; c < dk; ++c) S[i * dk + c] += u * k[c];
  }
  /* read of the updated state */
  for (i = 0; i < dv; ++i) {
    double acc = 0.0;
    for (c = 0; c < dk; ++c) acc += S[i * dk + c] * q[c];
    o[i] = acc;
  }
}

/* One Gated DeltaNet-2 step on the state W (dv x dk) of one head, in the
 * notation of the "Linear Attention Architectures" notes, section 2.6
 * (Eqs. 21-24): the erase and write controls of the delta rule are separate
 * vectors.
 *   W~ = W D_alpha          per-key-channel decay, from the right
 *   e  = b (.) kappa        erase direction, key side
 *   z  = w (.) v            new content, value side
 *   r  = z - W~ e           residual against the erase read-out
 *   W  = W~ + r kappa^T     the outer product takes the key itself, not e
 *   o  = W q                the query reads the updated state
 * With b = beta 1 and w = beta 1 this is the per-channel (KDA) step. */
static void oracle_step_gdn2(double* W, const double* q, const double* kappa,
                             const double* v, const double* alpha, const double* b,
                             const double* w, double* o, int dk, int dv, double* res) {
  int i, c;
  for (i = 0; i < dv; ++i)
    for (c = 0; c < dk; ++c) W[i * dk + c] *= alpha[c];
  for (i = 0; i < dv; ++i) {
    double read = 0.0;
    for (c = 0; c < dk; ++c) read += W[i * dk + c] * (b[c] * kappa[c]);
    res[i] = w[i] * v[i] - read;
  }
  for (i = 0; i < dv; ++i)
    for (c = 0; c < dk; ++c) W[i * dk + c] += res[i] * kappa[c];
  for (i = 0; i < dv; ++i) {
    double acc = 0.0;
    for (c = 0; c < dk; ++c) acc += W[i * dk + c] * q[c];
    o[i] = acc;
  }
}

/* One token of any variant: GDN2 reads the erase and write gates of the
 * token, the others its beta. */
static void oracle_token(double* S, const double* q, const double* k, const double* v,
                         const double* alpha, const double* beta, const double* erase,
                         const double* write, size_t tok, double* o, int dk, int dv, int mode,
                         double* p) {
  const double* a = NULL;
  if (mode == MODE_SCALAR) a = alpha + tok;
  if (mode == MODE_CHANNEL || mode == MODE_GDN2) a = alpha + tok * dk;
  if (mode == MODE_GDN2)
    oracle_step_gdn2(S, q + tok * dk, k + tok * dk, v + tok * dv, a, erase + tok * dk,
                     write + tok * dv, o + tok * dv, dk, dv, p);
  else
    oracle_step(S, q + tok * dk, k + tok * dk, v + tok * dv, a, beta[tok], o + tok * dv, dk, dv,
                mode, p);
}

/* Arguments every entry point checks the same way. */
static int bad_mode_args(int mode, const double* alpha, const double* beta, const double* erase,
                         const double* write, int has_tokens) {
  if (mode < MODE_NONE || mode > MODE_GDN2) return 1;
  if (!has_tokens) return 0;
  if (mode != MODE_NONE && alpha == NULL) return 1;
  if (mode == MODE_GDN2) return erase == NULL || write == NULL;
  return beta == NULL;
}

/* Prefill over T tokens.  Returns 0 on success, -1 on a bad argument.
 * erase [B, T, H, dk] and write [B, T, H, dv] are read by mode GDN2 only
 * (which ignores beta; its alpha is [B, T, H, dk]). */
int oracle_gdn_fwd_f64(const double* q, const double* k, const double* v,
                       const double* alpha, const double* beta, const double* erase,
                       const double* write, const double* S0, double* o, double* S_final,
                       int B, int T, int H, int dk, int dv, int mode) {
  long bh;
  int fail = 0;
  if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
  if (bad_mode_args(mode, alpha, beta, erase, write, T > 0)) return -1;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
  for (bh = 0; bh < (long)B * H; ++bh) {
    long b = bh / H, h = bh % H;
    double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
    double* p = (double*)malloc(sizeof(double) * (size_t)dv);
    if (S == NULL || p == NULL) {
      free(S);
      free(p);
      fail |= 1;
      continue;
    }
    if (S0 != NULL)
      memcpy(S, S0 + (size_t)bh * dv * dk, sizeof(double) * (size_t)dv * dk);
    else
      memset(S, 0, sizeof(double) * (size_t)dv * dk);
    for (long t = 0; t < T; ++t) {
      size_t tok = ((size_t)b * T + t) * H + h; /* index of (b, t, h) */
      oracle_token(S, q, k, v, alpha, beta, erase, write, tok, o, dk, dv, mode, p);
    }
    if (S_final != NULL)
      memcpy(S_final + (size_t)bh * dv * dk, S, sizeof(double) * (size_t)dv * dk);
    free(S);
    free(p);
  }
  return fail ? -1 : 0;
}

/* Prefill over a packed batch of N sequences of varying length.
 *
 * The tokens of all sequences lie back to back along one axis of length T:
 * sequence s holds tokens cu[s] .. cu[s+1]-1 (cu[0] = 0, non-decreasing,
 * cu[N] = T; empty sequences allowed).  The state starts again from S0[s]
 * (zeros when S0 is NULL) at the first token of every sequence and nowhere
 * else: a token that opens a document inside a sequence does not reset it
 * (NextTransformer "method sources" page, baseline section on the packed
 * rows of the recurrent mixers).
 *
 * The loop runs once over the whole token axis per head and performs the reset
 * when the token index reaches the next boundary; it is written independently
 * of oracle_gdn_fwd_f64 so that the two can be checked against each other.
 *
 * Layouts: q, k [T, H, dk]; v, o [T, H, dv]; alpha [T, H] or [T, H, dk];
 * beta [T, H]; S0, S_final [N, H, dv, dk].  Returns 0, or -1 on a bad argument
 * (including cu_seqlens that do not run from 0 to T without decreasing). */
int oracle_gdn_fwd_varlen_f64(const double* q, const double* k, const double* v,
                              const double* alpha, const double* beta, const double* erase,
                              const double* write, const double* S0, double* o,
                              double* S_final, const int* cu, int N, int T, int H, int dk,
                              int dv, int mode) {
  long h;
  int s, fail = 0;
  const size_t sz = (size_t)dv * dk;
  if (N < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || cu == NULL) return -1;
  if (bad_mode_args(mode, alpha, beta, erase, write, T > 0)) return -1;
  if (cu[0] != 0 || cu[N] != T) return -1;
  for (s = 0; s < N; ++s)
    if (cu[s + 1] < cu[s]) return -1;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
  for (h = 0; h < H; ++h) {
    double* S = (double*)malloc(sizeof(double) * sz);
    double* p = (double*)malloc(sizeof(double) * (size_t)dv);
    int seq = 0;
    long t;
    if (S == NULL || p == NULL) {
      free(S);
      free(p);
      fail |= 1;
      continue;
    }
    if (N > 0) {
      if (S0 != NULL) memcpy(S, S0 + (size_t)h * sz, sizeof(double) * sz);
      else memset(S, 0, sizeof(double) * sz);
    }
    for (t = 0; t <= T; ++t) {
      /* close every sequence that ends before token t, open the next one */
      while (seq < N && cu[seq + 1] == t) {
        if (S_final != NULL) memcpy(S_final + ((size_t)seq * H + h) * sz, S, sizeof(double) * sz);
        ++seq;
        if (seq < N) {
          if (S0 != NULL) memcpy(S, S0 + ((size_t)seq * H + h) * sz, sizeof(double) * sz);
          else memset(S, 0, sizeof(double) * sz);
        }
      }
      if (t == T) break;
      oracle_token(S, q, k, v, alpha, beta, erase, write, (size_t)t * H + h, o, dk, dv, mode, p);
    }
    free(S);
    free(p);
  }
  return fail ? -1 : 0;
}

/* One decode step on S in place.
 *   q, k [B, H, dk]; v, o [B, H, dv]; alpha [B, H] (mode 1) or [B, H, dk]
 *   (mode 2); beta [B, H]; S [B, H, dv, dk] in/out. */
int oracle_gdn_decode_f64(const double* q, const double* k, const double* v,
                          const double* alpha, const double* beta, const double* erase,
                          const double* write, double* S, double* o, int B, int H, int dk,
                          int dv, int mode) {
  long bh;
  int fail = 0;
  if (B < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
  if (bad_mode_args(mode, alpha, beta, erase, write, B > 0 && H > 0)) return -1;
#pragma omp parallel for schedule(static) reduction(| : fail)
  for (bh = 0; bh < (long)B * H; ++bh) {
    double* p = (double*)malloc(sizeof(double) * (size_t)dv);
    if (p == NULL) {
      fail |= 1;
      continue;
    }
    /* one token per head: the token index is the head index */
    oracle_token(S + (size_t)bh * dv * dk, q, k, v, alpha, beta, erase, write, (size_t)bh, o, dk,
                 dv, mode, p);
    free(p);
  }
  return fail ? -1 : 0;
}

/* Threads OpenMP would use (reported with the CPU baseline). */
int oracle_num_threads(void) {
  int n = 1;
#pragma omp parallel
  {
#pragma omp single
    {
#ifdef _OPENMP
      extern int omp_get_num_threads(void);
      n = omp_get_num_threads();
#endif
    }
  }
  return n;
}
