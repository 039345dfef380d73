// Chunk-level backward of the gated delta-rule prefill, bf16 operands, no,
// scalar or per-channel decay.  (fp32 operands take the token-level kernels of
// gdn_backward.hip.)  The per-channel kernels follow the scalar ones below.
//
// The forward per chunk of C = 64 tokens (the chunk form derived from the
// recurrence of the "Linear Attention Architectures" notes, sections 2.3-2.4;
// G_r the running sum of log alpha inside the chunk, gamma_r = exp(G_r),
// E[r][s] = exp(G_r - G_s), S = S_n the entry state, K~ = diag(exp(G_C - G)) K):
//
//   A = tril_-1(diag(beta) (E o K K^T)),  M = (I + A)^-1,  T = M diag(beta)
//   X = V - diag(gamma) K S^T,            U = T X
//   P = tril_0(E o Q K^T),                O = diag(gamma) Q S^T + P U
//   S_{n+1} = gamma_C S + U^T K~
//
// Reverse mode through one chunk, dS = dL/dS_{n+1}, dO = dL/dO:
//
//   dU  = P^T dO + K~ dS^T           dX = T^T dU = dV
//   dS_n = gamma_C dS + dO^T diag(gamma) Q - dX^T diag(gamma) K
//   dT  = dU X^T,  N1 = M^T dT,  dA = -tril_-1(N1 T^T),  dP = tril_0(dO U^T)
//   dbeta_r = N1[r][r] + sum_s dA[r][s] (E o K K^T)[r][s]
//   dQ = (dP o E) K + diag(gamma) dO S
//   dK = (W + W^T) K + (dP o E)^T Q - diag(gamma) dX S + diag(exp(G_C - G)) U dS,
//        W = diag(beta) (dA o E)
//   dG_r = rows(Z) - cols(Z) + rows(Y) - cols(Y), Z = dA o A, Y = dP o P,
//          + q_r . (gamma_r dO S)_r - k_r . (gamma_r dX S)_r - k_r . (exp(G_C - G_r) U dS)_r
//   dG_C += <dS, S_{n+1}> = gamma_C <dS, S> + sum_r k_r . (exp(G_C - G_r) U dS)_r
//   dlog alpha_t = sum_{r >= t} dG_r (inside the chunk),  dalpha = dlog alpha / alpha
//
// Only dS carries from chunk to chunk, so three kernels (after the forward's
// own prep kernel has written T and the gate rows of every chunk):
//   bc_states  the forward chain per (b, h, 32-column value slice), writing the
//              bf16 entry state S_n of every chunk to the workspace
//   bc_rev     the reverse chain per (b, h, value slice): writes dV and the
//              bf16 dS of every chunk's end to the workspace, and dS0
//   bc_grad    fully parallel, one 512-thread workgroup per chunk of every
//              head: M (the forward's triangular solve with unit beta),
//              then the value axis in 32-column slices (X, U, dU and their
//              products summed over the slices in MFMA accumulators), then
//              the C x C algebra and dq, dk, dbeta, dalpha.
// Every product is a bf16 MFMA with fp32 accumulation; the states cross from
// the chains to bc_grad as bf16.  dbeta and dalpha are short sums with
// cancellation (with one token each is one dot product), so dT takes X and dU
// as bf16 hi + lo pairs, and the chunks whose state is an fp32 input (S0 at
// the first chunk, dS_final at the last) take it whole.  The results are
// deterministic: every sum runs in a fixed order, no atomics.
#include <stdint.h>

#include "gdn_backward.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_solve.h"

namespace gdn {
namespace {

using bf = __bf16;
constexpr int C = 64;              // chunk length
constexpr int SL = 32;             // value columns per slice
constexpr int kChainThreads = 256;
constexpr int kGradThreads = 512;
constexpr float kLogFloor = -100.f;   // as the forward: log alpha below -100 acts as -100
constexpr int LDT = C + 8;         // bf16 rows of 64 (C x C tiles, transposed slices)
constexpr int LDO = SL + 8;        // bf16 rows of 32 (row-major value slices)

// bf16 chunk record of the prefill workspace: T [C][C] at element 0, then
// fp32 gate rows G, exp(G), exp(G_C - G), ... of C values each.
constexpr size_t kRecG = (size_t)C * C;
constexpr size_t kRecElems = (size_t)C * C + 5 * C * 2;
// Per-channel decay: T, P [C][C], then the rows K (.) Gamma, Q (.) Gamma and
// K (.) exp(G_C - G) [C][DK], then gamma_C (DK fp32).
template <int DK>
struct KRec {
  static constexpr size_t t = 0, p = (size_t)C * C, kg = 2 * (size_t)C * C, qg = kg + (size_t)C * DK,
                          kc = qg + (size_t)C * DK, g = kc + (size_t)C * DK, elems = g + 2 * (size_t)DK;
};
template <int DK, bool KDA>
constexpr size_t rec_elems() { return KDA ? KRec<DK>::elems : kRecElems; }

constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }

__device__ inline u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }
__device__ inline u32x4 ld16(const bf* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ inline void st16(bf* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// 16 bytes of bf16 scaled by s (rounded to bf16).
__device__ inline u32x4 scale16(const u32x4& u, float s) {
  bf16x8 x = __builtin_bit_cast(bf16x8, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (bf)((float)x[i] * s);
  return __builtin_bit_cast(u32x4, x);
}

// 8 floats as bf16 pairs: hi = bf16(x), lo = bf16(x - hi) (hi + lo carries 16
// significant bits).
__device__ inline void split8(const float* x, u32x4& hi, u32x4& lo) {
  bf16x8 h, l;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    h[i] = (bf)x[i];
    l[i] = (bf)(x[i] - (float)h[i]);
  }
  hi = __builtin_bit_cast(u32x4, h);
  lo = __builtin_bit_cast(u32x4, l);
}

__device__ inline void unpack8(const u32x4& u, float* x) {
  const bf16x8 h = __builtin_bit_cast(bf16x8, u);
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
}

// Four values stored as bf16 hi and lo parts (8 bytes each).
__device__ inline void store4_split(bf* hi, bf* lo, float a, float b, float c, float d) {
  const float x[4] = {a, b, c, d};
  float r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = x[i] - (float)(bf)x[i];
  store4(hi, a, b, c, d);
  store4(lo, r[0], r[1], r[2], r[3]);
}

// Sum over the 32 lanes of each half of the wave (result in all of them):
// quads, then row_half_mirror and row_mirror DPP, then one swap of 16.
__device__ inline float half_sum(float x) {
  x = quad_sum(x);
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
  x += __shfl_xor(x, 16);
  return x;
}

// Row sums of a 32x32 accumulator tile (rows r0 + acc_row) added to rows[],
// then, if COLS, column sums (columns c0 + lane % 32) subtracted from cols[].
// The 16 row sums are independent reductions; lane j < 16 of each half then
// adds the one of row acc_row(j / 4, j % 4) in a single read-modify-write.
// Only the calling wave touches rows[] and cols[], and the row and column
// updates are separate instructions, so the order of the sums is fixed.
template <bool COLS>
__device__ inline void tile_row_col_sums(const f32x16& x, float* rows, int r0, float* cols, int c0, int lane) {
  float s[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) s[v] = half_sum(x[v]);
  const int j = lane & 31;
  float mine = s[0];
#pragma unroll
  for (int v = 1; v < 16; ++v) mine = j == v ? s[v] : mine;
  if (j < 16) rows[r0 + acc_row(j >> 2, j & 3, lane)] += mine;
  if constexpr (COLS) {
    float c = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) c += x[v];
    c += __shfl_xor(c, 32);
    if (lane < 32) cols[c0 + lane] -= c;
  }
}

// The value slices of one head go to the same XCD (workgroups are dispatched
// to the 8 XCDs round-robin), so its K, Q and records come from HBM once.
__device__ inline void head_and_slice(int nheads, int nsl, int& head, int& sl) {
  const int bid = blockIdx.x;
  if ((nheads & 7) == 0) {
    const int x = bid & 7, j = bid >> 3;
    head = (j / nsl) * 8 + x;
    sl = j % nsl;
  } else {
    head = bid / nsl;
    sl = bid % nsl;
  }
}

// ---------------------------------------------------------------------------
// bc_states: S_n of every chunk (bf16) for one (b, h, value slice).
// ---------------------------------------------------------------------------
template <int DK, bool KDA>
struct StatesLds {
  static constexpr int LDK = DK + 8;
  static constexpr size_t kb = 0;                                // K rows [C][LDK] (per channel: K (.) Gamma)
  static constexpr size_t kc = kb + (size_t)C * LDK * 2;         // per channel: K (.) exp(G_C - G) rows
  static constexpr size_t tb = kc + (KDA ? (size_t)C * LDK * 2 : 0);   // T [C][LDT]
  static constexpr size_t sb = tb + (size_t)C * LDT * 2;         // S slice [SL][LDK]
  static constexpr size_t xt = sb + (size_t)SL * LDK * 2;        // X^T [SL][LDT]
  static constexpr size_t ut = xt + (size_t)SL * LDT * 2;        // (diag(exp(G_C - G)) U)^T [SL][LDT]
  static constexpr size_t vb = ut + (size_t)SL * LDT * 2;        // V slice [C][LDO]
  static constexpr size_t gs = vb + (size_t)C * LDO * 2;         // exp(G), exp(G_C - G); per channel: gamma_C
  static constexpr size_t total = gs + (KDA ? DK : 2 * C) * 4;
};

// Per-channel decay (KDA): the operands come decay-weighted from the record,
// X = V - (K (.) Gamma) S^T, S^T <- diag(gamma_C) S^T + (K (.) exp(G_C - G))^T U.
template <int DK, bool KDA>
__global__ __launch_bounds__(kChainThreads, 2) void bc_states(BackwardArgs a, const bf* __restrict__ recs,
                                                              bf* __restrict__ ssave) {
  using L = StatesLds<DK, KDA>;
  using KR = KRec<DK>;
  constexpr size_t RE = rec_elems<DK, KDA>();
  constexpr int LDK = L::LDK, CPR = DK / 8, KPT = C * CPR / kChainThreads;
  static_assert(C * CPR % kChainThreads == 0 && SL * CPR % kChainThreads == 0, "even split");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  bf* Kb = reinterpret_cast<bf*>(smem + L::kb);
  bf* Kcb = KDA ? reinterpret_cast<bf*>(smem + L::kc) : Kb;   // the state update's K operand
  bf* Tb = reinterpret_cast<bf*>(smem + L::tb);
  bf* Sb = reinterpret_cast<bf*>(smem + L::sb);
  bf* Xt = reinterpret_cast<bf*>(smem + L::xt);
  bf* Ut = reinterpret_cast<bf*>(smem + L::ut);
  bf* Vb = reinterpret_cast<bf*>(smem + L::vb);
  float* eG = reinterpret_cast<float*>(smem + L::gs);   // per channel: gamma_C [DK]
  float* eC = eG + C;

  // (the wave index in a scalar register: branches on it are uniform jumps)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int T = a.T, H = a.H, DV = a.dv_, NC = (T + C - 1) / C;
  int head, sl;
  head_and_slice(a.B * H, DV / SL, head, sl);
  const int b = head / H, h = head % H, i0 = sl * SL;
  const bf* kg = static_cast<const bf*>(a.k);
  const bf* vg = static_cast<const bf*>(a.v);

  // S^T tile of wave w < DK / 32: rows j = 32 w + acc_row, column i = col
  f32x16 S = zero16();
  if (wave < DK / 32 && a.S0) {
    const float* s0 = a.S0 + ((size_t)head * DV + i0 + col) * DK + 32 * wave;
#pragma unroll
    for (int v = 0; v < 16; ++v) S[v] = s0[acc_row(v >> 2, v & 3, lane)];
  }
  // Wait for those loads here: a load pending on entry to the loop would make
  // the compiler wait for every later load (the prefetches too) at the first
  // use of S in each step.
  __builtin_amdgcn_s_waitcnt(0);

  u32x4 kreg[KPT], kcreg[KDA ? KPT : 1], treg[2], vreg;
  float greg = 0.f;
  const int vrow = tid >> 2, vcc = tid & 3;   // this thread's piece of the V slice
  auto load = [&](int n) __attribute__((always_inline)) {
    const int t0 = n * C, cn = min(C, T - t0);
    const bf* rec = recs + ((size_t)head * NC + n) * RE;
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
      if constexpr (KDA) {   // (the record's rows past the sequence end are not zero)
        kreg[m] = r < cn ? ld16(rec + KR::kg + r * DK + cc * 8) : zero_u4();
        kcreg[m] = r < cn ? ld16(rec + KR::kc + r * DK + cc * 8) : zero_u4();
      } else {
        kreg[m] = r < cn ? ld16(kg + (((size_t)b * T + t0 + r) * H + h) * DK + cc * 8) : zero_u4();
      }
    }
    vreg = vrow < cn ? ld16(vg + (((size_t)b * T + t0 + vrow) * H + h) * DV + i0 + vcc * 8) : zero_u4();
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = tid + kChainThreads * m, r = q >> 3, cc = q & 7;
      treg[m] = ld16(rec + r * C + cc * 8);
    }
    if constexpr (KDA) {
      if (tid < DK) greg = reinterpret_cast<const float*>(rec + KR::g)[tid];
    } else {
      if (tid < 2 * C) greg = reinterpret_cast<const float*>(rec + kRecG)[C + tid];
    }
  };
  auto commit = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
      st16(Kb + r * LDK + cc * 8, kreg[m]);
      if constexpr (KDA) st16(Kcb + r * LDK + cc * 8, kcreg[m]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = tid + kChainThreads * m, r = q >> 3, cc = q & 7;
      st16(Tb + r * LDT + cc * 8, treg[m]);
    }
    if (tid < (KDA ? DK : 2 * C)) eG[tid] = greg;
    st16(Vb + vrow * LDO + vcc * 8, vreg);
  };

  // The next chunk's registers go to LDS at the end of each step, after its
  // last barrier: the loads were issued at the step's start and only its own
  // stores follow them, so the wait for them is exact.
  if (NC > 0) {
    load(0);
    commit();
  }
  for (int n = 0; n < NC; ++n) {
    if (n + 1 < NC) load(n + 1);
    if (wave < DK / 32) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(Sb + col * LDK + 32 * wave + 8 * g + 4 * hh, S[4 * g], S[4 * g + 1], S[4 * g + 2], S[4 * g + 3]);
    }
    __syncthreads();
    {   // the chunk's entry state -> workspace [head][n][DV][DK]
      bf* dst = ssave + (((size_t)head * NC + n) * DV + i0) * DK;
#pragma unroll
      for (int m = 0; m < SL * CPR / kChainThreads; ++m) {
        const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
        st16(dst + (size_t)r * DK + cc * 8, ld16(Sb + r * LDK + cc * 8));
      }
    }
    if (wave < 2) {   // X = V - diag(gamma) K S^T, rows 32 wave ..
      f32x16 y = zero16();
      tile_nt_k<DK / 16>(y, Kb + 32 * wave * LDK, LDK, Sb, LDK, lane);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = 32 * wave + 8 * g + 4 * hh;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = (float)Vb[(r0 + e) * LDO + col] - (KDA ? 1.f : eG[r0 + e]) * y[4 * g + e];
        store4(Xt + col * LDT + r0, x[0], x[1], x[2], x[3]);
      }
    }
    __syncthreads();
    if (wave < 2) {   // U = T X, stored decayed to the chunk end (per channel: the decay sits in K's rows)
      f32x16 u = zero16();
      tile_nt_k<C / 16>(u, Tb + 32 * wave * LDT, LDT, Xt, LDT, lane);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = 32 * wave + 8 * g + 4 * hh;
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = KDA ? 1.f : eC[r0 + e];
        store4(Ut + col * LDT + r0, w[0] * u[4 * g], w[1] * u[4 * g + 1], w[2] * u[4 * g + 2], w[3] * u[4 * g + 3]);
      }
    }
    __syncthreads();
    if (wave < DK / 32) {   // S^T <- gamma_C S^T + K^T (decayed U)
      if constexpr (KDA) {
#pragma unroll
        for (int v = 0; v < 16; ++v) S[v] *= eG[32 * wave + acc_row(v >> 2, v & 3, lane)];
      } else {
        const float gC = eG[C - 1];
#pragma unroll
        for (int v = 0; v < 16; ++v) S[v] *= gC;
      }
#pragma unroll
      for (int s = 0; s < C / 16; ++s)
        mma_bf16(S, frag_perm_tr(Kcb, LDK, 16 * s, 32 * wave, lane), frag_perm(Ut + col * LDT, 16 * s, hh));
    }
    __syncthreads();
    if (n + 1 < NC) commit();
  }
}

// ---------------------------------------------------------------------------
// bc_rev: dS backwards over the chunks of one (b, h, value slice); dV, the
// chunk-end dS (bf16) of every chunk, dS0.
// ---------------------------------------------------------------------------
template <int DK, bool KDA>
struct RevLds {
  static constexpr int LDK = DK + 8;
  static constexpr size_t kb = 0;                                // K rows [C][LDK] (per channel: K (.) Gamma)
  static constexpr size_t qb = kb + (size_t)C * LDK * 2;         // Q rows [C][LDK] (per channel: Q (.) Gamma)
  static constexpr size_t kc = qb + (size_t)C * LDK * 2;         // per channel: K (.) exp(G_C - G) rows
  static constexpr size_t tb = kc + (KDA ? (size_t)C * LDK * 2 : 0);   // T [C][LDT]
  static constexpr size_t dob = tb + (size_t)C * LDT * 2;        // dO slice [C][LDO]
  static constexpr size_t dog = dob + (size_t)C * LDO * 2;       // diag(gamma) dO slice [C][LDO] (per channel: dO)
  static constexpr size_t dsb = dog + (size_t)C * LDO * 2;       // dS slice [SL][LDK]
  static constexpr size_t pt = dsb + (size_t)SL * LDK * 2;       // P^T [C][LDT] (per channel: P); then (-diag(gamma) dX)^T [SL][LDT]
  static constexpr size_t dut = pt + (size_t)C * LDT * 2;        // dU^T [SL][LDT]
  static constexpr size_t gs = dut + (size_t)SL * LDT * 2;       // G, exp(G), exp(G_C - G); per channel: gamma_C
  static constexpr size_t total = gs + (KDA ? DK : 3 * C) * 4;
};

// Per-channel decay (KDA): P and the decay-weighted operands come from the
// record, dU = P^T dO + (K (.) exp(G_C - G)) dS^T and
// dS^T <- diag(gamma_C) dS^T + (Q (.) Gamma)^T dO - (K (.) Gamma)^T dX.
template <int DK, bool KDA>
__global__ __launch_bounds__(kChainThreads, 2) void bc_rev(BackwardArgs a, const bf* __restrict__ recs,
                                                           bf* __restrict__ dssave) {
  using L = RevLds<DK, KDA>;
  using KR = KRec<DK>;
  constexpr size_t RE = rec_elems<DK, KDA>();
  constexpr int LDK = L::LDK, CPR = DK / 8, KPT = C * CPR / kChainThreads;
  static_assert(C * SL / 8 == kChainThreads, "one dO piece per thread");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  bf* Kb = reinterpret_cast<bf*>(smem + L::kb);
  bf* Qb = reinterpret_cast<bf*>(smem + L::qb);
  bf* Tb = reinterpret_cast<bf*>(smem + L::tb);
  bf* dOb = reinterpret_cast<bf*>(smem + L::dob);
  bf* dOg = reinterpret_cast<bf*>(smem + L::dog);
  bf* dSb = reinterpret_cast<bf*>(smem + L::dsb);
  bf* Pt = reinterpret_cast<bf*>(smem + L::pt);   // per channel: P row-major
  bf* Xn = Pt;
  bf* Kcb = KDA ? reinterpret_cast<bf*>(smem + L::kc) : Kb;   // dU's K operand
  bf* dUt = reinterpret_cast<bf*>(smem + L::dut);
  float* Gs = reinterpret_cast<float*>(smem + L::gs);   // per channel: gamma_C [DK]
  float* eG = Gs + C;
  float* eC = Gs + 2 * C;

  // (the wave index in a scalar register: branches on it are uniform jumps)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int T = a.T, H = a.H, DV = a.dv_, NC = (T + C - 1) / C;
  int head, sl;
  head_and_slice(a.B * H, DV / SL, head, sl);
  const int b = head / H, h = head % H, i0 = sl * SL;
  const bf* kg = static_cast<const bf*>(a.k);
  const bf* qg = static_cast<const bf*>(a.q);
  const bf* dout_g = static_cast<const bf*>(a.dout);
  bf* dvg = static_cast<bf*>(a.dv);

  // dS^T tile of wave w < DK / 32: rows j = 32 w + acc_row, column i = col
  f32x16 dS = zero16();
  if (wave < DK / 32 && a.dS_final) {
    const float* s = a.dS_final + ((size_t)head * DV + i0 + col) * DK + 32 * wave;
#pragma unroll
    for (int v = 0; v < 16; ++v) dS[v] = s[acc_row(v >> 2, v & 3, lane)];
  }
  __builtin_amdgcn_s_waitcnt(0);   // (as in bc_states)

  u32x4 kreg[KPT], qreg[KPT], kcreg[KDA ? KPT : 1], treg[2], preg[KDA ? 2 : 1], oreg;
  float greg = 0.f, ograte = 0.f;
  const int orow = tid >> 2, occ = tid & 3;   // this thread's piece of the dO slice
  auto load = [&](int n) __attribute__((always_inline)) {
    const int t0 = n * C, cn = min(C, T - t0);
    const bf* rec = recs + ((size_t)head * NC + n) * RE;
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
      if constexpr (KDA) {   // (the record's rows past the sequence end are not zero)
        const uint32_t o = (uint32_t)r * DK + cc * 8;
        kreg[m] = r < cn ? ld16(rec + KR::kg + o) : zero_u4();
        qreg[m] = r < cn ? ld16(rec + KR::qg + o) : zero_u4();
        kcreg[m] = r < cn ? ld16(rec + KR::kc + o) : zero_u4();
      } else {
        const size_t off = (((size_t)b * T + t0 + r) * H + h) * DK + cc * 8;
        kreg[m] = r < cn ? ld16(kg + off) : zero_u4();
        qreg[m] = r < cn ? ld16(qg + off) : zero_u4();
      }
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = tid + kChainThreads * m, r = q >> 3, cc = q & 7;
      treg[m] = ld16(rec + r * C + cc * 8);
      if constexpr (KDA) preg[m] = ld16(rec + KR::p + r * C + cc * 8);
    }
    if constexpr (KDA) {
      if (tid < DK) greg = reinterpret_cast<const float*>(rec + KR::g)[tid];
    } else {
      const float* rg = reinterpret_cast<const float*>(rec + kRecG);
      if (tid < 3 * C) greg = rg[tid];
      ograte = rg[C + orow];
    }
    oreg = orow < cn ? ld16(dout_g + (((size_t)b * T + t0 + orow) * H + h) * DV + i0 + occ * 8) : zero_u4();
  };
  auto commit = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
      st16(Kb + r * LDK + cc * 8, kreg[m]);
      st16(Qb + r * LDK + cc * 8, qreg[m]);
      if constexpr (KDA) st16(Kcb + r * LDK + cc * 8, kcreg[m]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = tid + kChainThreads * m, r = q >> 3, cc = q & 7;
      st16(Tb + r * LDT + cc * 8, treg[m]);
      if constexpr (KDA) st16(Pt + r * LDT + cc * 8, preg[m]);
    }
    if (tid < (KDA ? DK : 3 * C)) Gs[tid] = greg;
    st16(dOb + orow * LDO + occ * 8, oreg);
    st16(dOg + orow * LDO + occ * 8, KDA ? oreg : scale16(oreg, ograte));
  };

  // P^T is zero where s >= 32 > r; nothing else writes there
  if (!KDA && wave == 3) {
#pragma unroll
    for (int g = 0; g < 4; ++g) store4(Pt + (32 + col) * LDT + 8 * g + 4 * hh, 0.f, 0.f, 0.f, 0.f);
  }
  // (the next chunk's registers go to LDS at the end of each step, as in bc_states)
  if (NC > 0) {
    load(NC - 1);
    commit();
  }
  for (int n = NC - 1; n >= 0; --n) {
    const int t0 = n * C, cn = min(C, T - t0);
    if (n > 0) load(n - 1);
    if (wave < DK / 32) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(dSb + col * LDK + 32 * wave + 8 * g + 4 * hh, dS[4 * g], dS[4 * g + 1], dS[4 * g + 2],
               dS[4 * g + 3]);
    }
    __syncthreads();
    {   // dS at the chunk's end -> workspace [head][n][DV][DK]
      bf* dst = dssave + (((size_t)head * NC + n) * DV + i0) * DK;
#pragma unroll
      for (int m = 0; m < SL * CPR / kChainThreads; ++m) {
        const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
        st16(dst + (size_t)r * DK + cc * 8, ld16(dSb + r * LDK + cc * 8));
      }
    }
    // P^T tiles: wave 0 (r, s < 32), wave 1 (r >= 32 > s), wave 2 (r, s >= 32)
    if (!KDA && wave < 3) {
      const int rr = wave >= 1 ? 1 : 0, sc = wave == 2 ? 1 : 0;
      f32x16 p = zero16();
      tile_nt_k<DK / 16>(p, Qb + 32 * rr * LDK, LDK, Kb + 32 * sc * LDK, LDK, lane);
      const int s = 32 * sc + col;
      const float gs = Gs[s];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = 32 * rr + 8 * g + 4 * hh;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = r0 + e >= s ? __expf(Gs[r0 + e] - gs) * p[4 * g + e] : 0.f;
        store4(Pt + s * LDT + r0, x[0], x[1], x[2], x[3]);
      }
    }
    f32x16 du = zero16();
    if (wave < 2) tile_nt_k<DK / 16>(du, Kcb + 32 * wave * LDK, LDK, dSb, LDK, lane);   // K dS^T
    __syncthreads();
    if (wave < 2) {   // dU = diag(exp(G_C - G)) K dS^T + P^T dO, rows s = 32 wave ..
      if constexpr (!KDA) {
#pragma unroll
        for (int v = 0; v < 16; ++v) du[v] *= eC[32 * wave + acc_row(v >> 2, v & 3, lane)];
      }
#pragma unroll
      for (int t = 0; t < C / 16; ++t)
        mma_bf16(du, KDA ? frag_perm_tr(Pt, LDT, 16 * t, 32 * wave, lane) : frag_perm(Pt + (32 * wave + col) * LDT, 16 * t, hh),
                 frag_perm_tr(dOb, LDO, 16 * t, 0, lane));
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(dUt + col * LDT + 32 * wave + 8 * g + 4 * hh, du[4 * g], du[4 * g + 1], du[4 * g + 2], du[4 * g + 3]);
    }
    __syncthreads();
    if (wave < 2) {   // dX = T^T dU = dV, row-major into dO's bytes (dO is dead)
      f32x16 dx = zero16();
#pragma unroll
      for (int t = 0; t < C / 16; ++t)
        mma_bf16(dx, frag_perm_tr(Tb, LDT, 16 * t, 32 * wave, lane), frag_perm(dUt + col * LDT, 16 * t, hh));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int s0 = 32 * wave + 8 * g + 4 * hh;
#pragma unroll
        for (int e = 0; e < 4; ++e) dOb[(s0 + e) * LDO + col] = (bf)dx[4 * g + e];
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = KDA ? -1.f : -eG[s0 + e];
        store4(Xn + col * LDT + s0, w[0] * dx[4 * g], w[1] * dx[4 * g + 1], w[2] * dx[4 * g + 2], w[3] * dx[4 * g + 3]);
      }
    }
    __syncthreads();
    // dV rows -> HBM, one 16-byte piece per thread
    if (orow < cn) st16(dvg + (((size_t)b * T + t0 + orow) * H + h) * DV + i0 + occ * 8, ld16(dOb + orow * LDO + occ * 8));
    if (wave < DK / 32) {   // dS^T <- gamma_C dS^T + Q^T diag(gamma) dO - K^T diag(gamma) dX
      if constexpr (KDA) {
#pragma unroll
        for (int v = 0; v < 16; ++v) dS[v] *= Gs[32 * wave + acc_row(v >> 2, v & 3, lane)];
      } else {
        const float gC = eG[C - 1];
#pragma unroll
        for (int v = 0; v < 16; ++v) dS[v] *= gC;
      }
#pragma unroll
      for (int t = 0; t < C / 16; ++t)
        mma_bf16(dS, frag_perm_tr(Qb, LDK, 16 * t, 32 * wave, lane), frag_perm_tr(dOg, LDO, 16 * t, 0, lane));
#pragma unroll
      for (int t = 0; t < C / 16; ++t)
        mma_bf16(dS, frag_perm_tr(Kb, LDK, 16 * t, 32 * wave, lane), frag_perm(Xn + col * LDT, 16 * t, hh));
    }
    __syncthreads();
    if (n > 0) commit();
  }
  if (wave < DK / 32 && a.dS0) {
    float* d = a.dS0 + ((size_t)head * DV + i0 + col) * DK + 32 * wave;
#pragma unroll
    for (int v = 0; v < 16; ++v) d[acc_row(v >> 2, v & 3, lane)] = dS[v];
  }
}

// ---------------------------------------------------------------------------
// bc_grad: dq, dk, dbeta, dalpha of one chunk of one head.
// ---------------------------------------------------------------------------
template <int DK>
struct GradLds {
  static constexpr int LDK = DK + 8;
  static constexpr int LDA = SolveLd<float>::LDA;   // fp32 C x C
  static constexpr size_t kb = 0;                                // K rows [C][LDK]
  static constexpr size_t qb = kb + (size_t)C * LDK * 2;         // Q rows [C][LDK]
  static constexpr size_t tb = qb + (size_t)C * LDK * 2;         // T [C][LDT]
  static constexpr size_t pt = tb + (size_t)C * LDT * 2;         // P^T [C][LDT]
  static constexpr size_t mb = pt + (size_t)C * LDT * 2;         // M [C][LDT]
  static constexpr size_t ek = mb + (size_t)C * LDT * 2;         // tril_-1(E o K K^T) [C][LDT]
  static constexpr size_t gs = ek + (size_t)C * LDT * 2;         // G, exp(G), exp(G_C - G), beta, ones
  static constexpr size_t gp = gs + 5 * C * 4;                   // dG partials [8][C]
  static constexpr size_t bp = gp + 8 * C * 4;                   // dbeta partials [4][C]
  static constexpr size_t misc = bp + 4 * C * 4;                 // per-wave sums [16]
  static constexpr size_t un = misc + 16 * 4;                    // region shared by three phases:
  // solve: A (in place L^-1 and scratch) fp32 [C][LDA], M fp32 [C][LDA]
  static constexpr size_t am = un;
  static constexpr size_t mf = am + (size_t)C * LDA * 4;
  static constexpr size_t solve_end = mf + (size_t)C * LDA * 4;
  // value slices: S, dS and their low parts [SL][LDK]; dO, dX [C][LDO];
  // X^T, U^T, dU^T and the low parts of X^T and dU^T [SL][LDT]
  static constexpr size_t ssl = un;
  static constexpr size_t dssl = ssl + (size_t)SL * LDK * 2;
  static constexpr size_t sslo = dssl + (size_t)SL * LDK * 2;
  static constexpr size_t dsslo = sslo + (size_t)SL * LDK * 2;
  static constexpr size_t dob = dsslo + (size_t)SL * LDK * 2;
  static constexpr size_t dxb = dob + (size_t)C * LDO * 2;
  static constexpr size_t xt = dxb + (size_t)C * LDO * 2;
  static constexpr size_t ut = xt + (size_t)SL * LDT * 2;
  static constexpr size_t dut = ut + (size_t)SL * LDT * 2;
  static constexpr size_t xtlo = dut + (size_t)SL * LDT * 2;
  static constexpr size_t dutlo = xtlo + (size_t)SL * LDT * 2;
  static constexpr size_t vb = dutlo + (size_t)SL * LDT * 2;     // V slice [C][LDO]
  static constexpr size_t slice_end = vb + (size_t)C * LDO * 2;
  // C x C algebra: dT^T, (dP o E)^T, N1^T, W^T [C][LDT]
  static constexpr size_t dtt = un;
  static constexpr size_t dpe = dtt + (size_t)C * LDT * 2;
  static constexpr size_t n1t = dpe + (size_t)C * LDT * 2;
  static constexpr size_t ws = n1t + (size_t)C * LDT * 2;
  static constexpr size_t stg = ws + (size_t)C * LDT * 2;           // dq, then dk, [C][LDK] bf16
  static constexpr size_t alg_end = stg + (size_t)C * LDK * 2;
  static constexpr size_t total = cmax(solve_end, cmax(slice_end, alg_end));
};

template <int DK, int DV>
__global__ __launch_bounds__(kGradThreads, 1) void bc_grad(BackwardArgs a, const bf* __restrict__ recs,
                                                           const bf* __restrict__ ssave,
                                                           const bf* __restrict__ dssave) {
  using L = GradLds<DK>;
  constexpr int LDK = L::LDK, LDA = L::LDA, CPR = DK / 8;
  constexpr int NT = 2 * DK / 32;   // C x DK tiles: wave w < NT owns rows 32 (w & 1) .., columns 32 (w >> 1) ..
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  bf* Kb = reinterpret_cast<bf*>(smem + L::kb);
  bf* Qb = reinterpret_cast<bf*>(smem + L::qb);
  bf* Tb = reinterpret_cast<bf*>(smem + L::tb);
  bf* Pt = reinterpret_cast<bf*>(smem + L::pt);
  bf* Mb = reinterpret_cast<bf*>(smem + L::mb);
  bf* EK = reinterpret_cast<bf*>(smem + L::ek);
  float* Gs = reinterpret_cast<float*>(smem + L::gs);
  float* eG = Gs + C;
  float* eC = Gs + 2 * C;
  float* Bt = Gs + 3 * C;
  float* ones = Gs + 4 * C;
  float* dGp = reinterpret_cast<float*>(smem + L::gp);
  float* dBp = reinterpret_cast<float*>(smem + L::bp);
  float* misc = reinterpret_cast<float*>(smem + L::misc);
  float* Am = reinterpret_cast<float*>(smem + L::am);
  float* Mf = reinterpret_cast<float*>(smem + L::mf);
  bf* Ssl = reinterpret_cast<bf*>(smem + L::ssl);
  bf* dSsl = reinterpret_cast<bf*>(smem + L::dssl);
  bf* dOb = reinterpret_cast<bf*>(smem + L::dob);
  bf* dXb = reinterpret_cast<bf*>(smem + L::dxb);
  bf* Xt = reinterpret_cast<bf*>(smem + L::xt);
  bf* Ut = reinterpret_cast<bf*>(smem + L::ut);
  bf* dUt = reinterpret_cast<bf*>(smem + L::dut);
  bf* Slo = reinterpret_cast<bf*>(smem + L::sslo);
  bf* dSlo = reinterpret_cast<bf*>(smem + L::dsslo);
  bf* Xtlo = reinterpret_cast<bf*>(smem + L::xtlo);
  bf* dUtlo = reinterpret_cast<bf*>(smem + L::dutlo);
  bf* Vb = reinterpret_cast<bf*>(smem + L::vb);
  bf* dTt = reinterpret_cast<bf*>(smem + L::dtt);
  bf* dPEt = reinterpret_cast<bf*>(smem + L::dpe);
  bf* N1t = reinterpret_cast<bf*>(smem + L::n1t);
  bf* Ws = reinterpret_cast<bf*>(smem + L::ws);
  bf* Stg = reinterpret_cast<bf*>(smem + L::stg);

  // (the wave index in a scalar register: branches on it are uniform jumps)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int T = a.T, H = a.H, NC = (T + C - 1) / C;
  // chunk index outermost, ascending: bc_rev visited the chunks in reverse,
  // so the first chunks of every head are the ones still in the last-level cache
  const int nheads = a.B * H;
  const int head = blockIdx.x % nheads, n = blockIdx.x / nheads;
  const int b = head / H, h = head % H, t0 = n * C, cn = min(C, T - t0);
  const bf* rec = recs + ((size_t)head * NC + n) * kRecElems;
  const float* rg = reinterpret_cast<const float*>(rec + kRecG);
  auto tok = [&](int r) { return ((size_t)b * T + t0 + r) * H + h; };

  // The first chunk's entry state is S0 and the last chunk's end gradient is
  // dS_final, both fp32 inputs: those chunks take them whole (hi + lo parts)
  // instead of the chains' bf16 copies.  (With one chunk, dbeta and dalpha
  // then rest on no rounded state at all.)
  const bool s_exact = n == 0, ds_exact = n == NC - 1;
  // Global inputs of a value slice, loaded one slice ahead into registers:
  // the bf16 S and dS pieces (one 16-byte piece of each per thread) and the
  // dO, dX, V pieces (768 over the 512 threads).
  static_assert(SL * CPR <= kGradThreads && 3 * C * SL / 8 <= 2 * kGradThreads, "slice pieces per thread");
  u32x4 pS = zero_u4(), pD = zero_u4(), pO0 = zero_u4(), pO1 = zero_u4();
  auto piece = [&](int p, int i0) __attribute__((always_inline)) {
    const int kind = p >> 8, q = p & 255, r = q >> 2, c4 = q & 3;
    const void* src = kind == 0 ? a.dout : kind == 1 ? a.dv : a.v;
    return r < cn ? ld16(static_cast<const bf*>(src) + tok(r) * DV + i0 + c4 * 8) : zero_u4();
  };
  auto load_slice = [&](int sl) __attribute__((always_inline)) {
    const int i0 = sl * SL;
    if (tid < SL * CPR) {
      const size_t off = (((size_t)head * NC + n) * DV + i0 + tid / CPR) * DK + (tid % CPR) * 8;
      if (!s_exact) pS = ld16(ssave + off);
      if (!ds_exact) pD = ld16(dssave + off);
    }
    pO0 = piece(tid, i0);
    if (tid < 3 * C * SL / 8 - kGradThreads) pO1 = piece(tid + kGradThreads, i0);
  };
  // ---- stage K, Q, gates (their loads go out before the first slice's); clear the partial sums ----
  {
    const bf* kg = static_cast<const bf*>(a.k);
    const bf* qg = static_cast<const bf*>(a.q);
    constexpr int KQ = (C * CPR + kGradThreads - 1) / kGradThreads;
    static_assert(C * CPR % kGradThreads == 0, "K rows split evenly");
    u32x4 kr[KQ], qr[KQ];
#pragma unroll
    for (int m = 0; m < KQ; ++m) {
      const int q = tid + kGradThreads * m, r = q / CPR, cc = q % CPR;
      const bool ok = r < cn;
      kr[m] = ok ? ld16(kg + tok(r) * DK + cc * 8) : zero_u4();
      qr[m] = ok ? ld16(qg + tok(r) * DK + cc * 8) : zero_u4();
    }
    const float gr = tid < 3 * C ? rg[tid] : 0.f;
    const float br = tid < cn ? a.beta[tok(tid)] : 0.f;
    load_slice(0);
#pragma unroll
    for (int m = 0; m < KQ; ++m) {
      const int q = tid + kGradThreads * m, r = q / CPR, cc = q % CPR;
      st16(Kb + r * LDK + cc * 8, kr[m]);
      st16(Qb + r * LDK + cc * 8, qr[m]);
    }
    if (tid < 3 * C) Gs[tid] = gr;
    if (tid < C) {
      Bt[tid] = br;
      ones[tid] = 1.f;
    }
    for (int q = tid; q < 12 * C + 16; q += kGradThreads) dGp[q] = 0.f;   // dGp, dBp, misc
  }
  __syncthreads();

  // ---- K K^T (waves 0-3) and Q K^T (waves 4-7), tile (rr, sc) of each ----
  {
    const int w4 = wave & 3, rr = w4 >> 1, sc = w4 & 1;
    const bool kk = wave < 4;
    if (rr == 0 && sc == 1) {   // above the diagonal: zero (A's is the solve's scratch)
      if (kk) {
#pragma unroll
        for (int v = 0; v < 16; ++v) EK[acc_row(v >> 2, v & 3, lane) * LDT + 32 + col] = (bf)0.f;
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) store4(Pt + (32 + col) * LDT + 8 * g + 4 * hh, 0.f, 0.f, 0.f, 0.f);
      }
    } else {
      f32x16 p = zero16();
      tile_nt_k<DK / 16>(p, (kk ? Kb : Qb) + 32 * rr * LDK, LDK, Kb + 32 * sc * LDK, LDK, lane);
      const int s = 32 * sc + col;
      const float gs = Gs[s];
      if (kk) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = 32 * rr + acc_row(v >> 2, v & 3, lane);
          const float x = s < r ? __expf(Gs[r] - gs) * p[v] : 0.f;
          EK[r * LDT + s] = (bf)x;
          Am[r * LDA + s] = Bt[r] * x;
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = 32 * rr + 8 * g + 4 * hh;
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = r0 + e >= s ? __expf(Gs[r0 + e] - gs) * p[4 * g + e] : 0.f;
          store4(Pt + s * LDT + r0, x[0], x[1], x[2], x[3]);
        }
      }
    }
  }
  __syncthreads();
  // ---- M = (I + A)^-1 (waves 0-3; the others pass the solve's four barriers) ----
  if (wave < 4) {
    tri_solve<float, LDA>(Am, Am, Am + 32, ones, Mf, tid);
  } else {
    __syncthreads();
    __syncthreads();
    __syncthreads();
    __syncthreads();
  }
  {   // M and T = M diag(beta) in bf16
    const int r = tid >> 3, c0 = (tid & 7) * 8;
    float m[8], t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      m[e] = Mf[r * LDA + c0 + e];
      t[e] = m[e] * Bt[c0 + e];
    }
    store4(Mb + r * LDT + c0, m[0], m[1], m[2], m[3]);
    store4(Mb + r * LDT + c0 + 4, m[4], m[5], m[6], m[7]);
    store4(Tb + r * LDT + c0, t[0], t[1], t[2], t[3]);
    store4(Tb + r * LDT + c0 + 4, t[4], t[5], t[6], t[7]);
  }
  __syncthreads();

  // ---- the value axis in slices of 32 columns ----
  const int rr = (wave & 3) >> 1, sc = wave & 1;        // C x C tile of this wave
  const int rt = wave & 1, jt = wave >> 1;              // C x DK tile of this wave (wave < NT)
  f32x16 cc_acc = zero16();   // waves 0-3: dT tile; waves 4-7: dP tile
  f32x16 dQi = zero16(), P1 = zero16(), P2 = zero16();
  float sd = 0.f;             // this thread's part of <dS, S>
  for (int sl = 0; sl < DV / SL; ++sl) {
    const int i0 = sl * SL;
    {
      if (tid < SL * CPR) {
        const int r = tid / CPR, cc = tid % CPR;
        float xs[8], xd[8];
        u32x4 hi, lo;
        if (s_exact) {
          const float* src = a.S0 ? a.S0 + ((size_t)head * DV + i0 + r) * DK + cc * 8 : nullptr;
#pragma unroll
          for (int e = 0; e < 8; ++e) xs[e] = src ? src[e] : 0.f;
          split8(xs, hi, lo);
          st16(Slo + r * LDK + cc * 8, lo);
        } else {
          hi = pS;
          unpack8(hi, xs);
        }
        st16(Ssl + r * LDK + cc * 8, hi);
        if (ds_exact) {
          const float* src = a.dS_final ? a.dS_final + ((size_t)head * DV + i0 + r) * DK + cc * 8 : nullptr;
#pragma unroll
          for (int e = 0; e < 8; ++e) xd[e] = src ? src[e] : 0.f;
          split8(xd, hi, lo);
          st16(dSlo + r * LDK + cc * 8, lo);
        } else {
          hi = pD;
          unpack8(hi, xd);
        }
        st16(dSsl + r * LDK + cc * 8, hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) sd += xs[e] * xd[e];
      }
      auto put = [&](int p, const u32x4& x) __attribute__((always_inline)) {
        const int kind = p >> 8, q = p & 255;
        st16((kind == 0 ? dOb : kind == 1 ? dXb : Vb) + (q >> 2) * LDO + (q & 3) * 8, x);
      };
      put(tid, pO0);
      if (tid < 3 * C * SL / 8 - kGradThreads) put(tid + kGradThreads, pO1);
    }
    if (sl + 1 < DV / SL) load_slice(sl + 1);
    __syncthreads();
    f32x16 y = zero16();
    if (wave < 2) {   // X = V - diag(gamma) K S^T -> X^T (hi and lo parts)
      tile_nt_k<DK / 16>(y, Kb + 32 * wave * LDK, LDK, Ssl, LDK, lane);
      if (s_exact) tile_nt_k<DK / 16>(y, Kb + 32 * wave * LDK, LDK, Slo, LDK, lane);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = 32 * wave + 8 * g + 4 * hh;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (float)Vb[(r0 + e) * LDO + col] - eG[r0 + e] * y[4 * g + e];
        store4_split(Xt + col * LDT + r0, Xtlo + col * LDT + r0, x[0], x[1], x[2], x[3]);
      }
    } else if (wave < 4) {   // K dS^T, rows 32 (wave - 2) ..
      tile_nt_k<DK / 16>(y, Kb + 32 * (wave - 2) * LDK, LDK, dSsl, LDK, lane);
      if (ds_exact) tile_nt_k<DK / 16>(y, Kb + 32 * (wave - 2) * LDK, LDK, dSlo, LDK, lane);
    }
    __syncthreads();
    if (wave < 2) {   // U = T X -> U^T
      f32x16 u = zero16();
      tile_nt_k<C / 16>(u, Tb + 32 * wave * LDT, LDT, Xt, LDT, lane);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(Ut + col * LDT + 32 * wave + 8 * g + 4 * hh, u[4 * g], u[4 * g + 1], u[4 * g + 2], u[4 * g + 3]);
    } else if (wave < 4) {   // dU = diag(exp(G_C - G)) K dS^T + P^T dO -> dU^T
      const int s0 = 32 * (wave - 2);
#pragma unroll
      for (int v = 0; v < 16; ++v) y[v] *= eC[s0 + acc_row(v >> 2, v & 3, lane)];
#pragma unroll
      for (int t = 0; t < C / 16; ++t)
        mma_bf16(y, frag_perm(Pt + (s0 + col) * LDT, 16 * t, hh), frag_perm_tr(dOb, LDO, 16 * t, 0, lane));
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4_split(dUt + col * LDT + s0 + 8 * g + 4 * hh, dUtlo + col * LDT + s0 + 8 * g + 4 * hh, y[4 * g],
                     y[4 * g + 1], y[4 * g + 2], y[4 * g + 3]);
    }
    __syncthreads();
    if (wave < 4) {   // dT += dU X^T, hi * hi + hi * lo + lo * hi (dbeta is a short sum of these)
#pragma unroll
      for (int t = 0; t < SL / 16; ++t) {
        const bf16x8 uh = frag_perm_tr(dUt, LDT, 16 * t, 32 * rr, lane);
        const bf16x8 xh = frag_perm_tr(Xt, LDT, 16 * t, 32 * sc, lane);
        mma_bf16(cc_acc, uh, xh);
        mma_bf16(cc_acc, uh, frag_perm_tr(Xtlo, LDT, 16 * t, 32 * sc, lane));
        mma_bf16(cc_acc, frag_perm_tr(dUtlo, LDT, 16 * t, 32 * rr, lane), xh);
      }
    } else if (rr >= sc) {   // dP += dO U^T (the tile above the diagonal stays zero)
#pragma unroll
      for (int t = 0; t < SL / 16; ++t)
        mma_bf16(cc_acc, frag_perm(dOb + (32 * rr + col) * LDO, 16 * t, hh), frag_perm_tr(Ut, LDT, 16 * t, 32 * sc, lane));
    }
    if (wave < NT) {   // dO S, dX S, U dS
#pragma unroll
      for (int t = 0; t < SL / 16; ++t) {
        const bf16x8 bs = frag_perm_tr(Ssl, LDK, 16 * t, 32 * jt, lane);
        mma_bf16(dQi, frag_perm(dOb + (32 * rt + col) * LDO, 16 * t, hh), bs);
        mma_bf16(P1, frag_perm(dXb + (32 * rt + col) * LDO, 16 * t, hh), bs);
        mma_bf16(P2, frag_perm_tr(Ut, LDT, 16 * t, 32 * rt, lane), frag_perm_tr(dSsl, LDK, 16 * t, 32 * jt, lane));
      }
    }
    __syncthreads();
  }

  // rows of the staging buffer -> [B, T, H, DK] in HBM, 16 bytes per thread and step
  auto store_rows = [&](void* dst) __attribute__((always_inline)) {
    bf* g = static_cast<bf*>(dst);
    for (int q = tid; q < C * CPR; q += kGradThreads) {
      const int r = q / CPR, cc = q % CPR;
      if (r < cn) st16(g + tok(r) * DK + cc * 8, ld16(Stg + r * LDK + cc * 8));
    }
  };
  // ---- C x C algebra ----
  float* myG = dGp + wave * C;
  if (wave < 4) {   // dT -> dT^T
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4(dTt + (32 * sc + col) * LDT + 32 * rr + 8 * g + 4 * hh, cc_acc[4 * g], cc_acc[4 * g + 1],
             cc_acc[4 * g + 2], cc_acc[4 * g + 3]);
  } else {   // dP: rows(Y) - cols(Y) into dG; (dP o E)^T
    const int s = 32 * sc + col;
    if (rr < sc) {
#pragma unroll
      for (int g = 0; g < 4; ++g) store4(dPEt + s * LDT + 32 * rr + 8 * g + 4 * hh, 0.f, 0.f, 0.f, 0.f);
    } else {
      f32x16 yv, pe;
      const float gs = Gs[s];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * rr + acc_row(v >> 2, v & 3, lane);
        const float d = r >= s ? cc_acc[v] : 0.f;
        yv[v] = d * (float)Pt[s * LDT + r];
        pe[v] = d * __expf(Gs[r] - gs);
      }
      tile_row_col_sums<true>(yv, myG, 32 * rr, myG, 32 * sc, lane);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(dPEt + s * LDT + 32 * rr + 8 * g + 4 * hh, pe[4 * g], pe[4 * g + 1], pe[4 * g + 2], pe[4 * g + 3]);
    }
  }
  f32x16 qv = zero16();   // Q o diag(gamma) dO S: its row sums go into dG with those of the dK terms
  if (wave < NT) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 32 * rt + acc_row(v >> 2, v & 3, lane);
      dQi[v] *= eG[r];
      qv[v] = (float)Qb[r * LDK + 32 * jt + col] * dQi[v];
    }
  }
  __syncthreads();
  if (wave < 4) {   // N1 = M^T dT; dbeta += diag(N1); N1 -> N1^T
    f32x16 n1 = zero16();
#pragma unroll
    for (int t = 0; t < C / 16; ++t)
      mma_bf16(n1, frag_perm_tr(Mb, LDT, 16 * t, 32 * rr, lane), frag_perm(dTt + (32 * sc + col) * LDT, 16 * t, hh));
    if (rr == sc) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (acc_row(v >> 2, v & 3, lane) == col) dBp[wave * C + 32 * rr + col] += n1[v];
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4(N1t + (32 * sc + col) * LDT + 32 * rr + 8 * g + 4 * hh, n1[4 * g], n1[4 * g + 1], n1[4 * g + 2],
             n1[4 * g + 3]);
  }
  if (wave < NT) {   // dQ = diag(gamma) dO S + (dP o E) K
#pragma unroll
    for (int t = 0; t < C / 16; ++t)
      mma_bf16(dQi, frag_perm_tr(dPEt, LDT, 16 * t, 32 * rt, lane), frag_perm_tr(Kb, LDK, 16 * t, 32 * jt, lane));
#pragma unroll
    for (int v = 0; v < 16; ++v) Stg[(32 * rt + acc_row(v >> 2, v & 3, lane)) * LDK + 32 * jt + col] = (bf)dQi[v];
  }
  __syncthreads();
  store_rows(a.dq);
  if (wave == 1) {   // W^T is zero where s >= 32 > r
#pragma unroll
    for (int g = 0; g < 4; ++g) store4(Ws + (32 + col) * LDT + 8 * g + 4 * hh, 0.f, 0.f, 0.f, 0.f);
  }
  if (wave < 4 && rr >= sc) {   // dA = -tril_-1(N1 T^T); dbeta, Z, W
    f32x16 da = zero16();
#pragma unroll
    for (int t = 0; t < C / 16; ++t)
      mma_bf16(da, frag_perm_tr(N1t, LDT, 16 * t, 32 * rr, lane), frag_perm(Tb + (32 * sc + col) * LDT, 16 * t, hh));
    const int s = 32 * sc + col;
    const float gs = Gs[s];
    f32x16 bz, zz, wv;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 32 * rr + acc_row(v >> 2, v & 3, lane);
      const float d = r > s ? -da[v] : 0.f;
      const float ekk = (float)EK[r * LDT + s];
      bz[v] = d * ekk;
      zz[v] = bz[v] * Bt[r];
      wv[v] = Bt[r] * d * __expf(Gs[r] - gs);
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)   // W^T[s][r], 8-byte stores
      store4(Ws + s * LDT + 32 * rr + 8 * g + 4 * hh, wv[4 * g], wv[4 * g + 1], wv[4 * g + 2], wv[4 * g + 3]);
    // Z = diag(beta) (dA o E o K K^T): its row sums are beta_r times those of bz
    float sr[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) sr[v] = half_sum(bz[v]);
    const int j = lane & 31;
    float mine = sr[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mine = j == v ? sr[v] : mine;
    if (j < 16) {
      const int r = 32 * rr + acc_row(j >> 2, j & 3, lane);
      dBp[wave * C + r] += mine;
      myG[r] += Bt[r] * mine;
    }
    float cz = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) cz += zz[v];
    cz += __shfl_xor(cz, 32);
    if (lane < 32) myG[32 * sc + lane] -= cz;
  }
  float gcp = 0.f;   // this wave's part of sum_r k_r . (exp(G_C - G_r) U dS)_r
  if (wave < NT) {   // dK so far: -diag(gamma) dX S + diag(exp(G_C - G)) U dS; dG terms of both
    f32x16 kv;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 32 * rt + acc_row(v >> 2, v & 3, lane);
      const float t1 = eG[r] * P1[v], t2 = eC[r] * P2[v];
      const float kr = (float)Kb[r * LDK + 32 * jt + col];
      kv[v] = qv[v] - kr * (t1 + t2);
      gcp += kr * t2;
      P1[v] = t2 - t1;
    }
    tile_row_col_sums<false>(kv, myG, 32 * rt, nullptr, 0, lane);
  }
  __syncthreads();
  if (wave < NT) {   // dK += W K + W^T K + (dP o E)^T Q (W^T is stored)
#pragma unroll
    for (int t = 0; t < C / 16; ++t) {
      const bf16x8 kf = frag_perm_tr(Kb, LDK, 16 * t, 32 * jt, lane);
      mma_bf16(P1, frag_perm_tr(Ws, LDT, 16 * t, 32 * rt, lane), kf);
      mma_bf16(P1, frag_perm(Ws + (32 * rt + col) * LDT, 16 * t, hh), kf);
    }
#pragma unroll
    for (int t = 0; t < C / 16; ++t)
      mma_bf16(P1, frag_perm(dPEt + (32 * rt + col) * LDT, 16 * t, hh), frag_perm_tr(Qb, LDK, 16 * t, 32 * jt, lane));
#pragma unroll
    for (int v = 0; v < 16; ++v) Stg[(32 * rt + acc_row(v >> 2, v & 3, lane)) * LDK + 32 * jt + col] = (bf)P1[v];
  }
  {   // per-wave sums: <dS, S> and gcp
    float x = sd, y = gcp;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      x += __shfl_xor(x, off);
      y += __shfl_xor(y, off);
    }
    if (lane == 0) {
      misc[wave] = x;
      misc[8 + wave] = y;
    }
  }
  __syncthreads();
  store_rows(a.dk);
  if (wave == 0) {   // dG -> dlog alpha (sum over the rows at or after each token), dbeta
    const int r = lane;
    float g = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) g += dGp[w * C + r];
    if (r == C - 1) {
      float sds = 0.f, gc = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        sds += misc[w];
        gc += misc[8 + w];
      }
      g += eG[C - 1] * sds + gc;
    }
    // suffix sum over the lanes
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_down(g, off);
      if (r + off < 64) g += o;
    }
    if (r < cn) {
      const size_t t = tok(r);
      a.dbeta[t] = dBp[r] + dBp[C + r] + dBp[2 * C + r] + dBp[3 * C + r];
      if (a.mode == 1) {
        const float al = static_cast<const float*>(a.alpha)[t];
        a.dalpha[t] = logf(al) < kLogFloor ? 0.f : g / al;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per-channel decay, after the two chains: bk_gradv (the value axis and the
// C x C algebra) and bk_chan (the channel-weighted contractions, dq, dk,
// dalpha).  With G the running sum of log alpha per channel inside the chunk,
// E3[r][s][c] = exp(G[r][c] - G[s][c]) (<= 1 for s <= r), At[r][s] =
// sum_c k_r[c] k_s[c] E3[r][s][c], A = tril_-1(diag(beta) At), P = tril_0(sum_c
// q_r[c] k_s[c] E3[r][s][c]) and the record's operands Kg = K (.) Gamma,
// Qg = Q (.) Gamma, Kc = K (.) exp(G_C - G):
//   dU = P^T dO + Kc dS^T,  dX = T^T dU,  dT = dU X^T,  N1 = M^T dT,
//   dA = -tril_-1(N1 T^T),  dP = tril_0(dO U^T),  W = diag(beta) dA
//   dbeta_r = N1[r][r] + sum_s dA[r][s] At[r][s]
//   R_Pq[r] = sum_s dP[r][s] k_s (.) E3[r][s]    R_Pk[s] = sum_r dP[r][s] q_r (.) E3[r][s]
//   R_Ar[r] = sum_s W[r][s] k_s (.) E3[r][s]     R_Ac[s] = sum_r W[r][s] k_r (.) E3[r][s]
//   dq = R_Pq + Gamma (.) dO S
//   dk = R_Pk + R_Ar + R_Ac - Gamma (.) dX S + exp(G_C - G) (.) U dS
//   dG = q (.) (R_Pq + Gamma (.) dO S) - k (.) (R_Pk - R_Ar + R_Ac + Gamma (.) dX S + exp(G_C - G) (.) U dS)
//   dG[last] += gamma_C (.) sum_i dS[i] (.) S[i] + sum_r k_r (.) exp(G_C - G_r) (.) (U dS)_r
//   dlog alpha_t = sum_{r >= t} dG_r inside the chunk.
// bk_gradv leaves dP, W, dO S, dX S, U dS and sum_i dS[i] (.) S[i] (fp32) in
// the workspace; bk_chan forms the four R terms on the vector ALUs.
// ---------------------------------------------------------------------------
template <int DK>
struct KGradOut {   // fp32 offsets inside one chunk's block
  static constexpr size_t dp = 0, w = (size_t)C * C, dqs = 2 * (size_t)C * C, dxs = dqs + (size_t)C * DK,
                          uds = dxs + (size_t)C * DK, d1 = uds + (size_t)C * DK, floats = d1 + DK;
};

template <int DK>
struct KGradLds {
  static constexpr int LDK = DK + 8;
  static constexpr int LDA = SolveLd<float>::LDA;
  static constexpr size_t kgb = 0;                                // Kg rows [C][LDK]
  static constexpr size_t kcb = kgb + (size_t)C * LDK * 2;        // Kc rows [C][LDK]
  static constexpr size_t tb = kcb + (size_t)C * LDK * 2;         // T [C][LDT]
  static constexpr size_t pb = tb + (size_t)C * LDT * 2;          // P [C][LDT], row-major
  static constexpr size_t mb = pb + (size_t)C * LDT * 2;          // M [C][LDT]
  static constexpr size_t ek = mb + (size_t)C * LDT * 2;          // At [C][LDT]
  static constexpr size_t gs = ek + (size_t)C * LDT * 2;          // beta, ones
  static constexpr size_t bp = gs + 2 * C * 4;                    // dbeta partials [4][C]
  static constexpr size_t d1p = bp + 4 * C * 4;                   // <dS, S> partials [8][DK]
  static constexpr size_t un = d1p + 8 * DK * 4;
  static constexpr size_t am = un;                                // solve: A, then M fp32 [C][LDA]
  static constexpr size_t mf = am + (size_t)C * LDA * 4;
  static constexpr size_t solve_end = mf + (size_t)C * LDA * 4;
  static constexpr size_t ssl = un;                               // value slices, as bc_grad
  static constexpr size_t dssl = ssl + (size_t)SL * LDK * 2;
  static constexpr size_t sslo = dssl + (size_t)SL * LDK * 2;
  static constexpr size_t dsslo = sslo + (size_t)SL * LDK * 2;
  static constexpr size_t dob = dsslo + (size_t)SL * LDK * 2;
  static constexpr size_t dxb = dob + (size_t)C * LDO * 2;
  static constexpr size_t xt = dxb + (size_t)C * LDO * 2;
  static constexpr size_t ut = xt + (size_t)SL * LDT * 2;
  static constexpr size_t dut = ut + (size_t)SL * LDT * 2;
  static constexpr size_t xtlo = dut + (size_t)SL * LDT * 2;
  static constexpr size_t dutlo = xtlo + (size_t)SL * LDT * 2;
  static constexpr size_t vb = dutlo + (size_t)SL * LDT * 2;
  static constexpr size_t slice_end = vb + (size_t)C * LDO * 2;
  static constexpr size_t dtt = un;                               // algebra: dT^T, N1^T [C][LDT]
  static constexpr size_t n1t = dtt + (size_t)C * LDT * 2;
  static constexpr size_t alg_end = n1t + (size_t)C * LDT * 2;
  static constexpr size_t total = cmax(solve_end, cmax(slice_end, alg_end));
};

template <int DK, int DV>
__global__ __launch_bounds__(kGradThreads, 1) void bk_gradv(BackwardArgs a, const bf* __restrict__ recs,
                                                            const float* __restrict__ atil,
                                                            const bf* __restrict__ ssave,
                                                            const bf* __restrict__ dssave, float* __restrict__ gout) {
  using L = KGradLds<DK>;
  using KR = KRec<DK>;
  using GO = KGradOut<DK>;
  constexpr int LDK = L::LDK, LDA = L::LDA, CPR = DK / 8;
  constexpr int NT = 2 * DK / 32;   // C x DK tiles: wave w < NT owns rows 32 (w & 1) .., columns 32 (w >> 1) ..
  static_assert(L::total <= 160 * 1024, "LDS plan exceeds 160 KiB");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  bf* Kgb = reinterpret_cast<bf*>(smem + L::kgb);
  bf* Kcb = reinterpret_cast<bf*>(smem + L::kcb);
  bf* Tb = reinterpret_cast<bf*>(smem + L::tb);
  bf* Pb = reinterpret_cast<bf*>(smem + L::pb);
  bf* Mb = reinterpret_cast<bf*>(smem + L::mb);
  bf* EK = reinterpret_cast<bf*>(smem + L::ek);
  float* Bt = reinterpret_cast<float*>(smem + L::gs);
  float* ones = Bt + C;
  float* dBp = reinterpret_cast<float*>(smem + L::bp);
  float* d1p = reinterpret_cast<float*>(smem + L::d1p);
  float* Am = reinterpret_cast<float*>(smem + L::am);
  float* Mf = reinterpret_cast<float*>(smem + L::mf);
  bf* Ssl = reinterpret_cast<bf*>(smem + L::ssl);
  bf* dSsl = reinterpret_cast<bf*>(smem + L::dssl);
  bf* dOb = reinterpret_cast<bf*>(smem + L::dob);
  bf* dXb = reinterpret_cast<bf*>(smem + L::dxb);
  bf* Xt = reinterpret_cast<bf*>(smem + L::xt);
  bf* Ut = reinterpret_cast<bf*>(smem + L::ut);
  bf* dUt = reinterpret_cast<bf*>(smem + L::dut);
  bf* Slo = reinterpret_cast<bf*>(smem + L::sslo);
  bf* dSlo = reinterpret_cast<bf*>(smem + L::dsslo);
  bf* Xtlo = reinterpret_cast<bf*>(smem + L::xtlo);
  bf* dUtlo = reinterpret_cast<bf*>(smem + L::dutlo);
  bf* Vb = reinterpret_cast<bf*>(smem + L::vb);
  bf* dTt = reinterpret_cast<bf*>(smem + L::dtt);
  bf* N1t = reinterpret_cast<bf*>(smem + L::n1t);

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, hh = lane >> 5;
  const int T = a.T, H = a.H, NC = (T + C - 1) / C;
  const int nheads = a.B * H;
  const int head = blockIdx.x % nheads, n = blockIdx.x / nheads;
  const int b = head / H, h = head % H, t0 = n * C, cn = min(C, T - t0);
  const size_t chunk = (size_t)head * NC + n;
  const bf* rec = recs + chunk * KR::elems;
  float* go = gout + chunk * GO::floats;
  auto tok = [&](int r) { return ((size_t)b * T + t0 + r) * H + h; };

  // (as bc_grad) the fp32 entry state and end gradient are taken whole where
  // they are inputs; the slice inputs are loaded one slice ahead
  const bool s_exact = n == 0, ds_exact = n == NC - 1;
  static_assert(SL * CPR <= kGradThreads && 3 * C * SL / 8 <= 2 * kGradThreads, "slice pieces per thread");
  u32x4 pS = zero_u4(), pD = zero_u4(), pO0 = zero_u4(), pO1 = zero_u4();
  auto piece = [&](int p, int i0) __attribute__((always_inline)) {
    const int kind = p >> 8, q = p & 255, r = q >> 2, c4 = q & 3;
    const void* src = kind == 0 ? a.dout : kind == 1 ? a.dv : a.v;
    return r < cn ? ld16(static_cast<const bf*>(src) + tok(r) * DV + i0 + c4 * 8) : zero_u4();
  };
  auto load_slice = [&](int sl) __attribute__((always_inline)) {
    const int i0 = sl * SL;
    if (tid < SL * CPR) {
      const size_t off = (chunk * DV + i0 + tid / CPR) * DK + (tid % CPR) * 8;
      if (!s_exact) pS = ld16(ssave + off);
      if (!ds_exact) pD = ld16(dssave + off);
    }
    pO0 = piece(tid, i0);
    if (tid < 3 * C * SL / 8 - kGradThreads) pO1 = piece(tid + kGradThreads, i0);
  };
  // ---- stage Kg, Kc, P, At, beta ----
  constexpr int KQ = C * CPR / kGradThreads;
  static_assert(C * CPR % kGradThreads == 0 && C * C / 8 == kGradThreads, "even split");
  float4 at4[2];
  {
    u32x4 kr[KQ], kc[KQ];
#pragma unroll
    for (int m = 0; m < KQ; ++m) {
      const int q = tid + kGradThreads * m, r = q / CPR, cc = q % CPR;
      const bool ok = r < cn;   // (the record's rows past the sequence end are not zero)
      kr[m] = ok ? ld16(rec + KR::kg + r * DK + cc * 8) : zero_u4();
      kc[m] = ok ? ld16(rec + KR::kc + r * DK + cc * 8) : zero_u4();
    }
    const u32x4 pr = ld16(rec + KR::p + (tid >> 3) * C + (tid & 7) * 8);
    const float4* ag = reinterpret_cast<const float4*>(atil + chunk * C * C);
    at4[0] = ag[tid];
    at4[1] = ag[tid + kGradThreads];
    const float br = tid < cn ? a.beta[tok(tid)] : 0.f;
    load_slice(0);
#pragma unroll
    for (int m = 0; m < KQ; ++m) {
      const int q = tid + kGradThreads * m, r = q / CPR, cc = q % CPR;
      st16(Kgb + r * LDK + cc * 8, kr[m]);
      st16(Kcb + r * LDK + cc * 8, kc[m]);
    }
    st16(Pb + (tid >> 3) * LDT + (tid & 7) * 8, pr);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int e = 4 * (tid + kGradThreads * m), r = e / C, s0 = e % C;
      store4(EK + r * LDT + s0, at4[m].x, at4[m].y, at4[m].z, at4[m].w);
    }
    if (tid < C) {
      Bt[tid] = br;
      ones[tid] = 1.f;
    }
    for (int q = tid; q < 4 * C + 8 * DK; q += kGradThreads) dBp[q] = 0.f;   // dBp, d1p
  }
  __syncthreads();
  // A = diag(beta) At below the diagonal (the upper-right block is the solve's scratch)
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int e = 4 * (tid + kGradThreads * m), r = e / C, s0 = e % C;
    if (r < 32 && s0 >= 32) continue;
    const float x[4] = {at4[m].x, at4[m].y, at4[m].z, at4[m].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) Am[r * LDA + s0 + j] = s0 + j < r ? Bt[r] * x[j] : 0.f;
  }
  __syncthreads();
  // ---- M = (I + A)^-1 (waves 0-3; the others pass the solve's four barriers) ----
  if (wave < 4) {
    tri_solve<float, LDA>(Am, Am, Am + 32, ones, Mf, tid);
  } else {
    __syncthreads();
    __syncthreads();
    __syncthreads();
    __syncthreads();
  }
  {   // M and T = M diag(beta) in bf16
    const int r = tid >> 3, c0 = (tid & 7) * 8;
    float m[8], t[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      m[e] = Mf[r * LDA + c0 + e];
      t[e] = m[e] * Bt[c0 + e];
    }
    store4(Mb + r * LDT + c0, m[0], m[1], m[2], m[3]);
    store4(Mb + r * LDT + c0 + 4, m[4], m[5], m[6], m[7]);
    store4(Tb + r * LDT + c0, t[0], t[1], t[2], t[3]);
    store4(Tb + r * LDT + c0 + 4, t[4], t[5], t[6], t[7]);
  }
  __syncthreads();

  // ---- the value axis in slices of 32 columns ----
  const int rr = (wave & 3) >> 1, sc = wave & 1;        // C x C tile of this wave
  const int rt = wave & 1, jt = wave >> 1;              // C x DK tile of this wave (wave < NT)
  f32x16 cc_acc = zero16();   // waves 0-3: dT tile; waves 4-7: dP tile
  f32x16 dQi = zero16(), P1 = zero16(), P2 = zero16();
  float sd[8];                // this thread's part of sum_i dS[i] (.) S[i], 8 channels
#pragma unroll
  for (int e = 0; e < 8; ++e) sd[e] = 0.f;
  for (int sl = 0; sl < DV / SL; ++sl) {
    const int i0 = sl * SL;
    {
      if (tid < SL * CPR) {
        const int r = tid / CPR, cc = tid % CPR;
        float xs[8], xd[8];
        u32x4 hi, lo;
        if (s_exact) {
          const float* src = a.S0 ? a.S0 + ((size_t)head * DV + i0 + r) * DK + cc * 8 : nullptr;
#pragma unroll
          for (int e = 0; e < 8; ++e) xs[e] = src ? src[e] : 0.f;
          split8(xs, hi, lo);
          st16(Slo + r * LDK + cc * 8, lo);
        } else {
          hi = pS;
          unpack8(hi, xs);
        }
        st16(Ssl + r * LDK + cc * 8, hi);
        if (ds_exact) {
          const float* src = a.dS_final ? a.dS_final + ((size_t)head * DV + i0 + r) * DK + cc * 8 : nullptr;
#pragma unroll
          for (int e = 0; e < 8; ++e) xd[e] = src ? src[e] : 0.f;
          split8(xd, hi, lo);
          st16(dSlo + r * LDK + cc * 8, lo);
        } else {
          hi = pD;
          unpack8(hi, xd);
        }
        st16(dSsl + r * LDK + cc * 8, hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) sd[e] += xs[e] * xd[e];
      }
      auto put = [&](int p, const u32x4& x) __attribute__((always_inline)) {
        const int kind = p >> 8, q = p & 255;
        st16((kind == 0 ? dOb : kind == 1 ? dXb : Vb) + (q >> 2) * LDO + (q & 3) * 8, x);
      };
      put(tid, pO0);
      if (tid < 3 * C * SL / 8 - kGradThreads) put(tid + kGradThreads, pO1);
    }
    if (sl + 1 < DV / SL) load_slice(sl + 1);
    __syncthreads();
    f32x16 y = zero16();
    if (wave < 2) {   // X = V - Kg S^T -> X^T (hi and lo parts)
      tile_nt_k<DK / 16>(y, Kgb + 32 * wave * LDK, LDK, Ssl, LDK, lane);
      if (s_exact) tile_nt_k<DK / 16>(y, Kgb + 32 * wave * LDK, LDK, Slo, LDK, lane);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = 32 * wave + 8 * g + 4 * hh;
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (float)Vb[(r0 + e) * LDO + col] - y[4 * g + e];
        store4_split(Xt + col * LDT + r0, Xtlo + col * LDT + r0, x[0], x[1], x[2], x[3]);
      }
    } else if (wave < 4) {   // Kc dS^T, rows 32 (wave - 2) ..
      tile_nt_k<DK / 16>(y, Kcb + 32 * (wave - 2) * LDK, LDK, dSsl, LDK, lane);
      if (ds_exact) tile_nt_k<DK / 16>(y, Kcb + 32 * (wave - 2) * LDK, LDK, dSlo, LDK, lane);
    }
    __syncthreads();
    if (wave < 2) {   // U = T X -> U^T
      f32x16 u = zero16();
      tile_nt_k<C / 16>(u, Tb + 32 * wave * LDT, LDT, Xt, LDT, lane);
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(Ut + col * LDT + 32 * wave + 8 * g + 4 * hh, u[4 * g], u[4 * g + 1], u[4 * g + 2], u[4 * g + 3]);
    } else if (wave < 4) {   // dU = Kc dS^T + P^T dO -> dU^T
      const int s0 = 32 * (wave - 2);
#pragma unroll
      for (int t = 0; t < C / 16; ++t)
        mma_bf16(y, frag_perm_tr(Pb, LDT, 16 * t, s0, lane), frag_perm_tr(dOb, LDO, 16 * t, 0, lane));
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4_split(dUt + col * LDT + s0 + 8 * g + 4 * hh, dUtlo + col * LDT + s0 + 8 * g + 4 * hh, y[4 * g],
                     y[4 * g + 1], y[4 * g + 2], y[4 * g + 3]);
    }
    __syncthreads();
    if (wave < 4) {   // dT += dU X^T, hi * hi + hi * lo + lo * hi
#pragma unroll
      for (int t = 0; t < SL / 16; ++t) {
        const bf16x8 uh = frag_perm_tr(dUt, LDT, 16 * t, 32 * rr, lane);
        const bf16x8 xh = frag_perm_tr(Xt, LDT, 16 * t, 32 * sc, lane);
        mma_bf16(cc_acc, uh, xh);
        mma_bf16(cc_acc, uh, frag_perm_tr(Xtlo, LDT, 16 * t, 32 * sc, lane));
        mma_bf16(cc_acc, frag_perm_tr(dUtlo, LDT, 16 * t, 32 * rr, lane), xh);
      }
    } else if (rr >= sc) {   // dP += dO U^T (the tile above the diagonal stays zero)
#pragma unroll
      for (int t = 0; t < SL / 16; ++t)
        mma_bf16(cc_acc, frag_perm(dOb + (32 * rr + col) * LDO, 16 * t, hh), frag_perm_tr(Ut, LDT, 16 * t, 32 * sc, lane));
    }
    if (wave < NT) {   // dO S, dX S, U dS
#pragma unroll
      for (int t = 0; t < SL / 16; ++t) {
        const bf16x8 bs = frag_perm_tr(Ssl, LDK, 16 * t, 32 * jt, lane);
        mma_bf16(dQi, frag_perm(dOb + (32 * rt + col) * LDO, 16 * t, hh), bs);
        mma_bf16(P1, frag_perm(dXb + (32 * rt + col) * LDO, 16 * t, hh), bs);
        mma_bf16(P2, frag_perm_tr(Ut, LDT, 16 * t, 32 * rt, lane), frag_perm_tr(dSsl, LDK, 16 * t, 32 * jt, lane));
      }
    }
    __syncthreads();
  }

  // ---- outputs of the value axis; C x C algebra ----
  if (wave < 4) {   // dT -> dT^T
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4(dTt + (32 * sc + col) * LDT + 32 * rr + 8 * g + 4 * hh, cc_acc[4 * g], cc_acc[4 * g + 1],
             cc_acc[4 * g + 2], cc_acc[4 * g + 3]);
  } else {   // dP (tril_0) -> workspace
    const int s = 32 * sc + col;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 32 * rr + acc_row(v >> 2, v & 3, lane);
      go[GO::dp + r * C + s] = rr >= sc && r >= s ? cc_acc[v] : 0.f;
    }
  }
  if (wave < NT) {   // dO S, dX S, U dS -> workspace
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 32 * rt + acc_row(v >> 2, v & 3, lane), c = 32 * jt + col;
      go[GO::dqs + r * DK + c] = dQi[v];
      go[GO::dxs + r * DK + c] = P1[v];
      go[GO::uds + r * DK + c] = P2[v];
    }
  }
  if (tid < SL * CPR) {   // sum_i dS[i] (.) S[i]: over the rows of the wave, then of the waves
#pragma unroll
    for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
      for (int e = 0; e < 8; ++e) sd[e] += __shfl_xor(sd[e], off);
    if (lane < CPR) {
#pragma unroll
      for (int e = 0; e < 8; ++e) d1p[wave * DK + lane * 8 + e] = sd[e];
    }
  }
  __syncthreads();
  if (wave < 4) {   // N1 = M^T dT; dbeta += diag(N1); N1 -> N1^T
    f32x16 n1 = zero16();
#pragma unroll
    for (int t = 0; t < C / 16; ++t)
      mma_bf16(n1, frag_perm_tr(Mb, LDT, 16 * t, 32 * rr, lane), frag_perm(dTt + (32 * sc + col) * LDT, 16 * t, hh));
    if (rr == sc) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (acc_row(v >> 2, v & 3, lane) == col) dBp[wave * C + 32 * rr + col] += n1[v];
    }
#pragma unroll
    for (int g = 0; g < 4; ++g)
      store4(N1t + (32 * sc + col) * LDT + 32 * rr + 8 * g + 4 * hh, n1[4 * g], n1[4 * g + 1], n1[4 * g + 2],
             n1[4 * g + 3]);
  }
  if (tid < DK) {
    float x = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      if (w * 64 < SL * CPR) x += d1p[w * DK + tid];
    go[GO::d1 + tid] = x;
  }
  __syncthreads();
  if (wave < 4) {   // dA = -tril_-1(N1 T^T); dbeta += rows(dA o At); W = diag(beta) dA -> workspace
    const int s = 32 * sc + col;
    if (rr < sc) {
#pragma unroll
      for (int v = 0; v < 16; ++v) go[GO::w + (32 * rr + acc_row(v >> 2, v & 3, lane)) * C + s] = 0.f;
    } else {
      f32x16 da = zero16();
#pragma unroll
      for (int t = 0; t < C / 16; ++t)
        mma_bf16(da, frag_perm_tr(N1t, LDT, 16 * t, 32 * rr, lane), frag_perm(Tb + (32 * sc + col) * LDT, 16 * t, hh));
      f32x16 bz;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = 32 * rr + acc_row(v >> 2, v & 3, lane);
        const float d = r > s ? -da[v] : 0.f;
        bz[v] = d * (float)EK[r * LDT + s];
        go[GO::w + r * C + s] = Bt[r] * d;
      }
      tile_row_col_sums<false>(bz, dBp + wave * C, 32 * rr, nullptr, 0, lane);
    }
  }
  __syncthreads();
  if (tid < cn) a.dbeta[tok(tid)] = dBp[tid] + dBp[C + tid] + dBp[2 * C + tid] + dBp[3 * C + tid];
}

// bk_chan: one 1024-thread workgroup per chunk of every head.  A wave takes
// the BR = 4 rows of one row block (NQ = 16 blocks) and 64 channels; with
// d_k = 128 the workgroup runs over the two halves of the channels in turn
// (more rows or channels per thread need more than the 128 registers a
// thread has here).  Off the diagonal blocks, exp(G_r - G_s) factors through
// an anchor row m with s <= m <= r: exp(G_r - G_m) exp(G_m - G_s), both at
// most 1, so the sums over the other blocks are plain multiply-adds of
// prescaled operands; inside the block every weight is formed directly.  Row
// block q takes its rows' sums over the earlier columns (R_Pq, R_Ar) and its
// columns' sums over the later rows (R_Pk + R_Ac): 64 - BR partners per
// thread in every block.
constexpr int kChanThreads = 1024;
constexpr int kChanBR = 4;
constexpr int kChanNQ = C / kChanBR;
static_assert(kChanNQ * 64 == kChanThreads, "a wave per row block");

template <int DK>
struct KChanLds {
  static constexpr int LDK = DK + 8;
  static constexpr int LDG = DK + 4;
  static constexpr int LDC = C + 4;
  static constexpr size_t kb = 0;                                 // K rows bf16 [C][LDK]
  static constexpr size_t qb = kb + (size_t)C * LDK * 2;          // Q rows bf16 [C][LDK]
  static constexpr size_t gb = qb + (size_t)C * LDK * 2;          // G fp32 [C][LDG]
  static constexpr size_t dpr = gb + (size_t)C * LDG * 4;         // dP [r][s] fp32 [C][LDC]
  static constexpr size_t dpt = dpr + (size_t)C * LDC * 4;        // dP^T [s][r]
  static constexpr size_t wr = dpt + (size_t)C * LDC * 4;         // W [r][s]
  static constexpr size_t wt = wr + (size_t)C * LDC * 4;          // W^T [s][r]
  static constexpr size_t tot = wt + (size_t)C * LDC * 4;         // block totals [NQ][64]
  static constexpr size_t total = tot + (size_t)kChanNQ * 64 * 4;
};

template <int DK>
__global__ __launch_bounds__(kChanThreads, 1) void bk_chan(BackwardArgs a, const bf* __restrict__ recs,
                                                           const float* __restrict__ gout) {
  using L = KChanLds<DK>;
  using GO = KGradOut<DK>;
  constexpr int NQ = kChanNQ, BR = kChanBR, LDK = L::LDK, LDG = L::LDG, LDC = L::LDC, CPR = DK / 8;
  static_assert(L::total <= 160 * 1024, "LDS plan exceeds 160 KiB");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  bf* Kb = reinterpret_cast<bf*>(smem + L::kb);
  bf* Qb = reinterpret_cast<bf*>(smem + L::qb);
  float* Gs = reinterpret_cast<float*>(smem + L::gb);
  float* dPr = reinterpret_cast<float*>(smem + L::dpr);
  float* dPt = reinterpret_cast<float*>(smem + L::dpt);
  float* Wr = reinterpret_cast<float*>(smem + L::wr);
  float* Wt = reinterpret_cast<float*>(smem + L::wt);
  float* Tot = reinterpret_cast<float*>(smem + L::tot);

  const int tid = threadIdx.x;
  const int T = a.T, H = a.H, NC = (T + C - 1) / C;
  const int nheads = a.B * H;
  const int head = blockIdx.x % nheads, n = blockIdx.x / nheads;
  const int b = head / H, h = head % H, t0 = n * C, cn = min(C, T - t0);
  const size_t chunk = (size_t)head * NC + n;
  const float* gi = gout + chunk * GO::floats;
  auto tok = [&](int r) { return ((size_t)b * T + t0 + r) * H + h; };
  const int q = __builtin_amdgcn_readfirstlane(tid >> 6), cl = tid & 63, r0 = q * BR;
  const bf* ag = static_cast<const bf*>(a.alpha);
  bf* __restrict__ dqg = static_cast<bf*>(a.dq);
  bf* __restrict__ dkg = static_cast<bf*>(a.dk);
  float* __restrict__ dag = a.dalpha;
  constexpr float L2E = 1.4426950408889634f;

  // ---- stage K, Q rows; dP and W in both orientations ----
  {
    const bf* kg = static_cast<const bf*>(a.k);
    const bf* qg = static_cast<const bf*>(a.q);
    for (int p = tid; p < C * CPR; p += kChanThreads) {
      const int r = p / CPR, cc = p % CPR;
      const bool ok = r < cn;
      st16(Kb + r * LDK + cc * 8, ok ? ld16(kg + tok(r) * DK + cc * 8) : zero_u4());
      st16(Qb + r * LDK + cc * 8, ok ? ld16(qg + tok(r) * DK + cc * 8) : zero_u4());
    }
    for (int p = tid; p < C * C / 4; p += kChanThreads) {
      const int r = p / (C / 4), s0 = 4 * (p % (C / 4));
      const float4 d = reinterpret_cast<const float4*>(gi + GO::dp)[p];
      const float4 w = reinterpret_cast<const float4*>(gi + GO::w)[p];
      *reinterpret_cast<float4*>(dPr + r * LDC + s0) = d;
      *reinterpret_cast<float4*>(Wr + r * LDC + s0) = w;
      dPt[(s0 + 0) * LDC + r] = d.x; dPt[(s0 + 1) * LDC + r] = d.y;
      dPt[(s0 + 2) * LDC + r] = d.z; dPt[(s0 + 3) * LDC + r] = d.w;
      Wt[(s0 + 0) * LDC + r] = w.x; Wt[(s0 + 1) * LDC + r] = w.y;
      Wt[(s0 + 2) * LDC + r] = w.z; Wt[(s0 + 3) * LDC + r] = w.w;
    }
  }

  for (int half = 0; half < DK / 64; ++half) {
    const int c = 64 * half + cl;
    // running sum of log alpha over this thread's rows, then the earlier blocks' totals
    float gl[BR];
#pragma unroll
    for (int i = 0; i < BR; ++i) gl[i] = (float)ag[tok(min(r0 + i, cn - 1)) * DK + c];
    {
      float run = 0.f;
#pragma unroll
      for (int i = 0; i < BR; ++i) {
        run += r0 + i < cn ? fmaxf(__logf(gl[i]), kLogFloor) : 0.f;
        gl[i] = run;
      }
      Tot[q * 64 + cl] = run;
    }
    __syncthreads();   // (also: the staging above, and the previous half's reads of Tot)
    {
      float off = 0.f;
      for (int j = 0; j < q; ++j) off += Tot[j * 64 + cl];
#pragma unroll
      for (int i = 0; i < BR; ++i) {
        gl[i] += off;
        Gs[(r0 + i) * LDG + c] = gl[i];
      }
    }
    __syncthreads();

    // ---- the channel-weighted sums for this thread's rows ----
    // (the column sums enter dk and dG only as R_Pk + R_Ac: one accumulator)
    float rpq[BR], rar[BR], rcol[BR];
#pragma unroll
    for (int i = 0; i < BR; ++i) rpq[i] = rar[i] = rcol[i] = 0.f;
    // rows r of the block against the columns s < r0 (anchor m = r0 - 1)
    if (q > 0) {
      const float gm = Gs[(r0 - 1) * LDG + c];
#pragma unroll 4
      for (int s = 0; s < r0; ++s) {
        const float ks = (float)Kb[s * LDK + c] * exp2f((gm - Gs[s * LDG + c]) * L2E);
        const float4 d4 = *reinterpret_cast<const float4*>(dPt + s * LDC + r0);
        const float4 w4 = *reinterpret_cast<const float4*>(Wt + s * LDC + r0);
        rpq[0] += d4.x * ks; rpq[1] += d4.y * ks; rpq[2] += d4.z * ks; rpq[3] += d4.w * ks;
        rar[0] += w4.x * ks; rar[1] += w4.y * ks; rar[2] += w4.z * ks; rar[3] += w4.w * ks;
      }
#pragma unroll
      for (int i = 0; i < BR; ++i) {
        const float f = exp2f((gl[i] - gm) * L2E);
        rpq[i] *= f;
        rar[i] *= f;
      }
    }
    // columns s of the block against the rows r > r0 + BR - 1 (anchor m = r0 + BR - 1)
    if (q < NQ - 1) {
      const float gm = gl[BR - 1];
#pragma unroll 4
      for (int r = r0 + BR; r < C; ++r) {
        const float f = exp2f((Gs[r * LDG + c] - gm) * L2E);
        const float qr = (float)Qb[r * LDK + c] * f, kr = (float)Kb[r * LDK + c] * f;
        const float4 d4 = *reinterpret_cast<const float4*>(dPr + r * LDC + r0);
        const float4 w4 = *reinterpret_cast<const float4*>(Wr + r * LDC + r0);
        rcol[0] += d4.x * qr + w4.x * kr;
        rcol[1] += d4.y * qr + w4.y * kr;
        rcol[2] += d4.z * qr + w4.z * kr;
        rcol[3] += d4.w * qr + w4.w * kr;
      }
#pragma unroll
      for (int i = 0; i < BR; ++i) rcol[i] *= exp2f((gm - gl[i]) * L2E);
    }
    // inside the block (s <= r): one weight per pair serves the row's sums and the column's
    float kv[BR], qv[BR];
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      kv[i] = (float)Kb[(r0 + i) * LDK + c];
      qv[i] = (float)Qb[(r0 + i) * LDK + c];
    }
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      const float4 d4 = *reinterpret_cast<const float4*>(dPr + (r0 + i) * LDC + r0);
      const float4 w4 = *reinterpret_cast<const float4*>(Wr + (r0 + i) * LDC + r0);
      const float dp[4] = {d4.x, d4.y, d4.z, d4.w}, w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
      for (int j = 0; j <= i; ++j) {
        const float e = exp2f((gl[i] - gl[j]) * L2E);
        const float de = dp[j] * e, we = w[j] * e;
        rpq[i] += de * kv[j];
        rar[i] += we * kv[j];
        rcol[j] += de * qv[i] + we * kv[i];
      }
    }

    // ---- dq, dk, dG; the last row's terms; suffix sums -> dalpha ----
    const float gC = Gs[(C - 1) * LDG + c];
    float dg[BR], gcp = 0.f;
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      const int r = r0 + i;
      const float gam = exp2f(gl[i] * L2E), gcr = exp2f((gC - gl[i]) * L2E);
      const float tq = gam * gi[GO::dqs + r * DK + c];
      const float tx = gam * gi[GO::dxs + r * DK + c];
      const float tu = gcr * gi[GO::uds + r * DK + c];
      const float dq = rpq[i] + tq;
      const float dk = rcol[i] + rar[i] - tx + tu;
      dg[i] = qv[i] * dq - kv[i] * (rcol[i] - rar[i] + tx + tu);
      gcp += kv[i] * tu;
      if (r < cn) {
        dqg[tok(r) * DK + c] = (bf)dq;
        dkg[tok(r) * DK + c] = (bf)dk;
      }
    }
    __syncthreads();   // Tot is free again
    Tot[q * 64 + cl] = gcp;
    __syncthreads();
    if (q == NQ - 1) {   // dG of the last row: gamma_C (.) <dS, S> + sum_r k_r (.) exp(G_C - G_r) (U dS)_r
      float x = exp2f(gC * L2E) * gi[GO::d1 + c];
      for (int j = 0; j < NQ; ++j) x += Tot[j * 64 + cl];
      dg[BR - 1] += x;
    }
    // suffix sums: inside the block, then the later blocks' totals
#pragma unroll
    for (int i = BR - 2; i >= 0; --i) dg[i] += dg[i + 1];
    __syncthreads();
    Tot[q * 64 + cl] = dg[0];
    __syncthreads();
    float later = 0.f;
    for (int j = q + 1; j < NQ; ++j) later += Tot[j * 64 + cl];
#pragma unroll
    for (int i = 0; i < BR; ++i) {
      const int r = r0 + i;
      const float al = (float)ag[tok(min(r, cn - 1)) * DK + c];
      if (r < cn) dag[tok(r) * DK + c] = __logf(al) < kLogFloor ? 0.f : (dg[i] + later) / al;
    }
    __syncthreads();   // (Tot before the next half)
  }
}

struct ChunkWs {
  size_t recs, atil, ss, dss, gout, total;
};

// Workspace: the chunk records, (per channel) At, the bf16 entry states and
// end gradients of every chunk, (per channel) bk_gradv's outputs.
ChunkWs chunk_ws(int B, int T, int H, int dk, int dv, bool kda) {
  const size_t nch = (size_t)B * H * (((size_t)T + C - 1) / C);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t rec = kda ? (dk == 128 ? KRec<128>::elems : KRec<64>::elems) : kRecElems;
  const size_t gfl = kda ? (dk == 128 ? KGradOut<128>::floats : KGradOut<64>::floats) : 0;
  ChunkWs w;
  w.recs = 0;
  w.atil = up(nch * rec * 2);
  w.ss = w.atil + (kda ? up(nch * C * C * 4) : 0);
  w.dss = w.ss + up(nch * (size_t)dv * dk * 2);
  w.gout = w.dss + up(nch * (size_t)dv * dk * 2);
  w.total = w.gout + up(nch * gfl * 4);
  return w;
}

template <int DK, int DV>
hipError_t launch_chunk(const BackwardArgs& a, void* ws, hipStream_t stream) {
  const bool kda = a.mode == 2;
  const ChunkWs w = chunk_ws(a.B, a.T, a.H, DK, DV, kda);
  unsigned char* base = static_cast<unsigned char*>(ws);
  const bf* recs = reinterpret_cast<const bf*>(base + w.recs);
  float* atil = reinterpret_cast<float*>(base + w.atil);
  bf* ss = reinterpret_cast<bf*>(base + w.ss);
  bf* dss = reinterpret_cast<bf*>(base + w.dss);
  float* gout = reinterpret_cast<float*>(base + w.gout);
  PrefillArgs p{a.q, a.k, a.v, a.alpha, a.beta, a.S0, nullptr, nullptr, a.B, a.T, a.H, DK, DV, 1, a.mode};
  if (kda) p.a_tilde = atil;
  hipError_t e = launch_prefill_prep(p, base + w.recs, stream);
  if (e != hipSuccess) return e;
  const int NC = (a.T + C - 1) / C;
  const dim3 chain((unsigned)((size_t)a.B * a.H * (DV / SL))), cblock(kChainThreads);
  const dim3 grid((unsigned)((size_t)a.B * a.H * NC)), gblock(kGradThreads);
  if (kda) {
    hipLaunchKernelGGL((bc_states<DK, true>), chain, cblock, 0, stream, a, recs, ss);
    hipLaunchKernelGGL((bc_rev<DK, true>), chain, cblock, 0, stream, a, recs, dss);
    hipLaunchKernelGGL((bk_gradv<DK, DV>), grid, gblock, 0, stream, a, recs, atil, ss, dss, gout);
    hipLaunchKernelGGL((bk_chan<DK>), grid, dim3(kChanThreads), 0, stream, a, recs, gout);
  } else {
    hipLaunchKernelGGL((bc_states<DK, false>), chain, cblock, 0, stream, a, recs, ss);
    hipLaunchKernelGGL((bc_rev<DK, false>), chain, cblock, 0, stream, a, recs, dss);
    hipLaunchKernelGGL((bc_grad<DK, DV>), grid, gblock, 0, stream, a, recs, ss, dss);
  }
  return hipGetLastError();
}

}  // namespace

bool chunk_backward_applies(int T, int dk, int dv, int dtype, int mode) {
  if (dtype != 1 || T <= 0 || (dk != 64 && dk != 128) || (dv != 64 && dv != 128)) return false;
  if (mode == 2)
    return prefill_record_bytes(dk, 1, mode) == (dk == 128 ? KRec<128>::elems : KRec<64>::elems) * 2;
  return (mode == 0 || mode == 1) && prefill_record_bytes(dk, 1, mode) == kRecElems * 2;
}

size_t chunk_backward_workspace_bytes(int B, int T, int H, int dk, int dv, int mode) {
  return chunk_ws(B, T, H, dk, dv, mode == 2).total;
}

hipError_t launch_chunk_backward(const BackwardArgs& a, void* workspace, hipStream_t stream) {
  if (a.dk_ == 128) return a.dv_ == 128 ? launch_chunk<128, 128>(a, workspace, stream)
                                        : launch_chunk<128, 64>(a, workspace, stream);
  return a.dv_ == 128 ? launch_chunk<64, 128>(a, workspace, stream) : launch_chunk<64, 64>(a, workspace, stream);
}

}  // namespace gdn
