// Chunk-level backward of the gated delta-rule prefill, bf16 operands, no or
// scalar decay.  (fp32 operands and per-channel decay take the token-level
// kernels of gdn_backward.hip.)
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
template <int DK>
struct StatesLds {
  static constexpr int LDK = DK + 8;
  static constexpr size_t kb = 0;                                // K rows [C][LDK]
  static constexpr size_t tb = kb + (size_t)C * LDK * 2;         // T [C][LDT]
  static constexpr size_t sb = tb + (size_t)C * LDT * 2;         // S slice [SL][LDK]
  static constexpr size_t xt = sb + (size_t)SL * LDK * 2;        // X^T [SL][LDT]
  static constexpr size_t ut = xt + (size_t)SL * LDT * 2;        // (diag(exp(G_C - G)) U)^T [SL][LDT]
  static constexpr size_t vb = ut + (size_t)SL * LDT * 2;        // V slice [C][LDO]
  static constexpr size_t gs = vb + (size_t)C * LDO * 2;         // exp(G), exp(G_C - G)
  static constexpr size_t total = gs + 2 * C * 4;
};

template <int DK>
__global__ __launch_bounds__(kChainThreads, 2) void bc_states(BackwardArgs a, const bf* __restrict__ recs,
                                                              bf* __restrict__ ssave) {
  using L = StatesLds<DK>;
  constexpr int LDK = L::LDK, CPR = DK / 8, KPT = C * CPR / kChainThreads;
  static_assert(C * CPR % kChainThreads == 0 && SL * CPR % kChainThreads == 0, "even split");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  bf* Kb = reinterpret_cast<bf*>(smem + L::kb);
  bf* Tb = reinterpret_cast<bf*>(smem + L::tb);
  bf* Sb = reinterpret_cast<bf*>(smem + L::sb);
  bf* Xt = reinterpret_cast<bf*>(smem + L::xt);
  bf* Ut = reinterpret_cast<bf*>(smem + L::ut);
  bf* Vb = reinterpret_cast<bf*>(smem + L::vb);
  float* eG = reinterpret_cast<float*>(smem + L::gs);
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

  u32x4 kreg[KPT], treg[2], vreg;
  float greg = 0.f;
  const int vrow = tid >> 2, vcc = tid & 3;   // this thread's piece of the V slice
  auto load = [&](int n) __attribute__((always_inline)) {
    const int t0 = n * C, cn = min(C, T - t0);
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
      kreg[m] = r < cn ? ld16(kg + (((size_t)b * T + t0 + r) * H + h) * DK + cc * 8) : zero_u4();
    }
    vreg = vrow < cn ? ld16(vg + (((size_t)b * T + t0 + vrow) * H + h) * DV + i0 + vcc * 8) : zero_u4();
    const bf* rec = recs + ((size_t)head * NC + n) * kRecElems;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = tid + kChainThreads * m, r = q >> 3, cc = q & 7;
      treg[m] = ld16(rec + r * C + cc * 8);
    }
    if (tid < 2 * C) greg = reinterpret_cast<const float*>(rec + kRecG)[C + tid];
  };
  auto commit = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
      st16(Kb + r * LDK + cc * 8, kreg[m]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = tid + kChainThreads * m, r = q >> 3, cc = q & 7;
      st16(Tb + r * LDT + cc * 8, treg[m]);
    }
    if (tid < 2 * C) eG[tid] = greg;
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
        for (int e = 0; e < 4; ++e) x[e] = (float)Vb[(r0 + e) * LDO + col] - eG[r0 + e] * y[4 * g + e];
        store4(Xt + col * LDT + r0, x[0], x[1], x[2], x[3]);
      }
    }
    __syncthreads();
    if (wave < 2) {   // U = T X, stored decayed to the chunk end
      f32x16 u = zero16();
      tile_nt_k<C / 16>(u, Tb + 32 * wave * LDT, LDT, Xt, LDT, lane);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = 32 * wave + 8 * g + 4 * hh;
        store4(Ut + col * LDT + r0, eC[r0] * u[4 * g], eC[r0 + 1] * u[4 * g + 1], eC[r0 + 2] * u[4 * g + 2],
               eC[r0 + 3] * u[4 * g + 3]);
      }
    }
    __syncthreads();
    if (wave < DK / 32) {   // S^T <- gamma_C S^T + K^T (decayed U)
      const float gC = eG[C - 1];
#pragma unroll
      for (int v = 0; v < 16; ++v) S[v] *= gC;
#pragma unroll
      for (int s = 0; s < C / 16; ++s)
        mma_bf16(S, frag_perm_tr(Kb, LDK, 16 * s, 32 * wave, lane), frag_perm(Ut + col * LDT, 16 * s, hh));
    }
    __syncthreads();
    if (n + 1 < NC) commit();
  }
}

// ---------------------------------------------------------------------------
// bc_rev: dS backwards over the chunks of one (b, h, value slice); dV, the
// chunk-end dS (bf16) of every chunk, dS0.
// ---------------------------------------------------------------------------
template <int DK>
struct RevLds {
  static constexpr int LDK = DK + 8;
  static constexpr size_t kb = 0;                                // K rows [C][LDK]
  static constexpr size_t qb = kb + (size_t)C * LDK * 2;         // Q rows [C][LDK]
  static constexpr size_t tb = qb + (size_t)C * LDK * 2;         // T [C][LDT]
  static constexpr size_t dob = tb + (size_t)C * LDT * 2;        // dO slice [C][LDO]
  static constexpr size_t dog = dob + (size_t)C * LDO * 2;       // diag(gamma) dO slice [C][LDO]
  static constexpr size_t dsb = dog + (size_t)C * LDO * 2;       // dS slice [SL][LDK]
  static constexpr size_t pt = dsb + (size_t)SL * LDK * 2;       // P^T [C][LDT]; then (-diag(gamma) dX)^T [SL][LDT]
  static constexpr size_t dut = pt + (size_t)C * LDT * 2;        // dU^T [SL][LDT]
  static constexpr size_t gs = dut + (size_t)SL * LDT * 2;       // G, exp(G), exp(G_C - G)
  static constexpr size_t total = gs + 3 * C * 4;
};

template <int DK>
__global__ __launch_bounds__(kChainThreads, 2) void bc_rev(BackwardArgs a, const bf* __restrict__ recs,
                                                           bf* __restrict__ dssave) {
  using L = RevLds<DK>;
  constexpr int LDK = L::LDK, CPR = DK / 8, KPT = C * CPR / kChainThreads;
  static_assert(C * SL / 8 == kChainThreads, "one dO piece per thread");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  bf* Kb = reinterpret_cast<bf*>(smem + L::kb);
  bf* Qb = reinterpret_cast<bf*>(smem + L::qb);
  bf* Tb = reinterpret_cast<bf*>(smem + L::tb);
  bf* dOb = reinterpret_cast<bf*>(smem + L::dob);
  bf* dOg = reinterpret_cast<bf*>(smem + L::dog);
  bf* dSb = reinterpret_cast<bf*>(smem + L::dsb);
  bf* Pt = reinterpret_cast<bf*>(smem + L::pt);
  bf* Xn = Pt;
  bf* dUt = reinterpret_cast<bf*>(smem + L::dut);
  float* Gs = reinterpret_cast<float*>(smem + L::gs);
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

  u32x4 kreg[KPT], qreg[KPT], treg[2], oreg;
  float greg = 0.f, ograte = 0.f;
  const int orow = tid >> 2, occ = tid & 3;   // this thread's piece of the dO slice
  auto load = [&](int n) __attribute__((always_inline)) {
    const int t0 = n * C, cn = min(C, T - t0);
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
      const size_t off = (((size_t)b * T + t0 + r) * H + h) * DK + cc * 8;
      kreg[m] = r < cn ? ld16(kg + off) : zero_u4();
      qreg[m] = r < cn ? ld16(qg + off) : zero_u4();
    }
    const bf* rec = recs + ((size_t)head * NC + n) * kRecElems;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = tid + kChainThreads * m, r = q >> 3, cc = q & 7;
      treg[m] = ld16(rec + r * C + cc * 8);
    }
    const float* rg = reinterpret_cast<const float*>(rec + kRecG);
    if (tid < 3 * C) greg = rg[tid];
    ograte = rg[C + orow];
    oreg = orow < cn ? ld16(dout_g + (((size_t)b * T + t0 + orow) * H + h) * DV + i0 + occ * 8) : zero_u4();
  };
  auto commit = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < KPT; ++m) {
      const int q = tid + kChainThreads * m, r = q / CPR, cc = q % CPR;
      st16(Kb + r * LDK + cc * 8, kreg[m]);
      st16(Qb + r * LDK + cc * 8, qreg[m]);
    }
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      const int q = tid + kChainThreads * m, r = q >> 3, cc = q & 7;
      st16(Tb + r * LDT + cc * 8, treg[m]);
    }
    if (tid < 3 * C) Gs[tid] = greg;
    st16(dOb + orow * LDO + occ * 8, oreg);
    st16(dOg + orow * LDO + occ * 8, scale16(oreg, ograte));
  };

  // P^T is zero where s >= 32 > r; nothing else writes there
  if (wave == 3) {
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
    if (wave < 3) {
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
    if (wave < 2) tile_nt_k<DK / 16>(du, Kb + 32 * wave * LDK, LDK, dSb, LDK, lane);   // K dS^T
    __syncthreads();
    if (wave < 2) {   // dU = diag(exp(G_C - G)) K dS^T + P^T dO, rows s = 32 wave ..
#pragma unroll
      for (int v = 0; v < 16; ++v) du[v] *= eC[32 * wave + acc_row(v >> 2, v & 3, lane)];
#pragma unroll
      for (int t = 0; t < C / 16; ++t)
        mma_bf16(du, frag_perm(Pt + (32 * wave + col) * LDT, 16 * t, hh), frag_perm_tr(dOb, LDO, 16 * t, 0, lane));
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
        store4(Xn + col * LDT + s0, -eG[s0] * dx[4 * g], -eG[s0 + 1] * dx[4 * g + 1], -eG[s0 + 2] * dx[4 * g + 2],
               -eG[s0 + 3] * dx[4 * g + 3]);
      }
    }
    __syncthreads();
    // dV rows -> HBM, one 16-byte piece per thread
    if (orow < cn) st16(dvg + (((size_t)b * T + t0 + orow) * H + h) * DV + i0 + occ * 8, ld16(dOb + orow * LDO + occ * 8));
    if (wave < DK / 32) {   // dS^T <- gamma_C dS^T + Q^T diag(gamma) dO - K^T diag(gamma) dX
      const float gC = eG[C - 1];
#pragma unroll
      for (int v = 0; v < 16; ++v) dS[v] *= gC;
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

struct ChunkWs {
  size_t recs, ss, dss, total;
};

ChunkWs chunk_ws(int B, int T, int H, int dk, int dv) {
  const size_t nch = (size_t)B * H * (((size_t)T + C - 1) / C);
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  ChunkWs w;
  w.recs = 0;
  w.ss = up(nch * kRecElems * 2);
  w.dss = w.ss + up(nch * (size_t)dv * dk * 2);
  w.total = w.dss + up(nch * (size_t)dv * dk * 2);
  return w;
}

template <int DK, int DV>
hipError_t launch_chunk(const BackwardArgs& a, void* ws, hipStream_t stream) {
  const ChunkWs w = chunk_ws(a.B, a.T, a.H, DK, DV);
  unsigned char* base = static_cast<unsigned char*>(ws);
  const bf* recs = reinterpret_cast<const bf*>(base + w.recs);
  bf* ss = reinterpret_cast<bf*>(base + w.ss);
  bf* dss = reinterpret_cast<bf*>(base + w.dss);
  PrefillArgs p{a.q, a.k, a.v, a.alpha, a.beta, a.S0, nullptr, nullptr, a.B, a.T, a.H, DK, DV, 1, a.mode};
  hipError_t e = launch_prefill_prep(p, base + w.recs, stream);
  if (e != hipSuccess) return e;
  const int NC = (a.T + C - 1) / C;
  const dim3 chain((unsigned)((size_t)a.B * a.H * (DV / SL))), cblock(kChainThreads);
  hipLaunchKernelGGL((bc_states<DK>), chain, cblock, 0, stream, a, recs, ss);
  hipLaunchKernelGGL((bc_rev<DK>), chain, cblock, 0, stream, a, recs, dss);
  hipLaunchKernelGGL((bc_grad<DK, DV>), dim3((unsigned)((size_t)a.B * a.H * NC)), dim3(kGradThreads), 0, stream, a,
                     recs, ss, dss);
  return hipGetLastError();
}

}  // namespace

bool chunk_backward_applies(int T, int dk, int dv, int dtype, int mode) {
  return dtype == 1 && (mode == 0 || mode == 1) && T > 0 && (dk == 64 || dk == 128) && (dv == 64 || dv == 128) &&
         prefill_record_bytes(dk, 1, mode) == kRecElems * 2;
}

size_t chunk_backward_workspace_bytes(int B, int T, int H, int dk, int dv) {
  return chunk_ws(B, T, H, dk, dv).total;
}

hipError_t launch_chunk_backward(const BackwardArgs& a, void* workspace, hipStream_t stream) {
  if (a.dk_ == 128) return a.dv_ == 128 ? launch_chunk<128, 128>(a, workspace, stream)
                                        : launch_chunk<128, 64>(a, workspace, stream);
  return a.dv_ == 128 ? launch_chunk<64, 128>(a, workspace, stream) : launch_chunk<64, 64>(a, workspace, stream);
}

}  // namespace gdn
