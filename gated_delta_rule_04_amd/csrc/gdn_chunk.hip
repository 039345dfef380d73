// Chunked prefill of the gated delta rule (DeltaNet and Gated DeltaNet decay).
//
// The token recurrence ("Linear Attention Architectures" notes, sections 2.3-2.4,
// Eqs. 9-10 and 15-17; state d_v x d_k as in the "On State Reduction" notes,
// section 2.1) is rewritten per chunk of C = 64 tokens.  With G_r the running sum
// of log alpha inside the chunk (gamma_r = exp(G_r)), entry state S_n and the
// chunk's row-stacked K, Q, V:
//
//   A[r][j] = beta_r exp(G_r - G_j) (k_r . k_j)      j < r     decay-weighted beta K K^T
//   T       = (I + A)^-1 diag(beta)                            unit-lower-triangular solve
//   X       = V - diag(gamma) K S_n^T                          write error before the chunk
//   U       = T X                                              pseudo-values u_r
//   P[r][j] = exp(G_r - G_j) (q_r . k_j)             j <= r    masked intra-chunk attention
//   O       = diag(gamma) Q S_n^T + P U                        inter-chunk + intra-chunk
//   S_{n+1} = gamma_C S_n + sum_r exp(G_C - G_r) u_r k_r^T     carried state
//
// (Unrolling the recurrence inside a chunk gives S_r = gamma_r S_n + sum_{j<=r}
// (gamma_r / gamma_j) u_j k_j^T; putting it into u_r = beta_r (v_r - S_{r-1}
// alpha_r k_r) gives (I + A) U = diag(beta) X.  The pseudo-value name u_t is the
// state-reduction notes' (section 2.2); the NextTransformer page names the
// triangular inverse of its chunked kernel in its numerics section.)
//
// One workgroup of 256 threads (four waves) owns one (b, h, d_v slice) and walks
// the chunks of its head in order; value rows are independent ("On State
// Reduction" notes, section 2.5), so slices of d_v never talk to each other.
// The fp32 state slice lives in MFMA accumulator registers for the whole
// sequence; a copy in the operand dtype is kept in LDS for the next chunk's
// K S^T and Q S^T.  Every product is a 32x32 MFMA tile fed from LDS; all
// intermediates (A, T, X, U, P) stay in LDS, so HBM sees q, k, v and beta/alpha
// once, o once, and S0 / S_final once per head.
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int C = 64;            // chunk length
constexpr int kThreads = 256;    // four waves
constexpr float kLogFloor = -100.f;  // gates below e^-100 act as e^-100 (= 0 in fp32 products)

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// LDS plan (byte offsets).  Lifetimes inside one chunk step:
//   Kr    K rows [64][LDK]              load .. phase 3b
//   Qr    Q rows [64][LDK]              load .. phase 3     } same region
//   Kt    K^T    [DK][LDT]              phase 3b .. 6       }
//   Sb    state copy S[i][c] [DVS][LDS] phase 6 .. next phase 3
//   Vt    V^T slice [DVS][LDT]          load .. phase 3
//   Pm    P [64][LDT]                   phase 1 .. 5
//   Tm    T [64][LDT]                   phase 2 .. 4 (fp32 mode: also the solve's L^-1)
//   Am    A fp32 [64][LDA]              phase 1 .. 2        } same region
//   Li    L^-1 fp32 [64][LDA] (bf16)    phase 2             }
//   Mt    3 x 16 x 16 fp32              phase 2             }
//   Xt, Ut, Uw  [DVS][LDT] each         phase 3 .. 6        }
//   G, Bt 64 fp32 each                  load .. 6
template <typename E, int DK, int DVS>
struct Plan {
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = DK + PAD;
  static constexpr int LDT = C + PAD;
  static constexpr int LDSB = DK + PAD;
  static constexpr int LDA = C + 4;
  static constexpr bool kF32 = sizeof(E) == 4;
  static constexpr size_t kr = 0;
  static constexpr size_t qr = kr + (size_t)C * LDK * sizeof(E);
  static constexpr size_t sb = qr + cmax((size_t)C * LDK, (size_t)DK * LDT) * sizeof(E);
  static constexpr size_t vt = sb + (size_t)DVS * LDSB * sizeof(E);
  static constexpr size_t pm = vt + (size_t)DVS * LDT * sizeof(E);
  static constexpr size_t tm = pm + (size_t)C * LDT * sizeof(E);
  static constexpr size_t region = tm + (size_t)C * LDT * sizeof(E);
  static constexpr size_t am = region;
  static constexpr size_t li = am + (size_t)C * LDA * 4;
  static constexpr size_t mt = kF32 ? li : li + (size_t)C * LDA * 4;
  static constexpr size_t solve_end = mt + 3 * 256 * 4;
  static constexpr size_t xu_end = region + 3 * (size_t)DVS * LDT * sizeof(E);
  static constexpr size_t g = cmax(solve_end, xu_end);
  static constexpr size_t total = g + 2 * C * 4;
  static_assert(!kF32 || LDT == LDA, "fp32 mode keeps L^-1 in the T buffer");
  static_assert(total <= 160 * 1024, "LDS plan exceeds 160 KiB");
};

template <typename E, int DK, int DVS, int MODE>
__global__ __launch_bounds__(kThreads) void chunk_kernel(PrefillArgs a) {
  using L = Plan<E, DK, DVS>;
  constexpr int NI = DVS / 32;       // 32-wide value blocks in the slice
  constexpr int NC = DK / 32;        // 32-wide key blocks
  constexpr int NT = NC * NI;        // state tiles
  constexpr int NST = (NT + 3) / 4;  // state tiles per wave
  constexpr int EPC = 16 / (int)sizeof(E);  // elements per 16-byte chunk
  constexpr int LDK = L::LDK, LDT = L::LDT, LDSB = L::LDSB, LDA = L::LDA;

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  E* Kr = reinterpret_cast<E*>(smem + L::kr);
  E* Qr = reinterpret_cast<E*>(smem + L::qr);
  E* Kt = Qr;
  E* Sb = reinterpret_cast<E*>(smem + L::sb);
  E* Vt = reinterpret_cast<E*>(smem + L::vt);
  E* Pm = reinterpret_cast<E*>(smem + L::pm);
  E* Tm = reinterpret_cast<E*>(smem + L::tm);
  float* Am = reinterpret_cast<float*>(smem + L::am);
  float* Li = L::kF32 ? reinterpret_cast<float*>(smem + L::tm) : reinterpret_cast<float*>(smem + L::li);
  float* Mt = reinterpret_cast<float*>(smem + L::mt);
  E* Xt = reinterpret_cast<E*>(smem + L::region);
  E* Ut = Xt + DVS * LDT;
  E* Uw = Ut + DVS * LDT;
  float* G = reinterpret_cast<float*>(smem + L::g);
  float* Bt = G + C;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31;
  const int H = a.H, T = a.T, dv = a.dv;
  const int nsl = dv / DVS;
  int bid = blockIdx.x;
  const int sl = bid % nsl;
  bid /= nsl;
  const int h = bid % H;
  const int b = bid / H;
  const int i0 = sl * DVS;

  const size_t qk_tok = (size_t)H * DK;   // stride between tokens in q, k
  const size_t v_tok = (size_t)H * dv;    // stride between tokens in v, o
  const E* qg = static_cast<const E*>(a.q) + ((size_t)b * T * H + h) * DK;
  const E* kg = static_cast<const E*>(a.k) + ((size_t)b * T * H + h) * DK;
  const E* vg = static_cast<const E*>(a.v) + ((size_t)b * T * H + h) * dv + i0;
  E* og = static_cast<E*>(a.o) + ((size_t)b * T * H + h) * dv + i0;
  const size_t sbase = ((size_t)b * H + h) * dv + i0;  // first state row of the slice

  // Tile ownership for phases 3-5: (row block rb, value block ib) of X, U, O.
  int own_rb = -1, own_ib = 0, x_rb = -1;
  if (NI == 2) {
    own_rb = wave >> 1;
    own_ib = wave & 1;
    x_rb = own_rb;
  } else {
    if (wave >= 2) own_rb = wave - 2;
    else x_rb = wave;
  }

  // Initial state: S0 or zeros, into registers and the operand copy.
  f32x16 Sacc[NST];
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    Sacc[st] = zero16();
    const int t = wave + 4 * st;
    if (t < NT) {
      const int cb = t / NI, ib = t % NI, i = ib * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = cb * 32 + acc_row(g, 0, lane);
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (a.S0) x = *reinterpret_cast<const float4*>(a.S0 + (sbase + i) * DK + c0);
        Sacc[st][4 * g + 0] = x.x;
        Sacc[st][4 * g + 1] = x.y;
        Sacc[st][4 * g + 2] = x.z;
        Sacc[st][4 * g + 3] = x.w;
        store4(Sb + i * LDSB + c0, x.x, x.y, x.z, x.w);
      }
    }
  }

  const int nchunks = (T + C - 1) / C;
  for (int n = 0; n < nchunks; ++n) {
    const int t0 = n * C;
    const int cn = min(C, T - t0);
    __syncthreads();

    // ---- phase 0: gates (log-decay prefix G, beta) and the K, Q, V tiles ----
    if (wave == 0) {
      const int r = lane;
      const bool ok = r < cn;
      const size_t tok = ((size_t)b * T + t0 + r) * H + h;
      const float bt = ok ? a.beta[tok] : 0.f;
      float la = 0.f;
      if (MODE == 1 && ok) la = fmaxf(logf(static_cast<const float*>(a.alpha)[tok]), kLogFloor);
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(la, off);
        if (lane >= off) la += y;
      }
      G[r] = la;
      Bt[r] = bt;
    }
    {
      constexpr int CPR = DK / EPC;  // 16-byte chunks per row
#pragma unroll
      for (int m = 0; m < C * CPR / kThreads; ++m) {
        const int qi = tid + kThreads * m, r = qi / CPR, cc = qi % CPR;
        uint4 kx = make_uint4(0, 0, 0, 0), qx = make_uint4(0, 0, 0, 0);
        if (r < cn) {
          kx = *reinterpret_cast<const uint4*>(kg + (size_t)(t0 + r) * qk_tok + cc * EPC);
          qx = *reinterpret_cast<const uint4*>(qg + (size_t)(t0 + r) * qk_tok + cc * EPC);
        }
        *reinterpret_cast<uint4*>(Kr + r * LDK + cc * EPC) = kx;
        *reinterpret_cast<uint4*>(Qr + r * LDK + cc * EPC) = qx;
      }
      constexpr int CPV = DVS / EPC;
      for (int qi = tid; qi < C * CPV; qi += kThreads) {
        const int r = qi / CPV, cc = qi % CPV;
        union { uint4 raw; E e[EPC]; } tmp;
        tmp.raw = make_uint4(0, 0, 0, 0);
        if (r < cn) tmp.raw = *reinterpret_cast<const uint4*>(vg + (size_t)(t0 + r) * v_tok + cc * EPC);
#pragma unroll
        for (int e = 0; e < EPC; ++e) Vt[(cc * EPC + e) * LDT + r] = tmp.e[e];
      }
    }
    __syncthreads();

    // ---- phase 1: A (fp32) and P from K K^T and K Q^T tiles ----
    // Tile (jb, rb) holds rows j of the j-block and columns r of the r-block, so
    // each lane writes four consecutive j of one row r.
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int tt = wave + 4 * rep;
      if (tt < 6) {
        const bool isA = tt < 3;
        const int idx = tt % 3;
        const int jb = idx == 2 ? 1 : 0, rb = idx == 0 ? 0 : 1;
        f32x16 acc = zero16();
        tile_nt(acc, Kr + jb * 32 * LDK, LDK, (isA ? Kr : Qr) + rb * 32 * LDK, LDK, DK / 16, lane);
        const int r = rb * 32 + col;
        const float Gr = G[r];
        if (isA) {
          const float br = Bt[r];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int j0 = jb * 32 + acc_row(g, 0, lane);
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[e] = (j0 + e < r) ? br * __expf(Gr - G[j0 + e]) * acc[4 * g + e] : 0.f;
            store4(Am + r * LDA + j0, x[0], x[1], x[2], x[3]);
          }
        } else {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int j0 = jb * 32 + acc_row(g, 0, lane);
            float x[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              x[e] = (j0 + e <= r) ? __expf(Gr - G[j0 + e]) * acc[4 * g + e] : 0.f;
            store4(Pm + r * LDT + j0, x[0], x[1], x[2], x[3]);
          }
        }
      }
    }
    __syncthreads();

    // ---- phase 2: T = (I + A)^-1 diag(beta), blocked by 16 ----
    // (a) inverse of each unit-lower 16x16 diagonal block, one column per thread
    if (tid < 64) {
      const int I = tid >> 4, c = tid & 15;
      const float* base = Am + (16 * I) * LDA + 16 * I;
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < i; ++j) s += base[i * LDA + j] * y[j];
        y[i] = i < c ? 0.f : (i == c ? 1.f : -s);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) Li[(16 * I + i) * LDA + 16 * I + c] = y[i];
    }
    __syncthreads();
    // (b) off-diagonal blocks by distance d: L^-1_IJ = -L^-1_II sum_{K=J}^{I-1} A_IK L^-1_KJ
    {
      const int i = tid >> 4, j = tid & 15;
      for (int d = 1; d < 4; ++d) {
        for (int bk = 0; bk < 4 - d; ++bk) {
          const int I = bk + d, J = bk;
          float s = 0.f;
          for (int K = J; K < I; ++K) {
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
              s += Am[(16 * I + i) * LDA + 16 * K + kk] * Li[(16 * K + kk) * LDA + 16 * J + j];
          }
          Mt[bk * 256 + i * 16 + j] = s;
        }
        __syncthreads();
        for (int bk = 0; bk < 4 - d; ++bk) {
          const int I = bk + d, J = bk;
          float s = 0.f;
#pragma unroll
          for (int m = 0; m < 16; ++m) s += Li[(16 * I + i) * LDA + 16 * I + m] * Mt[bk * 256 + m * 16 + j];
          Li[(16 * I + i) * LDA + 16 * J + j] = -s;
        }
        __syncthreads();
      }
    }
    // (c) T[r][j] = L^-1[r][j] beta_j on and below the diagonal, 0 above
    {
      const int r = tid >> 2, jc = (tid & 3) * 16;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = jc + e;
        const float x = j <= r ? Li[r * LDA + j] * Bt[j] : 0.f;
        Tm[r * LDT + j] = to_elem<E>(x);
      }
    }
    // phase 3 writes Xt over the solve's scratch region
    __syncthreads();

    // ---- phase 3: X = V - diag(gamma) K S^T  and  O_inter = diag(gamma) Q S^T ----
    f32x16 oacc = zero16();
    if (x_rb >= 0) {
      const int ib = NI == 2 ? own_ib : 0;
      f32x16 xacc = zero16();
      tile_nt(xacc, Kr + x_rb * 32 * LDK, LDK, Sb + ib * 32 * LDSB, LDSB, DK / 16, lane);
      const int i = ib * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = x_rb * 32 + acc_row(g, 0, lane);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          x[e] = load_elem(Vt + i * LDT + r0 + e) - __expf(G[r0 + e]) * xacc[4 * g + e];
        store4(Xt + i * LDT + r0, x[0], x[1], x[2], x[3]);
      }
    }
    if (own_rb >= 0) {
      tile_nt(oacc, Qr + own_rb * 32 * LDK, LDK, Sb + own_ib * 32 * LDSB, LDSB, DK / 16, lane);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = own_rb * 32 + acc_row(g, 0, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) oacc[4 * g + e] *= __expf(G[r0 + e]);
      }
    }
    __syncthreads();

    // ---- phase 3b: K^T into the Q region (4 rows x one 16-byte chunk per step) ----
    {
      constexpr int CPR = DK / EPC;
      for (int blk = tid; blk < (C / 4) * CPR; blk += kThreads) {
        const int rg = blk / CPR, cc = blk % CPR;
        union Row { uint4 raw; E e[EPC]; } v[4];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          v[m].raw = *reinterpret_cast<const uint4*>(Kr + (4 * rg + m) * LDK + cc * EPC);
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          E* dst = Kt + (cc * EPC + e) * LDT + 4 * rg;
          dst[0] = v[0].e[e];
          dst[1] = v[1].e[e];
          dst[2] = v[2].e[e];
          dst[3] = v[3].e[e];
        }
      }
    }

    // ---- phase 4: U = T X; store U^T and the decay-weighted copy for the state ----
    if (own_rb >= 0) {
      f32x16 uacc = zero16();
      tile_nt(uacc, Tm + own_rb * 32 * LDT, LDT, Xt + own_ib * 32 * LDT, LDT, (own_rb + 1) * 2, lane);
      const int i = own_ib * 32 + col;
      const float GC = G[C - 1];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = own_rb * 32 + acc_row(g, 0, lane);
        store4(Ut + i * LDT + r0, uacc[4 * g], uacc[4 * g + 1], uacc[4 * g + 2], uacc[4 * g + 3]);
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = uacc[4 * g + e] * __expf(GC - G[r0 + e]);
        store4(Uw + i * LDT + r0, w[0], w[1], w[2], w[3]);
      }
    }
    __syncthreads();

    // ---- phase 5: O = O_inter + P U, written to HBM ----
    if (own_rb >= 0) {
      tile_nt(oacc, Pm + own_rb * 32 * LDT, LDT, Ut + own_ib * 32 * LDT, LDT, (own_rb + 1) * 2, lane);
      const int i = own_ib * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = own_rb * 32 + acc_row(g, e, lane);
          if (r < cn) og[(size_t)(t0 + r) * v_tok + i] = to_elem<E>(oacc[4 * g + e]);
        }
      }
    }

    // ---- phase 6: S^T <- gamma_C S^T + K^T Uw  (fp32 accumulators), refresh Sb ----
    {
      const float gC = __expf(G[C - 1]);
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int t = wave + 4 * st;
        if (t < NT) {
          const int cb = t / NI, ib = t % NI;
#pragma unroll
          for (int v = 0; v < 16; ++v) Sacc[st][v] *= gC;
          tile_nt(Sacc[st], Kt + cb * 32 * LDT, LDT, Uw + ib * 32 * LDT, LDT, C / 16, lane);
          const int i = ib * 32 + col;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int c0 = cb * 32 + acc_row(g, 0, lane);
            store4(Sb + i * LDSB + c0, Sacc[st][4 * g], Sacc[st][4 * g + 1], Sacc[st][4 * g + 2],
                   Sacc[st][4 * g + 3]);
          }
        }
      }
    }
  }

  // Final state of the slice.
  if (a.S_final) {
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int t = wave + 4 * st;
      if (t < NT) {
        const int cb = t / NI, ib = t % NI, i = ib * 32 + col;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c0 = cb * 32 + acc_row(g, 0, lane);
          *reinterpret_cast<float4*>(a.S_final + (sbase + i) * DK + c0) =
              make_float4(Sacc[st][4 * g], Sacc[st][4 * g + 1], Sacc[st][4 * g + 2], Sacc[st][4 * g + 3]);
        }
      }
    }
  }
}

template <typename E, int DK, int DVS>
hipError_t launch_slices(const PrefillArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((size_t)a.B * a.H * (a.dv / DVS))), block(kThreads);
  if (a.mode == 0)
    hipLaunchKernelGGL((chunk_kernel<E, DK, DVS, 0>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((chunk_kernel<E, DK, DVS, 1>), grid, block, 0, stream, a);
  return hipGetLastError();
}

// Slice width: 64 value rows per workgroup when that still gives at least one
// workgroup per compute unit (256), else 32.
template <typename E, int DK>
hipError_t launch_dk(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (sizeof(E) == 4 && DK == 128) {
    return launch_slices<E, DK, 32>(a, stream);  // a 64-row fp32 slice does not fit in LDS
  } else {
    const long long wg64 = (long long)a.B * a.H * (a.dv / 64);
    if (wg64 >= 256) return launch_slices<E, DK, 64>(a, stream);
    return launch_slices<E, DK, 32>(a, stream);
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  if (a.mode == 2) return hipErrorNotSupported;
  if (a.dtype == 1) return a.dk == 128 ? launch_dk<__bf16, 128>(a, stream) : launch_dk<__bf16, 64>(a, stream);
  return a.dk == 128 ? launch_dk<float, 128>(a, stream) : launch_dk<float, 64>(a, stream);
}

}  // namespace gdn
