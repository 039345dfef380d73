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
// K S^T and Q S^T.  Every product is an MFMA tile fed from LDS and all
// intermediates (A, T, X, U, P) stay in LDS, so HBM sees q, k, v and the gates
// once, o once, and S0 / S_final once per head.  The next chunk's q, k, v and
// gates are loaded into registers while the current chunk computes.
//
// Per chunk step:
//   commit   prefetched registers -> LDS (K rows, K^T, Q rows, V^T, gates)
//   phase 1  A and P tiles (bf16/fp32 MFMA), X and diag(gamma) Q S^T tiles
//   solve    T = (I + A)^-1 diag(beta): 16x16 diagonal inverses by forward
//            substitution, then two levels of fp32 MFMA block products
//   phase 4  U = T X
//   phase 5  O = diag(gamma) Q S^T + P U  -> HBM
//   phase 6  S^T <- gamma_C S^T + K^T (diag(exp(G_C - G)) U)
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int C = 64;                // chunk length
constexpr int kThreads = 256;        // four waves
constexpr float kLogFloor = -100.f;  // gates below e^-100 act as e^-100 (= 0 in fp32 products)

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// LDS plan (byte offsets).  Lifetimes inside one chunk step:
//   Kr    K rows [64][LDK]               commit .. phase 1
//   Qr    Q rows [64][LDK]               commit .. phase 1
//   Kt    K^T    [DK][LDT]               commit (or after phase 1) .. phase 6
//         (fp32 with d_k = 128: shares Q's region to fit in 160 KiB)
//   Sb    state copy S[i][c] [DVS][LDSB] phase 6 .. next phase 1
//   Vt    V^T slice [DVS][LDT]           commit .. phase 1
//   Xt    X^T slice [DVS][LDT]           phase 1 .. phase 4
//   Pm    P [64][LDT]                    phase 1 .. phase 5
//   Tm    T [64][LDT]                    solve .. phase 4 (fp32: also the solve's L^-1)
//   Am    A fp32 [64][LDA]               phase 1 .. solve       } one region
//   Li    L^-1 fp32 [64][LDA] (bf16)     solve                  }
//   Mt    fp32 [32][LDM]                 solve                  }
//   Ut, Uw  [DVS][LDT] each              phase 4 .. phase 6     }
//   G, Bt, Eg, Ec  64 fp32 each          commit .. phase 6
template <typename E, int DK, int DVS, bool SEPKT>
struct Plan {
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = DK + PAD;
  static constexpr int LDT = C + PAD;
  static constexpr int LDSB = DK + PAD;
  static constexpr int LDA = C + 4;
  static constexpr int LDM = 32 + 4;
  static constexpr bool kF32 = sizeof(E) == 4;
  static constexpr size_t es = sizeof(E);
  static constexpr size_t kr = 0;
  static constexpr size_t qr = kr + (size_t)C * LDK * es;
  static constexpr size_t kt = SEPKT ? qr + (size_t)C * LDK * es : qr;
  static constexpr size_t sb = SEPKT ? kt + (size_t)DK * LDT * es
                                     : qr + cmax((size_t)C * LDK, (size_t)DK * LDT) * es;
  static constexpr size_t vt = sb + (size_t)DVS * LDSB * es;
  static constexpr size_t xt = vt + (size_t)DVS * LDT * es;
  static constexpr size_t pm = xt + (size_t)DVS * LDT * es;
  static constexpr size_t tm = pm + (size_t)C * LDT * es;
  static constexpr size_t region = tm + (size_t)C * LDT * es;
  static constexpr size_t am = region;
  static constexpr size_t li = am + (size_t)C * LDA * 4;
  static constexpr size_t mt = kF32 ? li : li + (size_t)C * LDA * 4;
  static constexpr size_t solve_end = mt + (size_t)32 * LDM * 4;
  static constexpr size_t ut = region;
  static constexpr size_t uw = ut + (size_t)DVS * LDT * es;
  static constexpr size_t u_end = uw + (size_t)DVS * LDT * es;
  static constexpr size_t g = cmax(solve_end, u_end);
  static constexpr size_t total = g + 4 * C * 4;
  static_assert(!kF32 || LDT == LDA, "fp32 mode keeps L^-1 in the T buffer");
};

template <typename E, int DK, int DVS>
constexpr bool sep_kt_fits() {
  return Plan<E, DK, DVS, true>::total <= 160 * 1024;
}

template <typename E, int DK, int DVS, int MODE>
__global__ __launch_bounds__(kThreads) void chunk_kernel(PrefillArgs a) {
  constexpr bool SEPKT = sep_kt_fits<E, DK, DVS>();
  using L = Plan<E, DK, DVS, SEPKT>;
  static_assert(L::total <= 160 * 1024, "LDS plan exceeds 160 KiB");
  constexpr int NI = DVS / 32;       // 32-wide value blocks in the slice
  constexpr int NC = DK / 32;        // 32-wide key blocks
  constexpr int NT = NC * NI;        // state tiles
  constexpr int NST = (NT + 3) / 4;  // state tiles per wave
  constexpr int EPC = 16 / (int)sizeof(E);  // elements per 16-byte chunk
  constexpr int LDK = L::LDK, LDT = L::LDT, LDSB = L::LDSB, LDA = L::LDA, LDM = L::LDM;
  // prefetch geometry: blocks of 4 rows x one 16-byte chunk, row group fastest
  constexpr int CPR = DK / EPC;              // chunks per q/k row
  constexpr int NKB = 16 * CPR;              // 4-row blocks per q/k tile
  constexpr int KBT = (NKB + kThreads - 1) / kThreads;
  constexpr int CPV = DVS / EPC;             // chunks per v row (slice)
  constexpr int NVB = 16 * CPV;
  constexpr int VBT = (NVB + kThreads - 1) / kThreads;

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  E* Kr = reinterpret_cast<E*>(smem + L::kr);
  E* Qr = reinterpret_cast<E*>(smem + L::qr);
  E* Kt = reinterpret_cast<E*>(smem + L::kt);
  E* Sb = reinterpret_cast<E*>(smem + L::sb);
  E* Vt = reinterpret_cast<E*>(smem + L::vt);
  E* Xt = reinterpret_cast<E*>(smem + L::xt);
  E* Pm = reinterpret_cast<E*>(smem + L::pm);
  E* Tm = reinterpret_cast<E*>(smem + L::tm);
  float* Am = reinterpret_cast<float*>(smem + L::am);
  float* Li = L::kF32 ? reinterpret_cast<float*>(smem + L::tm) : reinterpret_cast<float*>(smem + L::li);
  float* Mt = reinterpret_cast<float*>(smem + L::mt);
  E* Ut = reinterpret_cast<E*>(smem + L::ut);
  E* Uw = reinterpret_cast<E*>(smem + L::uw);
  float* G = reinterpret_cast<float*>(smem + L::g);
  float* Bt = G + C;
  float* Eg = G + 2 * C;   // exp(G_r)
  float* Ec = G + 3 * C;   // exp(G_C - G_r)

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

  // Tile ownership.  X, O_inter (phase 1), U (phase 4) and O (phase 5) tiles of
  // row block own_rb and value block own_ib belong to one wave; the three A/P
  // tile pairs (j block, r block) in {(0,0), (0,1), (1,1)} go to the waves with
  // the least other work.
  int own_rb = -1, own_ib = 0, ap = -1;
  if (NI == 2) {
    own_rb = wave >> 1;
    own_ib = wave & 1;
    ap = wave < 3 ? wave : -1;
  } else {
    if (wave < 2) own_rb = wave;
    ap = wave == 0 ? 2 : (wave >= 2 ? wave - 2 : -1);
  }
  const int ap_jb = ap == 2 ? 1 : 0, ap_rb = ap == 0 ? 0 : 1;

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

  // ---- prefetch registers ----
  // Loads are unconditional (rows past the sequence end re-read its last row and
  // are zeroed at commit) so the compiler keeps them in flight across the chunk.
  uint4 pk[KBT][4], pq[KBT][4], pv[VBT][4];
  float p_beta = 0.f, p_alpha = 1.f;
  int p_cn = 0;

  auto prefetch = [&](int n) __attribute__((always_inline)) {
    const int t0 = n * C;
    const int cn = min(C, T - t0);
    p_cn = cn;
#pragma unroll
    for (int m = 0; m < KBT; ++m) {
      const int blk = tid + kThreads * m;
      const int bq = blk < NKB ? blk : 0;
      const int rg = bq % 16, cc = bq / 16;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = min(4 * rg + rr, cn - 1);
        pk[m][rr] = *reinterpret_cast<const uint4*>(kg + (size_t)(t0 + r) * qk_tok + cc * EPC);
        pq[m][rr] = *reinterpret_cast<const uint4*>(qg + (size_t)(t0 + r) * qk_tok + cc * EPC);
      }
    }
#pragma unroll
    for (int m = 0; m < VBT; ++m) {
      const int blk = tid + kThreads * m;
      const int bq = blk < NVB ? blk : 0;
      const int rg = bq % 16, cc = bq / 16;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int r = min(4 * rg + rr, cn - 1);
        pv[m][rr] = *reinterpret_cast<const uint4*>(vg + (size_t)(t0 + r) * v_tok + cc * EPC);
      }
    }
    const size_t tok = ((size_t)b * T + t0 + min(lane, cn - 1)) * H + h;
    p_beta = a.beta[tok];
    if (MODE == 1) p_alpha = static_cast<const float*>(a.alpha)[tok];
  };

  auto commit = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < KBT; ++m) {
      const int blk = tid + kThreads * m;
      if (blk < NKB) {
        const int rg = blk % 16, cc = blk / 16;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const bool ok = 4 * rg + rr < p_cn;
          pk[m][rr] = keep_or_zero(pk[m][rr], ok);
          *reinterpret_cast<uint4*>(Kr + (4 * rg + rr) * LDK + cc * EPC) = pk[m][rr];
          *reinterpret_cast<uint4*>(Qr + (4 * rg + rr) * LDK + cc * EPC) = keep_or_zero(pq[m][rr], ok);
        }
        if (SEPKT) {
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            store_col4(Kt + (cc * EPC + e) * LDT + 4 * rg, pk[m][0], pk[m][1], pk[m][2], pk[m][3], e);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < VBT; ++m) {
      const int blk = tid + kThreads * m;
      if (blk < NVB) {
        const int rg = blk % 16, cc = blk / 16;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) pv[m][rr] = keep_or_zero(pv[m][rr], 4 * rg + rr < p_cn);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          store_col4(Vt + (cc * EPC + e) * LDT + 4 * rg, pv[m][0], pv[m][1], pv[m][2], pv[m][3], e);
      }
    }
    if (wave == 0) {
      const bool ok = lane < p_cn;
      float la = (MODE == 1 && ok) ? fmaxf(logf(p_alpha), kLogFloor) : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_up(la, off);
        if (lane >= off) la += y;
      }
      const float GC = __shfl(la, 63);
      G[lane] = la;
      Bt[lane] = ok ? p_beta : 0.f;
      Eg[lane] = __expf(la);
      Ec[lane] = __expf(GC - la);
    }
  };

  const int nchunks = (T + C - 1) / C;
  if (nchunks > 0) prefetch(0);
  for (int n = 0; n < nchunks; ++n) {
    const int t0 = n * C;
    const int cn = min(C, T - t0);
    __syncthreads();   // every reader of the previous chunk's buffers is done
    commit();
    if (n + 1 < nchunks) prefetch(n + 1);
    __syncthreads();

    // ---- phase 1: A, P tiles; X and O_inter tiles ----
    // A/P tile pair (jb, rb) holds rows j of the j-block and columns r of the
    // r-block (shared K_j operand), so each lane writes four consecutive j of one
    // row r.  The X and O_inter tiles of (own_rb, own_ib) share the S operand.
    f32x16 xacc = zero16(), oacc = zero16(), aacc = zero16(), pacc = zero16();
    {
      const E* Ax = Kr + (own_rb < 0 ? 0 : own_rb) * 32 * LDK;
      const E* Ao = Qr + (own_rb < 0 ? 0 : own_rb) * 32 * LDK;
      const E* Bs = Sb + own_ib * 32 * LDSB;
      const E* Aj = Kr + ap_jb * 32 * LDK;
      const E* C0 = Kr + ap_rb * 32 * LDK;
      const E* C1 = Qr + ap_rb * 32 * LDK;
      if (own_rb >= 0 && ap >= 0)
        tile_nt4<DK / 16>(xacc, oacc, aacc, pacc, Ax, Ao, Bs, Aj, C0, C1, LDK, LDSB, lane);
      else if (own_rb >= 0)
        tile_nt2_shared_b<DK / 16>(xacc, oacc, Ax, Ao, LDK, Bs, LDSB, lane);
      else if (ap >= 0)
        tile_nt2_shared_a<DK / 16>(aacc, pacc, Aj, LDK, C0, C1, LDK, lane);
    }
    if (ap >= 0) {
      const int r = ap_rb * 32 + col;
      const float Gr = G[r];
      const float br = Bt[r];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = ap_jb * 32 + acc_row(g, 0, lane);
        const float4 gj = *reinterpret_cast<const float4*>(G + j0);
        const float gjv[4] = {gj.x, gj.y, gj.z, gj.w};
        float xa[4], xp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float d = __expf(Gr - gjv[e]);
          xa[e] = (j0 + e < r) ? br * d * aacc[4 * g + e] : 0.f;
          xp[e] = (j0 + e <= r) ? d * pacc[4 * g + e] : 0.f;
        }
        store4(Am + r * LDA + j0, xa[0], xa[1], xa[2], xa[3]);
        store4(Pm + r * LDT + j0, xp[0], xp[1], xp[2], xp[3]);
      }
    }
    if (own_rb >= 0) {
      const int i = own_ib * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = own_rb * 32 + acc_row(g, 0, lane);
        const float4 eg = *reinterpret_cast<const float4*>(Eg + r0);
        store4(Xt + i * LDT + r0,
               load_elem(Vt + i * LDT + r0 + 0) - eg.x * xacc[4 * g + 0],
               load_elem(Vt + i * LDT + r0 + 1) - eg.y * xacc[4 * g + 1],
               load_elem(Vt + i * LDT + r0 + 2) - eg.z * xacc[4 * g + 2],
               load_elem(Vt + i * LDT + r0 + 3) - eg.w * xacc[4 * g + 3]);
        oacc[4 * g + 0] *= eg.x;
        oacc[4 * g + 1] *= eg.y;
        oacc[4 * g + 2] *= eg.z;
        oacc[4 * g + 3] *= eg.w;
      }
    }
    __syncthreads();

    // ---- K^T for phase 6 when it shares Q's region (fp32, d_k = 128) ----
    if (!SEPKT) {
      for (int blk = tid; blk < NKB; blk += kThreads) {
        const int rg = blk % 16, cc = blk / 16;
        uint4 v[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          v[rr] = *reinterpret_cast<const uint4*>(Kr + (4 * rg + rr) * LDK + cc * EPC);
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          store_col4(Kt + (cc * EPC + e) * LDT + 4 * rg, v[0], v[1], v[2], v[3], e);
      }
    }

    // ---- solve (a): inverses of the four unit-lower 16x16 diagonal blocks ----
    // Wave w owns block w; lane c (< 16) computes column c by forward substitution.
    {
      const int I = wave, c = lane & 15;
      const float* base = Am + (16 * I) * LDA + 16 * I;
      float y[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float s = 0.f;
#pragma unroll
        for (int jq = 0; jq < (i + 3) / 4; ++jq) {
          const float4 a4 = *reinterpret_cast<const float4*>(base + i * LDA + 4 * jq);
          const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (4 * jq + e < i) s += av[e] * y[4 * jq + e];
        }
        y[i] = i < c ? 0.f : (i == c ? 1.f : -s);
      }
      if (lane < 16) {
#pragma unroll
        for (int i = 0; i < 16; ++i) Li[(16 * I + i) * LDA + 16 * I + c] = y[i];
      }
    }
    __syncthreads();
    // ---- solve (b): L^-1_{b+1,b} = -L^-1_{b+1,b+1} (A_{b+1,b} L^-1_{b,b}), b = 0, 2 ----
    // fp32 MFMA 16x16x4; lane l uses k index 4 (l / 16) + s in step s, so the
    // first product's accumulator is directly the second product's B operand.
    if (wave < 2) {
      const int bb = 2 * wave, m = lane & 15, hq = lane >> 4;
      f32x4 mprod = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int k = 4 * hq + s;
        mprod = mma_f32_16x16(Am[(16 * (bb + 1) + m) * LDA + 16 * bb + k],
                              Li[(16 * bb + k) * LDA + 16 * bb + m], mprod);
      }
      f32x4 r = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s)
        r = mma_f32_16x16(Li[(16 * (bb + 1) + m) * LDA + 16 * (bb + 1) + 4 * hq + s], mprod[s], r);
#pragma unroll
      for (int v = 0; v < 4; ++v) Li[(16 * (bb + 1) + 4 * hq + v) * LDA + 16 * bb + m] = -r[v];
    }
    __syncthreads();
    // ---- solve (c): the 32x32 block L^-1_{1,0} = -L^-1_{11} (A_{10} L^-1_{00}) ----
    {
      const int mi = wave >> 1, ni = wave & 1, m = lane & 15, hq = lane >> 4;
      f32x4 acc = zero4();
      // L^-1_{00} is lower triangular: its rows 0..15 vanish in columns 16..31
      for (int s = ni ? 4 : 0; s < 8; ++s) {
        const int k = 4 * s + hq;
        acc = mma_f32_16x16(Am[(32 + 16 * mi + m) * LDA + k], Li[k * LDA + 16 * ni + m], acc);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) Mt[(16 * mi + 4 * hq + v) * LDM + 16 * ni + m] = acc[v];
    }
    __syncthreads();
    {
      const int mi = wave >> 1, ni = wave & 1, m = lane & 15, hq = lane >> 4;
      f32x4 acc = zero4();
      // L^-1_{11} is lower triangular: its rows 0..15 vanish in columns 16..31
      for (int s = 0; s < (mi ? 8 : 4); ++s) {
        const int k = 4 * s + hq;
        acc = mma_f32_16x16(Li[(32 + 16 * mi + m) * LDA + 32 + k], Mt[k * LDM + 16 * ni + m], acc);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) Li[(32 + 16 * mi + 4 * hq + v) * LDA + 16 * ni + m] = -acc[v];
    }
    __syncthreads();
    // ---- solve (d): T[r][j] = L^-1[r][j] beta_j on and below the diagonal, 0 above ----
    {
      const int r = tid >> 2, jc = (tid & 3) * 16;
      float x[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 l4 = *reinterpret_cast<const float4*>(Li + r * LDA + jc + 4 * q4);
        const float4 b4 = *reinterpret_cast<const float4*>(Bt + jc + 4 * q4);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * q4 + e] = (jc + 4 * q4 + e <= r) ? lv[e] * bv[e] : 0.f;
      }
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store4(Tm + r * LDT + jc + 4 * q4, x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]);
    }
    __syncthreads();

    // ---- phase 4: U = T X; store U^T and the decay-weighted copy for the state ----
    if (own_rb >= 0) {
      f32x16 uacc = zero16();
      if (own_rb == 0) tile_nt_k<2>(uacc, Tm, LDT, Xt + own_ib * 32 * LDT, LDT, lane);
      else tile_nt_k<4>(uacc, Tm + 32 * LDT, LDT, Xt + own_ib * 32 * LDT, LDT, lane);
      const int i = own_ib * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = own_rb * 32 + acc_row(g, 0, lane);
        const float4 ec = *reinterpret_cast<const float4*>(Ec + r0);
        store4(Ut + i * LDT + r0, uacc[4 * g], uacc[4 * g + 1], uacc[4 * g + 2], uacc[4 * g + 3]);
        store4(Uw + i * LDT + r0, uacc[4 * g] * ec.x, uacc[4 * g + 1] * ec.y,
               uacc[4 * g + 2] * ec.z, uacc[4 * g + 3] * ec.w);
      }
    }
    __syncthreads();

    // ---- phase 5: O = O_inter + P U, written to HBM ----
    if (own_rb >= 0) {
      if (own_rb == 0) tile_nt_k<2>(oacc, Pm, LDT, Ut + own_ib * 32 * LDT, LDT, lane);
      else tile_nt_k<4>(oacc, Pm + 32 * LDT, LDT, Ut + own_ib * 32 * LDT, LDT, lane);
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
      const float gC = Eg[C - 1];
#pragma unroll
      for (int st = 0; st < NST; ++st)
#pragma unroll
        for (int v = 0; v < 16; ++v) Sacc[st][v] *= gC;
      if (NST == 2 && wave + 4 < NT) {
        // tiles wave and wave + 4 share the value block: one Uw fragment, two MFMAs
        tile_nt2_shared_b<C / 16>(Sacc[0], Sacc[NST - 1], Kt + (wave / NI) * 32 * LDT,
                                  Kt + ((wave + 4) / NI) * 32 * LDT, LDT,
                                  Uw + (wave % NI) * 32 * LDT, LDT, lane);
      } else {
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const int t = wave + 4 * st;
          if (t < NT)
            tile_nt_k<C / 16>(Sacc[st], Kt + (t / NI) * 32 * LDT, LDT, Uw + (t % NI) * 32 * LDT,
                              LDT, lane);
        }
      }
#pragma unroll
      for (int st = 0; st < NST; ++st) {
        const int t = wave + 4 * st;
        if (t < NT) {
          const int cb = t / NI, ib = t % NI, i = ib * 32 + col;
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

// Slice width: 64 value rows per workgroup (bf16) when that still gives at least
// one workgroup per compute unit (256), else 32.  fp32 tiles take twice the LDS,
// so fp32 always uses 32-row slices.
template <typename E, int DK>
hipError_t launch_dk(const PrefillArgs& a, hipStream_t stream) {
  if constexpr (sizeof(E) == 4) {
    return launch_slices<E, DK, 32>(a, stream);
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
