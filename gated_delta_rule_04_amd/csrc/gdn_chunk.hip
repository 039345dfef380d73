// Chunked prefill of the gated delta rule: DeltaNet, Gated DeltaNet (scalar
// decay) and Kimi Delta Attention (per-channel decay).
//
// The token recurrence ("Linear Attention Architectures" notes, sections 2.3-2.5,
// Eqs. 9-10, 15-17 and 18-20; state d_v x d_k as in the "On State Reduction"
// notes, section 2.1) is rewritten per chunk of C = 64 tokens.  With G_r the
// running sum of log alpha inside the chunk (gamma_r = exp(G_r)), entry state
// S_n and the chunk's row-stacked K, Q, V:
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
// triangular inverse of its chunked kernel in its numerics section.  With
// per-channel decay the exponentials are per key channel; see chunk_prep_kda.)
//
// A, T and P depend only on the chunk's keys, queries and gates, never on the
// state, so they leave the state chain: a first, fully parallel kernel (one
// workgroup per chunk of every head) computes T (and P, except for scalar decay
// in bf16, where the state kernel's data waves form P from the K and Q rows
// they stage anyway) and hands it over through a workspace record per chunk.
// The sequential kernel then only carries the chain X -> U -> (O, S) per chunk.
//
// chunk_prep_kernel  (none / scalar decay; grid B * H * N_chunks)
//   K (fp32: and Q) tiles and gates -> A (and P) (MFMA) -> 16x16 diagonal
//   inverses (quad-DPP forward substitution) -> two levels of fp32 MFMA block
//   products -> T; T (P) and the gate rows -> record.
// chunk_prep_kda     (per-channel decay; grid B * H * N_chunks)
//   per-channel prefix of log alpha -> anchor-split decay factors -> A and P
//   (MFMA) -> T; T, P, the decay-scaled K / Q operands and exp(G_C) -> record.
// chunk_state_ws     (bf16; grid B * H * d_v / DVS, chunks in order)
//   Four chain waves carry the fp32 state slice in MFMA accumulators; four
//   data waves stream the chunks into LDS (and form P) and the outputs back
//   out.  Value
//   rows are independent ("On State Reduction" notes, section 2.5), so each
//   workgroup owns one (b, h, d_v slice).
// chunk_state_kernel (fp32; the same phases with four waves that also move
//   the data themselves)
#include <mutex>
#include <type_traits>

#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_solve.h"

namespace gdn {
namespace {

constexpr int C = 64;                // chunk length
constexpr int kThreads = 256;        // four waves
constexpr float kLogFloor = -100.f;  // gates below e^-100 act as e^-100 (about 3.7e-44, an fp32 subnormal)

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// Where the tokens of one sequence lie and where its chunk records start.
//   B rows of T tokens: sequence b is row b; its chunk n of head h has record
//     (b H + h) N_chunks + n.
//   packed batch: sequence b holds tokens cu[b] .. cu[b + 1] - 1 of the token
//     axis; its chunk n of head h has record h nslots + cu[b] / C + b + n.
//     Sequence b's records end at slot floor(cu[b + 1] / C) + b at most, below
//     the next sequence's first one, and every slot is below T / C + B.
// Offsets are clamped into [0, T] (each sequence to a range of its own start):
// malformed offsets then give unspecified results but never an access outside
// the buffers.
struct Span {
  size_t tok0;   // first token on the token axis ([B * T] for rows of T tokens)
  int len;       // tokens of the sequence
  size_t rec0;   // record of its chunk 0
};

__device__ inline Span seq_span(const PrefillArgs& a, int b, int h) {
  if (a.cu_seqlens) {
    const int s0 = min(max(a.cu_seqlens[b], 0), a.T);
    const int s1 = min(max(a.cu_seqlens[b + 1], s0), a.T);
    return Span{(size_t)s0, s1 - s0, (size_t)h * a.nslots + s0 / C + b};
  }
  return Span{(size_t)b * a.T, a.T, ((size_t)b * a.H + h) * (size_t)((a.T + C - 1) / C)};
}

// Packed batch: the sequence whose records may hold slot `slot`, i.e. the
// largest b with cu[b] / C + b <= slot (that bound grows strictly with b).  A
// 64-ary search, each wave on its own: 64 probes per round, as many rounds as
// the base-64 digits of B.
__device__ inline int seq_of_slot(const PrefillArgs& a, int slot) {
  const int lane = threadIdx.x & 63;
  int lo = 0, span = a.B;   // the answer lies in [lo, lo + span)
  while (span > 1) {
    const int stride = (span + 63) / 64;
    const int bq = lo + lane * stride;
    bool le = false;
    if (bq < lo + span) le = min(max(a.cu_seqlens[bq], 0), a.T) / C + bq <= slot;
    const int cnt = __popcll(__ballot(le));
    if (cnt == 0) return lo;
    const int nlo = lo + (cnt - 1) * stride;
    span = min(stride, lo + span - nlo);
    lo = nlo;
  }
  return lo;
}

// The chunk one prep workgroup handles: sequence b, head h, chunk n of the
// sequence (B rows of T tokens), or record slot n of head h (packed batch).
//   BY_CHUNK (scalar gates): the H heads of one chunk (slot) run back to back
//     on one XCD.  Workgroups are dispatched round-robin over the eight XCDs,
//     so workgroup i = 8 j + x takes head j % H of chunk (slot) 8 c + x of row
//     b, where j / H = b C8 + c (C8 = ceil(N / 8)).  The gates are [.., T, H]
//     fp32: the heads of a token share their cache lines, which then come
//     from HBM once per chunk rather than once per head.
//   otherwise (per-channel gates, contiguous per head and token): workgroup
//     (b H + h) N + n (slot: h nslots + slot), so that consecutive workgroups
//     write consecutive records.
// False for a workgroup past the last chunk (slot), or a packed slot that no
// chunk falls on.
struct PrepAt {
  int b, h, n;
  Span sp;
};

template <bool BY_CHUNK>
__host__ __device__ inline size_t prep_grid(int rows, int H, int nunits) {
  return BY_CHUNK ? (size_t)8 * rows * H * ((nunits + 7) / 8) : (size_t)rows * H * nunits;
}

template <bool BY_CHUNK>
__device__ inline bool prep_at(const PrefillArgs& a, int nchunks, PrepAt& p) {
  int unit, g;
  if (BY_CHUNK) {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int c8 = (nchunks + 7) / 8;
    p.h = j % a.H;
    unit = 8 * ((j / a.H) % c8) + x;
    g = j / a.H / c8;   // row
  } else {
    const int bh = blockIdx.x / nchunks;
    unit = blockIdx.x % nchunks;
    p.h = bh % a.H;
    g = bh / a.H;
  }
  if (unit >= nchunks) return false;
  if (!a.cu_seqlens) {
    p.b = g;
    p.n = unit;
    p.sp = seq_span(a, p.b, p.h);
    return true;
  }
  const int slot = unit;
  p.b = seq_of_slot(a, slot);
  p.sp = seq_span(a, p.b, p.h);
  p.n = slot - (int)(p.sp.rec0 - (size_t)p.h * a.nslots);
  return p.n >= 0 && p.n * C < p.sp.len;
}

// Tiles are moved between HBM, registers and LDS in blocks of 4 rows x one
// 16-byte chunk (used by the fp32 state kernel, which transposes from
// registers).  Block blk of a tile with cpr chunks per row covers rows
// 4 blk_row .. 4 blk_row + 3 and chunk blk_col.  Four consecutive blocks take
// four row groups of one chunk, the next four the next chunk, so a wave's
// global loads cover whole rows.
__device__ inline int blk_row(int blk, int cpr) { return (blk & 3) + 4 * (blk / (4 * cpr)); }
__device__ inline int blk_col(int blk, int cpr) { return (blk >> 2) % cpr; }

// 16-byte loads and stores of data touched once per kernel (inputs read once,
// workspace and outputs written once): non-temporal, so they do not displace
// the lines other workgroups still reuse.
__device__ inline u32x4 ld_once(const void* p) {
  return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}
__device__ inline void st_once(void* p, const u32x4& v) {
  __builtin_nontemporal_store(v, static_cast<u32x4*>(p));
}

// Workspace: one record per chunk of every head (chunk index = head *
// N_chunks + n).  Scalar or no decay, offsets in elements of the operand dtype:
//   T [C][C] (row-major), in fp32 also P [C][C], then five fp32 gate rows:
//     0  G_r
//     1  exp(G_r) nk_r          X = V - diag(row 1) K S^T
//     2  exp(G_C - G_r) nk_r    S_{n+1} = gamma_C S_n + U^T diag(row 2) K
//     3  exp(G_r) nq_r          O_inter = diag(row 3) Q S^T
//     4  G_r - ln nk_r          P[r][j] = exp(G_r - row 4_j) nq_r (q_r . k_j)
//   nk_r and nq_r are 1 / sqrt(|k_r|^2 + eps) and 1 / sqrt(|q_r|^2 + eps) when
//   the kernels normalise q and k, else 1.  The bf16 records hold nq = 1: that
//   state kernel forms P itself and applies nq to its output rows.
// (The per-channel record is KdaRec.)
constexpr int kGateRows = 5;
constexpr size_t kGateFloats = kGateRows * C;

template <typename E>
struct GateRec {
  static constexpr bool has_p = sizeof(E) == 4;
  static constexpr size_t t = 0;
  static constexpr size_t p = (size_t)C * C;   // fp32 only
  static constexpr size_t g = (has_p ? 2 : 1) * (size_t)C * C;   // fp32 region
  static constexpr size_t elems = g + kGateFloats * 4 / sizeof(E);
};


// Sum over aligned groups of N lanes (N = 4, 8, 16, 32), result in all of them.
template <int N>
__device__ inline float lane_group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group of 4, 8, 16 or 32 lanes");
  x = quad_sum(x);
  if constexpr (N >= 8)   // row_half_mirror: lane i of 8 takes lane 7 - i
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  if constexpr (N >= 16)  // row_mirror: lane i of 16 takes lane 15 - i
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// Sum of squares of a 16-byte piece of the operand dtype, accumulated onto s0
// (bf16: two products per dot instruction, summed in fp32; its clamp flag
// stays off, which would saturate the sum to [0, 1]).
template <typename E>
__device__ inline float sumsq16(const u32x4& u, float s0 = 0.f) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  float s = s0;
  if constexpr (sizeof(E) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      // (the word goes through a local first: a bit cast applied straight
      // to u[w] in this unrolled loop compiles to u[0] every time)
      const uint32_t uw = u[w];
      const bf16x2_t x = __builtin_bit_cast(bf16x2_t, uw);
      s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
    }
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float x = __uint_as_float(u[w]);
      s += x * x;
    }
  }
  return s;
}

// log alpha of one gate value of head h (channel c for a per-channel gate): the
// value itself, or a logit x with log alpha = -A[h] softplus(x + dt_bias)
// (a Mamba2-style decay); floored at kLogFloor.
__device__ inline float log_alpha(const Prologue& p, float x, int h, int bias_index) {
  const float la = p.alpha_logits
                       ? -p.A[h] * softplus_f(x + (p.dt_bias ? p.dt_bias[bias_index] : 0.f))
                       : logf(x);
  return fmaxf(la, kLogFloor);
}

// Gates of one chunk, lane r of the wave holding token r: inclusive prefix G of
// log alpha (la = 0 past the sequence end).
__device__ inline float chunk_prefix(float la) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float y = __shfl_up(la, off);
    if (lane >= off) la += y;
  }
  return la;
}


// ---------------------------------------------------------------------------
// chunk_prep_kernel: T = (I + A)^-1 diag(beta) (and in fp32 P) for one chunk of
// one head.
// ---------------------------------------------------------------------------
// Neither depends on the state, so both leave the sequential kernel.  (The bf16
// state kernel forms P from the K and Q rows it holds anyway, which spares
// this kernel the Q reads and the record the P bytes.)
// LDS: K rows [64][LDK] (then L^-1 fp32 [64][LDA]), Q rows [64][LDK] (then A
// fp32 [64][LDA], then T [64][LDT]), Mt fp32 [32][LDM], G, beta (and, when q
// and k are normalised, the inverse norms of the K and Q rows).  P goes to the
// record straight from the accumulators.
template <typename E, int DK, bool NORM>
struct PrepPlan {
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = DK + PAD;
  static constexpr int LDA = SolveLd<E>::LDA;
  static constexpr int LDT = SolveLd<E>::LDT;
  static constexpr int LDM = SolveLd<E>::LDM;
  static constexpr size_t es = sizeof(E);
  // bf16 (no Q): A takes the dead K rows' bytes and L^-1 overwrites A in
  // place, the solve's scratch tile sits in L^-1's unused upper-right block,
  // and T goes from the solve straight to the record; 17.9 KB, eight
  // workgroups per compute unit.
  // fp32: L^-1 over the K rows; Q, then A, then T in a second region.
  static constexpr bool inplace = sizeof(E) == 2;
  static constexpr size_t r1 = cmax((size_t)C * LDK * es, (size_t)C * LDA * 4);
  static constexpr size_t kr = 0;   // K rows, then L^-1
  static constexpr size_t am = inplace ? 0 : r1;
  static constexpr size_t tm = inplace ? r1 : am;   // (in place: no T in LDS)
  static constexpr int ldm = inplace ? LDA : LDM;
  static constexpr size_t mt = inplace ? (size_t)32 * 4   // A + 32 floats, leading dimension LDA
                                       : am + cmax((size_t)C * LDK * es, cmax((size_t)C * LDA * 4, (size_t)C * LDT * es));
  static constexpr size_t g = inplace ? r1 : mt + (size_t)32 * LDM * 4;
  // inverse norms (K, then Q in fp32)
  static constexpr size_t nk = g + 2 * C * 4;
  // squared K row norms (the transition bound of scalar decay)
  static constexpr size_t ksq = g + (NORM ? (inplace ? 3 : 4) : 2) * C * 4;
  // bf16, normalised: G_j - ln nk_j (the column factor of A inside its weight)
  static constexpr size_t gn = ksq + C * 4;
  static constexpr size_t total = gn + (NORM && inplace ? C * 4 : 0);
};

template <typename E, int DK, int MODE, bool NORM>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(8))) void chunk_prep_kernel(PrefillArgs a, E* __restrict__ tws,
                                                              int nchunks) {
  using L = PrepPlan<E, DK, NORM>;
  using R = GateRec<E>;
  constexpr bool WP = R::has_p;
  constexpr int EPC = 16 / (int)sizeof(E);
  constexpr int CPR = DK / EPC;
  constexpr int LDK = L::LDK, LDA = L::LDA, LDT = L::LDT;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  E* Kr = reinterpret_cast<E*>(smem + L::kr);
  float* Li = reinterpret_cast<float*>(smem + L::kr);
  E* Qr = reinterpret_cast<E*>(smem + L::am);
  float* Am = reinterpret_cast<float*>(smem + L::am);
  E* Tm = reinterpret_cast<E*>(smem + L::tm);
  float* Mt = reinterpret_cast<float*>(smem + L::mt);
  float* G = reinterpret_cast<float*>(smem + L::g);
  float* Bt = G + C;
  float* Nk = reinterpret_cast<float*>(smem + L::nk);   // NORM only
  float* Nq = Nk + C;                                   // NORM, fp32 only
  float* Ksq = reinterpret_cast<float*>(smem + L::ksq);  // scalar decay with a bound array only
  float* Gn = reinterpret_cast<float*>(smem + L::gn);    // bf16, normalised only

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 31;
  PrepAt at;
  if (!prep_at<true>(a, nchunks, at)) return;
  const int H = a.H, h = at.h, n = at.n;
  const int t0 = n * C, cn = min(C, at.sp.len - t0);
  const size_t tok0 = at.sp.tok0 + t0;   // first token of the chunk on the token axis
  E* rec = tws + (at.sp.rec0 + n) * R::elems;
  E* Pw = rec + R::p;

  // K (and Q) rows, consecutive threads along a row (rows past the sequence
  // end repeat its last row: beta = 0 there, so they never reach A or T, and
  // P's rows of them are never used).  K takes ordinary loads: the state
  // kernel reads it again right after this kernel, and K plus the records fit
  // the last-level cache at the batched workload's size (the non-temporal
  // hint cost that second read 3-4 % of the call).  Normalised q and k: the
  // inverse norms come from the loaded registers, summed over the CPR lanes
  // that hold a row.
  {
    const E* kg = static_cast<const E*>(a.k) + (tok0 * H + h) * DK;
    const E* qg = static_cast<const E*>(a.q) + (tok0 * H + h) * DK;
    const size_t ktok = (size_t)H * DK;
    static_assert(C * CPR % kThreads == 0, "K rows must split evenly over the threads");
  static_assert(L::inplace == !WP, "the in-place plan has no room for Q");
#pragma unroll
    for (int m = 0; m < C * CPR / kThreads; ++m) {
      const int q = tid + kThreads * m, r = q / CPR, cc = q % CPR;
      const size_t off = (size_t)min(r, cn - 1) * ktok + cc * EPC;
      const u32x4 kv = *reinterpret_cast<const u32x4*>(kg + off);
      *reinterpret_cast<u32x4*>(Kr + r * LDK + cc * EPC) = kv;
      u32x4 qv = kv;
      if constexpr (WP) {
        qv = ld_once(qg + off);
        *reinterpret_cast<u32x4*>(Qr + r * LDK + cc * EPC) = qv;
      }
      if constexpr (NORM && WP) {   // (bf16: the K norms come from the Gram tiles below)
        const float ks = lane_group_sum<CPR>(sumsq16<E>(kv));
        const float nk = __builtin_amdgcn_rsqf(ks + a.pro.norm_eps);
        const float nq = __builtin_amdgcn_rsqf(lane_group_sum<CPR>(sumsq16<E>(qv)) + a.pro.norm_eps);
        if (cc == 0) {
          Nk[r] = nk;
          Nq[r] = nq;
        }
      }
    }
  }
  if (wave == 0) {
    const bool ok = lane < cn;
    const size_t tok = (tok0 + min(lane, cn - 1)) * H + h;
    const float al = MODE == 1 ? static_cast<const float*>(a.alpha)[tok] : 1.f;
    const float braw = a.beta[tok];
    const float la = MODE == 1 ? log_alpha(a.pro, al, h, h) : 0.f;
    const float bt = a.pro.beta_logits ? sigmoid_f(braw) : braw;
    const float g = chunk_prefix(ok ? la : 0.f);
    const float gC = __shfl(g, C - 1);
    G[lane] = g;
    Bt[lane] = ok ? bt : 0.f;
    float* gw = reinterpret_cast<float*>(rec + R::g);
    gw[lane] = g;
    if constexpr (!NORM) {   // (normalised: the rows with norms follow once they are known)
      const float eg = __expf(g);
      gw[C + lane] = eg;
      gw[2 * C + lane] = __expf(gC - g);
      gw[3 * C + lane] = eg;
      gw[4 * C + lane] = g;
    }
  }
  __syncthreads();

  // A and P tiles (j block, r block) in {(0,0), (0,1), (1,1)}, rows j and
  // columns r; wave w < 3 takes tile w of both.
  const int jb = wave == 2 ? 1 : 0, rb = wave == 0 ? 0 : 1;
  f32x16 acca = zero16(), accp = zero16();
  if (wave < 3) {
    if constexpr (WP)
      tile_nt2_pairs<DK / 16>(acca, accp, Kr + jb * 32 * LDK, Kr + rb * 32 * LDK, Kr + jb * 32 * LDK,
                              Qr + rb * 32 * LDK, LDK, lane);
    else
      tile_nt_k<DK / 16>(acca, Kr + jb * 32 * LDK, LDK, Kr + rb * 32 * LDK, LDK, lane);
    // bf16: |k_r|^2 is the diagonal entry of a diagonal Gram tile (waves 0 and
    // 2), held by one lane: the inverse norms of normalised keys, or the
    // squared norms for the transition bound of scalar decay
    if (!WP && jb == rb && (NORM || (MODE == 1 && a.horizon))) {
      const int r = rb * 32 + col;
      float dg = 0.f;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e) dg = jb * 32 + acc_row(g, e, lane) == r ? acca[4 * g + e] : dg;
      if (((col >> 2) & 1) == (lane >> 5)) {
        if constexpr (NORM) {
          const float nk = __builtin_amdgcn_rsqf(dg + a.pro.norm_eps);
          Nk[r] = nk;
          Gn[r] = G[r] - __logf(nk);
          Ksq[r] = dg * nk * nk;   // |k|^2 of the normalised key
        } else {
          Ksq[r] = dg;
        }
      }
    }
  }
  __syncthreads();   // K and Q are dead: A takes their bytes
  // A[r][j] = beta_r exp(G_r - G_j) k_r.k_j (j < r); P[r][j] = exp(G_r - G_j) q_r.k_j
  // (j <= r).  Every weight is formed clamped to at most 1 before the masks
  // select (left conditional, its loads would sink into per-element branches).
  // Normalised q and k: A takes nk_r nk_j, P nq_r nk_j (the row factor joins
  // beta_r, the column factor the weight; in bf16 nk_j enters the exponent,
  // and the clamp, at e^88, then only keeps the masked weights finite).
  if (wave < 3) {
    constexpr bool GNJ = NORM && !WP;
    constexpr float WMAX = GNJ ? 88.f : 0.f;
    const float* Gj = GNJ ? Gn : G;
    const int r = rb * 32 + col;
    const float Gr = G[r];
    float br = Bt[r], pr = 1.f;
    if constexpr (NORM) {
      br *= Nk[r];
      if constexpr (WP) pr = Nq[r];
    }
    float w[16];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 gj = *reinterpret_cast<const float4*>(Gj + jb * 32 + acc_row(g, 0, lane));
      w[4 * g + 0] = __expf(fminf(Gr - gj.x, WMAX));
      w[4 * g + 1] = __expf(fminf(Gr - gj.y, WMAX));
      w[4 * g + 2] = __expf(fminf(Gr - gj.z, WMAX));
      w[4 * g + 3] = __expf(fminf(Gr - gj.w, WMAX));
      if constexpr (NORM && WP) {
        const float4 nj = *reinterpret_cast<const float4*>(Nk + jb * 32 + acc_row(g, 0, lane));
        w[4 * g + 0] *= nj.x;
        w[4 * g + 1] *= nj.y;
        w[4 * g + 2] *= nj.z;
        w[4 * g + 3] *= nj.w;
      }
    }
#pragma unroll
    for (int v = 0; v < 16; ++v) asm volatile("" ::"v"(w[v]));
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int j0 = jb * 32 + acc_row(g, 0, lane);
      float x[4], y[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = (j0 + e < r) ? br * w[4 * g + e] * acca[4 * g + e] : 0.f;
        y[e] = (j0 + e <= r) ? pr * w[4 * g + e] * accp[4 * g + e] : 0.f;
      }
      store4(Am + r * LDA + j0, x[0], x[1], x[2], x[3]);
      if constexpr (WP) store4(Pw + r * C + j0, y[0], y[1], y[2], y[3]);
    }
  } else {
    if constexpr (WP) {   // P rows 0..31, columns 32..63 are zero
      const int q = tid - 192, r = q >> 1, j0 = 32 + 16 * (q & 1);
#pragma unroll
      for (int e = 0; e < 16; e += 4) store4(Pw + r * C + j0 + e, 0.f, 0.f, 0.f, 0.f);
    }
    if constexpr (NORM) {   // the gate rows that carry the norms
      const float g = G[lane], eg = __expf(g), nk = Nk[lane];
      float* gw = reinterpret_cast<float*>(rec + R::g);
      gw[C + lane] = eg * nk;
      gw[2 * C + lane] = __expf(G[C - 1] - g) * nk;
      gw[3 * C + lane] = WP ? eg * Nq[lane] : eg;
      gw[4 * C + lane] = WP ? g - __logf(nk) : Gn[lane];
    }
  }
  __syncthreads();

  if constexpr (L::inplace) {
    tri_solve<E, L::ldm, true, true>(Am, Li, Mt, Bt, rec + R::t, tid);   // T straight to the record
    // The chunk's state transition S -> S prod_t alpha_t (I - beta_t k_t k_t^T)
    // has spectral norm at most prod_t alpha_t max(1, |1 - beta_t |k_t|^2|)
    // (each factor is symmetric with eigenvalues 1 and 1 - beta_t |k_t|^2); its
    // log goes to the bound array.  (Tokens past the sequence end: beta = 0.)
    // G, beta and |k|^2 outlive the solve, which writes neither.
    if (MODE == 1 && a.horizon && wave == 3) {
      float grow = __logf(fmaxf(1.f, fabsf(1.f - Bt[lane] * Ksq[lane])));
      grow = lane_group_sum<32>(grow);
      grow += __shfl_xor(grow, 32);
      if (lane == 0) a.horizon[at.sp.rec0 + n] = G[C - 1] + grow;
    }
  } else {
    tri_solve<E, L::ldm, false, true>(Am, Li, Mt, Bt, Tm, tid);
    // T -> the record, 64 x 64 contiguous, 16-byte stores
    constexpr int CPT = C / EPC;
    static_assert(C * CPT % kThreads == 0, "T must split evenly over the threads");
#pragma unroll
    for (int m = 0; m < C * CPT / kThreads; ++m) {
      const int q = tid + kThreads * m, r = q / CPT, cc = q % CPT;
      st_once(rec + R::t + r * C + cc * EPC, *reinterpret_cast<const u32x4*>(Tm + r * LDT + cc * EPC));
    }
  }
}

// ---------------------------------------------------------------------------
// chunk_prep_kda: per-channel decay (Kimi Delta Attention), one chunk of one head.
// ---------------------------------------------------------------------------
// With G_r[c] the running sum of log alpha_t[c] inside the chunk,
//   A[r][j] = beta_r sum_c k_r[c] k_j[c] exp(G_r[c] - G_j[c])      j < r
//   P[r][j] =        sum_c q_r[c] k_j[c] exp(G_r[c] - G_j[c])      j <= r
// The weight depends on the channel, so it cannot be applied after the
// contraction.  It is split at an anchor token m: exp(G_r - G_m) scales the
// r-side operand and exp(G_m - G_j) the j-side one, and each 32x32 tile is one
// MFMA product of two scaled operand tiles:
//   rows 32..63 x columns 0..31   m = 31: both factors are at most 1
//   diagonal blocks               m = 15 and 47: each factor spans at most 16
//                                 tokens of decay
// In a diagonal block, a channel whose decay on either side of the anchor
// exceeds exp(kSplitLimit) could overflow or underflow its factors; it is left
// out of the MFMA (zero operands) and its exact contribution, with the weight
// exp(G_r - G_j) <= 1 taken directly, is added by the wave that owns the tile.
// Masked entries (j > r) of the diagonal blocks may overflow; the epilogues
// replace them by zero with a select, never with arithmetic.
// Gated DeltaNet-2 ("Linear Attention Architectures" notes, section 2.6) runs
// through the same kernel: its erase direction e_r = b_r * k_r takes k_r's place
// on the row side of A and in Kg (the prediction reads e), beta is 1, and the
// state kernel scales V by the write gate (z = w * v); P, Kc and the state
// update keep k.
// Instead of gates, the state kernel gets decay-scaled operands (the chunk form
// with Diag(exp(G_r)) in place of gamma_r):
//   Kg = K . exp(G)          X = V - Kg S^T
//   Qg = Q . exp(G)          O_inter = Qg S^T
//   Kc = K . exp(G_C - G)    S_{n+1} = S Diag(gC) + U^T Kc
//   gC = exp(G_C)

// Per-chunk workspace record of the per-channel path (chunk index = head *
// N_chunks + n), offsets in elements of the operand dtype:
//   T [C][C], P [C][C], Kg [C][DK], Qg [C][DK], Kc [C][DK], then gC: DK fp32.
template <typename E, int DK>
struct KdaRec {
  static constexpr size_t t = 0;
  static constexpr size_t p = (size_t)C * C;
  static constexpr size_t kg = 2 * (size_t)C * C;
  static constexpr size_t qg = kg + (size_t)C * DK;
  static constexpr size_t kc = qg + (size_t)C * DK;
  static constexpr size_t g = kc + (size_t)C * DK;   // fp32 region
  static constexpr size_t elems = g + (size_t)DK * 4 / sizeof(E);
};

// The workspace record of a decay mode.
template <typename E, int DK, int MODE>
struct RecOf {
  using type = GateRec<E>;
};
template <typename E, int DK>
struct RecOf<E, DK, 2> {
  using type = KdaRec<E, DK>;
};
template <typename E, int DK>
struct RecOf<E, DK, 3> {   // Gated DeltaNet-2: Kg holds the decay-scaled erase rows
  using type = KdaRec<E, DK>;
};

// A 16-byte chunk of the operand dtype as fp32 values, and back (round to
// nearest even).
template <typename E>
__device__ inline void unpack16(const u32x4& u, float* f);
template <>
__device__ inline void unpack16<__bf16>(const u32x4& u, float* f) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    f[2 * w] = __uint_as_float(u[w] << 16);
    f[2 * w + 1] = __uint_as_float(u[w] & 0xffff0000u);
  }
}
template <>
__device__ inline void unpack16<float>(const u32x4& u, float* f) {
#pragma unroll
  for (int w = 0; w < 4; ++w) f[w] = __uint_as_float(u[w]);
}
template <typename E>
__device__ inline u32x4 pack16(const float* f);
template <>
__device__ inline u32x4 pack16<__bf16>(const float* f) {
  bf16x8 t;
#pragma unroll
  for (int i = 0; i < 8; ++i) t[i] = (__bf16)f[i];
  return __builtin_bit_cast(u32x4, t);
}
template <>
__device__ inline u32x4 pack16<float>(const float* f) {
  return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
}

// Element-wise product of two 16-byte pieces (rounded to the operand dtype).
template <typename E>
__device__ inline u32x4 mul16(const u32x4& a, const u32x4& b) {
  constexpr int N = 16 / (int)sizeof(E);
  float x[N], y[N];
  unpack16<E>(a, x);
  unpack16<E>(b, y);
#pragma unroll
  for (int i = 0; i < N; ++i) x[i] *= y[i];
  return pack16<E>(x);
}

constexpr float kSplitLimit = 64.f;

// LDS: region 1 holds G (fp32 [C][LDG]) while the operands are built, then A
// (fp32 [C][LDA], later T) and P [C][LDT]; region 2 holds the 32-row operand
// tiles; then prefix segment totals, beta and the bit masks of the channels
// left out of each diagonal block's MFMA.
//   bf16 (CMP, 52.5 KB: three workgroups per compute unit): two operand tiles,
//     the r-side one taking the K operand for the A tile and then the Q
//     operand for the P tile; the solve runs in place in A's bytes and writes
//     T straight to the record; the exact path of strongly decayed channels
//     reads the unscaled rows from global memory.
//   fp32: three operand tiles, then L^-1 and Mt of the solve; the unscaled K
//     and Q rows of the current diagonal block.
template <typename E, int DK, bool NORM>
struct KdaPrepPlan {
  static constexpr bool CMP = sizeof(E) == 2;
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = DK + PAD;
  static constexpr int LDG = DK + 4;
  static constexpr int LDA = SolveLd<E>::LDA;
  static constexpr int LDT = SolveLd<E>::LDT;
  static constexpr int LDM = SolveLd<E>::LDM;
  static constexpr int NSEG = kThreads / DK;   // prefix segments per channel
  static constexpr size_t g = 0;
  static constexpr size_t am = 0;
  static constexpr size_t pm = (size_t)C * LDA * 4;
  static constexpr size_t r1 = cmax((size_t)C * LDG * 4, pm + (size_t)C * LDT * sizeof(E));
  static constexpr size_t ops = r1;
  static constexpr size_t li = ops;
  static constexpr size_t mt = li + (size_t)C * LDA * 4;
  static constexpr size_t r2 = CMP ? (size_t)2 * 32 * LDK * sizeof(E)
                                   : cmax((size_t)3 * 32 * LDK * sizeof(E), (size_t)C * LDA * 4 + 32 * LDM * 4);
  static constexpr size_t raw = ops + r2;
  static constexpr size_t tot = raw + (CMP ? 0 : (size_t)2 * 32 * LDK * sizeof(E));
  static constexpr size_t bt = tot + (size_t)NSEG * DK * 4;
  static constexpr size_t msk = bt + C * 4;
  static constexpr size_t nrm = msk + (size_t)2 * (DK / 32) * 4;   // inverse norms of K, Q rows
  // (CMP) one channel's 32 unscaled K values of a diagonal block, for its exact path
  static constexpr size_t ksc = nrm + (NORM ? 2 * C * 4 : 0);
  static constexpr size_t total = ksc + (CMP ? 32 * 4 : 0);
};

template <typename E, int DK, bool NORM, bool G2>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(sizeof(E) == 2 ? 3 : 1)))
void chunk_prep_kda(PrefillArgs a, E* __restrict__ tws, int nchunks) {
  static_assert(!(NORM && G2), "the erase-gate variant takes no prologue");
  using L = KdaPrepPlan<E, DK, NORM>;
  using R = KdaRec<E, DK>;
  constexpr bool CMP = L::CMP;
  constexpr int EPC = 16 / (int)sizeof(E);
  constexpr int CPR = DK / EPC;
  constexpr int LDK = L::LDK, LDG = L::LDG, LDA = L::LDA, LDT = L::LDT;
  constexpr int NSEG = L::NSEG, RPS = C / NSEG;   // rows per prefix segment
  constexpr int IPT = 32 * CPR / kThreads;         // (row, chunk) items per thread per 32 rows
  static_assert(32 * CPR % kThreads == 0 && kThreads % CPR == 0, "item split");
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  float* Gl = reinterpret_cast<float*>(smem + L::g);
  float* Am = reinterpret_cast<float*>(smem + L::am);
  E* Tm = reinterpret_cast<E*>(smem + L::am);
  E* Pm = reinterpret_cast<E*>(smem + L::pm);
  E* Rop = reinterpret_cast<E*>(smem + L::ops);   // r-side K operand
  E* Qop = CMP ? Rop : Rop + 32 * LDK;             // r-side Q operand (CMP: after the A tile)
  E* Cop = Rop + (CMP ? 32 : 64) * LDK;            // j-side K operand
  float* Li = reinterpret_cast<float*>(smem + L::li);
  float* Mt = reinterpret_cast<float*>(smem + L::mt);
  E* Kraw = reinterpret_cast<E*>(smem + L::raw);   // unscaled rows of the current block (fp32)
  E* Qraw = Kraw + 32 * LDK;
  float* Tot = reinterpret_cast<float*>(smem + L::tot);
  float* Bt = reinterpret_cast<float*>(smem + L::bt);
  uint32_t* Msk = reinterpret_cast<uint32_t*>(smem + L::msk);   // [2][DK / 32]
  float* Nk = reinterpret_cast<float*>(smem + L::nrm);            // NORM only
  float* Nq = Nk + C;
  float* Ksc = reinterpret_cast<float*>(smem + L::ksc);           // CMP only

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, col = lane & 31;
  PrepAt at;
  if (!prep_at<false>(a, nchunks, at)) return;
  const int H = a.H, h = at.h, n = at.n;
  const int t0 = n * C, cn = min(C, at.sp.len - t0);
  const size_t tok0 = at.sp.tok0 + t0;
  const size_t qk_tok = (size_t)H * DK;
  const E* kgl = static_cast<const E*>(a.k) + (tok0 * H + h) * DK;
  const E* qgl = static_cast<const E*>(a.q) + (tok0 * H + h) * DK;
  const E* bgl = G2 ? static_cast<const E*>(a.erase) + (tok0 * H + h) * DK : nullptr;
  E* rec = tws + (at.sp.rec0 + n) * R::elems;

  // This thread's (row, 16-byte chunk) items of K and Q, loaded once for all
  // passes: item m is row (tid + kThreads m) / CPR (rows 0..31 for m < IPT,
  // 32..63 above), channels c0 = ((tid + kThreads m) % CPR) EPC.  Rows past the
  // sequence end repeat its last row.
  u32x4 kreg[2 * IPT], qreg[2 * IPT], breg[G2 ? 2 * IPT : 1];   // (erase gate rows: G2)
  float nkm[2 * IPT], nqm[2 * IPT];   // inverse norms of those rows (NORM)
  // G, per channel: thread (segment s, channel c) scans RPS rows, then adds the
  // totals of the segments before it.  Rows past the sequence end add nothing.
  {
    const int c = tid % DK, s = tid / DK;
    const E* ag = static_cast<const E*>(a.alpha) + (tok0 * H + h) * DK + c;
    // all loads first and unconditional (a load under the row test would be
    // waited for one at a time), then log and select
    float g[RPS];
#pragma unroll
    for (int i = 0; i < RPS; ++i) g[i] = (float)ag[(size_t)min(s * RPS + i, cn - 1) * qk_tok];
#pragma unroll
    for (int m = 0; m < 2 * IPT; ++m) {
      const int it = tid + kThreads * m;
      const uint32_t off = (uint32_t)min(it / CPR, cn - 1) * (uint32_t)qk_tok + (it % CPR) * EPC;
      kreg[m] = ld_once(kgl + off);
      qreg[m] = ld_once(qgl + off);
      if constexpr (G2) breg[m] = ld_once(bgl + off);
    }
    // (one branch around the loop: with the choice inside, both the logarithm
    // and the softplus would be formed for every value)
    if (a.pro.alpha_logits) {
      const float ah = a.pro.A[h], bc = a.pro.dt_bias ? a.pro.dt_bias[h * DK + c] : 0.f;
#pragma unroll
      for (int i = 0; i < RPS; ++i) {
        const float la = fmaxf(-ah * softplus_f(g[i] + bc), kLogFloor);
        g[i] = s * RPS + i < cn ? la : 0.f;
      }
    } else {
#pragma unroll
      for (int i = 0; i < RPS; ++i) {
        const float la = fmaxf(__logf(g[i]), kLogFloor);
        g[i] = s * RPS + i < cn ? la : 0.f;
      }
    }
#pragma unroll
    for (int i = 1; i < RPS; ++i) g[i] += g[i - 1];
    Tot[s * DK + c] = g[RPS - 1];
    if (tid < C) {   // (G2: beta is 1, the gates sit in the operands)
      const float bt = G2 ? 1.f : a.beta[(tok0 + min(tid, cn - 1)) * H + h];
      Bt[tid] = tid < cn ? (a.pro.beta_logits ? sigmoid_f(bt) : bt) : 0.f;
    }
    if constexpr (NORM) {
      // inverse norms of this thread's K and Q rows: a row's CPR pieces sit in
      // CPR consecutive lanes
#pragma unroll
      for (int m = 0; m < 2 * IPT; ++m) {
        const int it = tid + kThreads * m;
        nkm[m] = rsqrtf(lane_group_sum<CPR>(sumsq16<E>(kreg[m])) + a.pro.norm_eps);
        nqm[m] = rsqrtf(lane_group_sum<CPR>(sumsq16<E>(qreg[m])) + a.pro.norm_eps);
        if (it % CPR == 0) {
          Nk[it / CPR] = nkm[m];
          Nq[it / CPR] = nqm[m];
        }
      }
    }
    __syncthreads();
    float off = 0.f;
    for (int s2 = 0; s2 < s; ++s2) off += Tot[s2 * DK + c];
#pragma unroll
    for (int i = 0; i < RPS; ++i) Gl[(s * RPS + i) * LDG + c] = g[i] + off;
  }
  __syncthreads();
  if (tid < DK) reinterpret_cast<float*>(rec + R::g)[tid] = __expf(Gl[(C - 1) * LDG + tid]);
  // channels too strongly decayed inside a diagonal block for the anchor split:
  // thread (D, c) for D < 2; a wave covers 64 channels of one block
  if (tid < 2 * DK) {
    const int D = tid / DK, c = tid % DK, m = 32 * D + 15;
    const float gm = Gl[m * LDG + c];
    const bool out = Gl[32 * D * LDG + c] - gm > kSplitLimit || gm - Gl[(32 * D + 31) * LDG + c] > kSplitLimit;
    const unsigned long long bits = __ballot(out);
    if (lane == 0) {
      const int w0 = D * (DK / 32) + (c >> 5);
      Msk[w0] = (uint32_t)bits;
      Msk[w0 + 1] = (uint32_t)(bits >> 32);
    }
  }
  __syncthreads();

  // Three passes build operand tiles; after each, two waves take MFMA tiles:
  //   pass 0  rows 0..31, anchor 15    wave 0: A(0,0)   wave 1: P(0,0)
  //   pass 1  rows 32..63, anchor 47   wave 2: A(1,1)   wave 3: P(1,1)
  //   pass 2  anchor 31: j side rows 0..31, r side rows 32..63
  //                                    wave 0: A(1,0)   wave 1: P(1,0)
  // (tile (R, J): rows r of block R, columns j of block J).  Passes 0 and 1 also
  // write Kg, Qg and Kc.  Accumulators stay in registers until G is dead.
  // CMP: the A tile first; the Q operand waits in registers (yq) and then
  // takes the K operand's tile for the P tile.
  // Exact contributions of the channels left out of diagonal block D's MFMA
  // (the P tile with its Q rows when isp, else the A tile), onto acc.
  auto exact = [&](f32x16& acc, int D, bool isp) __attribute__((always_inline)) {
    const int r = 32 * D + col;
    const float xn = NORM ? (isp ? Nq[r] : Nk[r]) : 1.f;   // the rows are unscaled
    const E* xg = (isp ? qgl : kgl) + (size_t)min(r, cn - 1) * qk_tok;
#pragma unroll 1
    for (int wd = 0; wd < DK / 32; ++wd) {
      uint32_t bits = __builtin_amdgcn_readfirstlane(Msk[D * (DK / 32) + wd]);
      while (bits) {
        const int c = 32 * wd + __builtin_ctz(bits);
        bits &= bits - 1;
        const float gr = Gl[r * LDG + c];
        if constexpr (CMP) {   // the channel's K values of the block, one wave at a time
          if (lane < 32) Ksc[lane] = (float)kgl[(size_t)min(32 * D + lane, cn - 1) * qk_tok + c];
          __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's own row is written
        }
        float xv = (float)(CMP ? xg[c] : (isp ? Qraw : Kraw)[col * LDK + c]) * xn;
        // G2, A tiles: the row side is the erase direction; its gate comes
        // from HBM (a channel taking this path is rare)
        if (G2 && !isp) xv *= (float)bgl[(size_t)min(r, cn - 1) * qk_tok + c];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int jl = acc_row(v >> 2, v & 3, lane), j = 32 * D + jl;
          const float w = __expf(fminf(gr - Gl[j * LDG + c], 0.f)) * (NORM ? Nk[j] : 1.f);
          const float kj = CMP ? Ksc[jl] : (float)Kraw[jl * LDK + c];
          const float t = xv * kj * w;
          acc[v] += j <= r ? t : 0.f;
        }
      }
    }
  };
  f32x16 acc0 = zero16(), acc1 = zero16();
#pragma unroll
  for (int pass = 0; pass < 3; ++pass) {
    if (pass > 0) __syncthreads();   // the previous pass's tiles are consumed
    u32x4 yq[IPT];                   // (CMP) the r-side Q operand pieces of this pass
#pragma unroll
    for (int m = (pass == 1 ? IPT : 0); m < (pass == 0 ? IPT : 2 * IPT); ++m) {
      const int it = tid + kThreads * m, r = it / CPR, c0 = (it % CPR) * EPC;
      float kf[EPC], qf[EPC], gr[EPC], ga[EPC], x[EPC], y[EPC], z[EPC];
      const u32x4 kraw = kreg[m];
      const u32x4 qraw = qreg[m];
      unpack16<E>(kraw, kf);
      unpack16<E>(qraw, qf);
      // the row side of A and Kg: the key, or (G2) the erase direction b * k
      float ef[EPC];
      if constexpr (G2) {
        unpack16<E>(breg[m], ef);
#pragma unroll
        for (int e = 0; e < EPC; ++e) ef[e] *= kf[e];
      }
      if constexpr (NORM) {
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          kf[e] *= nkm[m];
          qf[e] *= nqm[m];
        }
      }
      const int anchor = pass == 2 ? 31 : (pass == 0 ? 15 : 47);
#pragma unroll
      for (int e = 0; e < EPC; e += 4) {
        const float4 g4 = *reinterpret_cast<const float4*>(Gl + r * LDG + c0 + e);
        const float4 a4 = *reinterpret_cast<const float4*>(Gl + anchor * LDG + c0 + e);
        gr[e] = g4.x; gr[e + 1] = g4.y; gr[e + 2] = g4.z; gr[e + 3] = g4.w;
        ga[e] = a4.x; ga[e + 1] = a4.y; ga[e + 2] = a4.z; ga[e + 3] = a4.w;
      }
      if (pass < 2) {
        float gl[EPC];
#pragma unroll
        for (int e = 0; e < EPC; e += 4) {
          const float4 l4 = *reinterpret_cast<const float4*>(Gl + (C - 1) * LDG + c0 + e);
          gl[e] = l4.x; gl[e + 1] = l4.y; gl[e + 2] = l4.z; gl[e + 3] = l4.w;
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const float w = __expf(gr[e]);
          x[e] = (G2 ? ef[e] : kf[e]) * w;
          y[e] = qf[e] * w;
          z[e] = kf[e] * __expf(gl[e] - gr[e]);
        }
        const size_t ro = (size_t)r * DK + c0;
        st_once(rec + R::kg + ro, pack16<E>(x));
        st_once(rec + R::qg + ro, pack16<E>(y));
        st_once(rec + R::kc + ro, pack16<E>(z));
      }
      const int lr = r & 31;
      // diagonal blocks: channels outside the split take zero operands
      uint32_t keep = ~0u;
      if (pass < 2) {
        if constexpr (!CMP) {
          *reinterpret_cast<u32x4*>(Kraw + lr * LDK + c0) = kraw;
          *reinterpret_cast<u32x4*>(Qraw + lr * LDK + c0) = qraw;
        }
        keep = ~(Msk[pass * (DK / 32) + (c0 >> 5)] >> (c0 & 31));
      }
      if (pass < 2 || r >= 32) {   // r side: exp(G_r - G_m)
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          const float w = __expf(gr[e] - ga[e]);
          const bool k1 = (keep >> e) & 1u;
          x[e] = k1 ? (G2 ? ef[e] : kf[e]) * w : 0.f;
          y[e] = k1 ? qf[e] * w : 0.f;
        }
        *reinterpret_cast<u32x4*>(Rop + lr * LDK + c0) = pack16<E>(x);
        if constexpr (CMP) yq[m % IPT] = pack16<E>(y);
        else *reinterpret_cast<u32x4*>(Qop + lr * LDK + c0) = pack16<E>(y);
      }
      if (pass < 2 || r < 32) {    // j side: exp(G_m - G_j)
#pragma unroll
        for (int e = 0; e < EPC; ++e) z[e] = ((keep >> e) & 1u) ? kf[e] * __expf(ga[e] - gr[e]) : 0.f;
        *reinterpret_cast<u32x4*>(Cop + lr * LDK + c0) = pack16<E>(z);
      }
    }
    __syncthreads();
    // tile (R, J) accumulates rows j (Cop) x columns r (Rop or Qop)
    const bool mine = pass == 2 ? wave < 2 : (wave >> 1) == pass;
    f32x16& acc = pass == 2 ? acc1 : acc0;
    if constexpr (CMP) {
      if (mine && !(wave & 1)) {
        tile_nt_k<DK / 16>(acc, Cop, LDK, Rop, LDK, lane);
        if (pass < 2) exact(acc, pass, false);
      }
      __syncthreads();   // the K operand is consumed: the Q operand takes its tile
#pragma unroll
      for (int m = (pass == 1 ? IPT : 0); m < (pass == 0 ? IPT : 2 * IPT); ++m) {
        const int it = tid + kThreads * m, r = it / CPR, c0 = (it % CPR) * EPC;
        if (pass < 2 || r >= 32) *reinterpret_cast<u32x4*>(Rop + (r & 31) * LDK + c0) = yq[m % IPT];
      }
      __syncthreads();
      if (mine && (wave & 1)) {
        tile_nt_k<DK / 16>(acc, Cop, LDK, Rop, LDK, lane);
        if (pass < 2) exact(acc, pass, true);
      }
    } else {
      if (mine) tile_nt_k<DK / 16>(acc, Cop, LDK, (wave & 1) ? Qop : Rop, LDK, lane);
      if (pass < 2 && mine) exact(acc, pass, wave & 1);
    }
  }
  __syncthreads();   // G is dead: A and P take region 1

  // Epilogues.  A[r][j] = beta_r acc for j < r; P[r][j] = acc for j <= r.
  {
    const bool isP = wave & 1;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (t == 1 && wave >= 2) break;
      const int Rb = t == 1 ? 1 : (wave >> 1), Jb = t == 1 ? 0 : (wave >> 1);
      const f32x16& acc = t == 1 ? acc1 : acc0;
      const int r = Rb * 32 + col;
      const float br = Bt[r];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = Jb * 32 + acc_row(g, 0, lane);
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float v = acc[4 * g + e];
          x[e] = isP ? (j0 + e <= r ? v : 0.f) : (j0 + e < r ? br * v : 0.f);
        }
        if (isP) {
          store4(Pm + r * LDT + j0, x[0], x[1], x[2], x[3]);
        } else {
          store4(Am + r * LDA + j0, x[0], x[1], x[2], x[3]);
          if (a.a_tilde) {   // (the backward) At itself, without beta
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = j0 + e < r ? acc[4 * g + e] : 0.f;
            *reinterpret_cast<float4*>(a.a_tilde + (at.sp.rec0 + n) * (size_t)(C * C) + r * C + j0) =
                make_float4(y[0], y[1], y[2], y[3]);
          }
        }
      }
    }
    if (a.a_tilde && wave == 2) {   // At rows 0..31, columns 32..63 are zero
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *reinterpret_cast<float4*>(a.a_tilde + (at.sp.rec0 + n) * (size_t)(C * C) + col * C + 32 +
                                   acc_row(g, 0, lane)) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (wave >= 2) {   // P rows 0..31, columns 32..63 are zero
      const int q = tid - 128, r = q >> 2, j0 = 32 + 8 * (q & 3);
      store4(Pm + r * LDT + j0, 0.f, 0.f, 0.f, 0.f);
      store4(Pm + r * LDT + j0 + 4, 0.f, 0.f, 0.f, 0.f);
    }
  }
  __syncthreads();

  // T (CMP: in place, straight to the record) and P -> the record, 64 x 64
  // contiguous each, 16-byte stores
  if constexpr (CMP)
    tri_solve<E, LDA, true, true>(Am, Am, Am + 32, Bt, rec + R::t, tid);
  else
    tri_solve<E, SolveLd<E>::LDM, false, true>(Am, Li, Mt, Bt, Tm, tid);
  {
    constexpr int CPT = C / EPC;
    for (int q = tid; q < C * CPT; q += kThreads) {
      const int r = q / CPT, cc = q % CPT;
      if constexpr (!CMP)
        st_once(rec + R::t + r * C + cc * EPC, *reinterpret_cast<const u32x4*>(Tm + r * LDT + cc * EPC));
      st_once(rec + R::p + r * C + cc * EPC, *reinterpret_cast<const u32x4*>(Pm + r * LDT + cc * EPC));
    }
  }
}

// ---------------------------------------------------------------------------
// chunk_state_kernel: the sequential pass over the chunks of one (b, h, slice).
// ---------------------------------------------------------------------------
// LDS plan.  Lifetimes inside one chunk step:
//   Kr    K rows [64][LDK]               commit .. phase 1
//   Qr    Q rows [64][LDK]               commit .. phase 1
//   Kt    K^T    [DK][LDT]               commit (or after phase 1) .. phase 6
//         (fp32 with d_k = 128: shares Q's region to fit in 160 KiB)
//   Sb    state copy S[i][c] [DVS][LDSB] phase 6 .. next phase 1
//   Vt    V^T slice [DVS][LDT]           commit .. phase 1
//   Xt    X^T slice [DVS][LDT]           phase 1 .. phase 4; then O staging
//   Pm    P [64][LDT]                    phase 1 .. phase 5
//   Tm    T [64][LDT]                    commit .. phase 4
//   Ut, Uw  [DVS][LDT] each              phase 4 .. phase 6
//   G, Eg, Ec  64 fp32 each              commit .. phase 6
template <typename E, int DK, int DVS, bool SEPKT>
struct StatePlan {
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = DK + PAD;
  static constexpr int LDT = C + PAD;
  static constexpr int LDSB = DK + PAD;
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
  static constexpr size_t ut = tm + (size_t)C * LDT * es;
  static constexpr size_t uw = ut + (size_t)DVS * LDT * es;
  static constexpr size_t g = uw + (size_t)DVS * LDT * es;
  static constexpr size_t total = g + 4 * C * 4;   // gate rows 0..3 (or DK per-channel values)
};

template <typename E, int DK, int DVS>
constexpr bool sep_kt_fits() {
  return StatePlan<E, DK, DVS, true>::total <= 160 * 1024;
}

// Element e of four 16-byte chunks (four consecutive rows), stored as four
// consecutive elements: the transpose used to build K^T and V^T.
__device__ inline void store_col4(__bf16* dst, const u32x4& r0, const u32x4& r1, const u32x4& r2,
                                  const u32x4& r3, int e) {
  const int w = e >> 1;
  const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
  const uint32_t lo = __builtin_amdgcn_perm(word_of(r1, w), word_of(r0, w), sel);
  const uint32_t hi = __builtin_amdgcn_perm(word_of(r3, w), word_of(r2, w), sel);
  *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
}
__device__ inline void store_col4(float* dst, const u32x4& r0, const u32x4& r1, const u32x4& r2,
                                  const u32x4& r3, int e) {
  *reinterpret_cast<u32x4*>(dst) = u32x4{word_of(r0, e), word_of(r1, e), word_of(r2, e), word_of(r3, e)};
}

template <typename E, int DK, int DVS, int MODE>
__global__ __launch_bounds__(kThreads) void chunk_state_kernel(PrefillArgs a, const E* __restrict__ tws) {
  constexpr bool SEPKT = sep_kt_fits<E, DK, DVS>();
  constexpr bool KDA = MODE >= 2;   // per-channel decay: operands come pre-scaled
  constexpr bool G2 = MODE == 3;    // Gated DeltaNet-2: V is scaled by the write gate
  using L = StatePlan<E, DK, DVS, SEPKT>;
  using R = typename RecOf<E, DK, MODE>::type;
  static_assert(L::total <= 160 * 1024, "LDS plan exceeds 160 KiB");
  constexpr int NI = DVS / 32;       // 32-wide value blocks in the slice
  constexpr int NC = DK / 32;        // 32-wide key blocks
  constexpr int NT = NC * NI;        // state tiles
  constexpr int NST = (NT + 3) / 4;  // state tiles per wave
  constexpr int EPC = 16 / (int)sizeof(E);  // elements per 16-byte chunk
  constexpr int LDK = L::LDK, LDT = L::LDT, LDSB = L::LDSB;
  // prefetch geometry: blocks of 4 rows x one 16-byte chunk (blk_row / blk_col)
  constexpr int CPR = DK / EPC;              // chunks per q/k row
  constexpr int NKB = 16 * CPR;              // 4-row blocks per q/k tile
  constexpr int KBT = (NKB + kThreads - 1) / kThreads;
  constexpr int CPV = DVS / EPC;             // chunks per v row (slice)
  constexpr int NVB = 16 * CPV;
  constexpr int VBT = (NVB + kThreads - 1) / kThreads;
  constexpr int CPT = C / EPC;               // chunks per T row
  constexpr int TBT = C * CPT / kThreads;    // T chunks per thread

  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  E* Kr = reinterpret_cast<E*>(smem + L::kr);
  E* Qr = reinterpret_cast<E*>(smem + L::qr);
  E* Kt = reinterpret_cast<E*>(smem + L::kt);
  E* Sb = reinterpret_cast<E*>(smem + L::sb);
  E* Vt = reinterpret_cast<E*>(smem + L::vt);
  E* Xt = reinterpret_cast<E*>(smem + L::xt);
  E* Pm = reinterpret_cast<E*>(smem + L::pm);
  E* Tm = reinterpret_cast<E*>(smem + L::tm);
  E* Ut = reinterpret_cast<E*>(smem + L::ut);
  E* Uw = reinterpret_cast<E*>(smem + L::uw);
  float* G = reinterpret_cast<float*>(smem + L::g);   // gate rows 0..3 of the record
  float* Eg = G + C;       // exp(G_r) nk_r
  float* Ec = G + 2 * C;   // exp(G_C - G_r) nk_r
  float* Eo = G + 3 * C;   // exp(G_r) nq_r
  float* Gc = G;           // per-channel decay: exp(G_C[c]), DK values
  // O staging (rows r, OST elements apart) reuses X^T's region, free after phase 4
  constexpr int OST = (sizeof(E) == 2 && DVS == 64) ? 72 : DVS;
  static_assert(C * OST <= DVS * LDT, "O staging does not fit in the X^T region");
  E* Os = Xt;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31;
  const int H = a.H, dv = a.dv;
  const int nsl = dv / DVS;
  const int nheads = a.B * H;
  // Workgroups are dispatched round-robin over the eight XCDs: give the slices
  // of one head the same XCD (same L2) when the head count allows it.
  int head, sl;
  if ((nheads & 7) == 0) {
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    head = xcd + 8 * (j / nsl);
    sl = j % nsl;
  } else {
    head = blockIdx.x / nsl;
    sl = blockIdx.x % nsl;
  }
  const int h = head % H, b = head / H;
  const int i0 = sl * DVS;
  const Span sp = seq_span(a, b, h);
  const int T = sp.len;   // tokens of this sequence
  const int nchunks = (T + C - 1) / C;

  const size_t qk_tok = (size_t)H * DK;   // stride between tokens in q, k
  const size_t v_tok = (size_t)H * dv;    // stride between tokens in v, o
  const E* qg = static_cast<const E*>(a.q) + (sp.tok0 * H + h) * DK;
  const E* kg = static_cast<const E*>(a.k) + (sp.tok0 * H + h) * DK;
  const E* vg = static_cast<const E*>(a.v) + (sp.tok0 * H + h) * dv + i0;
  const E* wg = G2 ? static_cast<const E*>(a.write) + (sp.tok0 * H + h) * dv + i0 : nullptr;
  const E* recs = tws + sp.rec0 * R::elems;   // per-chunk records
  E* og = static_cast<E*>(a.o) + (sp.tok0 * H + h) * dv + i0;
  const size_t sbase = ((size_t)b * H + h) * dv + i0;  // first state row of the slice

  // Tile ownership: X, O_inter (phase 1), U (phase 4) and O (phase 5) tiles of
  // row block own_rb and value block own_ib belong to one wave.
  int own_rb = -1, own_ib = 0;
  if (NI == 2) {
    own_rb = wave >> 1;
    own_ib = wave & 1;
  } else if (wave < 2) {
    own_rb = wave;
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

  // ---- prefetch registers ----
  // Loads are unconditional, so the compiler keeps them in flight across the
  // chunk.  Rows past the sequence end re-read its last row: T's rows and
  // columns of those tokens are zero (their beta is zero), so they never reach
  // U, O or S, and their O rows are not written.
  u32x4 pk[KBT][4], pq[KBT][4], pv[VBT][4], pt[TBT];
  u32x4 pw[G2 ? VBT : 1][4];   // write-gate rows (G2)
  u32x4 pg = u32x4{0u, 0u, 0u, 0u};   // gate block: rows 0..3, threads 0..63 (gC: DK / 4)
  u32x4 pkc[KDA && SEPKT ? KBT : 1][4], pp[TBT];   // Kc rows (per-channel decay) and P

  auto prefetch = [&](int n) __attribute__((always_inline)) {
    const int t0 = n * C;
    const int rmax = min(C, T - t0) - 1;
    const E* vq = vg + (size_t)t0 * v_tok;
    if constexpr (KDA) {
      // every row of a record is written (rows past the end are finite copies)
      const E* rq = recs + (size_t)n * R::elems;
#pragma unroll
      for (int m = 0; m < KBT; ++m) {
        const int blk = tid + kThreads * m;
        const int bq = blk < NKB ? blk : 0;
        const int rb4 = blk_row(bq, CPR), cc = blk_col(bq, CPR);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t off = (uint32_t)(4 * rb4 + rr) * DK + cc * EPC;
          pk[m][rr] = *reinterpret_cast<const u32x4*>(rq + R::kg + off);
          pq[m][rr] = *reinterpret_cast<const u32x4*>(rq + R::qg + off);
          if constexpr (SEPKT) pkc[m][rr] = *reinterpret_cast<const u32x4*>(rq + R::kc + off);
        }
      }
    } else {
      const E* kq = kg + (size_t)t0 * qk_tok;
      const E* qq = qg + (size_t)t0 * qk_tok;
#pragma unroll
      for (int m = 0; m < KBT; ++m) {
        const int blk = tid + kThreads * m;
        const int bq = blk < NKB ? blk : 0;
        const int rg = blk_row(bq, CPR), cc = blk_col(bq, CPR);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const uint32_t off = (uint32_t)min(4 * rg + rr, rmax) * (uint32_t)qk_tok + cc * EPC;
          pk[m][rr] = *reinterpret_cast<const u32x4*>(kq + off);
          pq[m][rr] = *reinterpret_cast<const u32x4*>(qq + off);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < VBT; ++m) {
      const int blk = tid + kThreads * m;
      const int bq = blk < NVB ? blk : 0;
      const int rg = blk_row(bq, CPV), cc = blk_col(bq, CPV);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const uint32_t off = (uint32_t)min(4 * rg + rr, rmax) * (uint32_t)v_tok + cc * EPC;
        pv[m][rr] = ld_once(vq + off);
        if constexpr (G2) pw[m][rr] = ld_once(wg + (size_t)t0 * v_tok + off);
      }
    }
    {
      const E* rq = recs + (size_t)n * R::elems;
#pragma unroll
      for (int m = 0; m < TBT; ++m) {
        pt[m] = *reinterpret_cast<const u32x4*>(rq + R::t + (tid + kThreads * m) * EPC);
        pp[m] = *reinterpret_cast<const u32x4*>(rq + R::p + (tid + kThreads * m) * EPC);
      }
      constexpr int NG4 = (KDA ? DK : 4 * C) / 4;   // 16-byte chunks of the fp32 rows used
      pg = *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(rq + R::g) + 4 * min(tid, NG4 - 1));
    }
  };

  auto commit = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < KBT; ++m) {
      const int blk = tid + kThreads * m;
      if (blk < NKB) {
        const int rg = blk_row(blk, CPR), cc = blk_col(blk, CPR);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          *reinterpret_cast<u32x4*>(Kr + (4 * rg + rr) * LDK + cc * EPC) = pk[m][rr];
          *reinterpret_cast<u32x4*>(Qr + (4 * rg + rr) * LDK + cc * EPC) = pq[m][rr];
        }
        if constexpr (SEPKT) {
          const auto& src = KDA ? pkc[m] : pk[m];
#pragma unroll
          for (int e = 0; e < EPC; ++e)
            store_col4(Kt + (cc * EPC + e) * LDT + 4 * rg, src[0], src[1], src[2], src[3], e);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < VBT; ++m) {
      const int blk = tid + kThreads * m;
      if (blk < NVB) {
        const int rg = blk_row(blk, CPV), cc = blk_col(blk, CPV);
        if constexpr (G2) {   // z = w * v
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) pv[m][rr] = mul16<E>(pv[m][rr], pw[m][rr]);
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          store_col4(Vt + (cc * EPC + e) * LDT + 4 * rg, pv[m][0], pv[m][1], pv[m][2], pv[m][3], e);
      }
    }
#pragma unroll
    for (int m = 0; m < TBT; ++m) {
      const int q = tid + kThreads * m, r = q / CPT, cc = q % CPT;
      *reinterpret_cast<u32x4*>(Tm + r * LDT + cc * EPC) = pt[m];
      *reinterpret_cast<u32x4*>(Pm + r * LDT + cc * EPC) = pp[m];
    }
    if (tid < (KDA ? DK / 4 : C)) *reinterpret_cast<u32x4*>(G + 4 * tid) = pg;
  };

  // Staged O rows of a chunk -> HBM, 16-byte stores along each row.
  auto flush_o = [&](int t0f, int cnf) __attribute__((always_inline)) {
    constexpr int CPO = DVS / EPC;
    E* oq = og + (size_t)t0f * v_tok;
    for (int q = tid; q < C * CPO; q += kThreads) {
      const int r = q / CPO, cc = q % CPO;
      if (r < cnf)
        st_once(oq + (uint32_t)r * (uint32_t)v_tok + cc * EPC, *reinterpret_cast<const u32x4*>(Os + r * OST + cc * EPC));
    }
  };

  // Iteration -1 only issues the first prefetch (one call site per helper keeps
  // the prefetch registers in registers).  Later prefetches are issued at the
  // start of phase 1, where the memory pipe works under the MFMA chains.
  for (int n = -1; n < nchunks; ++n) {
    if (n >= 0) {
      __syncthreads();   // every reader of the previous chunk's buffers is done
      if (n > 0) flush_o((n - 1) * C, C);
      commit();
      __syncthreads();
    }
    if (n + 1 < nchunks) prefetch(n + 1);
    if (n < 0) continue;

    // ---- phase 1: X and O_inter tiles (they share the S operand) ----
    f32x16 xacc = zero16(), oacc = zero16();
    if (own_rb >= 0)
      tile_nt2_shared_b<DK / 16>(xacc, oacc, Kr + own_rb * 32 * LDK, Qr + own_rb * 32 * LDK, LDK, LDK,
                                 Sb + own_ib * 32 * LDSB, LDSB, lane);
    if (own_rb >= 0) {
      const int i = own_ib * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = own_rb * 32 + acc_row(g, 0, lane);
        const float4 eg = KDA ? make_float4(1.f, 1.f, 1.f, 1.f) : *reinterpret_cast<const float4*>(Eg + r0);
        const float4 eo = KDA ? make_float4(1.f, 1.f, 1.f, 1.f) : *reinterpret_cast<const float4*>(Eo + r0);
        const float4 v4 = load4_elem(Vt + i * LDT + r0);
        store4(Xt + i * LDT + r0, v4.x - eg.x * xacc[4 * g + 0], v4.y - eg.y * xacc[4 * g + 1],
               v4.z - eg.z * xacc[4 * g + 2], v4.w - eg.w * xacc[4 * g + 3]);
        oacc[4 * g + 0] *= eo.x;
        oacc[4 * g + 1] *= eo.y;
        oacc[4 * g + 2] *= eo.z;
        oacc[4 * g + 3] *= eo.w;
      }
    }
    __syncthreads();

    // ---- K^T for phase 6 when it shares Q's region (fp32, d_k = 128) ----
    if constexpr (!SEPKT) {
      for (int blk = tid; blk < NKB; blk += kThreads) {
        const int rg4 = blk_row(blk, CPR), cc = blk_col(blk, CPR);
        u32x4 v[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          if constexpr (KDA) {   // per-channel decay: the decay-scaled Kc rows
            const E* kcq = recs + (size_t)n * R::elems + R::kc;
            v[rr] = *reinterpret_cast<const u32x4*>(kcq + (4 * rg4 + rr) * DK + cc * EPC);
          } else {
            v[rr] = *reinterpret_cast<const u32x4*>(Kr + (4 * rg4 + rr) * LDK + cc * EPC);
          }
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e)
          store_col4(Kt + (cc * EPC + e) * LDT + 4 * rg4, v[0], v[1], v[2], v[3], e);
      }
    }

    // ---- phase 4: U = T X; store U^T and the decay-weighted copy for the state ----
    if (own_rb >= 0) {
      f32x16 uacc = zero16();
      if (own_rb == 0) tile_nt_k<2>(uacc, Tm, LDT, Xt + own_ib * 32 * LDT, LDT, lane);
      else tile_nt_k<4>(uacc, Tm + 32 * LDT, LDT, Xt + own_ib * 32 * LDT, LDT, lane);
      const int i = own_ib * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int r0 = own_rb * 32 + acc_row(g, 0, lane);
        store4(Ut + i * LDT + r0, uacc[4 * g], uacc[4 * g + 1], uacc[4 * g + 2], uacc[4 * g + 3]);
        if constexpr (!KDA) {
          const float4 ec = *reinterpret_cast<const float4*>(Ec + r0);
          store4(Uw + i * LDT + r0, uacc[4 * g] * ec.x, uacc[4 * g + 1] * ec.y,
                 uacc[4 * g + 2] * ec.z, uacc[4 * g + 3] * ec.w);
        }
      }
    }
    __syncthreads();

    // ---- phase 5: O = O_inter + P U, staged in LDS (rows r, OST apart) ----
    if (own_rb >= 0) {
      if (own_rb == 0) tile_nt_k<2>(oacc, Pm, LDT, Ut + own_ib * 32 * LDT, LDT, lane);
      else tile_nt_k<4>(oacc, Pm + 32 * LDT, LDT, Ut + own_ib * 32 * LDT, LDT, lane);
      const int i = own_ib * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          Os[(own_rb * 32 + acc_row(g, e, lane)) * OST + i] = to_elem<E>(oacc[4 * g + e]);
    }

    // ---- phase 6: S^T <- gamma_C S^T + K^T Uw  (fp32 accumulators), refresh Sb ----
    // (per-channel decay: S^T <- Diag(gC) S^T + Kc^T U)
    {
      if constexpr (KDA) {
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const int cb = (wave + 4 * st) / NI;
          if (cb < NC) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const float4 d = *reinterpret_cast<const float4*>(Gc + cb * 32 + acc_row(g, 0, lane));
              Sacc[st][4 * g + 0] *= d.x;
              Sacc[st][4 * g + 1] *= d.y;
              Sacc[st][4 * g + 2] *= d.z;
              Sacc[st][4 * g + 3] *= d.w;
            }
          }
        }
      } else {
        const float gC = __expf(G[C - 1]);
#pragma unroll
        for (int st = 0; st < NST; ++st)
#pragma unroll
          for (int v = 0; v < 16; ++v) Sacc[st][v] *= gC;
      }
      const E* Ub = KDA ? Ut : Uw;
      if (NST == 2 && wave + 4 < NT) {
        // tiles wave and wave + 4 share the value block: one Uw fragment, two MFMAs
        tile_nt2_shared_b<C / 16>(Sacc[0], Sacc[NST - 1], Kt + (wave / NI) * 32 * LDT,
                                  Kt + ((wave + 4) / NI) * 32 * LDT, LDT, LDT,
                                  Ub + (wave % NI) * 32 * LDT, LDT, lane);
      } else {
#pragma unroll
        for (int st = 0; st < NST; ++st) {
          const int t = wave + 4 * st;
          if (t < NT)
            tile_nt_k<C / 16>(Sacc[st], Kt + (t / NI) * 32 * LDT, LDT, Ub + (t % NI) * 32 * LDT,
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
  if (nchunks > 0) {
    __syncthreads();
    flush_o((nchunks - 1) * C, T - (nchunks - 1) * C);
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

// ---------------------------------------------------------------------------
// chunk_state_ws: the sequential pass in bf16 with eight waves.
// ---------------------------------------------------------------------------
// Waves 0-3 carry the state chain; waves 4-7 move data: while the chain works
// on chunk n they load later chunks from HBM into registers, write each LDS
// buffer in an interval in which nobody reads it, and write the staged O rows
// out.  (Issuing the loads costs the compute unit about 40 bytes per clock;
// here it runs beside the MFMA chain instead of inside it.)
//
// Every buffer the data waves fill is row-major, written with 16-byte stores.
// Where the chain needs a column-wise operand (K^T of the state update, V in
// the X epilogue) it reads the rows with gfx950's transposed LDS read.
//
// Scalar or no decay: three data waves form P = (Q K^T masked, times
// exp(G_r - G_j)) for chunk n + 1 from the K and Q rows in LDS while the chain
// is in interval B of chunk n (the per-channel P comes with the record).
//
// The chain wave of row block rb and value block ib computes the X and the
// O_inter^T tiles (rb, ib) in phase 1 (both from one S fragment, which serves
// as the B operand of X = K S^T and the A operand of O^T = S Q^T).  After one
// barrier every chain wave computes U for the value block of its state tiles,
// both row blocks, and keeps it in registers: a 32x32 accumulator tile is an
// operand of the next product as it stands (frag_acc, with the other operand
// read in the matching k order), so O^T += U^T P^T and the state update take U
// and the decay-weighted U straight from the accumulators.  O is staged
// transposed-back in LDS with 8-byte stores.  Two barriers per chunk:
//   interval  chain waves                          data waves
//   A         phase 1: X, O_inter^T (X^T -> LDS)   K, Q, V rows, gates of n+1;
//                                                  T (per-channel: P) of n;
//                                                  O(n-1) -> HBM; load K,
//                                                  gates of n+2
//   B         U = T X; O^T += U^T P^T (staged);    load T (P) of n+1, Q, V of
//             S^T <- decay S^T + K^T Uw            n+2; P of n+1 (scalar)
// The row buffers are double-buffered (those of n+1 are written while the
// chain reads those of n); O has a staging buffer of its own.  The chain
// issues all LDS fragment loads of interval B before its first MFMA there.
// The two roles run separate loops with the same barrier count, so their
// registers do not add up.
template <typename E, int DK, int DVS, bool KDA, bool NORM>
struct WsPlan {
  static constexpr int PAD = 16 / (int)sizeof(E);
  static constexpr int LDK = DK + PAD;
  // The state update's K rows are also read transposed: a row stride of 16
  // mod 64 dwords, with row-swizzled chunks, serves both read shapes.
  static constexpr int LDKS = DK + 32;
  static constexpr int LDT = C + PAD;
  static constexpr int LDSB = DK + PAD;
  static constexpr int LDV = DVS + 16;   // 4-row transposed reads fall in fewer banks
  // P and the O staging rows are accessed 8 bytes per lane, a row per lane:
  // a row stride of 2 mod 4 dwords puts 32 rows in distinct banks.
  static constexpr int LDP = C + 4;
  static constexpr int OST = DVS + 4;
  static constexpr size_t es = sizeof(E);
  static constexpr size_t rows = (size_t)C * LDK * es;     // one [C][LDK] row buffer
  static constexpr size_t srows = (size_t)C * LDKS * es;   // one [C][LDKS] row buffer
  static constexpr size_t vrows = (size_t)C * LDV * es;    // one [C][LDV] V buffer
  static constexpr size_t pmat = (size_t)C * LDP * es;     // one [C][LDP] P matrix
  // Q rows, the state update's K rows and (per-channel) the phase-1 K rows, V
  // rows, the gates: two buffers each (n and n + 1).  P: two buffers when the
  // data waves form it during the chain's use of the previous one.
  // Per-channel decay with 64-row slices: one buffer each for Q and the
  // phase-1 K rows, which only phase 1 reads (the data waves write those of
  // n + 1 while the chain runs interval B of n).
  static constexpr bool single = KDA && DVS == 64;
  static constexpr size_t qr = 0;
  static constexpr size_t ks = qr + (single ? 1 : 2) * rows;
  static constexpr size_t kr = ks + 2 * srows;
  static constexpr size_t sb = kr + (KDA ? (single ? 1 : 2) * rows : 0);
  static constexpr size_t vr = sb + (size_t)DVS * LDSB * es;
  static constexpr size_t xt = vr + 2 * vrows;
  static constexpr size_t os = xt + (size_t)DVS * LDT * es;
  static constexpr size_t pm = os + (size_t)C * OST * es;
  static constexpr size_t tm = pm + (KDA ? 1 : 2) * pmat;
  static constexpr size_t g = tm + (size_t)C * LDT * es;
  // per buffer: gate rows 0..2 of the record (normalised q, k: rows 0..4 and
  // the chunk's inverse Q norms); per-channel: exp(G_C), DK values
  static constexpr int gstride = NORM ? 6 * C : 3 * C;
  static_assert(DK <= 3 * C, "per-channel decay row must fit a gate buffer");
  static constexpr size_t total = g + 2 * (size_t)gstride * 4;
};

constexpr int kWsThreads = 512;
constexpr int kP1Ahead = 2;   // phase-1 fragments loaded this many k steps ahead
constexpr int kFormPAhead = 2;   // fragments of P's product loaded this many k steps ahead

// One workgroup's share of a value slice: a lead-in over chunks [lead0, n_so)
// that runs the state recurrence alone (no Q, P or O), with the same products
// in the same order as the full pass, then the full pass over [n_so, n_end).
// The lead-in starts from S0 when lead0 = 0, else from a zero state; the last
// part of the slice writes S_final.  smem holds WsPlan::total bytes.
template <typename E, int DK, int DVS, int MODE, bool NORM>
__device__ __forceinline__ void state_ws_body(const PrefillArgs& a, const E* __restrict__ tws,
                                              unsigned char* __restrict__ smem, int head, int sl, const Span& sp,
                                              bool last, int lead0, int n_so, int n_end) {
  static_assert(sizeof(E) == 2, "the eight-wave kernel is bf16");
  constexpr bool KDA = MODE >= 2;
  constexpr bool G2 = MODE == 3;   // Gated DeltaNet-2: V is scaled by the write gate
  static_assert(!(KDA && NORM), "per-channel records carry normalised operands already");
  using L = WsPlan<E, DK, DVS, KDA, NORM>;
  constexpr int GS = L::gstride;
  static_assert(L::total <= 160 * 1024, "LDS plan exceeds 160 KiB");
  using R = typename RecOf<E, DK, MODE>::type;
  constexpr int NI = DVS / 32;       // 32-wide value blocks in the slice
  constexpr int NC = DK / 32;        // 32-wide key blocks
  constexpr int NT = NC * NI;        // state tiles
  constexpr int NST = (NT + 3) / 4;  // state tiles per chain wave
  constexpr int EPC = 8;
  constexpr int LDK = L::LDK, LDKS = L::LDKS, LDT = L::LDT, LDSB = L::LDSB, LDV = L::LDV, LDP = L::LDP,
                OST = L::OST;
  // data-wave geometry (256 threads): every row buffer in 16-byte pieces,
  // consecutive threads along a row (coalesced loads, conflict-free writes)
  constexpr int PT = 256;
  constexpr int CPR = DK / EPC;
  constexpr int KPT = C * CPR / PT;
  static_assert(C * CPR % PT == 0, "K rows must split evenly over the data threads");
  constexpr int CPV = DVS / EPC;
  constexpr int VPT = C * CPV / PT;
  static_assert(C * CPV % PT == 0, "V rows must split evenly over the data threads");
  constexpr int CPT = C / EPC;
  constexpr int TBT = C * CPT / PT;
  constexpr int NG4 = (KDA ? DK : (NORM ? 5 : 3) * C) / 4;   // 16-byte chunks of the fp32 rows

  // Buffer pairs are C * LDK (rows; C * LDKS for Ks), C * LDV (V), C * LDP (P) elements and
  // GS floats apart.
  E* Qrb = reinterpret_cast<E*>(smem + L::qr);
  E* Ksb = reinterpret_cast<E*>(smem + L::ks);   // K rows of the state update (K, or Kc), row-swizzled
  E* Krb = reinterpret_cast<E*>(smem + L::kr);   // per-channel: the K operand of phase 1
  E* Sb = reinterpret_cast<E*>(smem + L::sb);
  E* Vrb = reinterpret_cast<E*>(smem + L::vr);
  E* Xt = reinterpret_cast<E*>(smem + L::xt);
  E* Os = reinterpret_cast<E*>(smem + L::os);
  E* Pmb = reinterpret_cast<E*>(smem + L::pm);
  E* Tm = reinterpret_cast<E*>(smem + L::tm);
  float* Gbuf = reinterpret_cast<float*>(smem + L::g);  // gate rows (or gC rows)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, hh = lane >> 5;
  const int H = a.H, dv = a.dv;
  const int h = head % H, b = head / H;
  const int i0 = sl * DVS;
  const int T = sp.len;   // tokens of this sequence
  using Full = std::false_type;
  using Lead = std::true_type;
  const size_t v_tok = (size_t)H * dv;
  const size_t sbase = ((size_t)b * H + h) * dv + i0;

  if (wave >= 4) {
    // ======================= data waves =======================
    const int ptid = tid - 256;
    const size_t qk_tok = (size_t)H * DK;
    const E* qg = static_cast<const E*>(a.q) + (sp.tok0 * H + h) * DK;
    const E* kg = static_cast<const E*>(a.k) + (sp.tok0 * H + h) * DK;
    const E* vg = static_cast<const E*>(a.v) + (sp.tok0 * H + h) * dv + i0;
    const E* wg = G2 ? static_cast<const E*>(a.write) + (sp.tok0 * H + h) * dv + i0 : nullptr;
    const E* recs = tws + sp.rec0 * R::elems;
    E* og = static_cast<E*>(a.o) + (sp.tok0 * H + h) * dv + i0;

    u32x4 pk[KPT], pq[KPT], pv[VPT], pkc[KDA ? KPT : 1];   // rows of a chunk
    u32x4 pw[G2 ? VPT : 1];                                  // write-gate rows (G2)
    u32x4 pg = u32x4{0u, 0u, 0u, 0u};
    u32x4 pt[TBT], pp[KDA ? TBT : 1];                                // T (and P) of a chunk

    // The loads are split in two groups so that both intervals issue about
    // the same number of bytes: the K operands and the gates of chunk n, and
    // Q and V of chunk n (issued one chunk earlier).  Every thread issues the
    // same loads (surplus threads repeat a valid block), so the wait counts
    // the compiler derives are exact; rows past the sequence end re-read its
    // last row, whose T rows and columns are zero.
    // Row groups (parts): 1 the state update's K rows (K, or Kc), V and the
    // gates; 2 Q and the per-channel phase-1 K rows; 3 both.
    using AllRows = std::integral_constant<int, 3>;
    using RowsA = std::integral_constant<int, 1>;
    using RowsB = std::integral_constant<int, 2>;
    auto load_k = [&](int n, auto parts) __attribute__((always_inline)) {
      constexpr int PARTS = decltype(parts)::value;
      const int t0 = n * C;
      const int rmax = min(C, T - t0) - 1;
      const E* rq = recs + (size_t)n * R::elems;
      const E* kq = kg + (size_t)t0 * qk_tok;
#pragma unroll
      for (int m = 0; m < KPT; ++m) {
        const int q = ptid + PT * m, r = q / CPR, cc = q % CPR;
        if constexpr (KDA) {
          const uint32_t off = (uint32_t)r * DK + cc * EPC;
          if constexpr ((PARTS & 2) != 0) pk[m] = *reinterpret_cast<const u32x4*>(rq + R::kg + off);
          if constexpr ((PARTS & 1) != 0) pkc[m] = *reinterpret_cast<const u32x4*>(rq + R::kc + off);
        } else if constexpr ((PARTS & 1) != 0) {
          pk[m] = *reinterpret_cast<const u32x4*>(kq + (uint32_t)min(r, rmax) * (uint32_t)qk_tok + cc * EPC);
        }
      }
      if constexpr ((PARTS & 1) != 0)
        pg = *reinterpret_cast<const u32x4*>(reinterpret_cast<const float*>(rq + R::g) + 4 * min(ptid, NG4 - 1));
    };
    // (so: the lead-in, which needs no Q and no P)
    auto load_qv = [&](int n, auto so) __attribute__((always_inline)) {
      const int t0 = n * C;
      const int rmax = min(C, T - t0) - 1;
      const E* rq = recs + (size_t)n * R::elems;
      const E* qq = qg + (size_t)t0 * qk_tok;
#pragma unroll
      for (int m = 0; m < (decltype(so)::value ? 0 : KPT); ++m) {
        const int q = ptid + PT * m, r = q / CPR, cc = q % CPR;
        if constexpr (KDA)
          pq[m] = *reinterpret_cast<const u32x4*>(rq + R::qg + (uint32_t)r * DK + cc * EPC);
        else
          pq[m] = *reinterpret_cast<const u32x4*>(qq + (uint32_t)min(r, rmax) * (uint32_t)qk_tok + cc * EPC);
      }
      const E* vq = vg + (size_t)t0 * v_tok;
#pragma unroll
      for (int m = 0; m < VPT; ++m) {
        const int q = ptid + PT * m, r = q / CPV, cc = q % CPV;
        pv[m] = ld_once(vq + (uint32_t)min(r, rmax) * (uint32_t)v_tok + cc * EPC);
        if constexpr (G2)
          pw[m] = ld_once(wg + (size_t)t0 * v_tok + (uint32_t)min(r, rmax) * (uint32_t)v_tok + cc * EPC);
      }
    };
    auto load_tp = [&](int n, auto so) __attribute__((always_inline)) {
      const E* rq = recs + (size_t)n * R::elems;
#pragma unroll
      for (int m = 0; m < TBT; ++m) {
        pt[m] = *reinterpret_cast<const u32x4*>(rq + R::t + (ptid + PT * m) * EPC);
        if constexpr (KDA && !decltype(so)::value) pp[m] = *reinterpret_cast<const u32x4*>(rq + R::p + (ptid + PT * m) * EPC);
      }
    };
    // Rows of a chunk into buffer gb: Q, the state update's K operand (K, or
    // Kc), the per-channel phase-1 K operand, V, and the gates (the row groups
    // of load_k; single Q and phase-1 K buffers take buffer 0).
    auto commit_rows = [&](int gb, auto so, auto parts) __attribute__((always_inline)) {
      constexpr int PARTS = decltype(parts)::value;
      const int gq = L::single ? 0 : gb;
      E* Qr = Qrb + gq * C * LDK;
      E* Ks = Ksb + gb * C * LDKS;
      E* Kr = Krb + gq * C * LDK;
      E* Vr = Vrb + gb * C * LDV;
#pragma unroll
      for (int m = 0; m < KPT; ++m) {
        const int q = ptid + PT * m, r = q / CPR, cc = q % CPR;
        const int o = r * LDK + cc * EPC;
        if constexpr ((PARTS & 2) != 0 && !decltype(so)::value) *reinterpret_cast<u32x4*>(Qr + o) = pq[m];
        if constexpr ((PARTS & 1) != 0)
          *reinterpret_cast<u32x4*>(Ks + r * LDKS + swz_col(r, cc * EPC)) = KDA ? pkc[m] : pk[m];
        if constexpr (KDA && (PARTS & 2) != 0) *reinterpret_cast<u32x4*>(Kr + o) = pk[m];
      }
      if constexpr ((PARTS & 1) != 0) {
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
          const int q = ptid + PT * m, r = q / CPV, cc = q % CPV;
          *reinterpret_cast<u32x4*>(Vr + r * LDV + cc * EPC) = G2 ? mul16<E>(pv[m], pw[m]) : pv[m];
        }
        if (ptid < NG4) *reinterpret_cast<u32x4*>(Gbuf + gb * GS + 4 * ptid) = pg;
      }
    };
    // T (and the per-channel P) of a chunk.
    auto commit_tp = [&](auto so) __attribute__((always_inline)) {
#pragma unroll
      for (int m = 0; m < TBT; ++m) {
        const int q = ptid + PT * m, r = q / CPT, cc = q % CPT;
        *reinterpret_cast<u32x4*>(Tm + r * LDT + cc * EPC) = pt[m];
        if constexpr (KDA && !decltype(so)::value) {
          uint2* d = reinterpret_cast<uint2*>(Pmb + r * LDP + cc * EPC);
          d[0] = make_uint2(pp[m][0], pp[m][1]);
          d[1] = make_uint2(pp[m][2], pp[m][3]);
        }
      }
    };
    // P of the chunk in row buffers gb (scalar or no decay): data wave d < 3
    // takes the 32 x 32 tile (column block, row block) (0,0), (0,1), (1,1) of
    // P^T = K Q^T, so that each lane holds four consecutive columns j of one
    // row r: P[r][j] = exp(G_r - G_j) q_r.k_j for j <= r, else 0 (a select:
    // the weight of a masked entry may overflow).
    auto form_p = [&](int gb) __attribute__((always_inline)) {
      const int d = wave - 4;
      if (d >= 3) return;
      const int jb = d == 2 ? 1 : 0, rb = d == 0 ? 0 : 1;
      f32x16 acc = zero16();
      tile_nt_k<DK / 16, E, true, kFormPAhead>(acc, Ksb + gb * C * LDKS + jb * 32 * LDKS, LDKS,
                                  Qrb + gb * C * LDK + rb * 32 * LDK, LDK, lane);
      const float* Gl = Gbuf + gb * GS;
      E* Pm = Pmb + gb * C * LDP;
      const int r = rb * 32 + col;
      const float Gr = Gl[r];
      // Every weight is formed (clamped to at most 1) before the mask selects:
      // left conditional, the gate loads sink into per-element branches.
      // Normalised q and k: the column factor nk_j joins the exponent (the
      // record's row 4 holds G_j - ln nk_j; the clamp then only keeps masked
      // weights finite) and nq_r is applied to the output rows.
      constexpr int GJ = NORM ? 4 * C : 0;
      constexpr float WMAX = NORM ? 88.f : 0.f;
      float w[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 gj = *reinterpret_cast<const float4*>(Gl + GJ + jb * 32 + acc_row(g, 0, lane));
        w[4 * g + 0] = __expf(fminf(Gr - gj.x, WMAX));
        w[4 * g + 1] = __expf(fminf(Gr - gj.y, WMAX));
        w[4 * g + 2] = __expf(fminf(Gr - gj.z, WMAX));
        w[4 * g + 3] = __expf(fminf(Gr - gj.w, WMAX));
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) asm volatile("" ::"v"(w[v]));
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int j0 = jb * 32 + acc_row(g, 0, lane);
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = (j0 + e <= r) ? w[4 * g + e] * acc[4 * g + e] : 0.f;
        store4(Pm + r * LDP + j0, y[0], y[1], y[2], y[3]);
      }
    };
    // Staged O rows of a whole chunk -> HBM, 16-byte stores along each row.
    constexpr int CPO = DVS / EPC;
    auto os_piece = [&](int r, int cc) __attribute__((always_inline)) {   // rows are 8-byte aligned
      const uint2* p = reinterpret_cast<const uint2*>(Os + r * OST + cc * EPC);
      const uint2 lo = p[0], hi = p[1];
      return u32x4{lo.x, lo.y, hi.x, hi.y};
    };
    static_assert(C * CPO % PT == 0, "O rows must split evenly over the data threads");
    auto flush_o = [&](int t0f) __attribute__((always_inline)) {
      E* oq = og + (size_t)t0f * v_tok;
#pragma unroll
      for (int m = 0; m < C * CPO / PT; ++m) {
        const int q = ptid + PT * m, r = q / CPO, cc = q % CPO;
        st_once(oq + (uint32_t)r * (uint32_t)v_tok + cc * EPC, os_piece(r, cc));
      }
    };
    // One chunk step of a pass whose last chunk is nlast.  The LDS writes of
    // interval A use data loaded at least one interval earlier; the first step
    // (nothing to flush) is peeled so that no global access in the loop is
    // conditional.
    // With single Q and phase-1 K buffers, Q and the phase-1 K rows of n + 1
    // go in during interval B (phase 1 of n, their only reader, is over), and
    // the phase-1 K rows of n + 2 are loaded there once those of n + 1 are in.
    auto step = [&](int n, int nlast, auto first, auto so) __attribute__((always_inline)) {
      constexpr bool SO = decltype(so)::value;
      if constexpr (L::single) {
        // interval A: the chain runs phase 1 of chunk n
        if (n + 1 <= nlast) commit_rows((n + 1) & 1, so, RowsA{});
        commit_tp(so);                 // T (and P) of chunk n
        if constexpr (!SO && !decltype(first)::value) flush_o((n - 1) * C);
        load_k(min(n + 2, nlast), RowsA{});
        __syncthreads();
        // interval B: the chain runs U, O and S of chunk n
        if (n + 1 <= nlast) commit_rows((n + 1) & 1, so, RowsB{});
        load_tp(min(n + 1, nlast), so);
        load_qv(min(n + 2, nlast), so);
        load_k(min(n + 2, nlast), RowsB{});
        __syncthreads();
      } else {
        // interval A: the chain runs phase 1 of chunk n
        if (n + 1 <= nlast) commit_rows((n + 1) & 1, so, AllRows{});
        commit_tp(so);                 // T (and P) of chunk n
        if constexpr (!SO && !decltype(first)::value) flush_o((n - 1) * C);
        load_k(min(n + 2, nlast), AllRows{});
        __syncthreads();
        // interval B: the chain runs U, O and S of chunk n
        load_tp(min(n + 1, nlast), so);
        load_qv(min(n + 2, nlast), so);
        if constexpr (!KDA && !SO) {
          if (n + 1 <= nlast) form_p((n + 1) & 1);
        }
        __syncthreads();
      }
    };
    auto prologue = [&](int n0, int nlast, auto so) __attribute__((always_inline)) {
      load_k(n0, AllRows{});
      load_qv(n0, so);
      commit_rows(n0 & 1, so, AllRows{});
      load_k(min(n0 + 1, nlast), AllRows{});
      load_qv(min(n0 + 1, nlast), so);
      load_tp(n0, so);
    };

    if (n_so > lead0) {   // lead-in: the state alone over chunks [lead0, n_so)
      prologue(lead0, n_so - 1, Lead{});
      __syncthreads();
      __syncthreads();
      for (int n = lead0; n < n_so; ++n) step(n, n_so - 1, std::true_type{}, Lead{});
    }
    if (n_end > n_so) prologue(n_so, n_end - 1, Full{});
    __syncthreads();
    if constexpr (!KDA) {
      if (n_end > n_so) form_p(n_so & 1);
    }
    __syncthreads();
    if (n_end > n_so) step(n_so, n_end - 1, std::true_type{}, Full{});
    for (int n = n_so + 1; n < n_end; ++n) step(n, n_end - 1, std::false_type{}, Full{});
    if (n_end > n_so) {   // the last chunk's rows
      const int t0f = (n_end - 1) * C, cnf = min(C, T - t0f);
      E* oq = og + (size_t)t0f * v_tok;
      for (int q = ptid; q < C * CPO; q += PT) {
        const int r = q / CPO, cc = q % CPO;
        if (r < cnf)
          st_once(oq + (uint32_t)r * (uint32_t)v_tok + cc * EPC, os_piece(r, cc));
      }
    }
    return;
  }

  // ======================= chain waves =======================
  // Phase-1 tiles of value block own_ib: the X tile of row block x_rb and the
  // O tile of row block o_rb.  Two value blocks: wave (rb, ib) takes both
  // tiles of (rb, ib), the two products sharing their S fragments.  One value
  // block: waves 0 and 1 take the X tiles, waves 2 and 3 the O tiles, one
  // product each (half the MFMA chain per wave; S is read twice).  The wave's
  // state tiles t = wave + 4 st all lie in value block ub.
  int x_rb = -1, o_rb = -1, own_ib = 0;
  if (NI == 2) {
    x_rb = o_rb = wave >> 1;
    own_ib = wave & 1;
  } else if (wave < 2) {
    x_rb = wave;
  } else {
    o_rb = wave - 2;
  }
  const int ub = NI == 2 ? (wave & 1) : 0;

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
        if (a.S0 && lead0 == 0) x = *reinterpret_cast<const float4*>(a.S0 + (sbase + i) * DK + c0);
        Sacc[st][4 * g + 0] = x.x;
        Sacc[st][4 * g + 1] = x.y;
        Sacc[st][4 * g + 2] = x.z;
        Sacc[st][4 * g + 3] = x.w;
        store4(Sb + i * LDSB + c0, x.x, x.y, x.z, x.w);
      }
    }
  }
  // One chunk of the chain (so: a lead-in chunk, X, U and S only).
  auto chunk = [&](int n, auto so) __attribute__((always_inline)) {
    constexpr bool SO = decltype(so)::value;
    const int nb = n & 1;
    const float* G = Gbuf + nb * GS;
    const float* Eg = G + C;       // exp(G_r) nk_r
    const float* Ec = G + 2 * C;   // exp(G_C - G_r) nk_r
    const E* Ks = Ksb + nb * C * LDKS;
    const E* K1 = KDA ? Krb + (L::single ? 0 : nb) * C * LDK : Ks;   // K operand of phase 1 (scalar: swizzled)
    const E* Qr = Qrb + (L::single ? 0 : nb) * C * LDK;
    const E* Vr = Vrb + nb * C * LDV;
    const E* Pm = Pmb + (KDA ? 0 : nb) * C * LDP;

    // ---- interval A, phase 1: X = V - diag(gamma) K S^T, O_inter^T = S (diag(gamma) Q)^T ----
    f32x16 xacc = zero16(), oacc = zero16();
    const bool do_x = x_rb >= 0, do_o = o_rb >= 0 && !SO;
    if (do_x || do_o) {
      // the V columns and gate rows of the epilogue are read before the product
      const int vc = own_ib * 32 + 16 * ((lane >> 4) & 1);
      uint2 vw[4];
      float4 eg[4];
      if (do_x) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = x_rb * 32 + acc_row(g, 0, lane);
          vw[g] = tr_read4(Vr, LDV, r0, vc, lane);   // V[r0 .. r0 + 3][i]
          eg[g] = KDA ? make_float4(1.f, 1.f, 1.f, 1.f) : *reinterpret_cast<const float4*>(Eg + r0);
        }
      }
      // O^T columns are the chunk rows r: exp(G_r) (normalised q: exp(G_r) and,
      // after the intra-chunk part, nq_r)
      const float egr = KDA || !do_o ? 1.f : (NORM ? G[3 * C + o_rb * 32 + col] : Eg[o_rb * 32 + col]);
      const E* Sf = Sb + own_ib * 32 * LDSB;
      if (NI == 1 || SO) {
        if (do_x)
          tile_nt_k<DK / 16, E, !KDA, kP1Ahead>(xacc, K1 + x_rb * 32 * (KDA ? LDK : LDKS), KDA ? LDK : LDKS, Sf,
                                               LDSB, lane);
        else   // (the operand order of the shared-fragment product's second tile)
          tile_nt_k<DK / 16, E, false, kP1Ahead>(oacc, Sf, LDSB, Qr + o_rb * 32 * LDK, LDK, lane);
      } else {
        tile_nt2_shared_b<DK / 16, E, true, kP1Ahead, !KDA>(xacc, oacc, K1 + x_rb * 32 * (KDA ? LDK : LDKS),
                                                             Qr + o_rb * 32 * LDK, KDA ? LDK : LDKS, LDK, Sf,
                                                             LDSB, lane);
      }
      if (do_x) {
        const int i = own_ib * 32 + col;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = x_rb * 32 + acc_row(g, 0, lane);
          const float4 v4 = make_float4(__uint_as_float(vw[g].x << 16), __uint_as_float(vw[g].x & 0xffff0000u),
                                        __uint_as_float(vw[g].y << 16), __uint_as_float(vw[g].y & 0xffff0000u));
          store4(Xt + i * LDT + r0, v4.x - eg[g].x * xacc[4 * g + 0], v4.y - eg[g].y * xacc[4 * g + 1],
                 v4.z - eg[g].z * xacc[4 * g + 2], v4.w - eg[g].w * xacc[4 * g + 3]);
        }
      }
      if constexpr (!KDA && !SO) {
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[v] *= egr;
      }
    }
    // Normalised q: the inverse norms of the chunk's Q rows, for its output
    // rows in interval B (the chain waits for the data waves here anyway):
    // wave w takes rows 16 w .. 16 w + 15, four lanes per row, a quarter of
    // the row's 16-byte pieces each (at d_k = 128, 16 rows x 4 pieces in
    // distinct banks per read).
    if constexpr (NORM && !SO) {
      const int r = 16 * wave + (lane >> 2), p = lane & 3;
      const E* row = Qr + r * LDK + p * (CPR / 4) * EPC;
      float ss[2] = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < CPR / 4; ++i) ss[i & 1] = sumsq16<E>(*reinterpret_cast<const u32x4*>(row + i * EPC), ss[i & 1]);
      const float nq = __builtin_amdgcn_rsqf(quad_sum(ss[0] + ss[1]) + a.pro.norm_eps);
      if (p == 0) Gbuf[nb * GS + 5 * C + r] = nq;
    }
    __syncthreads();

    // ---- interval B: every LDS fragment of the interval first ----
    Frag<E> ta0[2], ta1[4], xb[4];   // T rows 0..31 (k < 32), T rows 32..63, X^T of block ub
    {
      const int ko = (lane >> 5) * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (s < 2) ta0[s] = frag_load(Tm + col * LDT + ko + 16 * s);
        ta1[s] = frag_load(Tm + (32 + col) * LDT + ko + 16 * s);
        xb[s] = frag_load(Xt + (ub * 32 + col) * LDT + ko + 16 * s);
      }
    }
    bf16x8 pa[2][2], ka[NST][2][2];  // P rows of the wave's O tile; K^T of its state tiles
    if (o_rb >= 0 && !SO) {
      const E* prow = Pm + (o_rb * 32 + col) * LDP;
#pragma unroll
      for (int rj = 0; rj < 2; ++rj)
#pragma unroll
        for (int s = 0; s < 2; ++s) pa[rj][s] = frag_perm(prow, 32 * rj + 16 * s, hh);
    }
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int cb = min((wave + 4 * st) / NI, NC - 1);
#pragma unroll
      for (int rj = 0; rj < 2; ++rj)
#pragma unroll
        for (int s = 0; s < 2; ++s) ka[st][rj][s] = frag_perm_tr<true>(Ks, LDKS, 32 * rj + 16 * s, cb * 32, lane);
    }
    sched_fence();

    // U = T X for value block ub, both row blocks, in registers (T is lower
    // triangular: row block 0 needs k < 32)
    f32x16 u0 = zero16(), u1 = zero16();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s < 2) mma16(u0, ta0[s], xb[s]);
      mma16(u1, ta1[s], xb[s]);
    }
    bf16x8 uf[2][2], wf[2][2];   // U and the decay-weighted U as operands (k = token)
    uf[0][0] = frag_acc(u0, 0);
    uf[0][1] = frag_acc(u0, 1);
    uf[1][0] = frag_acc(u1, 0);
    uf[1][1] = frag_acc(u1, 1);
    if constexpr (KDA) {
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        wf[q][0] = uf[q][0];
        wf[q][1] = uf[q][1];
      }
    } else {   // rows r times exp(G_C - G_r)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 e0 = *reinterpret_cast<const float4*>(Ec + acc_row(g, 0, lane));
        const float4 e1 = *reinterpret_cast<const float4*>(Ec + 32 + acc_row(g, 0, lane));
        u0[4 * g + 0] *= e0.x; u0[4 * g + 1] *= e0.y; u0[4 * g + 2] *= e0.z; u0[4 * g + 3] *= e0.w;
        u1[4 * g + 0] *= e1.x; u1[4 * g + 1] *= e1.y; u1[4 * g + 2] *= e1.z; u1[4 * g + 3] *= e1.w;
      }
      wf[0][0] = frag_acc(u0, 0);
      wf[0][1] = frag_acc(u0, 1);
      wf[1][0] = frag_acc(u1, 0);
      wf[1][1] = frag_acc(u1, 1);
    }

    // ---- O^T = O_inter^T + U^T P^T for the wave's tile, staged for the data waves ----
    if (o_rb >= 0 && !SO) {
#pragma unroll
      for (int rj = 0; rj < 2; ++rj) {
        if (rj > o_rb) break;
#pragma unroll
        for (int s = 0; s < 2; ++s) mma_bf16(oacc, uf[rj][s], pa[rj][s]);
      }
      const int r = o_rb * 32 + col;
      if constexpr (NORM) {
        const float nq = G[5 * C + r];
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[v] *= nq;
      }
#pragma unroll
      for (int g = 0; g < 4; ++g)
        store4(Os + r * OST + own_ib * 32 + acc_row(g, 0, lane), oacc[4 * g], oacc[4 * g + 1], oacc[4 * g + 2],
               oacc[4 * g + 3]);
    }

    // ---- S^T <- gamma_C S^T + K^T Uw (per-channel: Diag(gC) S^T + Kc^T U), refresh Sb ----
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const int t = wave + 4 * st;
      if (t >= NT) continue;
      const int cb = t / NI;
      if constexpr (KDA) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 d = *reinterpret_cast<const float4*>(G + cb * 32 + acc_row(g, 0, lane));
          Sacc[st][4 * g + 0] *= d.x;
          Sacc[st][4 * g + 1] *= d.y;
          Sacc[st][4 * g + 2] *= d.z;
          Sacc[st][4 * g + 3] *= d.w;
        }
      } else {
        const float gC = NORM ? G[3 * C + C - 1] : Eg[C - 1];   // (exp(G_r) is row 3 when normalised)
#pragma unroll
        for (int v = 0; v < 16; ++v) Sacc[st][v] *= gC;
      }
#pragma unroll
      for (int rj = 0; rj < 2; ++rj)
#pragma unroll
        for (int s = 0; s < 2; ++s) mma_bf16(Sacc[st], ka[st][rj][s], wf[rj][s]);
      const int i = ub * 32 + col;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int c0 = cb * 32 + acc_row(g, 0, lane);
        store4(Sb + i * LDSB + c0, Sacc[st][4 * g], Sacc[st][4 * g + 1], Sacc[st][4 * g + 2],
               Sacc[st][4 * g + 3]);
      }
    }
    __syncthreads();
  };

  if (n_so > lead0) {   // lead-in
    __syncthreads();
    __syncthreads();
    for (int n = lead0; n < n_so; ++n) chunk(n, Lead{});
  }
  __syncthreads();
  __syncthreads();   // the data waves form P of the first chunk
  for (int n = n_so; n < n_end; ++n) chunk(n, Full{});

  if (a.S_final && last) {
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

// Workgroups are dispatched round-robin over the eight XCDs: give the
// workgroups of one head the same XCD (same L2) when the head count allows it.
__device__ inline void ws_head(const PrefillArgs& a, int per_head, int& head, int& rw) {
  if (((a.B * a.H) & 7) == 0) {
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    head = xcd + 8 * (j / per_head);
    rw = j % per_head;
  } else {
    head = blockIdx.x / per_head;
    rw = blockIdx.x % per_head;
  }
}

// Parts of a value slice with lead-ins from chunk 0: part p writes the outputs
// of chunks [m_p, m_p+1) and reaches its starting state by the state
// recurrence alone over [0, m_p), the very state the unsplit pass holds there.
// With a lead-in chunk costing r of a full one, m_p = N (1 - (1 - r)^p) /
// (1 - (1 - r)^npart) gives every part the same time.
__device__ inline int geometric_split(int nchunks, int p, int npart, float r) {
  if (p <= 0) return 0;
  if (p >= npart) return nchunks;
  const float q = 1.f - r;
  const float f = (1.f - __powf(q, (float)p)) / (1.f - __powf(q, (float)npart));
  return min(nchunks, max(0, (int)((float)nchunks * f + 0.5f)));
}

// The history horizon of a split slice (scalar decay).  With every chunk's
// transition bounded in norm by e^{c_n} (the prep kernel's bound array), the
// state at chunk m is S_s Phi(s, m) + (the recurrence over [s, m) from a zero
// state), with |S_s Phi(s, m)| <= e^{c_s + ... + c_{m-1}} |S_s|.  A lead-in from
// the last s at which that sum is at most -kHorizon, started from zero, thus
// reaches the state at m up to a part below e^-40 (4e-18) of |S_s|: ten orders
// of magnitude below the resolution of the fp32 state itself (a threshold at
// the gate floor's e^-100 takes 2.5 times the lead-in chunks: 4 % more time on
// the long-context workload).  Strongly decaying gates forget the far past
// within a few chunks, so the parts of a slice no longer need lead-ins from
// chunk 0.
constexpr float kHorizon = 40.f;

// Lead-in length (chunks) for a part whose outputs start at chunk m: the
// smallest L with c_{m-L} + ... + c_{m-1} <= -kHorizon, or m (a lead-in from
// chunk 0 and S0, exact) when no L <= min(m, cap) qualifies.  One wave; every
// lane returns the same value.  hz: the sequence's bound array.
__device__ inline int horizon_lead(const float* __restrict__ hz, int m, int cap) {
  const int lane = threadIdx.x & 63;
  const int lim = min(m, cap);
  float carry = 0.f;
  for (int base = 0; base < lim; base += 256) {
    float c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {   // four blocks of 64 chunks in flight, latest chunks first
      const int off = base + 64 * u + lane;
      c[u] = off < lim ? hz[m - 1 - off] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float sfx = chunk_prefix(c[u]) + carry;   // c_{m-1-off} + ... + c_{m-1}
      const unsigned long long hit = __ballot(base + 64 * u + lane < lim && sfx <= -kHorizon);
      if (hit) return base + 64 * u + __ffsll((long long)hit);
      carry = __shfl(sfx, 63);
    }
  }
  return m;
}

// Packed batch of up to 64 sequences: the sequence of rank k when they are
// ordered by length, longest first (ties by index).  One wave, every lane
// returns the same value.
__device__ inline int seq_by_length_rank(const PrefillArgs& a, int k) {
  const int lane = threadIdx.x & 63, N = a.B;
  int len = -1;
  if (lane < N) {   // (as seq_span clamps the offsets)
    const int s0 = min(max(a.cu_seqlens[lane], 0), a.T);
    len = min(max(a.cu_seqlens[lane + 1], s0), a.T) - s0;
  }
  int rank = 0;
  for (int j = 0; j < N; ++j) {
    const int lj = __shfl(len, j);
    rank += (lj > len || (lj == len && j < lane)) ? 1 : 0;
  }
  const unsigned long long hit = __ballot(lane < N && rank == k);
  return hit ? __ffsll((long long)hit) - 1 : k;
}

// Value slices in npart parts each (geometric split, lead-ins from chunk 0).
// Packed batch of up to 64 sequences with at least half as many slices as
// compute units (split_above >= 0): the workgroups take the sequences longest first, so
// that the longest slices start in the first round and the short ones fill in
// behind them; the slices of a sequence of more than split_above chunks run
// in two parts, the second reaching its start by a lead-in (from the history
// horizon when the bound array is there); the grid has room for the parts of
// split_max sequences.  Workgroup i takes head x + 8 k of
// that order on XCD x = i % 8 (its slices and parts back to back in that
// XCD's queue, which then shares their K, Q and records in its L2); the split
// heads come first, and the workgroups past the last head, at the end of the
// grid, return at once.
template <typename E, int DK, int DVS, int MODE, bool NORM>
__global__ __launch_bounds__(kWsThreads) void chunk_state_ws(PrefillArgs a, const E* __restrict__ tws, int npart,
                                                             float lead_r, int split_above, int split_max) {
  __shared__ __attribute__((aligned(16))) unsigned char smem[WsPlan<E, DK, DVS, (MODE >= 2), NORM>::total];
  const int nsl = a.dv / DVS;
  if (split_above < 0) {
    int head, rw;
    ws_head(a, nsl * npart, head, rw);
    const int sl = rw % nsl, part = rw / nsl;
    const Span sp = seq_span(a, head / a.H, head % a.H);
    const int nchunks = (sp.len + C - 1) / C;
    state_ws_body<E, DK, DVS, MODE, NORM>(a, tws, smem, head, sl, sp, part == npart - 1, 0,
                                          geometric_split(nchunks, part, npart, lead_r),
                                          geometric_split(nchunks, part + 1, npart, lead_r));
    return;
  }
  // sequences (ranks 0 .. nsq - 1) whose slices are split
  const int lane = threadIdx.x & 63;
  int nsq = 0;
  {
    bool longer = false;
    if (lane < a.B) {
      const int s0 = min(max(a.cu_seqlens[lane], 0), a.T);
      longer = (min(max(a.cu_seqlens[lane + 1], s0), a.T) - s0 + C - 1) / C > split_above;
    }
    nsq = min(__popcll(__ballot(longer)), split_max);   // (the grid's room)
  }
  const int nh = a.B * a.H, ks = nsq * a.H;   // heads; split heads (ranks 0 .. ks - 1)
  const int x = blockIdx.x & 7, q = blockIdx.x >> 3, w2 = 2 * nsl;
  const int sx = ks > x ? (ks - x + 7) / 8 : 0;   // split heads on this XCD
  int k, within;
  if (q < sx * w2) {
    k = q / w2;
    within = q % w2;
  } else {
    k = sx + (q - sx * w2) / nsl;
    within = (q - sx * w2) % nsl;
  }
  const int hr = x + 8 * k;   // head rank
  if (hr >= nh) return;
  const int sl = within % nsl, part = within / nsl;
  const int head = seq_by_length_rank(a, hr / a.H) * a.H + hr % a.H;
  const Span sp = seq_span(a, head / a.H, head % a.H);
  const int nchunks = (sp.len + C - 1) / C;
  int lead0 = 0, n_so = 0, n_end = nchunks;
  bool last = true;
  if (hr < ks) {
    // two parts: part 0 takes chunks [0, m), part 1 a lead-in of l chunks and
    // [m, N), m balancing m against r l + N - m
    int m = geometric_split(nchunks, 1, 2, lead_r), lead = m;
    if (MODE == 1 && a.horizon) {
      const float* hz = a.horizon + sp.rec0;
      const int l0 = horizon_lead(hz, nchunks / 2, nchunks / 2);
      m = min(nchunks - 1, (int)(0.5f * ((float)nchunks + lead_r * (float)l0) + 0.5f));
      lead = horizon_lead(hz, m, m);
    }
    n_so = part == 0 ? 0 : m;
    n_end = part == 0 ? m : nchunks;
    lead0 = part == 0 ? 0 : m - lead;
    last = part == 1;
  }
  state_ws_body<E, DK, DVS, MODE, NORM>(a, tws, smem, head, sl, sp, last, lead0, n_so, n_end);
}

// Lead-in chunk cost relative to a full chunk of the eight-wave kernel
// (measured on the long-context workload): sets where the parts of a value
// slice split the sequence.
constexpr float kLeadCost = 0.65f;
// Per-chunk cost of a 64-row value slice relative to a 32-row one.
constexpr float kSlice64Cost = 1.35f;

// Scalar decay with split slices: per head, either 32-row slices in npart32
// parts with lead-ins from chunk 0 (as chunk_state_ws), or 64-row slices in
// twice as many parts of equal length with lead-ins from the history horizon,
// whichever the cost model gives less time.  Same workgroup count per head;
// every workgroup of a head reads the same bounds and takes the same choice.
template <typename E, int DK, bool NORM>
__global__ __launch_bounds__(kWsThreads) void chunk_state_ws_horizon(PrefillArgs a, const E* __restrict__ tws,
                                                                     int npart32, float lead_r) {
  using L32 = WsPlan<E, DK, 32, false, NORM>;
  using L64 = WsPlan<E, DK, 64, false, NORM>;
  __shared__ __attribute__((aligned(16))) unsigned char smem[cmax(L32::total, L64::total)];
  const int nsl32 = a.dv / 32, nsl64 = a.dv / 64;
  const int per_head = nsl32 * npart32, npart64 = per_head / nsl64;
  int head, rw;
  ws_head(a, per_head, head, rw);
  const Span sp = seq_span(a, head / a.H, head % a.H);
  const int nchunks = (sp.len + C - 1) / C;
  // time of the 32-row plan (its first part has no lead-in); past the lead-in
  // length at which the 64-row plan cannot win, the scan stops
  const float t32 = (float)geometric_split(nchunks, 1, npart32, lead_r);
  const float span64 = (float)nchunks / (float)npart64;
  const int cap = max(0, (int)((t32 / kSlice64Cost - span64) / lead_r) + 1);
  const float* hz = a.horizon + sp.rec0;
  int lmax = 0;   // longest lead-in of an equal split
  for (int q = 1; q < npart64; ++q)
    lmax = max(lmax, horizon_lead(hz, (int)((long long)q * nchunks / npart64), cap));
  if (kSlice64Cost * (span64 + lead_r * (float)lmax) < t32) {
    // Part 0 has no lead-in: it takes the outputs the others' lead-ins cost,
    // m_q = q tau - (q - 1) r L with tau = (N + (P - 1) r L) / P; the lead-ins
    // are then taken at these boundaries (scanned a little further than L).
    const float sh = lead_r * (float)lmax;
    const float tau = ((float)nchunks + (float)(npart64 - 1) * sh) / (float)npart64;
    auto bound = [&](int q) {
      if (q <= 0) return 0;
      if (q >= npart64) return nchunks;
      return min(nchunks, max(0, (int)((float)q * tau - (float)(q - 1) * sh + 0.5f)));
    };
    const int part64 = rw / nsl64;
    const int so = bound(part64), end = max(so, bound(part64 + 1));
    const int lead = horizon_lead(hz, so, 2 * lmax + 64);
    state_ws_body<E, DK, 64, 1, NORM>(a, tws, smem, head, rw % nsl64, sp, part64 == npart64 - 1, so - lead, so,
                                      end);
  } else {
    const int part = rw / nsl32;
    state_ws_body<E, DK, 32, 1, NORM>(a, tws, smem, head, rw % nsl32, sp, part == npart32 - 1, 0,
                                      geometric_split(nchunks, part, npart32, lead_r),
                                      geometric_split(nchunks, part + 1, npart32, lead_r));
  }
}

// Parts per value slice: while the slices fill at most half of the compute
// units, each slice is split in two parts more.
inline int state_parts(size_t slices) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return 1;
  int np = 1;
  while (np < 4 && slices * (size_t)(2 * np) <= (size_t)cus) np *= 2;
  return np;
}

template <typename E, int DK, int DVS>
hipError_t launch_state(const PrefillArgs& a, const E* tws, hipStream_t stream) {
  const size_t slices = (size_t)a.B * a.H * (a.dv / DVS);
  dim3 grid((unsigned)slices), block(kThreads);
  if constexpr (sizeof(E) == 2) {
    const int np = state_parts(slices);
    // packed batch of at least half as many slices as compute units (one
    // part each otherwise): longest sequences first,
    // the slices longer than an even share of chunks per compute unit in two
    // parts (Sum ceil(len_s / C) <= T / C + N bounds the chunks; at most
    // (T / C + N) / (split + 1) sequences exceed split chunks)
    int split = -1, nsq = 0;
    grid = dim3((unsigned)(slices * np));
    if (a.cu_seqlens && np == 1 && a.B > 1 && a.B <= 64) {
      int dev = 0, cus = 256;
      if (hipGetDevice(&dev) != hipSuccess ||
          hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
      const long long chunks = (long long)a.T / C + a.B, nsl = a.dv / DVS;
      split = (int)(chunks * (long long)slices / ((long long)a.B * cus)) + 1;
      nsq = (int)std::min<long long>(a.B, chunks / (split + 1));
      const long long heads8 = ((long long)a.B * a.H + 7) / 8, split8 = (nsq * a.H + 7) / 8;
      grid = dim3((unsigned)(8 * (heads8 * nsl + split8 * nsl)));
    }
    const float r = kLeadCost;
    dim3 wblock(kWsThreads);
    // (normalised q and k: the per-channel records carry normalised operands, so
    // only the scalar / no-decay state kernel has a variant of its own)
    const bool nrm = a.pro.qk_norm != 0;
    if (DVS == 32 && a.mode == 1 && np > 1 && a.horizon && np <= 4) {
      if (nrm)
        hipLaunchKernelGGL((chunk_state_ws_horizon<E, DK, true>), grid, wblock, 0, stream, a, tws, np, r);
      else
        hipLaunchKernelGGL((chunk_state_ws_horizon<E, DK, false>), grid, wblock, 0, stream, a, tws, np, r);
    } else if (a.mode == 0 && !nrm)
      hipLaunchKernelGGL((chunk_state_ws<E, DK, DVS, 0, false>), grid, wblock, 0, stream, a, tws, np, r, split, nsq);
    else if (a.mode == 0)
      hipLaunchKernelGGL((chunk_state_ws<E, DK, DVS, 0, true>), grid, wblock, 0, stream, a, tws, np, r, split, nsq);
    else if (a.mode == 1 && !nrm)
      hipLaunchKernelGGL((chunk_state_ws<E, DK, DVS, 1, false>), grid, wblock, 0, stream, a, tws, np, r, split, nsq);
    else if (a.mode == 1)
      hipLaunchKernelGGL((chunk_state_ws<E, DK, DVS, 1, true>), grid, wblock, 0, stream, a, tws, np, r, split, nsq);
    else if (a.mode == 2)
      hipLaunchKernelGGL((chunk_state_ws<E, DK, DVS, 2, false>), grid, wblock, 0, stream, a, tws, np, r, split, nsq);
    else
      hipLaunchKernelGGL((chunk_state_ws<E, DK, DVS, 3, false>), grid, wblock, 0, stream, a, tws, np, r, split, nsq);
  } else {
    if (a.mode == 0)
      hipLaunchKernelGGL((chunk_state_kernel<E, DK, DVS, 0>), grid, block, 0, stream, a, tws);
    else if (a.mode == 1)
      hipLaunchKernelGGL((chunk_state_kernel<E, DK, DVS, 1>), grid, block, 0, stream, a, tws);
    else if (a.mode == 2)
      hipLaunchKernelGGL((chunk_state_kernel<E, DK, DVS, 2>), grid, block, 0, stream, a, tws);
    else
      hipLaunchKernelGGL((chunk_state_kernel<E, DK, DVS, 3>), grid, block, 0, stream, a, tws);
  }
  return hipGetLastError();
}

// Slice width: 64 value rows per workgroup (bf16) when that still gives at least
// one workgroup per compute unit (256; per-channel decay: 128, in two parts),
// else 32.  fp32 tiles take twice the LDS, so fp32 always uses 32-row slices.
// One prep workgroup per chunk of every head; a packed batch takes one per
// record slot (slots that no chunk falls on return at once).
template <typename E, int DK>
hipError_t launch_prep(const PrefillArgs& a, E* tws, hipStream_t stream) {
  const int nchunks = a.cu_seqlens ? a.nslots : (a.T + C - 1) / C;
  const bool by_chunk = a.mode < 2;   // (the prep kernel of none or scalar decay)
  const int rows = a.cu_seqlens ? 1 : a.B;
  const size_t nprep = a.cu_seqlens && a.T == 0 ? 0
                       : (by_chunk ? prep_grid<true>(rows, a.H, nchunks) : prep_grid<false>(rows, a.H, nchunks));
  if (nprep > 0) {
    dim3 grid((unsigned)nprep), block(kThreads);
    if (a.pro.qk_norm) {
      if (a.mode == 0)
        hipLaunchKernelGGL((chunk_prep_kernel<E, DK, 0, true>), grid, block, 0, stream, a, tws, nchunks);
      else if (a.mode == 1)
        hipLaunchKernelGGL((chunk_prep_kernel<E, DK, 1, true>), grid, block, 0, stream, a, tws, nchunks);
      else
        hipLaunchKernelGGL((chunk_prep_kda<E, DK, true, false>), grid, block, 0, stream, a, tws, nchunks);
    } else {
      if (a.mode == 0)
        hipLaunchKernelGGL((chunk_prep_kernel<E, DK, 0, false>), grid, block, 0, stream, a, tws, nchunks);
      else if (a.mode == 1)
        hipLaunchKernelGGL((chunk_prep_kernel<E, DK, 1, false>), grid, block, 0, stream, a, tws, nchunks);
      else if (a.mode == 2)
        hipLaunchKernelGGL((chunk_prep_kda<E, DK, false, false>), grid, block, 0, stream, a, tws, nchunks);
      else
        hipLaunchKernelGGL((chunk_prep_kda<E, DK, false, true>), grid, block, 0, stream, a, tws, nchunks);
    }
    return hipGetLastError();
  }
  return hipSuccess;
}

template <typename E, int DK>
hipError_t launch_dk(const PrefillArgs& a0, void* workspace, hipStream_t stream) {
  E* tws = static_cast<E*>(workspace);
  PrefillArgs a = a0;
  const long long wg64 = (long long)a.B * a.H * (a.dv / 64);
  // 64-row value slices (bf16): none or scalar decay, and Gated DeltaNet-2,
  // when they give every compute unit a workgroup; per-channel decay already
  // when two parts per slice do (its 32-row slices load the whole chunk record
  // for half the rows: B=4 H=16 T=8192 458.8 -> 440.7 us with two parts,
  // packed 16 rows 478 -> 420 us, Gated DeltaNet-2 at B=8 H=16 T=4096 503 ->
  // 436 us; Gated DeltaNet-2 with two parts 498 -> 504 us).
  const bool dvs64 = sizeof(E) == 2 && (wg64 >= 256 || (a.mode == 2 && wg64 >= 128));
  // Scalar decay in bf16 with split value slices (a head's, or a packed
  // batch's longest rows'): the prep kernel also writes the transition
  // bounds, after the records.
  if (sizeof(E) == 2 && a.mode == 1 &&
      (a.cu_seqlens || (!dvs64 && state_parts((size_t)a.B * a.H * (a.dv / 32)) > 1))) {
    const size_t nrec = a.cu_seqlens ? (size_t)a.H * a.nslots : (size_t)a.B * a.H * ((a.T + C - 1) / C);
    a.horizon = reinterpret_cast<float*>(tws + nrec * GateRec<E>::elems);
  }
  const hipError_t e = launch_prep<E, DK>(a, tws, stream);
  if (e != hipSuccess) return e;
  if constexpr (sizeof(E) == 4) {
    return launch_state<E, DK, 32>(a, tws, stream);
  } else {
    if (dvs64) return launch_state<E, DK, 64>(a, tws, stream);
    return launch_state<E, DK, 32>(a, tws, stream);
  }
}

}  // namespace

// Bytes of one chunk record.
static size_t record_bytes(int dk, int dtype, int mode) {
  const size_t es = dtype == 1 ? 2 : 4;
  if (mode >= 2) return (2 * (size_t)C * C + 3 * (size_t)C * dk) * es + 4 * (size_t)dk;
  return (es == 4 ? 2 : 1) * (size_t)C * C * es + kGateFloats * 4;   // bf16: no P
}

// The transition bounds of scalar decay in bf16 (one fp32 per record) follow
// the records, 256-byte aligned.
static size_t horizon_bytes(size_t nrec, int dtype, int mode) {
  return dtype == 1 && mode == 1 ? (nrec * 4 + 255) & ~(size_t)255 : 0;
}

size_t prefill_workspace_bytes(int B, int T, int H, int dk, int dtype, int mode) {
  const size_t nrec = (size_t)B * H * (((size_t)T + C - 1) / C);
  return nrec * record_bytes(dk, dtype, mode) + horizon_bytes(nrec, dtype, mode);
}

int varlen_slots(int N, int T) { return T / C + N; }

size_t prefill_varlen_workspace_bytes(int N, int T, int H, int dk, int dtype, int mode) {
  if (T == 0) return 0;
  const size_t nrec = (size_t)H * varlen_slots(N, T);
  return nrec * record_bytes(dk, dtype, mode) + horizon_bytes(nrec, dtype, mode);
}

size_t prefill_record_bytes(int dk, int dtype, int mode) { return record_bytes(dk, dtype, mode); }

// Chunk records of the prefill entry point that allocates nothing: one copy
// of this array per device, alive until the process ends.  In host code its
// name is only a stand-in; kernels get the device address looked up below.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_prefill_prep(const PrefillArgs& a, void* workspace, hipStream_t stream) {
  if (a.dtype == 1)
    return a.dk == 128 ? launch_prep<__bf16, 128>(a, static_cast<__bf16*>(workspace), stream)
                       : launch_prep<__bf16, 64>(a, static_cast<__bf16*>(workspace), stream);
  return a.dk == 128 ? launch_prep<float, 128>(a, static_cast<float*>(workspace), stream)
                     : launch_prep<float, 64>(a, static_cast<float*>(workspace), stream);
}

hipError_t launch_prefill(const PrefillArgs& a, void* workspace, hipStream_t stream) {
  if (a.dtype == 1)
    return a.dk == 128 ? launch_dk<__bf16, 128>(a, workspace, stream) : launch_dk<__bf16, 64>(a, workspace, stream);
  return a.dk == 128 ? launch_dk<float, 128>(a, workspace, stream) : launch_dk<float, 64>(a, workspace, stream);
}

}  // namespace gdn
