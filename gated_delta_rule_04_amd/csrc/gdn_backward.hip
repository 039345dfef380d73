// Backward of the gated delta-rule prefill: the gradients of
//   L = sum(do . o) + sum(dS_final . S_T)
// with respect to q, k, v, alpha, beta and S0, for the three decay families.
//
// The pages train these mixers with a custom first-order backward that keeps
// the state history (NextTransformer "method sources" page, KDA entry).  Here
// the history is rebuilt instead of stored: it would be d_v x d_k fp32 per
// token.  Per token, with S~ = S_{t-1} D_t, p = S~ k, u = beta (v - p) and
// S_t = S~ + u k^T (the forward loop), the reverse step is, per state row i:
//
//   dS_i  += do_i q                 o = S_t q
//   dq    += S_t^T do               (a sum over rows)
//   du_i   = dS_i . k
//   dk    += dS^T u + S~^T dp,      dp_i = -beta du_i
//   dbeta  = sum_i du_i (v_i - p_i),   dv_i = beta du_i
//   dS~_i  = dS_i + dp_i k
//   dalpha = sum_i dS~_i . S_{t-1,i}   (per channel: the column sums)
//   dS_{t-1,i} = dS~_i D_t
//
// Three kernels:
//   bwd_checkpoint  the forward token loop from S0, storing S every 8 tokens
//                   (one workgroup per (b, h, 32-row value slice); rows are
//                   independent: "On State Reduction" notes, section 2.5)
//   bwd_reverse     chunks of 64 tokens in reverse order: the chunk's K, V, dO
//                   and gates are staged in LDS, each 4-token block's states
//                   are recomputed into registers from the checkpoint at most
//                   4 tokens before it, then the reverse steps run over the
//                   block.  (Blocks of 4 and LDS below 80 KB let two
//                   workgroups share a compute unit and hide each other's
//                   latency.)  dv and dS0 are complete
//                   per slice; the sums over rows (dq, dk, per-channel dalpha,
//                   dbeta, scalar dalpha) are complete per slice and go to a
//                   workspace, one partial per value slice
//   bwd_reduce      adds the slices' partials in a fixed order (deterministic,
//                   no atomics) and writes dq, dk, dalpha, dbeta.
// Layout of the work inside a workgroup: 8 rows per wave, 32 rows per
// workgroup, 8 lanes per state row; lane 8 c + r of a wave holds row r of the
// wave and the columns 4 c + 32 j .. + 3.  The sums over rows (three per token,
// 4 d_k / 32 values each) are then DPP sums over 8 adjacent lanes, and only
// the dot products over a row (two or three per token) need lane shuffles;
// across the four waves the sums go through LDS.  (Measured with 8-token
// blocks: 21 ms against 25 ms with 8 adjacent lanes per row, at B=8, H=16,
// T=4096, d=128.)
#include <stdint.h>

#include "gdn_backward.h"

namespace gdn {
namespace {

constexpr int C = 64;                  // tokens staged in LDS at a time
constexpr int CK = 8;                  // tokens between state checkpoints
constexpr int SUB = 4;                 // tokens whose states are held in registers at a time
static_assert(C % CK == 0 && CK % SUB == 0, "checkpoints at block boundaries");
constexpr int kThreads = 256;
constexpr int LPR = 8;                 // lanes per state row
constexpr int DVS = kThreads / LPR;    // state rows per workgroup

__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(__bf16 x) { return (float)x; }
__device__ inline void from_f32(float* p, float x) { *p = x; }
__device__ inline void from_f32(__bf16* p, float x) { *p = (__bf16)x; }

// Sum over the 8 lanes of a row (lanes 8 apart), result in all of them: lanes
// 8 apart inside a 16-lane DPP row (row_ror:8), then across the DPP rows.
__device__ inline float row_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, true));
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Sum over the 8 rows of a wave (aligned groups of 8 lanes), result in all of them.
__device__ inline float rows_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));
  return x;
}

__device__ inline float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline float4 ld4(const __bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

__device__ inline float dot4(const float4& a, const float4& b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}
__device__ inline float4 mul4(const float4& a, const float4& b) {
  return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w);
}
__device__ inline float4 scale4(const float4& a, float s) {
  return make_float4(a.x * s, a.y * s, a.z * s, a.w * s);
}
__device__ inline float4 fma4(float s, const float4& a, const float4& b) {   // s a + b
  return make_float4(s * a.x + b.x, s * a.y + b.y, s * a.z + b.z, s * a.w + b.w);
}

// LDS of the two sequential kernels: the chunk's K rows and per-channel gates
// (operand dtype), V and dO slices and the gate scalars (fp32); then (reverse
// kernel) the block's Q rows, the four waves' partial sums over rows and the
// block's dv.  Below 80 KB (bf16; fp32 without per-channel gates): two
// workgroups per compute unit.
template <typename E, int DK, int MODE>
struct BwdLds {
  static constexpr int NCOL = MODE == 2 ? 3 : 2;   // dq, dk (, dalpha per channel)
  static constexpr size_t es = sizeof(E);
  static constexpr size_t k = 0;                   // K and per-channel gates in the operand dtype
  static constexpr size_t a = k + (size_t)C * DK * es;
  static constexpr size_t v = a + (MODE == 2 ? (size_t)C * DK * es : 0);
  static constexpr size_t d = v + (size_t)C * DVS * 4;
  static constexpr size_t g = d + (size_t)C * DVS * 4;   // beta [C], scalar alpha [C]
  static constexpr size_t q = g + 2 * C * 4;
  static constexpr size_t col = q + (size_t)SUB * DK * 4;                 // [4][SUB][NCOL][DK]
  static constexpr size_t sc = col + (size_t)4 * SUB * NCOL * DK * 4;     // [4][SUB][2]
  static constexpr size_t dvb = sc + (size_t)4 * SUB * 2 * 4;             // [SUB][DVS]
  static constexpr size_t total = dvb + (size_t)SUB * DVS * 4;
  static_assert(total <= 160 * 1024, "backward LDS plan exceeds 160 KiB");
};

// Where a workgroup works: head (b, h), value rows i0 .. i0 + 31, and the
// thread's row g inside them and its column group l8 (columns 4 l8 + 32 j).
struct Place {
  int b, h, sl, i0, g, l8, wave, lane;
};
__device__ inline Place place(const BackwardArgs& a) {
  const int nsl = a.dv_ / DVS;
  Place p;
  p.sl = blockIdx.x % nsl;
  const int bh = blockIdx.x / nsl;
  p.h = bh % a.H;
  p.b = bh / a.H;
  p.i0 = p.sl * DVS;
  p.wave = threadIdx.x >> 6;
  p.lane = threadIdx.x & 63;
  p.g = p.wave * 8 + (p.lane & 7);
  p.l8 = p.lane >> 3;
  return p;
}

// The chunk's rows into LDS (rows past the sequence end repeat its last row;
// the loops below never reach them).
template <typename E, int DK, int MODE, bool WITH_DO>
__device__ inline void stage_chunk(const BackwardArgs& a, const Place& P, int t0, int cn, E* kst,
                                   E* ast, float* vst, float* dst, float* gst) {
  const size_t tok0 = (size_t)P.b * a.T + t0;
  const int H = a.H;
  for (int idx = threadIdx.x; idx < C * DK; idx += kThreads) {
    const int r = idx / DK, c = idx % DK;
    const size_t tk = ((tok0 + min(r, cn - 1)) * H + P.h) * DK + c;
    kst[idx] = static_cast<const E*>(a.k)[tk];
    if constexpr (MODE == 2) ast[idx] = static_cast<const E*>(a.alpha)[tk];
  }
  for (int idx = threadIdx.x; idx < C * DVS; idx += kThreads) {
    const int r = idx / DVS, i = idx % DVS;
    const size_t tv = ((tok0 + min(r, cn - 1)) * H + P.h) * (size_t)a.dv_ + P.i0 + i;
    vst[idx] = to_f32(static_cast<const E*>(a.v)[tv]);
    if constexpr (WITH_DO) dst[idx] = to_f32(static_cast<const E*>(a.dout)[tv]);
  }
  for (int r = threadIdx.x; r < C; r += kThreads) {
    const size_t tb = (tok0 + min(r, cn - 1)) * H + P.h;
    gst[r] = a.beta[tb];
    gst[C + r] = MODE == 1 ? static_cast<const float*>(a.alpha)[tb] : 1.f;
  }
}

// One forward token step on this lane's piece of its row.
template <typename E, int DK, int MODE>
__device__ inline void fstep(float4 (&S)[DK / 32], int r, int g, int l8, const E* kst,
                             const E* ast, const float* vst, const float* gst) {
  constexpr int NQ = DK / 32;
  float4 kk[NQ];
  float p = 0.f;
  const float as = gst[C + r];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    kk[j] = ld4(kst + r * DK + 4 * l8 + 32 * j);
    if constexpr (MODE == 2) S[j] = mul4(S[j], ld4(ast + r * DK + 4 * l8 + 32 * j));
    if constexpr (MODE == 1) S[j] = scale4(S[j], as);
    p += dot4(S[j], kk[j]);
  }
  p = row_sum(p);
  const float u = gst[r] * (vst[r * DVS + g] - p);
#pragma unroll
  for (int j = 0; j < NQ; ++j) S[j] = fma4(u, kk[j], S[j]);
}

template <typename E, int DK, int MODE>
__global__ __launch_bounds__(kThreads, 2) void bwd_checkpoint(BackwardArgs a, float* __restrict__ ck) {
  using L = BwdLds<E, DK, MODE>;
  constexpr int NQ = DK / 32;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  E* kst = reinterpret_cast<E*>(smem + L::k);
  E* ast = reinterpret_cast<E*>(smem + L::a);
  float* vst = reinterpret_cast<float*>(smem + L::v);
  float* gst = reinterpret_cast<float*>(smem + L::g);
  const Place P = place(a);
  const int nch = (a.T + C - 1) / C;
  const size_t row = ((size_t)P.b * a.H + P.h) * a.dv_ + P.i0 + P.g;   // state row in [B, H, dv]
  float4 S[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
    S[j] = a.S0 ? *reinterpret_cast<const float4*>(a.S0 + row * DK + 4 * P.l8 + 32 * j)
                : make_float4(0.f, 0.f, 0.f, 0.f);
  const int nck = (a.T + CK - 1) / CK;
  for (int n = 0; n < nch; ++n) {
    const int t0 = n * C, cn = min(C, a.T - t0);
    __syncthreads();
    stage_chunk<E, DK, MODE, false>(a, P, t0, cn, kst, ast, vst, nullptr, gst);
    __syncthreads();
    for (int r = 0; r < cn; ++r) {
      if ((r & (CK - 1)) == 0) {   // checkpoint: the state before token t0 + r, [B, H][t / CK][dv][dk]
        float* cp = ck + ((((size_t)P.b * a.H + P.h) * nck + (t0 + r) / CK) * a.dv_ + P.i0 + P.g) * DK;
#pragma unroll
        for (int j = 0; j < NQ; ++j) *reinterpret_cast<float4*>(cp + 4 * P.l8 + 32 * j) = S[j];
      }
      fstep<E, DK, MODE>(S, r, P.g, P.l8, kst, ast, vst, gst);
    }
  }
}

template <typename E, int DK, int MODE>
__global__ __launch_bounds__(kThreads, 2) void bwd_reverse(BackwardArgs a, const float* __restrict__ ck,
                                                        float* __restrict__ part, float* __restrict__ spart) {
  using L = BwdLds<E, DK, MODE>;
  constexpr int NQ = DK / 32, NCOL = L::NCOL;
  __shared__ __attribute__((aligned(16))) unsigned char smem[L::total];
  E* kst = reinterpret_cast<E*>(smem + L::k);
  E* ast = reinterpret_cast<E*>(smem + L::a);
  float* vst = reinterpret_cast<float*>(smem + L::v);
  float* dst = reinterpret_cast<float*>(smem + L::d);
  float* gst = reinterpret_cast<float*>(smem + L::g);
  float* qst = reinterpret_cast<float*>(smem + L::q);
  float* col = reinterpret_cast<float*>(smem + L::col);
  float* sc = reinterpret_cast<float*>(smem + L::sc);
  float* dvb = reinterpret_cast<float*>(smem + L::dvb);

  const Place P = place(a);
  const int nsl = a.dv_ / DVS;
  const int nch = (a.T + C - 1) / C;
  const int nck = (a.T + CK - 1) / CK;
  const size_t NTH = (size_t)a.B * a.T * a.H;   // token-heads
  const size_t row = ((size_t)P.b * a.H + P.h) * a.dv_ + P.i0 + P.g;
  float4 dS[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j)
    dS[j] = a.dS_final ? *reinterpret_cast<const float4*>(a.dS_final + row * DK + 4 * P.l8 + 32 * j)
                       : make_float4(0.f, 0.f, 0.f, 0.f);

  // Sum over the wave's rows of a lane piece, stored by the wave's first row.
  auto col_store = [&](float4 x, float* dstp) __attribute__((always_inline)) {
    x.x = rows_sum(x.x);
    x.y = rows_sum(x.y);
    x.z = rows_sum(x.z);
    x.w = rows_sum(x.w);
    if ((P.lane & 7) == 0) *reinterpret_cast<float4*>(dstp) = x;
  };

  // One reverse token step: Sp is the state before token r (chunk row r), jb
  // the token's place in the block.
  auto bstep = [&](const float4 (&Sp)[NQ], int r, int jb) __attribute__((always_inline)) {
    float4 kk[NQ], qq[NQ], dd[NQ], St[NQ], Sd[NQ];
    const float as = gst[C + r], bt = gst[r];
    float p = 0.f;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      kk[j] = ld4(kst + r * DK + 4 * P.l8 + 32 * j);
      qq[j] = *reinterpret_cast<const float4*>(qst + jb * DK + 4 * P.l8 + 32 * j);
      dd[j] = MODE == 2 ? ld4(ast + r * DK + 4 * P.l8 + 32 * j) : make_float4(as, as, as, as);
      Sd[j] = MODE == 0 ? Sp[j] : mul4(Sp[j], dd[j]);   // S~
      p += dot4(Sd[j], kk[j]);
    }
    p = row_sum(p);
    const float vi = vst[r * DVS + P.g], doi = dst[r * DVS + P.g];
    const float u = bt * (vi - p);
    float du = 0.f;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      St[j] = fma4(u, kk[j], Sd[j]);
      dS[j] = fma4(doi, qq[j], dS[j]);
      du += dot4(dS[j], kk[j]);
    }
    du = row_sum(du);
    const float dp = -bt * du;
    float* cw = col + (size_t)((P.wave * SUB + jb) * NCOL) * DK;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      col_store(scale4(St[j], doi), cw + 4 * P.l8 + 32 * j);                                     // dq
      col_store(fma4(dp, Sd[j], scale4(dS[j], u)), cw + DK + 4 * P.l8 + 32 * j);                   // dk
    }
    const float dbeta_w = rows_sum(du * (vi - p));   // every lane of a row holds the row's value
    if (P.l8 == 0) dvb[jb * DVS + P.g] = bt * du;
    float da = 0.f;
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      const float4 dsd = fma4(dp, kk[j], dS[j]);   // dS~
      if constexpr (MODE == 2) col_store(mul4(dsd, Sp[j]), cw + 2 * DK + 4 * P.l8 + 32 * j);
      if constexpr (MODE == 1) da += dot4(dsd, Sp[j]);
      dS[j] = MODE == 0 ? dsd : mul4(dsd, dd[j]);
    }
    if constexpr (MODE == 1) da = rows_sum(row_sum(da));
    if (P.lane == 0) {
      sc[(P.wave * SUB + jb) * 2] = dbeta_w;
      sc[(P.wave * SUB + jb) * 2 + 1] = da;
    }
  };

  // The checkpoint and the Q rows of a block, into registers: the next block's
  // are loaded while the current one is computed.
  constexpr int QPT = SUB * DK / kThreads;
  static_assert(SUB * DK % kThreads == 0, "Q rows of a block must split evenly");
  auto load_block = [&](int t0, int cn, int sb, E (&qv)[QPT], float4 (&sc4)[NQ]) __attribute__((always_inline)) {
    const int r0 = sb * SUB, nv = min(SUB, cn - r0), rs = r0 & ~(CK - 1);
    const float* cp = ck + ((((size_t)P.b * a.H + P.h) * nck + (t0 + rs) / CK) * a.dv_ + P.i0 + P.g) * DK;
#pragma unroll
    for (int j = 0; j < NQ; ++j) sc4[j] = *reinterpret_cast<const float4*>(cp + 4 * P.l8 + 32 * j);
    const size_t tok0 = (size_t)P.b * a.T + t0 + r0;
#pragma unroll
    for (int m = 0; m < QPT; ++m) {
      const int idx = threadIdx.x + kThreads * m, j = idx / DK, c = idx % DK;
      qv[m] = static_cast<const E*>(a.q)[((tok0 + min(j, nv - 1)) * a.H + P.h) * DK + c];
    }
  };

  for (int n = nch - 1; n >= 0; --n) {
    const int t0 = n * C, cn = min(C, a.T - t0);
    __syncthreads();   // the previous chunk's readers are done with LDS
    stage_chunk<E, DK, MODE, true>(a, P, t0, cn, kst, ast, vst, dst, gst);
    const int nsub = (cn + SUB - 1) / SUB;
    E qv[QPT];
    float4 Sc[NQ];
    load_block(t0, cn, nsub - 1, qv, Sc);
    for (int sb = nsub - 1; sb >= 0; --sb) {
      const int r0 = sb * SUB, nv = min(SUB, cn - r0);
      const int rs = r0 & ~(CK - 1);   // the checkpoint at or before the block
#pragma unroll
      for (int m = 0; m < QPT; ++m) qst[threadIdx.x + kThreads * m] = to_f32(qv[m]);
      __syncthreads();
      E qn[QPT];
      float4 Sn[NQ];
      load_block(t0, cn, max(sb - 1, 0), qn, Sn);   // the next block's (unconditional: exact waits)
      // states before each token of the block, recomputed from the checkpoint
      float4 S[NQ];
#pragma unroll
      for (int j = 0; j < NQ; ++j) S[j] = Sc[j];
      for (int r = rs; r < r0; ++r) fstep<E, DK, MODE>(S, r, P.g, P.l8, kst, ast, vst, gst);
      float4 Sp[SUB][NQ];
#pragma unroll
      for (int jb = 0; jb < SUB; ++jb) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) Sp[jb][j] = S[j];
        if (jb < nv) fstep<E, DK, MODE>(S, r0 + jb, P.g, P.l8, kst, ast, vst, gst);
      }
#pragma unroll
      for (int jb = SUB - 1; jb >= 0; --jb)
        if (jb < nv) bstep(Sp[jb], r0 + jb, jb);
      __syncthreads();
      // the four waves' sums, in a fixed order, to this slice's partials
      const size_t th0 = ((size_t)P.b * a.T + t0 + r0) * a.H + P.h;   // token-head of the block's first token
      for (int idx = threadIdx.x; idx < nv * NCOL * DK; idx += kThreads) {
        const int jb = idx / (NCOL * DK), qc = (idx / DK) % NCOL, c = idx % DK;
        const float* s0 = col + (size_t)(jb * NCOL + qc) * DK + c;
        const size_t wstride = (size_t)SUB * NCOL * DK;
        const float s = ((s0[0] + s0[wstride]) + s0[2 * wstride]) + s0[3 * wstride];
        part[((size_t)qc * nsl + P.sl) * NTH * DK + (th0 + (size_t)jb * a.H) * DK + c] = s;
      }
      for (int idx = threadIdx.x; idx < nv * 2; idx += kThreads) {
        const int jb = idx >> 1, qs = idx & 1;
        const float s = ((sc[(0 * SUB + jb) * 2 + qs] + sc[(1 * SUB + jb) * 2 + qs]) + sc[(2 * SUB + jb) * 2 + qs]) +
                        sc[(3 * SUB + jb) * 2 + qs];
        spart[((size_t)qs * nsl + P.sl) * NTH + th0 + (size_t)jb * a.H] = s;
      }
      for (int idx = threadIdx.x; idx < nv * DVS; idx += kThreads) {
        const int jb = idx / DVS, i = idx % DVS;
        from_f32(static_cast<E*>(a.dv) + (th0 + (size_t)jb * a.H) * a.dv_ + P.i0 + i, dvb[idx]);
      }
#pragma unroll
      for (int m = 0; m < QPT; ++m) qv[m] = qn[m];
#pragma unroll
      for (int j = 0; j < NQ; ++j) Sc[j] = Sn[j];
    }
  }
  if (a.dS0) {
#pragma unroll
    for (int j = 0; j < NQ; ++j) *reinterpret_cast<float4*>(a.dS0 + row * DK + 4 * P.l8 + 32 * j) = dS[j];
  }
}

// dq, dk (and per-channel dalpha) per (token-head, 4 columns); dbeta and scalar
// dalpha by the first thread of each token-head.
template <typename E, int DK, int MODE>
__global__ __launch_bounds__(256) void bwd_reduce(BackwardArgs a, const float* __restrict__ part,
                                                  const float* __restrict__ spart) {
  constexpr int NCOL = BwdLds<E, DK, MODE>::NCOL;
  const int nsl = a.dv_ / DVS;
  const size_t NTH = (size_t)a.B * a.T * a.H;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= NTH * (DK / 4)) return;
  const size_t th = idx / (DK / 4);
  const int c = (int)(idx % (DK / 4)) * 4;
#pragma unroll
  for (int qc = 0; qc < NCOL; ++qc) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int sl = 0; sl < nsl; ++sl) {
      const float4 x = *reinterpret_cast<const float4*>(part + ((size_t)qc * nsl + sl) * NTH * DK + th * DK + c);
      s = make_float4(s.x + x.x, s.y + x.y, s.z + x.z, s.w + x.w);
    }
    if (qc < 2) {
      E* o = static_cast<E*>(qc == 0 ? a.dq : a.dk) + th * DK + c;
      from_f32(o + 0, s.x);
      from_f32(o + 1, s.y);
      from_f32(o + 2, s.z);
      from_f32(o + 3, s.w);
    } else {
      *reinterpret_cast<float4*>(a.dalpha + th * DK + c) = s;
    }
  }
  if (c == 0) {
    float sb = 0.f, sa = 0.f;
    for (int sl = 0; sl < nsl; ++sl) {
      sb += spart[(size_t)sl * NTH + th];
      sa += spart[((size_t)nsl + sl) * NTH + th];
    }
    a.dbeta[th] = sb;
    if (MODE == 1) a.dalpha[th] = sa;
  }
}

struct BwdWs {
  size_t ck, part, spart, total;
};
BwdWs bwd_ws(int B, int T, int H, int dk, int dv, int mode) {
  const size_t nck = ((size_t)T + CK - 1) / CK, NTH = (size_t)B * T * H, nsl = dv / DVS;
  const size_t ncol = mode == 2 ? 3 : 2;
  BwdWs w;
  w.ck = 0;
  w.part = w.ck + (size_t)B * H * nck * dv * dk * 4;
  w.spart = w.part + ncol * nsl * NTH * dk * 4;
  w.total = w.spart + 2 * nsl * NTH * 4;
  return w;
}

template <typename E, int DK, int MODE>
hipError_t launch_mode(const BackwardArgs& a, void* ws, hipStream_t stream) {
  const BwdWs w = bwd_ws(a.B, a.T, a.H, DK, a.dv_, MODE);
  unsigned char* base = static_cast<unsigned char*>(ws);
  float* ck = reinterpret_cast<float*>(base + w.ck);
  float* part = reinterpret_cast<float*>(base + w.part);
  float* spart = reinterpret_cast<float*>(base + w.spart);
  const dim3 grid((unsigned)((size_t)a.B * a.H * (a.dv_ / DVS))), block(kThreads);
  if (a.T > 0) hipLaunchKernelGGL((bwd_checkpoint<E, DK, MODE>), grid, block, 0, stream, a, ck);
  hipLaunchKernelGGL((bwd_reverse<E, DK, MODE>), grid, block, 0, stream, a, ck, part, spart);
  const size_t n = (size_t)a.B * a.T * a.H * (DK / 4);
  if (n > 0)
    hipLaunchKernelGGL((bwd_reduce<E, DK, MODE>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, a,
                       part, spart);
  return hipGetLastError();
}

template <typename E, int DK>
hipError_t launch_dk(const BackwardArgs& a, void* ws, hipStream_t stream) {
  if (a.mode == 0) return launch_mode<E, DK, 0>(a, ws, stream);
  if (a.mode == 1) return launch_mode<E, DK, 1>(a, ws, stream);
  return launch_mode<E, DK, 2>(a, ws, stream);
}

}  // namespace

size_t backward_workspace_bytes(int B, int T, int H, int dk, int dv, int dtype, int mode) {
  if (chunk_backward_applies(T, dk, dv, dtype, mode)) return chunk_backward_workspace_bytes(B, T, H, dk, dv, mode);
  return bwd_ws(B, T, H, dk, dv, mode).total;
}

hipError_t launch_backward(const BackwardArgs& a, void* workspace, hipStream_t stream) {
  if (chunk_backward_applies(a.T, a.dk_, a.dv_, a.dtype, a.mode)) return launch_chunk_backward(a, workspace, stream);
  if (a.dtype == 1)
    return a.dk_ == 128 ? launch_dk<__bf16, 128>(a, workspace, stream) : launch_dk<__bf16, 64>(a, workspace, stream);
  return a.dk_ == 128 ? launch_dk<float, 128>(a, workspace, stream) : launch_dk<float, 64>(a, workspace, stream);
}

}  // namespace gdn
