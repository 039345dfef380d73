// Decode step of the gated delta rule: one token, state updated in place.
//
// Per state row i (a value channel) the step is the recurrence body:
//   s_k = S_i D k,  s_q = S_i D q,  u_i = beta (v_i - s_k),
//   o_i = s_q + u_i (k . q),        S_i <- S_i D + u_i k^T
// which is the predict/correct reading of the Gated DeltaNet output ("Enhancing
// Linear Attention with Residual Learning" notes, section 1.2, Table 1) and needs
// the row only once for both dot products.  Rows are independent linear systems
// that share the key-side transition ("On State Reduction in Linear Attention"
// notes, section 2.5), so every row is handled by its own group of lanes with
// no cross-row communication.
//
// Layout of the work: LPR lanes share a state row (8 at d_k = 128, 16 at
// d_k = 64) and lane l owns its float4 columns {4l + 4 LPR j}, so each load
// instruction of a wave covers whole rows as contiguous segments (coalesced
// 128-bit accesses).  A thread holds one row at d_k = 128 (four float4; one
// 256-thread workgroup takes 32 rows of a (b, h) head) and d_v / 16 rows at
// d_k = 64 (one float4 each; one workgroup per head).  The fp32 rows are held
// in registers between the read and the write, and the two row dot products
// are finished with xor-shuffles over the row's lanes.
// Gated DeltaNet-2 (MODE 3; "Linear Attention Architectures" notes, section
// 2.6): the prediction reads the erase direction e = b * k, the target is
// w_i v_i and there is no beta: s_k = S_i D e, u_i = w_i v_i - s_k; the write
// and the output keep k.
// With the prologue on, q and k are normalised in fp32 registers (their norms
// are sums over the row's lanes like the dot products) and beta, alpha come
// from logits; the state traffic is unchanged.
// The state is touched once per step, so its loads and stores are marked
// non-temporal (they do not displace cached lines); with more, smaller
// workgroups than heads the reads of later workgroups overlap the writes of
// earlier ones.  Both raise the streaming rate (about 5.3 -> 6.0 TB/s for an
// HBM-resident state on MI355X).
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
// Lanes that share a state row and 16-byte state pieces per thread: d_k = 128
// takes 8 lanes per 512-byte row, one row per thread; d_k = 64 takes 16 lanes
// per 256-byte row (measured: 12.04 against 12.22 us per step with 8 lanes,
// batch 64, 16 heads, d_v = 128) and a whole head per workgroup, d_v / 16 rows
// per thread: with the vector gate loads and the staged token loads below,
// 12.5 -> 11.9 us per step with HBM-resident states and a fresh token per step
// (the layout alone about 12.55 us, the gate loads alone 12.4).  d_k = 128 keeps 32 rows per workgroup and issues all its loads at
// once: 2 or 4 rows per thread measured 23.8 and 24.8 us against 22.5, and
// with the staged loads below 24.2 and 24.5 (one row per thread: 24.3).
template <int DK> constexpr int lanes_per_row() { return DK == 64 ? 16 : 8; }
template <int DK, int DV> constexpr int f4_per_thread() { return DK == 64 ? DV / 16 : 4; }

// Wait until every vector memory load this wave has issued is back
// (s_waitcnt vmcnt(0); the other counters at their maximum: expcnt 7,
// lgkmcnt 15 in gfx9's encoding); the scheduling barriers keep the compiler
// from moving loads across it.
__device__ inline void wait_for_loads() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __builtin_amdgcn_sched_barrier(0);
}

// A zero the compiler cannot prove uniform: indexing the per-head gates with it
// turns their loads into vector loads.  A uniform index makes them scalar
// loads, whose round trip to memory is longer than the state rows' (measured:
// about 0.15 us per step of 12.5 with fresh tokens from HBM) and which every
// row's update waits for.
__device__ inline int lane_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline float4 load_state(const float* p) {
  const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(t.x, t.y, t.z, t.w);
}
__device__ inline void store_state(float* p, float4 v) {
  const f32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<f32x4*>(p));
}

__device__ inline float bf16_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Token values as loaded: four elements (fp32: a float4; bf16: two words) or
// one, converted to fp32 separately.
template <typename E> struct Raw;
template <> struct Raw<float> {
  using four = float4;
  using one = float;
};
template <> struct Raw<__bf16> {
  using four = uint2;
  using one = uint16_t;
};
__device__ inline float4 load_raw4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline uint2 load_raw4(const __bf16* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ inline float load_raw1(const float* p) { return *p; }
__device__ inline uint16_t load_raw1(const __bf16* p) { return *reinterpret_cast<const uint16_t*>(p); }
__device__ inline float4 to_f32x4(float4 x) { return x; }
__device__ inline float4 to_f32x4(uint2 w) {
  return make_float4(bf16_to_f32(w.x & 0xffff), bf16_to_f32(w.x >> 16), bf16_to_f32(w.y & 0xffff),
                     bf16_to_f32(w.y >> 16));
}
__device__ inline float to_f32(float x) { return x; }
__device__ inline float to_f32(uint16_t x) { return bf16_to_f32(x); }

__device__ inline float dot4(const float4& a, const float4& b) {
  return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w;
}

__device__ inline void store1(float* p, float x) { *p = x; }
__device__ inline void store1(__bf16* p, float x) { *p = (__bf16)x; }

// Sum over the LPR lanes that share a row (an aligned group of LPR lanes), by
// DPP moves inside a row of 16 lanes: the two quad steps, then the half-row
// and row mirrors (lane i of 8 takes lane 7 - i, lane i of 16 lane 15 - i);
// every lane of the group ends with the sum.  (Cross-lane moves through LDS
// would put an LDS round trip on each step of the reduction.)
template <int LPR>
__device__ inline float group_sum(float x) {
  static_assert(LPR == 8 || LPR == 16, "groups of 8 or 16 lanes");
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  if constexpr (LPR == 16)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));  // row_mirror
  return x;
}

template <typename E, int DK, int DV, int MODE, bool PRO>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  constexpr int LPR = lanes_per_row<DK>();               // lanes per row
  constexpr int NQ = DK / (4 * LPR);                     // float4 per lane per row
  constexpr int NR = f4_per_thread<DK, DV>() / NQ;       // rows per thread
  constexpr int RPW = kThreads / LPR;                    // rows per pass of the workgroup
  constexpr int RPG = RPW * NR;                          // rows per workgroup
  constexpr int GPH = DV / RPG;                          // workgroups per head
  static_assert(NQ >= 1 && NR >= 1 && GPH >= 1 && DV % RPG == 0, "unsupported head size");
  // Rows of a lane group: g + RPW m, so that every load instruction of a wave
  // covers whole rows that are consecutive in memory.  (Consecutive rows per
  // group, g NR + m, would make a group's v and o entries one 16-byte run, but
  // the waves' state accesses then become 256-byte pieces 2 KB apart: 12.29
  // against 12.08 us per step at d_k = 64 with HBM-resident states.)
  auto row = [](int g, int m) { return g + RPW * m; };
  // The token's and the gates' loads are issued only once the state rows are
  // in (an explicit wait): issued beside the state rows, these small loads
  // from the token arrays slowed the step by about 0.9 us of 12.7 at d_k = 64
  // (HBM-resident states, a fresh token per step from HBM).
  constexpr bool STAGE = DK == 64;

  const size_t bh = blockIdx.x / GPH;
  const int r0 = (blockIdx.x % GPH) * RPG;               // first state row of this workgroup
  const int l8 = threadIdx.x % LPR;                      // lane within the row's group
  const int g = threadIdx.x / LPR;                       // row within the workgroup

  const E* q = static_cast<const E*>(a.q) + bh * DK;
  const E* k = static_cast<const E*>(a.k) + bh * DK;
  const E* v = static_cast<const E*>(a.v) + bh * DV + r0;
  float* S = a.S + (bh * DV + r0) * (size_t)DK;
  E* o = static_cast<E*>(a.o) + bh * DV + r0;

  // State rows first: these are the bytes that matter, issue them early.
  float4 s[NR][NQ];
#pragma unroll
  for (int m = 0; m < NR; ++m)
#pragma unroll
    for (int j = 0; j < NQ; ++j) s[m][j] = load_state(S + (size_t)row(g, m) * DK + 4 * l8 + 4 * LPR * j);
  if constexpr (STAGE) wait_for_loads();

  // The token's values and gates: every load is issued, as loaded words,
  // before the first conversion (a conversion placed between the loads waits
  // for its own load while the later ones are not yet issued; 0.2 us per step
  // at d_k = 64 with a fresh token from HBM).
  using R4 = typename Raw<E>::four;
  using R1 = typename Raw<E>::one;
  R4 kw[NQ], qw[NQ], aw[NQ], bw[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    kw[j] = load_raw4(k + 4 * l8 + 4 * LPR * j);
    qw[j] = load_raw4(q + 4 * l8 + 4 * LPR * j);
    if (MODE >= 2) aw[j] = load_raw4(static_cast<const E*>(a.alpha) + bh * DK + 4 * l8 + 4 * LPR * j);
    if (MODE == 3) bw[j] = load_raw4(static_cast<const E*>(a.erase) + bh * DK + 4 * l8 + 4 * LPR * j);
  }
  const int z = DK == 64 ? lane_zero() : 0;   // (d_k = 128: scalar loads measured 0.2 us faster)
  float beta = MODE == 3 ? 1.f : a.beta[bh + z];
  float alpha = 1.f;
  if (MODE == 1) alpha = static_cast<const float*>(a.alpha)[bh + z];
  R1 vw[NR], ww[NR];
  auto load_v = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      vw[m] = load_raw1(v + row(g, m));
      if (MODE == 3) ww[m] = load_raw1(static_cast<const E*>(a.write) + bh * DV + r0 + row(g, m));   // target w_i v_i
    }
  };
  // (d_k = 128: the v loads after the gates' arithmetic and no barrier; with
  // the d_k = 64 order 0.1 - 0.4 us slower)
  if constexpr (STAGE) {
    load_v();
    __builtin_amdgcn_sched_barrier(0);
  }
  float4 kf[NQ], qf[NQ], af[NQ], bf[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    kf[j] = to_f32x4(kw[j]);
    qf[j] = to_f32x4(qw[j]);
    if (MODE >= 2) af[j] = to_f32x4(aw[j]);
    if (MODE == 3) bf[j] = to_f32x4(bw[j]);
  }
  if constexpr (PRO) {
    const Prologue& p = a.pro;
    const int h = (int)(bh % a.H);
    if (p.beta_logits) beta = sigmoid_f(beta);
    if (MODE == 1 && p.alpha_logits)
      alpha = __expf(fmaxf(-p.A[h] * softplus_f(alpha + (p.dt_bias ? p.dt_bias[h] : 0.f)), -100.f));
    if (MODE == 2 && p.alpha_logits) {
      const float ah = p.A[h];
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const int c = 4 * l8 + 4 * LPR * j;
        float4 b4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (p.dt_bias) {
          const float* bp = p.dt_bias + (size_t)h * DK + c;
          b4 = make_float4(bp[0], bp[1], bp[2], bp[3]);
        }
        af[j].x = __expf(fmaxf(-ah * softplus_f(af[j].x + b4.x), -100.f));
        af[j].y = __expf(fmaxf(-ah * softplus_f(af[j].y + b4.y), -100.f));
        af[j].z = __expf(fmaxf(-ah * softplus_f(af[j].z + b4.z), -100.f));
        af[j].w = __expf(fmaxf(-ah * softplus_f(af[j].w + b4.w), -100.f));
      }
    }
    if (p.qk_norm) {   // fp32, exact scaling of the loaded values
      float sk = dot4(kf[0], kf[0]), sq = dot4(qf[0], qf[0]);
#pragma unroll
      for (int j = 1; j < NQ; ++j) {
        sk += dot4(kf[j], kf[j]);
        sq += dot4(qf[j], qf[j]);
      }
      const float nk = rsqrtf(group_sum<LPR>(sk) + p.norm_eps);
      const float nq = rsqrtf(group_sum<LPR>(sq) + p.norm_eps);
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        kf[j] = make_float4(kf[j].x * nk, kf[j].y * nk, kf[j].z * nk, kf[j].w * nk);
        qf[j] = make_float4(qf[j].x * nq, qf[j].y * nq, qf[j].z * nq, qf[j].w * nq);
      }
    }
  }

  if constexpr (!STAGE) load_v();

  // k . q over the head (every group computes it; it is tiny)
  float kq = dot4(kf[0], qf[0]);
#pragma unroll
  for (int j = 1; j < NQ; ++j) kq += dot4(kf[j], qf[j]);
  kq = group_sum<LPR>(kq);

  // D k and D q for the per-channel decay (the scalar decay is applied to the sums)
  float4 kd[NQ], qd[NQ];
#pragma unroll
  for (int j = 0; j < NQ; ++j) {
    if (MODE == 3) {   // the prediction reads D e = D (b * k)
      kd[j] = make_float4(kf[j].x * bf[j].x * af[j].x, kf[j].y * bf[j].y * af[j].y,
                          kf[j].z * bf[j].z * af[j].z, kf[j].w * bf[j].w * af[j].w);
      qd[j] = make_float4(qf[j].x * af[j].x, qf[j].y * af[j].y, qf[j].z * af[j].z, qf[j].w * af[j].w);
    } else if (MODE == 2) {
      kd[j] = make_float4(kf[j].x * af[j].x, kf[j].y * af[j].y, kf[j].z * af[j].z, kf[j].w * af[j].w);
      qd[j] = make_float4(qf[j].x * af[j].x, qf[j].y * af[j].y, qf[j].z * af[j].z, qf[j].w * af[j].w);
    } else {
      kd[j] = kf[j];
      qd[j] = qf[j];
    }
  }

#pragma unroll
  for (int m = 0; m < NR; ++m) {
    // (sums start from their first term: an fp32 sum started at 0 keeps an
    // add of +0 per sum, which the compiler may not drop)
    float pk = dot4(s[m][0], kd[0]), pq = dot4(s[m][0], qd[0]);
#pragma unroll
    for (int j = 1; j < NQ; ++j) {
      pk += dot4(s[m][j], kd[j]);
      pq += dot4(s[m][j], qd[j]);
    }
    pk = group_sum<LPR>(pk);
    pq = group_sum<LPR>(pq);
    if (MODE == 1) {
      pk *= alpha;
      pq *= alpha;
    }
    // (v converted here, row by row: each row waits only for its own v)
    const float vm = MODE == 3 ? to_f32(vw[m]) * to_f32(ww[m]) : to_f32(vw[m]);
    const float u = beta * (vm - pk);
    const float out = pq + u * kq;
    if (l8 == 0) store1(o + row(g, m), out);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
      float4 d = MODE >= 2 ? af[j] : make_float4(alpha, alpha, alpha, alpha);
      float4 r;
      r.x = s[m][j].x * d.x + u * kf[j].x;
      r.y = s[m][j].y * d.y + u * kf[j].y;
      r.z = s[m][j].z * d.z + u * kf[j].z;
      r.w = s[m][j].w * d.w + u * kf[j].w;
      store_state(S + (size_t)row(g, m) * DK + 4 * l8 + 4 * LPR * j, r);
    }
  }
}

template <typename E, int DK, int DV>
hipError_t launch_mode(const DecodeArgs& a, hipStream_t stream) {
  constexpr int LPR = lanes_per_row<DK>();
  constexpr int RPG = kThreads / LPR * (f4_per_thread<DK, DV>() / (DK / (4 * LPR)));
  dim3 grid((unsigned)(a.B * a.H * (DV / RPG))), block(kThreads);
  const bool pro = a.pro.qk_norm || a.pro.beta_logits || a.pro.alpha_logits;
  switch (a.mode * 2 + (pro ? 1 : 0)) {
    case 0: hipLaunchKernelGGL((decode_kernel<E, DK, DV, 0, false>), grid, block, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((decode_kernel<E, DK, DV, 0, true>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((decode_kernel<E, DK, DV, 1, false>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((decode_kernel<E, DK, DV, 1, true>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((decode_kernel<E, DK, DV, 2, false>), grid, block, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((decode_kernel<E, DK, DV, 2, true>), grid, block, 0, stream, a); break;
    default: hipLaunchKernelGGL((decode_kernel<E, DK, DV, 3, false>), grid, block, 0, stream, a); break;
  }
  return hipGetLastError();
}

template <typename E>
hipError_t launch_dtype(const DecodeArgs& a, hipStream_t stream) {
  if (a.dk == 128 && a.dv == 128) return launch_mode<E, 128, 128>(a, stream);
  if (a.dk == 64 && a.dv == 128) return launch_mode<E, 64, 128>(a, stream);
  if (a.dk == 128 && a.dv == 64) return launch_mode<E, 128, 64>(a, stream);
  return launch_mode<E, 64, 64>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  return a.dtype == 1 ? launch_dtype<__bf16>(a, stream) : launch_dtype<float>(a, stream);
}

}  // namespace gdn
