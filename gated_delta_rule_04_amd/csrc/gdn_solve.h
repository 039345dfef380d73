// Unit-lower-triangular solve of one 64-token chunk, shared by the prefill's
// prep kernel and the chunk-level backward.
#pragma once

#include <hip/hip_runtime.h>

#include "gdn_mfma.h"

namespace gdn {
namespace solve_detail {

constexpr int C = 64;   // chunk length

// Sum over the four lanes of a quad (lanes 4c .. 4c + 3), result in all four.
__device__ inline float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));
  return x;
}

// T = (I + A)^-1 diag(beta) for one chunk, in LDS.
//   Am  A, fp32 [C][LDA]: read below the diagonal; inside the 16x16 diagonal
//       blocks the entries on and above the diagonal must be zero
//   Bt  beta [C] (zero for rows past the sequence end)
//   Li  scratch for L^-1 = (I + A)^-1, fp32 [C][LDA]; may be Am itself (every
//       step overwrites only blocks of A that it has finished reading)
//   Mt  scratch, fp32 [32][ldm]; in place it may be Am + 32 with ldm = LDA
//       (rows 0..31, columns 32..63 of L^-1 are above the diagonal and never
//       read)
//   Tm  T in the operand dtype: LDS [C][LDT] (it may
//       share Am's bytes unless Li is Am), or (DIRECT) the chunk record in
//       global memory, [C][C]
// All threads of the workgroup take part; it ends with a barrier unless DIRECT.
// COLUMNS: the diagonal blocks are inverted by wave 0 alone, one column per
// lane (a quarter of the vector instructions, a longer dependent chain: for
// kernels that run many workgroups per compute unit).
template <typename E>
struct SolveLd {
  static constexpr int LDA = C + 4;
  static constexpr int LDT = C + 16 / (int)sizeof(E);
  static constexpr int LDM = 32 + 4;
};

template <typename E, int LDM = SolveLd<E>::LDM, bool DIRECT = false, bool COLUMNS = false>
__device__ __attribute__((always_inline)) inline void tri_solve(const float* Am, float* Li, float* Mt,
                                                                const float* Bt, E* Tm, int tid) {
  constexpr int LDA = SolveLd<E>::LDA, LDT = DIRECT ? C : SolveLd<E>::LDT;
  const int lane = tid & 63, wave = tid >> 6;
  if constexpr (COLUMNS) {
    // (a) inverse of each unit-lower 16x16 diagonal block by forward
    // substitution down one column: lane 16 I + c of wave 0 takes column c of
    // block I, y_c = 1 and y_i = -sum_{j < i} A_ij y_j below it (y_j = 0 above
    // c, so every lane runs the same rows; above the diagonal y_i is -0).
    if (wave == 0) {
      const int I = lane >> 4, c = lane & 15;
      const float* ab = Am + (16 * I) * LDA + 16 * I;
      float y[16];
      y[0] = c == 0 ? 1.f : 0.f;
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        float s0 = 0.f, s1 = 0.f;   // (two partial sums: a shorter chain)
#pragma unroll
        for (int j4 = 0; j4 < i; j4 += 4) {
          const float4 a4 = *reinterpret_cast<const float4*>(ab + i * LDA + j4);
          const float av[4] = {a4.x, a4.y, a4.z, a4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (j4 + e >= i) break;
            if ((j4 + e) & 1)
              s1 += av[e] * y[j4 + e];
            else
              s0 += av[e] * y[j4 + e];
          }
        }
        y[i] = i == c ? 1.f : -(s0 + s1);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) Li[(16 * I + i) * LDA + 16 * I + c] = y[i];
    }
  } else {
    // (a) inverse of each unit-lower 16x16 diagonal block: wave w owns block w;
    // lane 4c + p computes column c, rows 4p .. 4p + 3, summing its part of each
    // row's dot product and finishing it across the quad.
    const int I = wave, c = lane >> 2, p = lane & 3;
    const float* arow = Am + (16 * I) * LDA + 16 * I + 4 * p;
    float y[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 a4 = *reinterpret_cast<const float4*>(arow + i * LDA);
      float part = a4.x * y[0] + a4.y * y[1] + a4.z * y[2] + a4.w * y[3];
      part = quad_sum(part);
      const float yi = i < c ? 0.f : (i == c ? 1.f : -part);
      if (p == (i >> 2)) y[i & 3] = yi;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Li[(16 * I + 4 * p + e) * LDA + 16 * I + c] = y[e];
  }
  __syncthreads();
  // (b) L^-1_{b+1,b} = -L^-1_{b+1,b+1} (A_{b+1,b} L^-1_{b,b}), b = 0, 2, fp32 MFMA
  // 16x16x4; lane l uses k index 4 (l / 16) + s in step s, so the first
  // product's accumulator is directly the second product's B operand.
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
  // (c) the 32x32 block L^-1_{1,0} = -L^-1_{11} (A_{10} L^-1_{00}).  L^-1_{00} and
  // L^-1_{11} are lower triangular: their rows 0..15 vanish in columns 16..31,
  // so those k steps take zero operands (selected, never read as data).
  const int mi = wave >> 1, ni = wave & 1, m16 = lane & 15, hq = lane >> 4;
  {
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int k = 4 * s + hq;
      const bool live = ni == 0 || s >= 4;
      const float av = Am[(32 + 16 * mi + m16) * LDA + k];
      const float bv = Li[k * LDA + 16 * ni + m16];
      acc = mma_f32_16x16(live ? av : 0.f, live ? bv : 0.f, acc);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) Mt[(16 * mi + 4 * hq + v) * LDM + 16 * ni + m16] = acc[v];
  }
  __syncthreads();   // A is dead from here: T takes its bytes
  {
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int k = 4 * s + hq;
      const bool live = mi == 1 || s < 4;
      const float av = Li[(32 + 16 * mi + m16) * LDA + 32 + k];
      const float bv = Mt[k * LDM + 16 * ni + m16];
      acc = mma_f32_16x16(live ? av : 0.f, live ? bv : 0.f, acc);
    }
    const float bj = Bt[16 * ni + m16];
#pragma unroll
    for (int v = 0; v < 4; ++v)
      Tm[(32 + 16 * mi + 4 * hq + v) * LDT + 16 * ni + m16] = to_elem<E>(-acc[v] * bj);
    // T on the two diagonal 32x32 blocks, zeros above them: 8 columns per thread
    const int q = tid >> 7, r = 32 * q + ((tid & 127) >> 2), jc = 32 * q + (tid & 3) * 8;
    float x[8];
#pragma unroll
    for (int q4 = 0; q4 < 2; ++q4) {
      const float4 l4 = *reinterpret_cast<const float4*>(Li + r * LDA + jc + 4 * q4);
      const float4 b4 = *reinterpret_cast<const float4*>(Bt + jc + 4 * q4);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) x[4 * q4 + e] = (jc + 4 * q4 + e <= r) ? lv[e] * bv[e] : 0.f;
    }
    store4(Tm + r * LDT + jc, x[0], x[1], x[2], x[3]);
    store4(Tm + r * LDT + jc + 4, x[4], x[5], x[6], x[7]);
    if (q == 0) {
      store4(Tm + r * LDT + 32 + (tid & 3) * 8, 0.f, 0.f, 0.f, 0.f);
      store4(Tm + r * LDT + 36 + (tid & 3) * 8, 0.f, 0.f, 0.f, 0.f);
    }
  }
  if constexpr (!DIRECT) __syncthreads();
}

}  // namespace solve_detail

using solve_detail::quad_sum;
using solve_detail::SolveLd;
using solve_detail::tri_solve;

}  // namespace gdn
