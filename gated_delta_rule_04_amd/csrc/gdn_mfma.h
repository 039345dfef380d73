// MFMA tile helpers for gfx950 (CDNA4), wave64.
//
// All products in the chunk kernels are "NT" products with both operands stored
// in LDS with the contraction index contiguous:
//     C[m][n] += sum_k A[m][k] * B[n][k]
// One call computes one 32x32 fp32 tile.  Operand fragments: lane l reads the
// eight consecutive k values A[l % 32][k0 + 8 (l / 32) + 0..7] (one 16-byte LDS
// read for bf16, two for fp32) and the same for B.
//   bf16: one v_mfma_f32_32x32x16_bf16 per 16 k values.
//   fp32: eight v_mfma_f32_32x32x2f32 per 16 k values; MFMA m consumes k value
//         8 (l / 32) + m of each lane, which is a permutation of the k order of
//         the sum and leaves the result a full-fp32 dot product.
// Accumulator element v of lane l holds C[row][col] with
//     row = 8 (v / 4) + 4 (l / 32) + (v % 4),   col = l % 32.
// (Layouts checked on the device against a host product.)
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes moved as one value (a native vector, so copies stay in registers).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename E>
struct Frag;

template <>
struct Frag<__bf16> {
  bf16x8 v;
};

template <>
struct Frag<float> {
  float4 lo, hi;
};

__device__ inline Frag<__bf16> frag_load(const __bf16* p) {
  Frag<__bf16> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}

__device__ inline Frag<float> frag_load(const float* p) {
  Frag<float> f;
  f.lo = *reinterpret_cast<const float4*>(p);
  f.hi = *reinterpret_cast<const float4*>(p + 4);
  return f;
}

__device__ inline void mma16(f32x16& acc, const Frag<__bf16>& a, const Frag<__bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ inline void mma16(f32x16& acc, const Frag<float>& a, const Frag<float>& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
}

// The helpers below are fully unrolled over the NK k steps.  The fragments of
// step s + kAhead are loaded before the MFMAs of step s are issued, and
// scheduling fences keep that order (left alone, the scheduler moves each
// load next to its MFMA and the LDS latency of every step is exposed).
constexpr int kAhead = 2;

__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Rows of a row-swizzled bf16 LDS buffer keep their 16-byte chunks at index
// chunk ^ swz(row), swz(row) = (row / 4) % 4.  For a row stride of 16 mod 64
// dwords this puts the 16-byte reads of 16 consecutive rows and the transposed
// reads of 4 consecutive rows into distinct banks.
__device__ inline int swz(int row) { return (row >> 2) & 3; }
__device__ inline int swz_col(int row, int col) { return (((col >> 3) ^ swz(row)) << 3) | (col & 7); }

// acc += A[0:32, 0:16 NK] * B[0:32, 0:16 NK]^T, A and B in LDS with leading
// dimensions lda and ldb (elements), k contiguous.  With SWA the rows of A are
// row-swizzled (the tile's first row a multiple of 16).  Fragments are loaded
// AH k steps ahead.
template <int NK, typename E, bool SWA = false, int AH = kAhead>
__device__ inline void tile_nt_k(f32x16& acc, const E* A, int lda, const E* B, int ldb, int lane) {
  const int sa = SWA ? swz(lane & 31) : 0;
  const E* pa = A + (lane & 31) * lda;
  const E* pb = B + (lane & 31) * ldb + (lane >> 5) * 8;
  auto oa = [&](int s) { return (((2 * s + (lane >> 5)) ^ sa) << 3); };
  Frag<E> fa[NK], fb[NK];
#pragma unroll
  for (int s = 0; s < AH && s < NK; ++s) {
    fa[s] = frag_load(pa + oa(s));
    fb[s] = frag_load(pb + 16 * s);
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    if (s + AH < NK) {
      fa[s + AH] = frag_load(pa + oa(s + AH));
      fb[s + AH] = frag_load(pb + 16 * (s + AH));
    }
    sched_fence();
    mma16(acc, fa[s], fb[s]);
    sched_fence();
  }
}

// Two tiles that share the B operand: acc0 += A0 B^T, acc1 += A1 B^T, or with
// T1 the second one transposed, acc1 += B A1^T (a fragment has the same
// register layout as an A and as a B operand).  Fragments are loaded AH k
// steps ahead.  A0 has leading dimension lda0 and, with SW0, row-swizzled rows
// (the tile's first row a multiple of 16).
template <int NK, typename E, bool T1 = false, int AH = kAhead, bool SW0 = false>
__device__ inline void tile_nt2_shared_b(f32x16& acc0, f32x16& acc1, const E* A0, const E* A1,
                                         int lda0, int lda, const E* B, int ldb, int lane) {
  const int ra = (lane & 31) * lda + (lane >> 5) * 8;
  const E* pb = B + (lane & 31) * ldb + (lane >> 5) * 8;
  const int s0 = SW0 ? swz(lane & 31) : 0;
  const E* p0 = A0 + (lane & 31) * lda0;
  auto o0 = [&](int s) { return (((2 * s + (lane >> 5)) ^ s0) << 3); };
  Frag<E> fb[NK], f0[NK], f1[NK];
#pragma unroll
  for (int s = 0; s < AH && s < NK; ++s) {
    fb[s] = frag_load(pb + 16 * s);
    f0[s] = frag_load(p0 + o0(s));
    f1[s] = frag_load(A1 + ra + 16 * s);
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    if (s + AH < NK) {
      const int t = s + AH;
      fb[t] = frag_load(pb + 16 * t);
      f0[t] = frag_load(p0 + o0(t));
      f1[t] = frag_load(A1 + ra + 16 * t);
    }
    sched_fence();
    mma16(acc0, f0[s], fb[s]);
    if constexpr (T1) mma16(acc1, fb[s], f1[s]);
    else mma16(acc1, f1[s], fb[s]);
    sched_fence();
  }
}

// Two independent tiles, interleaved: acc0 += A0 B0^T, acc1 += A1 B1^T.
template <int NK, typename E>
__device__ inline void tile_nt2_pairs(f32x16& acc0, f32x16& acc1, const E* A0, const E* B0,
                                      const E* A1, const E* B1, int ld, int lane) {
  const int ro = (lane & 31) * ld + (lane >> 5) * 8;
  Frag<E> a0[NK], b0[NK], a1[NK], b1[NK];
#pragma unroll
  for (int s = 0; s < kAhead && s < NK; ++s) {
    a0[s] = frag_load(A0 + ro + 16 * s);
    b0[s] = frag_load(B0 + ro + 16 * s);
    a1[s] = frag_load(A1 + ro + 16 * s);
    b1[s] = frag_load(B1 + ro + 16 * s);
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    if (s + kAhead < NK) {
      const int o = ro + 16 * (s + kAhead), t = s + kAhead;
      a0[t] = frag_load(A0 + o);
      b0[t] = frag_load(B0 + o);
      a1[t] = frag_load(A1 + o);
      b1[t] = frag_load(B1 + o);
    }
    sched_fence();
    mma16(acc0, a0[s], b0[s]);
    mma16(acc1, a1[s], b1[s]);
    sched_fence();
  }
}

// Three tiles at once (independent accumulation chains):
//   x += Ax B^T, o += Ao B^T   (shared B; A leading dimension lda, B ldb)
//   p += Pa Pb^T               (both leading dimension lda)
template <int NK, typename E>
__device__ inline void tile_nt3(f32x16& x, f32x16& o, f32x16& p, const E* Ax, const E* Ao,
                                const E* B, const E* Pa, const E* Pb, int lda, int ldb, int lane) {
  const int ra = (lane & 31) * lda + (lane >> 5) * 8;
  const int rb = (lane & 31) * ldb + (lane >> 5) * 8;
  Frag<E> fb[NK], fx[NK], fo[NK], fpa[NK], fpb[NK];
#pragma unroll
  for (int s = 0; s < kAhead && s < NK; ++s) {
    fb[s] = frag_load(B + rb + 16 * s);
    fx[s] = frag_load(Ax + ra + 16 * s);
    fo[s] = frag_load(Ao + ra + 16 * s);
    fpa[s] = frag_load(Pa + ra + 16 * s);
    fpb[s] = frag_load(Pb + ra + 16 * s);
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    if (s + kAhead < NK) {
      const int t = s + kAhead, oa = ra + 16 * t;
      fb[t] = frag_load(B + rb + 16 * t);
      fx[t] = frag_load(Ax + oa);
      fo[t] = frag_load(Ao + oa);
      fpa[t] = frag_load(Pa + oa);
      fpb[t] = frag_load(Pb + oa);
    }
    sched_fence();
    mma16(x, fx[s], fb[s]);
    mma16(p, fpa[s], fpb[s]);
    mma16(o, fo[s], fb[s]);
    sched_fence();
  }
}

// ---- products whose B operand is an accumulator tile (bf16) ----
// A 32x32 accumulator tile can be the B operand of the next product as it
// stands: lane l holds rows 8g + 4h + e (g, e = 0..3, h = l / 32) of column
// l % 32, so the 16-row k step s takes the lane's rows 16s + 4h + 0..3 and
// 16s + 8 + 4h + 0..3.  The A operand is then read from LDS in that same k
// order; the sum over k is unchanged.

// A fragment (row-major bf16 row of lane l % 32) for the k step covering
// k0 .. k0 + 15, in the accumulator's k order.
__device__ inline bf16x8 frag_perm(const __bf16* row, int k0, int h) {
  const uint2 lo = *reinterpret_cast<const uint2*>(row + k0 + 4 * h);
  const uint2 hi = *reinterpret_cast<const uint2*>(row + k0 + 8 + 4 * h);
  return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
}

// B fragment for k step s (rows 16s .. 16s + 15) of an fp32 accumulator tile,
// rounded to bf16.
__device__ inline bf16x8 frag_acc(const f32x16& acc, int s) {
  bf16x8 f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f[j] = (__bf16)acc[8 * s + j];
    f[4 + j] = (__bf16)acc[8 * s + 4 + j];
  }
  return f;
}

// Transposed LDS read (ds_read_b64_tr_b16, gfx950) of a row-major bf16 matrix:
// every 16-lane group g of the wave receives a 4 x 16 block, lane l getting
// M[r0 + e][c0 + (l & 15)] for e = 0..3, where r0 and c0 are the group's (the
// same in all its lanes).  The instruction has lane s of a group read the 8
// bytes at row r0 + s / 4, columns c0 + 4 (s % 4) .. + 3, and hands element j
// of that read to lane 4 (s % 4) + j of the group as its element s / 4.
template <bool SW = false>
__device__ inline uint2 tr_read4(const __bf16* M, int ld, int r0, int c0, int lane) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const int s = lane & 15, r = r0 + (s >> 2), c = c0 + 4 * (s & 3);
  const __bf16* p = M + r * ld + (SW ? swz_col(r, c) : c);
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(uint2, v);
}

// A fragment for the k step covering k0 .. k0 + 15 in the accumulator's k order
// (as frag_perm) taken down a column: lane l receives M[k][c0 + l % 32] for the
// rows k of that order, out of a row-major matrix whose rows are the k index
// (with SW, row-swizzled).
template <bool SW = false>
__device__ inline bf16x8 frag_perm_tr(const __bf16* M, int ld, int k0, int c0, int lane) {
  const int h = lane >> 5, c = c0 + 16 * ((lane >> 4) & 1);
  const uint2 lo = tr_read4<SW>(M, ld, k0 + 4 * h, c, lane);
  const uint2 hi = tr_read4<SW>(M, ld, k0 + 8 + 4 * h, c, lane);
  return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
}

__device__ inline void mma_bf16(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
}

// fp32 16x16 tile step, four k values: lane l supplies A[l % 16][kappa] and
// B[kappa][l % 16] for one k index kappa of its choice (A and B must agree);
// accumulator element v of lane l is C[4 (l / 16) + v][l % 16].
__device__ inline f32x4 mma_f32_16x16(float a, float b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

__device__ inline f32x4 zero4() {
  f32x4 z;
  z[0] = z[1] = z[2] = z[3] = 0.f;
  return z;
}

// 32-bit word i (compile-time after unrolling) of a 16-byte chunk.
__device__ inline uint32_t word_of(const u32x4& u, int i) { return u[i]; }

__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row of accumulator element (4 g + e) for this lane: 8 g + 4 (lane / 32) + e.
__device__ inline int acc_row(int g, int e, int lane) { return 8 * g + 4 * (lane >> 5) + e; }

__device__ inline float bf16_bits_to_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

template <typename E>
__device__ inline E to_elem(float x);
template <>
__device__ inline float to_elem<float>(float x) { return x; }
template <>
__device__ inline __bf16 to_elem<__bf16>(float x) { return (__bf16)x; }

// Store four consecutive elements (8 or 16 bytes).
__device__ inline void store4(__bf16* p, float a, float b, float c, float d) {
  bf16x4 t;
  t[0] = (__bf16)a; t[1] = (__bf16)b; t[2] = (__bf16)c; t[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(p) = t;
}
__device__ inline void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

// Four consecutive elements as fp32 (one 8- or 16-byte LDS read).
__device__ inline float4 load4_elem(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ inline float4 load4_elem(const __bf16* p) {
  const uint2 w = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                     __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

}  // namespace gdn
