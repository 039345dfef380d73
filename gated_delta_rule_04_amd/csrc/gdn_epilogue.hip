// Output epilogue of the Gated DeltaNet mixer: a gated RMSNorm of every
// (token, head) output row (NextTransformer "method sources" page, baseline
// section, Gated DeltaNet entry: the output passes an RMSNorm, a gain and a
// SiLU gate; backend section: the output-gated RMSNorm):
//
//     y = o / sqrt(mean(o^2) + eps) * w * silu(g),   silu(g) = g / (1 + e^-g)
//
// over the d_v values of the row, w one gain per value channel.  The state
// kernels split d_v over workgroups, so the norm of a row is not known where
// its pieces are produced; this is its own streaming pass.  A row is spread
// over the 16-byte pieces of LPR lanes (its sum of squares is a sum over
// that lane group), loads and stores are non-temporal (every byte is touched
// once), arithmetic is fp32 and the output is rounded once to the dtype.
#include "gdn_epilogue.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4e __attribute__((ext_vector_type(4)));

template <typename E>
__device__ inline void unpack(const u32x4e& u, float* x);
template <>
__device__ inline void unpack<float>(const u32x4e& u, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(u[i]);
}
template <>
__device__ inline void unpack<__bf16>(const u32x4e& u, float* x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(u[i] << 16);
    x[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
  }
}

template <typename E>
__device__ inline u32x4e pack(const float* x);
template <>
__device__ inline u32x4e pack<float>(const float* x) {
  return u32x4e{__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]), __float_as_uint(x[3])};
}
template <>
__device__ inline u32x4e pack<__bf16>(const float* x) {
  u32x4e u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 lo = (__bf16)x[2 * i], hi = (__bf16)x[2 * i + 1];
    u[i] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  return u;
}

// Sum over aligned groups of N lanes (N = 8, 16 or 32), every lane of the
// group ending with the sum: DPP moves inside rows of 16 lanes (the two quad
// steps, then the half-row and row mirrors), one swap across rows for 32.
template <int N>
__device__ inline float group_sum(float x) {
  static_assert(N == 8 || N == 16 || N == 32, "groups of 8, 16 or 32 lanes");
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));   // quad [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));   // quad [2,3,0,1]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, true));  // row_half_mirror
  if constexpr (N >= 16)
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x140, 0xF, 0xF, true));  // row_mirror
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// 1 / sqrt(m) for m >= 0 by the hardware reciprocal square root (about 1 ulp);
// a mean square below 2^-100 (down to subnormals) is scaled into range first.
__device__ inline float rsqrt_scaled(float m) {
  const bool tiny = m < 0x1p-100f;
  const float r = __builtin_amdgcn_rsqf(tiny ? m * 0x1p64f : m);
  return tiny ? r * 0x1p32f : r;
}

constexpr int kRowsPerThread = 4;

// RPT rows per thread: lane group g of the workgroup takes rows g + RPW m, so
// that each load instruction of a wave covers consecutive rows; every row's
// loads are issued before the first row is computed.  Rows past the end
// re-read the last row and are not stored.
template <typename E, int DV>
__global__ __launch_bounds__(kThreads) void gated_rmsnorm_kernel(const E* o, const E* __restrict__ g,
                                                                 const float* __restrict__ w, E* y,
                                                                 long long rows, float eps) {
  constexpr int EPL = 16 / (int)sizeof(E);   // values per lane
  constexpr int LPR = DV / EPL;              // lanes per row
  constexpr int RPW = kThreads / LPR;        // rows per pass of the workgroup
  constexpr int RPT = kRowsPerThread;
  static_assert(LPR >= 8 && LPR <= 32 && (LPR & (LPR - 1)) == 0, "row lane group");
  const long long row0 = (long long)blockIdx.x * RPW * RPT + threadIdx.x / LPR;
  const int l = threadIdx.x % LPR;
  u32x4e ro[RPT], rg[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const size_t off = (size_t)min(row0 + RPW * m, rows - 1) * DV + (size_t)l * EPL;
    ro[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4e*>(o + off));
    rg[m] = __builtin_nontemporal_load(reinterpret_cast<const u32x4e*>(g + off));
  }
  float wv[EPL];
#pragma unroll
  for (int i = 0; i < EPL; i += 4) {
    const float4 t = *reinterpret_cast<const float4*>(w + l * EPL + i);
    wv[i] = t.x; wv[i + 1] = t.y; wv[i + 2] = t.z; wv[i + 3] = t.w;
  }
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    float x[EPL], gv[EPL];
    unpack<E>(ro[m], x);
    unpack<E>(rg[m], gv);
    float ss = x[0] * x[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) ss += x[i] * x[i];
    const float r = rsqrt_scaled(group_sum<LPR>(ss) * (1.f / DV) + eps);
    float z[EPL];
    // silu(g) = g / (1 + e^-g) by the hardware reciprocal (e^-g = inf gives -0, as the division)
#pragma unroll
    for (int i = 0; i < EPL; ++i) z[i] = x[i] * r * wv[i] * (gv[i] * __builtin_amdgcn_rcpf(1.f + __expf(-gv[i])));
    const long long row = row0 + RPW * m;
    if (row < rows)
      __builtin_nontemporal_store(pack<E>(z), reinterpret_cast<u32x4e*>(y + (size_t)row * DV + (size_t)l * EPL));
  }
}

template <typename E, int DV>
hipError_t launch_dv(const void* o, const void* g, const float* w, void* y, long long rows, float eps,
                     hipStream_t stream) {
  constexpr int RPB = kThreads / (DV / (16 / (int)sizeof(E))) * kRowsPerThread;   // rows per workgroup
  const long long blocks = (rows + RPB - 1) / RPB;
  hipLaunchKernelGGL((gated_rmsnorm_kernel<E, DV>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const E*>(o), static_cast<const E*>(g), w, static_cast<E*>(y), rows, eps);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_rmsnorm(const void* o, const void* g, const float* w, void* y, long long rows, int dv,
                                float eps, int dtype, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  if (dtype == 1)
    return dv == 128 ? launch_dv<__bf16, 128>(o, g, w, y, rows, eps, stream)
                     : launch_dv<__bf16, 64>(o, g, w, y, rows, eps, stream);
  return dv == 128 ? launch_dv<float, 128>(o, g, w, y, rows, eps, stream)
                   : launch_dv<float, 64>(o, g, w, y, rows, eps, stream);
}

}  // namespace gdn
