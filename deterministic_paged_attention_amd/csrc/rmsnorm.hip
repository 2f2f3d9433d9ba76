// Per-row RMSNorm with a reduction tree fixed by the hidden size alone.
//
// Record "Deterministic and bit-exact inference" (field technical, Invariance):
// RMSNorm is made batch-invariant by giving each row one reduction order that
// does not depend on how many rows are in the call.  One workgroup owns one
// row; thread i owns the 8-element chunks i, i + 256, i + 512, ... and sums
// their squares in that order; the 64 lanes of a wave combine by a fixed xor
// butterfly; the four wave sums are added in wave order.  Nothing here depends
// on M or on the row index.
//   y = x * (sum x^2 / H + eps)^(-1/2) * gamma, fp32 throughout, one bf16 rounding.

#include "bi_internal.h"

namespace bi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

// ADD = false: x is the row.  ADD = true: the row is s = bf16(a + b)
// (elementwise fp32 add, one bf16 rounding, the residual add of a decoder
// block), written to s and then normalised: the values and the reduction
// tree are exactly those of the add followed by the plain kernel on s.
// Each thread reads back only the chunks it wrote, so s may alias a or b.
template <bool ADD>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* x, int64_t ldx, const uint16_t* xb,
                                                      int64_t ldxb, uint16_t* s, int64_t lds,
                                                      const uint16_t* gamma, float eps, int64_t H, uint16_t* y,
                                                      int64_t ldy) {
  __shared__ float wsum[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* xr = x + row * ldx;
  uint16_t* yr = y + row * ldy;
  const int64_t nchunk = H / 8;

  float ss = 0.f;
  for (int64_t c = tid; c < nchunk; c += 256) {
    u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * c);
    if constexpr (ADD) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(xb + row * ldxb + 8 * c);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = pack_bf16(bf16_lo(v[e]) + bf16_lo(w[e]), bf16_hi(v[e]) + bf16_hi(w[e]));
      *reinterpret_cast<u32x4*>(s + row * lds + 8 * c) = v;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float lo = bf16_lo(v[e]);
      const float hi = bf16_hi(v[e]);
      ss = __builtin_fmaf(lo, lo, ss);
      ss = __builtin_fmaf(hi, hi, ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = ss;
  __syncthreads();
  const float total = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  const float inv = 1.0f / __builtin_sqrtf(total / (float)H + eps);

  const uint16_t* rr = ADD ? (const uint16_t*)(s + row * lds) : xr;
  for (int64_t c = tid; c < nchunk; c += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(rr + 8 * c);
    const u32x4 g = *reinterpret_cast<const u32x4*>(gamma + 8 * c);
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = (__bf16)((bf16_lo(v[e]) * inv) * bf16_lo(g[e]));
      o[2 * e + 1] = (__bf16)((bf16_hi(v[e]) * inv) * bf16_hi(g[e]));
    }
    *reinterpret_cast<bf16x8*>(yr + 8 * c) = o;
  }
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps, int64_t M,
                          int64_t H, uint16_t* y, int64_t ldy, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel<false>, dim3((unsigned)M), dim3(256), 0, stream, x, ldx, nullptr, (int64_t)0,
                     nullptr, (int64_t)0, gamma, eps, H, y, ldy);
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, uint16_t* s,
                              int64_t lds, const uint16_t* gamma, float eps, int64_t M, int64_t H, uint16_t* y,
                              int64_t ldy, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  hipLaunchKernelGGL(rmsnorm_kernel<true>, dim3((unsigned)M), dim3(256), 0, stream, a, lda, b, ldb, s, lds, gamma,
                     eps, H, y, ldy);
  return hipGetLastError();
}

}  // namespace bi
