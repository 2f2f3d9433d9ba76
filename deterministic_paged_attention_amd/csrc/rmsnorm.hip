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

__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                                                      float eps, int64_t H, uint16_t* y, int64_t ldy) {
  __shared__ float wsum[4];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* xr = x + row * ldx;
  uint16_t* yr = y + row * ldy;
  const int64_t nchunk = H / 8;

  float ss = 0.f;
  for (int64_t c = tid; c < nchunk; c += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * c);
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

  for (int64_t c = tid; c < nchunk; c += 256) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(xr + 8 * c);
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
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)M), dim3(256), 0, stream, x, ldx, gamma, eps, H, y, ldy);
  return hipGetLastError();
}

}  // namespace bi
