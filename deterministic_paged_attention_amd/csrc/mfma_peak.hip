// MFMA throughput reference kernel, for measurement only.
//
// The GEMM's utilisation is quoted against MI355X's published dense bf16
// peak and, beside it, against what the matrix cores sustain on this GPU:
// every wave of a full grid issues long runs of the GEMM's own instruction
// (v_mfma_f32_16x16x32_bf16) into eight independent accumulators, so nothing
// but the MFMA pipes bounds it.  Each wave then adds element 0 of its
// accumulators into sink[wave] (so the MFMAs cannot be dropped); with
// fragments of all ones every MFMA adds 32 to each accumulator element, which
// is how the tests check the instruction count.

#include "bi_internal.h"

namespace bi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kPeakThreads = 256;
constexpr int kPeakAcc = 8;      // independent accumulators per wave
constexpr int kPeakUnroll = 4;   // MFMA rounds per loop iteration

__global__ __launch_bounds__(kPeakThreads) void mfma_peak_kernel(float value, int32_t rounds, float* sink) {
  bf16x8 x;
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (__bf16)value;
  f32x4 acc[kPeakAcc];
#pragma unroll
  for (int j = 0; j < kPeakAcc; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r = 0; r < rounds; r += kPeakUnroll) {
#pragma unroll
    for (int u = 0; u < kPeakUnroll; ++u)
#pragma unroll
      for (int j = 0; j < kPeakAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x, x, acc[j], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int j = 0; j < kPeakAcc; ++j) t += acc[j][0];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kPeakThreads / 64) + (threadIdx.x >> 6)] = t;
}

}  // namespace

hipError_t launch_mfma_peak(float value, int32_t rounds, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(kMfmaPeakGroups), dim3(kPeakThreads), 0, stream, value, rounds, sink);
  return hipGetLastError();
}

int64_t mfma_peak_flops(int32_t rounds) {
  // waves x rounds x accumulators x (16 x 16 x 32 multiply-adds = 16384 flops)
  return (int64_t)kMfmaPeakGroups * (kPeakThreads / 64) * rounds * kPeakAcc * 16384;
}

}  // namespace bi
