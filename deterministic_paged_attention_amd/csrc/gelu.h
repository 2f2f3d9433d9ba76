// Gated GELU of one element, tanh form (the decoder's MLP activation):
//   gelu(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))),  result gelu(gate) * up
// in fp32 from bf16 inputs.  gated_gelu_kernel and the GEMM that applies it in
// its epilogue both call this one expression, so both round the same fp32
// value once to bf16.
#pragma once

#include <hip/hip_runtime.h>

namespace bi {

__device__ __forceinline__ float gated_gelu_f32(float x, float u) {
  const float inner = 0.7978845608028654f * (x + 0.044715f * x * x * x);
  const float gl = 0.5f * x * (1.0f + tanhf(inner));
  return gl * u;
}

}  // namespace bi
