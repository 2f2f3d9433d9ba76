// Streaming-read reference kernel, for measurement only.
//
// The decode split kernel is bound by HBM bandwidth; its roofline is quoted
// against MI355X's published 8 TB/s and, beside it, against what a plain
// read of one large contiguous buffer reaches on the same GPU.  This kernel
// is that plain read: each workgroup reads one contiguous chunk of the
// buffer, 16-byte non-temporal loads, sixteen per thread in flight (a probe
// of read kernels on MI355X: contiguous per-workgroup chunks reached about
// 7.1 TB/s where a grid-stride loop over the whole buffer stayed at 6.2-6.9);
// the chunks are xor-folded so that no load can be dropped, and each
// workgroup writes the xor of what it read to sink[workgroup].  The xor of all
// sink words equals the xor of all 32-bit words of the buffer, which is how the
// tests check that every byte was read.

#include "bi_internal.h"

namespace bi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 16;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                 uint32_t* __restrict__ sink) {
  // Chunk [b, e) of this workgroup, in 16-byte units.
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b = min((int64_t)blockIdx.x * per, n16);
  const int64_t e = min(b + per, n16);
  int64_t i = b + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kReadUnroll - 1) * kReadThreads < e; i += kReadUnroll * kReadThreads) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) v[j] = __builtin_nontemporal_load(src + i + j * kReadThreads);
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) acc ^= v[j];
  }
  for (; i < e; i += kReadThreads) acc ^= __builtin_nontemporal_load(src + i);
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x ^= __shfl_xor(x, off);
  __shared__ uint32_t wave_x[kReadThreads / 64];
  if ((threadIdx.x & 63) == 0) wave_x[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kReadThreads / 64; ++w) t ^= wave_x[w];
    sink[blockIdx.x] = t;
  }
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(kStreamReadGroups), dim3(kReadThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace bi
