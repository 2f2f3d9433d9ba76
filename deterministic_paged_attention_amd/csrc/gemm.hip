// Matrix product c[m,n] = sum_k a[m,k] w[n,k] with a K path fixed independently of M.
//
// Vosti deep-dive blog (深入解析 Vosti), §6.1: the matmul contract asks that
// row x of c depend only on row x of a and on b, bitwise, for any M; its proof
// obligations are a zero-initialised accumulator, the same iteration order and
// the same reduction order over a shared K.  Here every output element has one
// fp32 accumulator, starts at zero, and is updated by one 16x16x32 bf16 MFMA
// per 32-wide K step, in increasing K order — the same instruction sequence
// whatever M is and wherever the row sits in its tile.  There is no split of K.
//
// Mapping: one wave owns a 16 (n) x 16 (m) output block and computes C^T =
// W A^T, so that a lane ends with four consecutive n of one m (one vector
// store).  A operand = 16 rows of w, B operand = 16 rows of a; both are read
// straight from global memory as 16-byte runs along K (K-major storage).
//
// The split-K comparator (measurement only) runs the same kernel over K
// sub-ranges into fp32 partials and sums them in split order afterwards, so
// its reduction order follows the number of splits.

#include "bi_internal.h"

namespace bi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;    // waves per workgroup, side by side along n
constexpr int kUnroll = 8;   // K steps whose operands are loaded together

// out_kind: 0 = bf16 c, 1 = fp32 c.  K range [k_begin, k_begin + k_count).
__global__ __launch_bounds__(64 * kWaves) void gemm_kernel(const uint16_t* a, int64_t lda, const uint16_t* w,
                                                           int64_t ldw, void* c, int64_t ldc, int out_kind,
                                                           int64_t M, int64_t N, int64_t k_count,
                                                           int64_t split_stride_elems) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;
  const int g4 = lane >> 4;
  const int64_t n0 = ((int64_t)blockIdx.x * kWaves + wave) * 16;
  const int64_t m0 = (int64_t)blockIdx.y * 16;
  if (n0 >= N) return;
  const int64_t k_begin = (int64_t)blockIdx.z * k_count;

  const bool n_ok = n0 + r < N;
  const bool m_ok = m0 + r < M;
  const uint16_t* wp = w + (n_ok ? (n0 + r) : 0) * ldw + k_begin + 8 * g4;
  const uint16_t* ap = a + (m_ok ? (m0 + r) : 0) * lda + k_begin + 8 * g4;

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const int64_t nsteps = k_count / 32;
  int64_t st = 0;
  for (; st + kUnroll <= nsteps; st += kUnroll) {
    u32x4 wf[kUnroll], af[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      wf[u] = n_ok ? *reinterpret_cast<const u32x4*>(wp + (st + u) * 32) : u32x4{0u, 0u, 0u, 0u};
      af[u] = m_ok ? *reinterpret_cast<const u32x4*>(ap + (st + u) * 32) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[u]),
                                                    __builtin_bit_cast(bf16x8, af[u]), acc, 0, 0, 0);
  }
  for (; st < nsteps; ++st) {
    const u32x4 wf = n_ok ? *reinterpret_cast<const u32x4*>(wp + st * 32) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 af = m_ok ? *reinterpret_cast<const u32x4*>(ap + st * 32) : u32x4{0u, 0u, 0u, 0u};
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf), __builtin_bit_cast(bf16x8, af),
                                                  acc, 0, 0, 0);
  }

  // Lane holds C^T[n0 + 4*g4 + i][m0 + r], i = 0..3.
  if (!m_ok) return;
  const int64_t m = m0 + r;
  const int64_t nb = n0 + 4 * g4;
  if (out_kind == 1) {
    float* cp = reinterpret_cast<float*>(c) + (int64_t)blockIdx.z * split_stride_elems + m * ldc + nb;
    if (nb + 4 <= N && ((reinterpret_cast<uintptr_t>(cp) & 15) == 0)) {
      *reinterpret_cast<f32x4*>(cp) = acc;
    } else {
      for (int i = 0; i < 4; ++i)
        if (nb + i < N) cp[i] = acc[i];
    }
  } else {
    uint16_t* cp = reinterpret_cast<uint16_t*>(c) + m * ldc + nb;
    bf16x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = (__bf16)acc[i];
    if (nb + 4 <= N && ((reinterpret_cast<uintptr_t>(cp) & 7) == 0)) {
      *reinterpret_cast<bf16x4*>(cp) = o;
    } else {
      const u32x2 bits = __builtin_bit_cast(u32x2, o);
      for (int i = 0; i < 4; ++i)
        if (nb + i < N) cp[i] = (uint16_t)((i & 1) ? (bits[i >> 1] >> 16) : (bits[i >> 1] & 0xffffu));
    }
  }
}

// c[m,n] = sum over splits z = 0..k_splits-1, in order, of partial[z][m][n].
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* partial, int32_t k_splits, int64_t M,
                                                            int64_t N, void* c, int64_t ldc, int out_kind) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= M * N) return;
  const int64_t m = gid / N, n = gid % N;
  float s = 0.f;
  for (int z = 0; z < k_splits; ++z) s += partial[(int64_t)z * M * N + gid];
  if (out_kind == 1) reinterpret_cast<float*>(c)[m * ldc + n] = s;
  else reinterpret_cast<__bf16*>(c)[m * ldc + n] = (__bf16)s;
}

}  // namespace

hipError_t launch_gemm(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c, int64_t ldc,
                       int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 16 * kWaves - 1) / (16 * kWaves)), (unsigned)((M + 15) / 16), 1);
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(64 * kWaves), 0, stream, a, lda, w, ldw, c, ldc, out_kind, M, N, K,
                     (int64_t)0);
  return hipGetLastError();
}

hipError_t launch_gemm_splitk(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, float* partial,
                              int64_t M, int64_t N, int64_t K, int32_t k_splits, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((unsigned)((N + 16 * kWaves - 1) / (16 * kWaves)), (unsigned)((M + 15) / 16), (unsigned)k_splits);
  hipLaunchKernelGGL(gemm_kernel, grid, dim3(64 * kWaves), 0, stream, a, lda, w, ldw, (void*)partial, N, 1, M, N,
                     K / k_splits, M * N);
  return hipGetLastError();
}

hipError_t launch_gemm_splitk_reduce(const float* partial, int32_t k_splits, int64_t M, int64_t N, void* c,
                                     int64_t ldc, int out_kind, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((M * N + 255) / 256)), dim3(256), 0, stream, partial,
                     k_splits, M, N, c, ldc, out_kind);
  return hipGetLastError();
}

}  // namespace bi
