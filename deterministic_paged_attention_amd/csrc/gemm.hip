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
// Two work mappings share that per-element arithmetic exactly (same
// instruction, same K steps in the same order, same k-slot layout per lane
// group), so which one runs never changes a bit of any output row:
//  * gemm_kernel (M <= 32): one wave per 16 (n) x 16 (m) block, operands read
//    straight from global memory — weight streaming for decode-sized M;
//  * gemm_tiled_kernel<BM, BN> (larger M): a workgroup owns a BM x BN tile,
//    stages 64-wide K slices of both operands through LDS (double-buffered),
//    and each of its four waves computes a (BM/2) x (BN/2) sub-tile; tiles are
//    ordered so that the workgroups sharing a slice of w run on one XCD (one
//    L2).
//
// The split-K comparator (measurement only) runs gemm_kernel over K
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

// ---------------------------------------------------------------------------
// LDS-tiled mapping.
// ---------------------------------------------------------------------------
constexpr int kBK = 64;          // K slice staged per iteration (two MFMA K steps)
constexpr int kLdsRow = kBK + 8; // padded LDS row (elements): conflict-free fragment reads
constexpr int kXcds = 8;         // workgroups are dispatched round-robin over 8 XCDs

template <int BM, int BN>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(const uint16_t* a, int64_t lda, const uint16_t* w,
                                                         int64_t ldw, void* c, int64_t ldc, int out_kind, int64_t M,
                                                         int64_t N, int64_t K) {
  constexpr int MB = BM / 32;                 // 16-row m blocks per wave
  constexpr int NB = BN / 32;                 // 16-row n blocks per wave
  constexpr int A_CHUNKS = BM * (kBK / 8) / 256;  // 16-byte chunks per thread per slice
  constexpr int W_CHUNKS = BN * (kBK / 8) / 256;
  __shared__ __attribute__((aligned(16))) uint16_t lds_a[2][BM * kLdsRow];
  __shared__ __attribute__((aligned(16))) uint16_t lds_w[2][BN * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int r = lane & 15, g4 = lane >> 4;
  const int wm = wave & 1, wn = wave >> 1;

  // XCD-aware tile order: workgroup ids id and id + 8 share an XCD; each XCD
  // gets a contiguous run of tiles, m fastest, so the m tiles that read the
  // same slice of w are served by one L2.
  const int64_t nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN;
  const int64_t per = (nM * nN + kXcds - 1) / kXcds;
  const int64_t tile = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= nM * nN) return;
  const int64_t m0 = (tile % nM) * BM;
  const int64_t n0 = (tile / nM) * BN;

  // Global -> register staging of one K slice.
  u32x4 ra[A_CHUNKS], rw[W_CHUNKS];
  auto load_slice = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int ch = tid + 256 * i, row = ch >> 3, col = (ch & 7) * 8;
      const int64_t m = m0 + row;
      ra[i] = (m < M && k0 + col < K) ? *reinterpret_cast<const u32x4*>(a + m * lda + k0 + col)
                                      : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < W_CHUNKS; ++i) {
      const int ch = tid + 256 * i, row = ch >> 3, col = (ch & 7) * 8;
      const int64_t n = n0 + row;
      rw[i] = (n < N && k0 + col < K) ? *reinterpret_cast<const u32x4*>(w + n * ldw + k0 + col)
                                      : u32x4{0u, 0u, 0u, 0u};
    }
  };
  auto store_slice = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
      const int ch = tid + 256 * i, row = ch >> 3, col = (ch & 7) * 8;
      *reinterpret_cast<u32x4*>(&lds_a[buf][row * kLdsRow + col]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < W_CHUNKS; ++i) {
      const int ch = tid + 256 * i, row = ch >> 3, col = (ch & 7) * 8;
      *reinterpret_cast<u32x4*>(&lds_w[buf][row * kLdsRow + col]) = rw[i];
    }
  };

  f32x4 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int64_t nsteps = K / 32;              // MFMA K steps in total
  const int64_t nslices = (nsteps + 1) / 2;
  load_slice(0);
  store_slice(0);
  __syncthreads();
  for (int64_t sl = 0; sl < nslices; ++sl) {
    const int buf = (int)(sl & 1);
    if (sl + 1 < nslices) load_slice((sl + 1) * kBK);
    const int ksteps = (int)min<int64_t>(2, nsteps - 2 * sl);  // 1 only on an odd final slice
    for (int ks = 0; ks < ksteps; ++ks) {
      bf16x8 fw[NB], fa[MB];
#pragma unroll
      for (int i = 0; i < NB; ++i)
        fw[i] = *reinterpret_cast<const bf16x8*>(&lds_w[buf][(wn * (BN / 2) + 16 * i + r) * kLdsRow + ks * 32 + 8 * g4]);
#pragma unroll
      for (int j = 0; j < MB; ++j)
        fa[j] = *reinterpret_cast<const bf16x8*>(&lds_a[buf][(wm * (BM / 2) + 16 * j + r) * kLdsRow + ks * 32 + 8 * g4]);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fw[i], fa[j], acc[i][j], 0, 0, 0);
    }
    if (sl + 1 < nslices) store_slice(buf ^ 1);
    __syncthreads();
  }

  // Lane holds C^T[n + 4*g4 + i][m + r] of each block.
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int64_t m = m0 + wm * (BM / 2) + 16 * j + r;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t nb = n0 + wn * (BN / 2) + 16 * i + 4 * g4;
      if (out_kind == 1) {
        float* cp = reinterpret_cast<float*>(c) + m * ldc + nb;
        if (nb + 4 <= N && ((reinterpret_cast<uintptr_t>(cp) & 15) == 0)) {
          *reinterpret_cast<f32x4*>(cp) = acc[i][j];
        } else {
          for (int e = 0; e < 4; ++e)
            if (nb + e < N) cp[e] = acc[i][j][e];
        }
      } else {
        uint16_t* cp = reinterpret_cast<uint16_t*>(c) + m * ldc + nb;
        bf16x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[i][j][e];
        if (nb + 4 <= N && ((reinterpret_cast<uintptr_t>(cp) & 7) == 0)) {
          *reinterpret_cast<bf16x4*>(cp) = o;
        } else {
          const u32x2 bits = __builtin_bit_cast(u32x2, o);
          for (int e = 0; e < 4; ++e)
            if (nb + e < N) cp[e] = (uint16_t)((e & 1) ? (bits[e >> 1] >> 16) : (bits[e >> 1] & 0xffffu));
        }
      }
    }
  }
}

template <int BM, int BN>
hipError_t tiled_launch(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c, int64_t ldc,
                        int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t groups = (tiles + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN>), dim3((unsigned)groups), dim3(256), 0, stream, a, lda, w, ldw, c,
                     ldc, out_kind, M, N, K);
  return hipGetLastError();
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
  // The mapping follows M; the arithmetic of every output element does not.
  if (M > 512) return tiled_launch<128, 128>(a, lda, w, ldw, c, ldc, out_kind, M, N, K, stream);
  if (M > 32) return tiled_launch<64, 64>(a, lda, w, ldw, c, ldc, out_kind, M, N, K, stream);
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
