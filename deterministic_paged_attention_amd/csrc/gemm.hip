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
// Fragments: an output block is 16 (n) x 16 (m); a wave computes C^T = W A^T
// for it, so that a lane ends with four consecutive n of one m (one vector
// store).  The MFMA A operand is 16 rows of w, the B operand 16 rows of a;
// lane l supplies k-slots 8*(l>>4) .. 8*(l>>4)+7 of the 32-wide K step, both
// operands K-major as stored.
//
// The product mapping, gemm_ring_kernel<BM, BN, WM, BK, STAGES>: a workgroup
// owns a BM x BN tile and streams BK-wide K slices of both operands into an
// LDS ring with direct-to-LDS buffer loads.  The tile configuration is chosen
// from M and N; every configuration performs the same per-element instruction
// sequence (same instruction, same K steps in the same order, same k-slot
// layout per lane group), so which one runs never changes a bit of any
// output row.
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

// ---------------------------------------------------------------------------
// LDS ring mapping.
//
// A workgroup (four waves) owns a BM x BN output tile.  K is consumed in
// BK-wide slices; slice s of both operands is copied straight from global
// memory into LDS stage s % STAGES by buffer loads that write LDS directly
// (each wave instruction moves 1 KiB: 512/BK rows x 2*BK bytes; lane i of it
// writes the i-th 16-byte LDS slot).  STAGES - 1 slices are in flight while one is being
// multiplied, which is what keeps HBM busy when there are few workgroups per
// CU (skinny M) and the K loop is long.  Rows past M or N are fetched through
// a buffer descriptor whose range ends at the last valid element, so they
// arrive as zeros without touching memory.
//
// LDS layout of one operand slice: row-major, BK/8 chunks of 16 bytes per
// row, chunk c of row R stored at slot R*BK/8 + (c ^ (R & 7)), so that the
// 8 rows a group of fragment-reading lanes touches fall in distinct banks.
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;         // workgroups are dispatched round-robin over 8 XCDs

// s_waitcnt with vmcnt = n and the other counters left free (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] in bits [15:14]).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}

typedef __attribute__((address_space(3))) void lds_void;

// 16-byte LDS read at byte address addr (result valid after lds_wait).  The
// bodies are GPU assembly; the host pass of the compiler only sees stubs.
__device__ __forceinline__ u32x4 lds_read16(uint32_t addr) {
  u32x4 v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
#else
  v = u32x4{addr, 0u, 0u, 0u};
#endif
  return v;
}

// Waits for every outstanding LDS read of this wave; x and y are tied to
// the wait so no use of them can be scheduled above it.
template <int pending, int NA, int NB>
__device__ __forceinline__ void lds_wait(u32x4 (&x)[NA], u32x4 (&y)[NB]) {
  static_assert(pending == 0, "the reads are consumed right after they land");
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < NA; ++i) asm volatile("" : "+v"(x[i]));
#pragma unroll
  for (int i = 0; i < NB; ++i) asm volatile("" : "+v"(y[i]));
#endif
}

// Buffer descriptor over `rows` rows (ld elements apart) of K valid elements
// starting at base; everything past the last valid element reads as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int64_t rows, int64_t ld,
                                                            int64_t K) {
  const int64_t bytes = rows > 0 ? ((rows - 1) * ld + K) * 2 : 0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, (int)(uint32_t)bytes,
                                           0x00020000);
}

// Split launches (ksplit_len > 0, grid y = number of splits): workgroup row y
// multiplies the K range [y*ksplit_len, min((y+1)*ksplit_len, K)) into fp32
// partial y (c + y*M*N, row stride ldc), all splits at once.
template <int BM, int BN, int WM, int BK, int STAGES>
__global__ __launch_bounds__(256) void gemm_ring_kernel(const uint16_t* a, int64_t lda, const uint16_t* w,
                                                        int64_t ldw, void* c, int64_t ldc, int out_kind, int64_t M,
                                                        int64_t N, int64_t K, int64_t ksplit_len) {
#if defined(__HIP_DEVICE_COMPILE__)  // LDS address-space casts and buffer-to-LDS copies exist on the GPU only
  if (ksplit_len > 0) {
    const int64_t k0 = (int64_t)blockIdx.y * ksplit_len;
    a += k0;
    w += k0;
    K = min(ksplit_len, K - k0);
    c = reinterpret_cast<float*>(c) + (int64_t)blockIdx.y * M * N;
  }
  constexpr int WN = 4 / WM;
  constexpr int MB = BM / WM / 16;            // 16-row m blocks per wave
  constexpr int NB = BN / WN / 16;            // 16-row n blocks per wave
  constexpr int CPR = BK / 8;                 // 16-byte chunks per row of a slice
  constexpr int RPI = 64 / CPR;               // rows moved by one copy instruction
  constexpr int G = (BM + BN) / RPI;          // copy instructions per slice
  constexpr int IPW = (G + 3) / 4;            // per slice for waves 0 .. G%4-1 (all if G%4 == 0)
  constexpr int STAGE = (BM + BN) * BK;       // elements per stage
  constexpr int SPS = BK / 32;                // MFMA K steps per slice
  static_assert(WM * WN == 4 && MB >= 1 && NB >= 1, "tile shape");
  static_assert((BK == 64 || BK == 128 || BK == 256 || BK == 512) && (BM + BN) % RPI == 0, "slice shape");
  static_assert(STAGES >= 2, "ring depth");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g4 = lane >> 4;
  const int wm = wave % WM, wn = wave / WM;

  // XCD-aware tile order: workgroup ids id and id + 8 share an XCD; each XCD
  // gets a contiguous run of tiles, m fastest, so the m tiles that read the
  // same slice of w are served by one L2.
  const int64_t nM = (M + BM - 1) / BM, nN = (N + BN - 1) / BN;
  const int64_t per = (nM * nN + kXcds - 1) / kXcds;
  const int64_t tile = (int64_t)(blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
  if (tile >= nM * nN) return;
  const int64_t m0 = (tile % nM) * BM;
  const int64_t n0 = (tile / nM) * BN;

  // Copy plan: instruction j of this wave moves rows RPI*gi .. RPI*gi+RPI-1
  // of the stacked [a rows; w rows] slice, gi = wave + 4j, if gi < G.
  const __amdgpu_buffer_rsrc_t ra = rows_rsrc(a + m0 * lda, min<int64_t>(BM, M - m0), lda, K);
  const __amdgpu_buffer_rsrc_t rw = rows_rsrc(w + n0 * ldw, min<int64_t>(BN, N - n0), ldw, K);
  const __amdgpu_buffer_rsrc_t rzero = rows_rsrc(a, 0, lda, K);
  uint32_t voff[IPW];
  __amdgpu_buffer_rsrc_t rsj[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int srow = RPI * (wave + 4 * j) + lane / CPR;    // row of the stacked slice
    const bool is_a = srow < BM;
    const int row = is_a ? srow : srow - BM;
    const int chunk = (lane % CPR) ^ (srow & 7);           // logical chunk landing in this lane's slot
    voff[j] = (uint32_t)(row * (is_a ? lda : ldw) * 2 + chunk * 16);
    rsj[j] = is_a ? ra : rw;
  }
  const int64_t nsteps = K / 32;
  const int64_t nslices = (nsteps + SPS - 1) / SPS;
  // Slice s into stage s % STAGES; slices past the end copy nothing (a
  // zero-range descriptor) so that every iteration issues the same count.
  auto issue = [&](int64_t s) {
    const int st = (int)(s % STAGES);
    const bool live = s < nslices;
#pragma unroll
    for (int j = 0; j < IPW; ++j) {
      if (G % 4 != 0 && wave + 4 * j >= G) break;  // wave-uniform
      lds_void* dst = (lds_void*)(lds + st * STAGE + (wave + 4 * j) * 512);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rsj[j] : rzero, dst, 16,
                                               voff[j] + (uint32_t)(s * BK * 2), 0, 0, 0);
    }
  };
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;

  f32x4 acc[NB][MB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p) issue(p);
  for (int64_t s = 0; s < nslices; ++s) {
    // The copies land in LDS behind the compiler's back, so the fragment
    // reads below are explicit ds_read instructions and the waits are ours:
    // this wave's copies of slice s are done (vmcnt), then everyone's are and
    // nobody still reads slice s-1 (barrier).
    if (G % 4 == 0 || wave < G % 4) wait_vmcnt<IPW * (STAGES - 2)>();
    else wait_vmcnt<(IPW - 1) * (STAGES - 2)>();
    __builtin_amdgcn_s_barrier();
    issue(s + STAGES - 1);                   // into the stage slice s-1 used
    const uint32_t sa = lds_base + (uint32_t)((s % STAGES) * STAGE * 2);
    const uint32_t sw = sa + BM * BK * 2;
    const int ksteps = (int)min<int64_t>(SPS, nsteps - SPS * s);  // fewer only on a ragged final slice
    // One K step at a time: its fragments are read and waited for in full
    // before its MFMAs.  (The reads are not prefetched a step ahead: the
    // compiler does not know these registers fill asynchronously and may copy
    // them before the wait.)
    for (int ks = 0; ks < ksteps; ++ks) {
      const uint32_t cs = (uint32_t)(((4 * ks + g4) ^ (r & 7)) * 16);
      u32x4 fw[NB], fa[MB];
#pragma unroll
      for (int i = 0; i < NB; ++i)
        fw[i] = lds_read16(sw + (uint32_t)((wn * (BN / WN) + 16 * i + r) * BK * 2) + cs);
#pragma unroll
      for (int j = 0; j < MB; ++j)
        fa[j] = lds_read16(sa + (uint32_t)((wm * (BM / WM) + 16 * j + r) * BK * 2) + cs);
      lds_wait<0>(fw, fa);
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fw[i]),
                                                             __builtin_bit_cast(bf16x8, fa[j]), acc[i][j], 0, 0, 0);
    }
  }
  wait_vmcnt<0>();                           // drain the trailing (empty) copies

  // Lane holds C^T[n + 4*g4 + i][m + r] of each block.
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int64_t m = m0 + wm * (BM / WM) + 16 * j + r;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int64_t nb = n0 + wn * (BN / WN) + 16 * i + 4 * g4;
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
#endif
}

// nsplit > 1: split launch over K ranges of ksplit_len into fp32 partials
// (see the kernel).
template <int BM, int BN, int WM, int BK, int STAGES>
hipError_t ring_launch(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c, int64_t ldc,
                       int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t stream, int64_t ksplit_len,
                       int64_t nsplit) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t groups = (tiles + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((gemm_ring_kernel<BM, BN, WM, BK, STAGES>), dim3((unsigned)groups, (unsigned)nsplit), dim3(256),
                     0, stream, a, lda, w, ldw, c, ldc, out_kind, M, N, K, nsplit > 1 ? ksplit_len : (int64_t)0);
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

namespace {
// Tile configuration by (M, N); with nsplit > 1 the K ranges of ksplit_len
// run as one launch into fp32 partials.  N here is the partial's width.
hipError_t launch_gemm_impl(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c, int64_t ldc,
                            int out_kind, int64_t M, int64_t N, int64_t K, int64_t ksplit_len, int64_t nsplit,
                            hipStream_t stream) {
  // The mapping follows M (and N, which every call of a given weight
  // shares); the arithmetic of every output element does not.  Tile shape,
  // slice width and ring depth come from a measured sweep on MI355X: skinny
  // M wants long contiguous row runs and many slices in flight; larger M
  // wants larger tiles to cut operand re-reads.
  auto L = [&](auto kernel_cfg) {
    return kernel_cfg(a, lda, w, ldw, c, ldc, out_kind, M, N, K, stream, ksplit_len, nsplit);
  };
  if (M <= 32) {
    if (N >= 8192) return L(ring_launch<32, 32, 2, 256, 2>);
    return L(ring_launch<32, 32, 2, 512, 2>);
  }
  if (M <= 64) {
    if (N >= 16384) return L(ring_launch<64, 128, 2, 128, 3>);
    if (N >= 8192) return L(ring_launch<64, 64, 2, 128, 4>);
    return L(ring_launch<32, 32, 2, 256, 4>);
  }
  if (M <= 128) {
    if (N >= 16384) return L(ring_launch<128, 128, 2, 64, 4>);
    if (N >= 8192) return L(ring_launch<64, 64, 2, 128, 2>);
    return L(ring_launch<32, 32, 2, 256, 2>);
  }
  if (M <= 256) {
    if (N >= 16384) return L(ring_launch<256, 128, 4, 64, 3>);
    if (N >= 8192) return L(ring_launch<128, 128, 2, 64, 4>);
    return L(ring_launch<64, 64, 2, 128, 4>);
  }
  if (N >= 8192) return L(ring_launch<256, 128, 4, 64, 3>);
  return L(ring_launch<128, 128, 2, 64, 4>);
}

}  // namespace

hipError_t launch_gemm(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c, int64_t ldc,
                       int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  return launch_gemm_impl(a, lda, w, ldw, c, ldc, out_kind, M, N, K, 0, 1, stream);
}

hipError_t launch_gemm_splitk(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, float* partial,
                              int64_t M, int64_t N, int64_t K, int32_t k_splits, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  // Split z multiplies the K range [z*kc, (z+1)*kc) with the product kernel
  // into fp32 partial[z]; all splits in one launch, the tile configuration
  // being the product's for (M, N).
  return launch_gemm_impl(a, lda, w, ldw, partial, N, 1, M, N, K, K / k_splits, k_splits, stream);
}

hipError_t launch_gemm_splitk_reduce(const float* partial, int32_t k_splits, int64_t M, int64_t N, void* c,
                                     int64_t ldc, int out_kind, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((M * N + 255) / 256)), dim3(256), 0, stream, partial,
                     k_splits, M, N, c, ldc, out_kind);
  return hipGetLastError();
}


}  // namespace bi
