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
// The product mappings: gemm_ring_kernel<BM, BN, WM, BK, STAGES> (a
// workgroup owns a BM x BN tile and streams BK-wide K slices of both operands
// into an LDS ring with direct-to-LDS buffer loads) and, for M <= 16,
// gemm_skinny_kernel<STAGES> (a workgroup owns 16 weight rows; three waves
// stream them through the ring while one wave computes).  The kernel and its
// configuration are chosen from M and N; every choice performs the same
// per-element instruction sequence (same instruction, same K steps in the
// same order, same k-slot layout per lane group), so which one runs never
// changes a bit of any output row.
//
// The split-K comparator (measurement only) runs the same kernel over K
// sub-ranges into fp32 partials and sums them in split order afterwards, so
// its reduction order follows the number of splits.

#include "bi_internal.h"
#include "gelu.h"

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
// A workgroup (NW = four or eight waves) owns a BM x BN output tile.  K is consumed in
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
template <int BM, int BN, int WM, int BK, int STAGES, int NW = 4>
__global__ __launch_bounds__(64 * NW) void gemm_ring_kernel(const uint16_t* a, int64_t lda, const uint16_t* w,
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
  constexpr int WN = NW / WM;
  constexpr int MB = BM / WM / 16;            // 16-row m blocks per wave
  constexpr int NB = BN / WN / 16;            // 16-row n blocks per wave
  constexpr int CPR = BK / 8;                 // 16-byte chunks per row of a slice
  constexpr int RPI = 64 / CPR;               // rows moved by one copy instruction
  constexpr int G = (BM + BN) / RPI;          // copy instructions per slice
  constexpr int IPW = (G + NW - 1) / NW;      // per slice for waves 0 .. G%NW-1 (all if G%NW == 0)
  constexpr int STAGE = (BM + BN) * BK;       // elements per stage
  constexpr int SPS = BK / 32;                // MFMA K steps per slice
  // K steps whose fragments are read together: all of a slice for the small
  // tiles of skinny M (where one LDS round trip per step would dominate),
  // one step at a time for the large, register-heavy tiles.
  constexpr int GK = (NB + MB) <= 4 ? (SPS < 32 / (NB + MB) ? SPS : 32 / (NB + MB)) : 1;
  static_assert(SPS % GK == 0, "K-step groups tile the slice");
  static_assert(WM * WN == NW && MB >= 1 && NB >= 1, "tile shape");
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
  // of the stacked [a rows; w rows] slice, gi = wave + NW*j, if gi < G.
  const __amdgpu_buffer_rsrc_t ra = rows_rsrc(a + m0 * lda, min<int64_t>(BM, M - m0), lda, K);
  const __amdgpu_buffer_rsrc_t rw = rows_rsrc(w + n0 * ldw, min<int64_t>(BN, N - n0), ldw, K);
  const __amdgpu_buffer_rsrc_t rzero = rows_rsrc(a, 0, lda, K);
  uint32_t voff[IPW];
  __amdgpu_buffer_rsrc_t rsj[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int srow = RPI * (wave + NW * j) + lane / CPR;   // row of the stacked slice
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
      if (G % NW != 0 && wave + NW * j >= G) break;  // wave-uniform
      lds_void* dst = (lds_void*)(lds + st * STAGE + (wave + NW * j) * 512);
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

  // Fragments of one group of GK K steps, all read from one stage.
  auto read_group = [&](uint32_t sa, int kg, u32x4 (&fw)[GK * NB], u32x4 (&fa)[GK * MB]) {
    const uint32_t sw = sa + BM * BK * 2;
#pragma unroll
    for (int q = 0; q < GK; ++q) {
      const uint32_t cs = (uint32_t)(((4 * (kg + q) + g4) ^ (r & 7)) * 16);
#pragma unroll
      for (int i = 0; i < NB; ++i)
        fw[q * NB + i] = lds_read16(sw + (uint32_t)((wn * (BN / WN) + 16 * i + r) * BK * 2) + cs);
#pragma unroll
      for (int j = 0; j < MB; ++j)
        fa[q * MB + j] = lds_read16(sa + (uint32_t)((wm * (BM / WM) + 16 * j + r) * BK * 2) + cs);
    }
  };
  auto mfma_group = [&](const u32x4 (&fw)[GK * NB], const u32x4 (&fa)[GK * MB]) {
#pragma unroll
    for (int q = 0; q < GK; ++q)
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fw[q * NB + i]),
                                                             __builtin_bit_cast(bf16x8, fa[q * MB + j]),
                                                             acc[i][j], 0, 0, 0);
  };

  // Software pipeline over groups of K steps: the fragments of group g + 1
  // are read while the MFMAs of group g run, and waited for (in full) before
  // the next group; the last group of a slice is carried into the next
  // iteration, whose first reads (after the barrier) overlap it.  The carried
  // fragments start as zeros: their MFMAs add exact zeros to the zero
  // accumulators (+0 + +0 = +0), which changes no bit.  Every element still
  // sees one MFMA per K step, in increasing K.  The wait closes each group
  // inside the iteration, so every copy the compiler makes of these registers
  // (the loop-carried ones included) happens after their data has landed.
  u32x4 cw[GK * NB], ca[GK * MB];
#pragma unroll
  for (int i = 0; i < GK * NB; ++i) cw[i] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < GK * MB; ++j) ca[j] = u32x4{0u, 0u, 0u, 0u};

  bool carried = true;                       // wave-uniform

#pragma unroll
  for (int p = 0; p < STAGES - 1; ++p) issue(p);
  for (int64_t s = 0; s < nslices; ++s) {
    // The copies land in LDS behind the compiler's back, so the fragment
    // reads below are explicit ds_read instructions and the waits are ours:
    // this wave's copies of slice s are done (vmcnt), then everyone's are and
    // nobody still reads slice s-1 (barrier; the carried group is already in
    // registers).
    if (G % NW == 0 || wave < G % NW) wait_vmcnt<IPW * (STAGES - 2)>();
    else wait_vmcnt<(IPW - 1) * (STAGES - 2)>();
    __builtin_amdgcn_s_barrier();
    issue(s + STAGES - 1);                   // into the stage slice s-1 used
    const uint32_t sa = lds_base + (uint32_t)((s % STAGES) * STAGE * 2);
    const int ksteps = (int)min<int64_t>(SPS, nsteps - SPS * s);  // fewer only on a ragged final slice
    if (ksteps == SPS) {
#pragma unroll
      for (int kg = 0; kg < SPS; kg += GK) {
        u32x4 fw[GK * NB], fa[GK * MB];
        read_group(sa, kg, fw, fa);
        __builtin_amdgcn_sched_barrier(0);   // all reads issued before the MFMAs they overlap,
        mfma_group(cw, ca);
        __builtin_amdgcn_sched_barrier(0);   // and waited for only after those MFMAs
        lds_wait<0>(fw, fa);
#pragma unroll
        for (int i = 0; i < GK * NB; ++i) cw[i] = fw[i];
#pragma unroll
        for (int j = 0; j < GK * MB; ++j) ca[j] = fa[j];
      }
    } else {
      // Ragged final slice: finish the carried group, then one step at a time.
      mfma_group(cw, ca);
      carried = false;
      const uint32_t sw = sa + BM * BK * 2;
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
  }
  if (carried) mfma_group(cw, ca);           // the last group (none after a ragged slice)
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

// ---------------------------------------------------------------------------
// Skinny mapping (M <= 16): a workgroup owns 16 rows of w (one output block).
// Waves 1..3 stream those rows through an LDS ring of STAGES 512-wide slices
// (one 1 KiB contiguous run of one row per copy instruction; STAGES - 1
// slices in flight), wave 0 loads the rows of a straight into registers one
// slice ahead and runs the MFMAs — the same per-element instruction sequence
// as the ring mapping (A operand = 16 rows of w, B operand = the rows of a,
// k-slots 8*(lane>>4) .. +7 of each 32-wide step, increasing K).  Rows of a
// past M are not loaded: they only feed output columns that are discarded.
//
// GLU: the gated form for a [gate | up] weight (up half from row up_row): a
// workgroup owns output features n0 .. n0 + 15, streams gate rows n0 .. and up
// rows up_row + n0 .. (32 LDS rows per stage), runs two MFMA chains over the
// same rows of a, and writes bf16(gated_gelu(gate, up)) from the bf16-rounded
// gate and up values — the bits of this GEMM's bf16 output followed by
// gated_gelu_kernel, in one launch.  Its slices are 256 wide (BK), so that a
// ring of four 32-row stages fits the 64 KiB of the 16-row form and two
// workgroups share a compute unit; a copy instruction then carries the half
// KiB runs of two rows.
// ---------------------------------------------------------------------------
constexpr int kSkinnyBK = 512;

template <int STAGES, bool GLU = false, int BK = kSkinnyBK>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const uint16_t* a, int64_t lda, const uint16_t* w,
                                                          int64_t ldw, void* c, int64_t ldc, int out_kind, int64_t M,
                                                          int64_t N, int64_t K, int64_t ksplit_len,
                                                          int64_t up_row = 0) {
#if defined(__HIP_DEVICE_COMPILE__)
  static_assert(BK == 512 || BK == 256, "a copy instruction moves 1 KiB: one 512-wide row run or two 256-wide");
  constexpr int SPS = BK / 32;                // MFMA K steps per slice
  constexpr int WR = GLU ? 32 : 16;           // weight rows per stage
  constexpr int STAGE = WR * BK;              // elements per stage: WR rows x BK
  constexpr int RPI = 512 / BK;               // rows per copy instruction
  constexpr int CPR = BK / 8;                 // 16-byte chunks per row of a slice
  __shared__ __attribute__((aligned(1024))) uint16_t lds[STAGES * STAGE];
  if (ksplit_len > 0) {
    const int64_t k0 = (int64_t)blockIdx.y * ksplit_len;
    a += k0;
    w += k0;
    K = min(ksplit_len, K - k0);
    c = reinterpret_cast<float*>(c) + (int64_t)blockIdx.y * M * N;
  }
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g4 = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  if (n0 >= N) return;
  const int64_t nsteps = K / 32;
  const int64_t nslices = (nsteps + SPS - 1) / SPS;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(lds_void*)lds;

  if (wave != 0) {
    // Copy waves: copy units (one instruction: RPI rows of a slice) [ub, ub +
    // cnt) of the WR / RPI = 16 per stage, about a third each (0..5, 6..10,
    // 11..15); LDS rows 16.. are the GLU form's up rows.
    constexpr int UNITS = WR / RPI;
    constexpr int MAXC = (UNITS + 2) / 3;
    const int ub = ((wave - 1) * UNITS + 2) / 3;
    const int cnt = (wave * UNITS + 2) / 3 - ub;
    // One resource from weight row n0: the block's rows (GLU: gate rows, then
    // the up rows up_row further on, the rows between never read); it ends at
    // the block's last valid element, so rows past N read as zero.
    const int64_t nvalid = min<int64_t>(16, N - n0);
    const __amdgpu_buffer_rsrc_t rw = rows_rsrc(w + n0 * ldw, GLU ? up_row + nvalid : nvalid, ldw, K);
    const __amdgpu_buffer_rsrc_t rzero = rows_rsrc(w, 0, ldw, K);
    uint32_t voff[MAXC];
#pragma unroll
    for (int i = 0; i < MAXC; ++i) {
      const int row = RPI * (ub + i) + lane / CPR;  // this lane's LDS row
      const int64_t wrow = (GLU && row >= 16) ? up_row + (row - 16) : row;
      // chunk c of LDS row R lands in slot c ^ (R & 7)
      voff[i] = (uint32_t)(wrow * ldw * 2 + (((lane % CPR) ^ (row & 7)) * 16));
    }
    auto issue = [&](int64_t s) {
      const int st = (int)(s % STAGES);
      const bool live = s < nslices;
#pragma unroll
      for (int i = 0; i < MAXC; ++i) {
        if (i >= cnt) break;                  // wave-uniform
        lds_void* dst = (lds_void*)(lds + st * STAGE + RPI * (ub + i) * BK);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(live ? rw : rzero, dst, 16, voff[i] + (uint32_t)(s * BK * 2), 0,
                                                 0, 0);
      }
    };
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p) issue(p);
    for (int64_t s = 0; s < nslices; ++s) {
      if (cnt == MAXC) wait_vmcnt<MAXC * (STAGES - 2)>();
      else wait_vmcnt<(MAXC - 1) * (STAGES - 2)>();
      __builtin_amdgcn_s_barrier();           // slice s is in LDS; slice s-1 is no longer read
      issue(s + STAGES - 1);
    }
    wait_vmcnt<0>();
    return;
  }

  // Compute wave.  B operand: row r of a, k-slots 8*g4 .. 8*g4+7 of each step,
  // read through a descriptor ending at the last valid element of a: rows
  // past M (and anything past the end) read as zero without memory traffic;
  // steps past K on the last slice read data no MFMA uses.  The loads are
  // unconditional so that their waits stay counted, not serialized.
  const bool m_ok = r < M;
  const __amdgpu_buffer_rsrc_t ra = rows_rsrc(a, min<int64_t>(16, M), lda, K);
  const uint32_t aoff = (uint32_t)(r * lda * 2 + 16 * g4);
  u32x4 af[2][SPS];
  auto load_a = [&](int64_t s, u32x4 (&dst)[SPS]) {
#pragma unroll
    for (int ks = 0; ks < SPS; ++ks)
      dst[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                              ra, aoff + (uint32_t)((s * BK + 32 * ks) * 2), 0, 0));
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  f32x4 acc_up = {0.f, 0.f, 0.f, 0.f};  // GLU: the up rows' chain (LDS rows 16..31)
  auto slice = [&](int64_t s, u32x4 (&cur)[SPS], u32x4 (&nxt)[SPS]) {
    load_a(s + 1, nxt);                      // next slice's rows of a, in flight during this one
    __builtin_amdgcn_s_barrier();            // slice s of w is in LDS
    const uint32_t sw = lds_base + (uint32_t)((s % STAGES) * STAGE * 2);
    const int ksteps = (int)min<int64_t>(SPS, nsteps - SPS * s);
    // A full slice reads all of its w fragments at once (one LDS round trip
    // per slice, straight-line code), then runs its MFMAs in step order; a
    // ragged final slice goes one step at a time.
    if (ksteps == SPS) {
      u32x4 fw[SPS];
#pragma unroll
      for (int ks = 0; ks < SPS; ++ks)
        fw[ks] = lds_read16(sw + (uint32_t)(r * BK * 2) + (uint32_t)(((4 * ks + g4) ^ (r & 7)) * 16));
      lds_wait<0>(fw, cur);
#pragma unroll
      for (int ks = 0; ks < SPS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fw[ks]),
                                                      __builtin_bit_cast(bf16x8, cur[ks]), acc, 0, 0, 0);
      if constexpr (GLU) {
        const uint32_t su = sw + (uint32_t)((16 + r) * BK * 2);
#pragma unroll
        for (int ks = 0; ks < SPS; ++ks) fw[ks] = lds_read16(su + (uint32_t)(((4 * ks + g4) ^ (r & 7)) * 16));
        lds_wait<0>(fw, cur);
#pragma unroll
        for (int ks = 0; ks < SPS; ++ks)
          acc_up = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fw[ks]),
                                                           __builtin_bit_cast(bf16x8, cur[ks]), acc_up, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < SPS; ++ks) {    // static register indices; the guard is wave-uniform
        if (ks < ksteps) {
          u32x4 fw[1] = {lds_read16(sw + (uint32_t)(r * BK * 2) + (uint32_t)(((4 * ks + g4) ^ (r & 7)) * 16))};
          u32x4 fa[1] = {cur[ks]};
          lds_wait<0>(fw, fa);
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fw[0]),
                                                        __builtin_bit_cast(bf16x8, fa[0]), acc, 0, 0, 0);
          if constexpr (GLU) {
            u32x4 fu[1] = {lds_read16(sw + (uint32_t)((16 + r) * BK * 2) +
                                      (uint32_t)(((4 * ks + g4) ^ (r & 7)) * 16))};
            lds_wait<0>(fu, fa);
            acc_up = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fu[0]),
                                                             __builtin_bit_cast(bf16x8, fa[0]), acc_up, 0, 0, 0);
          }
        }
      }
    }
  };
  load_a(0, af[0]);
  int64_t s = 0;
  for (; s + 1 < nslices; s += 2) {
    slice(s, af[0], af[1]);
    slice(s + 1, af[1], af[0]);
  }
  if (s < nslices) slice(s, af[0], af[1]);

  // Lane holds C^T[n0 + 4*g4 + i][r].
  if (!m_ok) return;
  const int64_t nb = n0 + 4 * g4;
  if constexpr (GLU) {
    // gate and up rounded to bf16 as this GEMM's bf16 output is, then the
    // gated GELU of gated_gelu_kernel, one more bf16 rounding.
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g = (float)(__bf16)acc[e], u = (float)(__bf16)acc_up[e];
      acc[e] = gated_gelu_f32(g, u);
    }
  }
  if (out_kind == 1) {
    float* cp = reinterpret_cast<float*>(c) + (int64_t)r * ldc + nb;
    if (nb + 4 <= N && ((reinterpret_cast<uintptr_t>(cp) & 15) == 0)) {
      *reinterpret_cast<f32x4*>(cp) = acc;
    } else {
      for (int e = 0; e < 4; ++e)
        if (nb + e < N) cp[e] = acc[e];
    }
  } else {
    uint16_t* cp = reinterpret_cast<uint16_t*>(c) + (int64_t)r * ldc + nb;
    bf16x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (__bf16)acc[e];
    if (nb + 4 <= N && ((reinterpret_cast<uintptr_t>(cp) & 7) == 0)) {
      *reinterpret_cast<bf16x4*>(cp) = o;
    } else {
      const u32x2 bits = __builtin_bit_cast(u32x2, o);
      for (int e = 0; e < 4; ++e)
        if (nb + e < N) cp[e] = (uint16_t)((e & 1) ? (bits[e >> 1] >> 16) : (bits[e >> 1] & 0xffffu));
    }
  }
#endif
}

template <int STAGES>
hipError_t skinny_launch(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c, int64_t ldc,
                         int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t stream, int64_t ksplit_len,
                         int64_t nsplit) {
  hipLaunchKernelGGL(gemm_skinny_kernel<STAGES>, dim3((unsigned)((N + 15) / 16), (unsigned)nsplit), dim3(256), 0,
                     stream, a, lda, w, ldw, c, ldc, out_kind, M, N, K, nsplit > 1 ? ksplit_len : (int64_t)0,
                     (int64_t)0);
  return hipGetLastError();
}

// nsplit > 1: split launch over K ranges of ksplit_len into fp32 partials
// (see the kernel).
template <int BM, int BN, int WM, int BK, int STAGES, int NW = 4>
hipError_t ring_launch(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c, int64_t ldc,
                       int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t stream, int64_t ksplit_len,
                       int64_t nsplit) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t groups = (tiles + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((gemm_ring_kernel<BM, BN, WM, BK, STAGES, NW>), dim3((unsigned)groups, (unsigned)nsplit),
                     dim3(64 * NW), 0, stream, a, lda, w, ldw, c, ldc, out_kind, M, N, K,
                     nsplit > 1 ? ksplit_len : (int64_t)0);
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
// Workgroups of one ring configuration the current device keeps resident at
// once (all compute units; computed once per device; 0 if unknown).
template <int BM, int BN, int WM, int BK, int STAGES, int NW = 4>
int64_t ring_capacity() {
  static int64_t cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] > 0) return cached[dev];
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gemm_ring_kernel<BM, BN, WM, BK, STAGES, NW>, 64 * NW, 0) !=
      hipSuccess)
    return 0;
  cached[dev] = (int64_t)cus * per_cu;
  return cached[dev];
}

// True when every workgroup of the configuration is resident at once (one
// round), as in ring_launch's grid.
template <int BM, int BN, int WM, int BK, int STAGES, int NW = 4>
bool ring_fits(int64_t M, int64_t N) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t groups = (tiles + kXcds - 1) / kXcds * kXcds;
  const int64_t cap = ring_capacity<BM, BN, WM, BK, STAGES, NW>();
  return cap == 0 || groups <= cap;
}

// Tile configuration by (M, N); with nsplit > 1 the K ranges of ksplit_len
// run as one launch into fp32 partials.  N here is the partial's width.
hipError_t launch_gemm_impl(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c, int64_t ldc,
                            int out_kind, int64_t M, int64_t N, int64_t K, int64_t ksplit_len, int64_t nsplit,
                            hipStream_t stream) {
  // The mapping follows M (and N, which every call of a given weight
  // shares); the arithmetic of every output element does not.  Kernel, tile
  // shape, slice width and ring depth come from a measured sweep on MI355X:
  // skinny M wants long contiguous weight-row runs, many slices in flight and
  // few LDS round trips per slice; larger M wants larger tiles to cut operand
  // re-reads.
  auto L = [&](auto kernel_cfg) {
    return kernel_cfg(a, lda, w, ldw, c, ldc, out_kind, M, N, K, stream, ksplit_len, nsplit);
  };
  if (M <= 16) {
    if (N <= 8192 || (N >= 16384 && M <= 4)) return L(skinny_launch<4>);
    if (N < 16384) return L(ring_launch<32, 32, 2, 256, 2>);
    return L(ring_launch<64, 64, 2, 128, 2>);
  }
  // Up to N = 8192 the tiles are small and the run is latency-bound: a
  // configuration whose workgroups do not all fit on the GPU at once runs a
  // second, partly empty round, so the deeper ring (one workgroup per CU)
  // gives way to a shallower one (two per CU) or to larger tiles.
  if (M <= 32) {
    if (N <= 8192) {
      if (ring_fits<32, 32, 2, 256, 4>(M, N)) return L(ring_launch<32, 32, 2, 256, 4>);
      return L(ring_launch<32, 32, 2, 256, 2>);
    }
    if (N < 16384) return L(ring_launch<32, 64, 2, 128, 5>);
    return L(ring_launch<64, 64, 2, 128, 2>);
  }
  if (M <= 64) {
    if (N <= 8192) {
      if (ring_fits<32, 32, 2, 256, 4>(M, N)) return L(ring_launch<32, 32, 2, 256, 4>);
      return L(ring_launch<32, 32, 2, 256, 2>);
    }
    // One round of eight-wave 64 x 64 tiles where it fits (14336 x 4096 at
    // M = 64: 31.3 -> 29.5 us against four waves).
    if (N < 16384 && ring_fits<64, 64, 2, 128, 4, 8>(M, N)) return L(ring_launch<64, 64, 2, 128, 4, 8>);
    if (N < 16384) return L(ring_launch<64, 64, 2, 128, 4>);
    return L(ring_launch<64, 128, 2, 128, 3>);
  }
  // Above M = 64, eight-wave workgroups (two waves per SIMD) let one wave's
  // LDS reads overlap another's MFMAs.
  if (M <= 128) {
    if (N <= 8192) {
      if (ring_fits<32, 32, 2, 256, 2>(M, N)) return L(ring_launch<32, 32, 2, 256, 2>);
      // 6144 x 4096 at M = 100..128: 29.2 -> 27.1 us with eight waves.
      if (ring_fits<64, 64, 2, 128, 4, 8>(M, N)) return L(ring_launch<64, 64, 2, 128, 4, 8>);
      return L(ring_launch<64, 64, 2, 128, 4>);
    }
    if (N < 16384) return L(ring_launch<64, 128, 2, 128, 3>);
    if (N < 65536) return L(ring_launch<128, 128, 2, 64, 4, 8>);
    return L(ring_launch<128, 256, 2, 64, 3, 8>);
  }
  if (M <= 256) {
    if (N <= 8192) {
      // Two-wave 32 x 80 tiles while they all fit in one round: N = 2560 makes
      // 256 of them at M = 256 (Gemma-shaped down projection 2560 x 10240:
      // 62 -> 50 us; 2560 x 2048: 18 -> 15 us); with a second round they lose.
      if (ring_fits<32, 80, 2, 128, 4, 2>(M, N)) return L(ring_launch<32, 80, 2, 128, 4, 2>);
      // One round of tiles, as few bytes per compute unit as that allows (each
      // unit pulls (BM + BN) K 2 bytes through LDS at ~50 GB/s): 64 x 64 tiles
      // with eight waves (4096 x 4096 at M = 256: 29.4 -> 27.4 us; 4096 x 2560
      // 22.1 -> 20.4 us), else 64 x 96 tiles (6144 wide: 256 of them at
      // M = 256; 6144 x 4096 38.6 -> 30.4 us, 6144 x 2560 29.9 -> 23.0 us).
      if (ring_fits<64, 64, 2, 128, 4, 8>(M, N)) return L(ring_launch<64, 64, 2, 128, 4, 8>);
      if (ring_fits<64, 96, 2, 128, 4>(M, N)) return L(ring_launch<64, 96, 2, 128, 4>);
      return L(ring_launch<64, 64, 2, 128, 2>);
    }
    if (N < 16384) return L(ring_launch<128, 128, 2, 64, 4, 8>);
    // 128 x 160 tiles: a 20480-wide weight makes exactly 256 of them (Gemma-
    // shaped gate/up projection at M = 256: 53 -> 44 us against 256 x 128).
    if (N < 65536) return L(ring_launch<128, 160, 2, 64, 3, 4>);
    return L(ring_launch<256, 128, 4, 64, 3, 8>);
  }
  if (M <= 512 && N >= 16384 && N < 65536) return L(ring_launch<128, 160, 2, 64, 3, 4>);  // M = 512: 97 -> 80 us
  if (N <= 8192) {
    // 128 x 128 tiles while they fit in one round, else 128 x 256 (M = 2048:
    // 2560 x 10240 220 -> 188 us; 6144 x 4096 at M = 1024 99 -> 82 us)
    if (ring_fits<128, 128, 2, 64, 4, 8>(M, N)) return L(ring_launch<128, 128, 2, 64, 4, 8>);
    return L(ring_launch<128, 256, 2, 64, 3, 8>);
  }
  // 256 x 128 tiles of 64 x 64 per wave (M = 1024: 14336 x 4096 146 -> 140 us
  // against 128 x 256; 128256 x 4096 1239 -> 1060 us against 32 x 128 per wave).
  return L(ring_launch<256, 128, 4, 64, 3, 8>);
}

}  // namespace

hipError_t launch_gemm(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c, int64_t ldc,
                       int out_kind, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  return launch_gemm_impl(a, lda, w, ldw, c, ldc, out_kind, M, N, K, 0, 1, stream);
}

// Ring of the gated skinny form: four stages of 32 weight rows x 256 (16 KiB).
constexpr int kGluStages = 4;
constexpr int kGluBK = 256;

hipError_t launch_gemm_gated_gelu(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, uint16_t* out,
                                  int64_t ldo, int64_t M, int64_t F, int64_t K, hipStream_t stream) {
  if (M == 0 || F == 0) return hipSuccess;
  if (M > 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_skinny_kernel<kGluStages, true, kGluBK>), dim3((unsigned)((F + 15) / 16), 1u), dim3(256), 0,
                     stream, a, lda, w, ldw, (void*)out, ldo, 0, M, F, K, (int64_t)0, F);
  return hipGetLastError();
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
