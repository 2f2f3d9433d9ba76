// Batch-invariant paged attention for gfx950: split phase and merge phase.
//
// What is computed (Vosti deep-dive blog (深入解析 Vosti), §6.2, attention causal
// contract): the query row at position p = k_len - q_len + i sees keys [lo, p],
// lo = max(0, p - w + 1) under a sliding window, and its output depends only on
// that row of Q and those keys and values — not on the query length, the row
// index, the batch or the physical page table.
//
// How the arithmetic of a row is fixed by logical key positions alone:
//  * keys are cut into splits of a fixed SIZE S, [sS, (s+1)S), never a fixed
//    count (record "Deterministic and bit-exact inference", field technical,
//    Invariance);
//  * a split is a pass over 32-key tiles in increasing order with an online
//    softmax (deep-dive blog, §6.2: the tiles meeting a row's range are visited
//    in the same order by every invocation);
//  * a tile where a row sees no key leaves that row's (m, l, acc) bit-for-bit
//    unchanged, by select (deep-dive blog, §6.2, value rules: masked score
//    -inf, masked weight 0, an all-false row copies its incoming state);
//  * masking is a select, never an additive bias, so keys outside [lo, p] —
//    including never-written slots holding NaN — cannot reach the result;
//    values of keys at or past k_len are zero-filled on load;
//  * decode rows and prefill rows go through the same MFMA instructions: a
//    query-row block is 16 MFMA columns = (16 / G) tokens x G heads of one KV
//    head, and a decode block simply leaves columns empty;
//  * splits are merged in increasing split order (merge kernel), and a -0
//    result is stored as +0.
//
// Data path per wave (no LDS): the K tile is read straight into the A operand
// of v_mfma_f32_16x16x32_bf16 (S^T = K Q^T), the score fragments that come out
// are exactly the B operand of the PV product (O^T = V^T P^T), and the V
// fragments are read straight into its A operand.  The cache layouts
// (K [page][h][D/8][16][8], V [page][h][D][16]) make every one of these reads
// a fully used contiguous run of 512 B or 1 KiB per wave instruction.

#include "bi_internal.h"

#include <math.h>

namespace bi {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Largest s with start(s) <= x, start(s) = qsl[s] / tq + s (monotone in s).
__device__ __forceinline__ int find_block_seq(const int32_t* qsl, int num_seqs, int tq, int x) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] / tq + mid <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Largest s with qsl[s] <= t.
__device__ __forceinline__ int find_token_seq(const int32_t* qsl, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Split phase.  Grid: x = query-row block (global numbering qsl[s]/Tq + s + b),
// y = KV head, z = group of kSplitWaves splits; one wave per split.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64 * kSplitWaves) void attn_split_kernel(const AttnSplitArgs a) {
  constexpr int NSTEP = D / 32;  // 32-wide head-dim steps of QK^T
  constexpr int NBLK = D / 16;   // 16-row head-dim blocks of O^T
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane & 15;       // MFMA column = query row of the block
  const int g4 = lane >> 4;      // lane group = k-slot group of the MFMA operands
  const int kvh = blockIdx.y;
  const int sigma = blockIdx.z * kSplitWaves + wave;
  if (sigma >= a.ns) return;

  const int G = 1 << a.log2_group;
  const int tq = kRowsPerBlock >> a.log2_group;  // tokens per row block
  const int xb = blockIdx.x;
  const int s = find_block_seq(a.qsl, a.num_seqs, tq, xb);
  const int q0 = a.qsl[s];
  const int q_len = a.qsl[s + 1] - q0;
  const int k_len = a.seq_lens[s];
  const int local = xb - (q0 / tq + s);
  const int tq0 = local * tq;
  if (local < 0 || tq0 >= q_len) return;

  const int nrow_tok = min(tq, q_len - tq0);
  const int p_first = k_len - q_len + tq0;
  const int p_last = p_first + nrow_tok - 1;
  if (p_last < 0) return;
  const int lo_first = a.window > 0 ? max(0, p_first - a.window + 1) : 0;
  const int S = a.split;
  if (sigma < max(lo_first, 0) / S || sigma > p_last / S) return;
  const int split_lo = sigma * S;
  const int key_begin = max(split_lo, max(lo_first, 0));
  const int key_end = min(split_lo + S, p_last + 1);  // exclusive
  const int tile_begin = key_begin >> 5;
  const int tile_end = (key_end + 31) >> 5;

  // This lane's query row: token t of the block, head hh of the GQA group.
  const int t = r >> a.log2_group;
  const int hh = r & (G - 1);
  const bool row_ok = (t < nrow_tok) && (q0 + tq0 + t < a.num_tokens);
  const int p = p_first + t;
  int rk_lo = max(a.window > 0 ? max(0, p - a.window + 1) : 0, split_lo);
  int rk_hi = min(p, split_lo + S - 1);
  if (!row_ok || p < 0) { rk_lo = 1; rk_hi = 0; }

  // Q fragment (B operand of S^T = K Q^T): step st, lane group g4 holds the
  // head-dim chunk 4*st + g4 (8 elements) of this lane's row.
  bf16x8 qf[NSTEP];
  {
    const int tok = q0 + tq0 + (row_ok ? t : 0);
    const uint16_t* qrow = a.q + (int64_t)tok * a.q_stride + (int64_t)((kvh << a.log2_group) + hh) * D;
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (row_ok) v = *reinterpret_cast<const u32x4*>(qrow + (4 * st + g4) * 8);
      qf[st] = __builtin_bit_cast(bf16x8, v);
    }
  }

  float m_run = -INFINITY;
  float l_run = 0.f;
  f32x4 acc[NBLK];
#pragma unroll
  for (int n = 0; n < NBLK; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int32_t* pt_row = a.page_table + (int64_t)s * a.pt_stride;
  const int64_t head_elems = (int64_t)D * 16;  // one page of one KV head

  for (int tile = tile_begin; tile < tile_end; ++tile) {
    const int kb = tile << 5;
    u32x4 kf[2][NSTEP];
    u32x2 vf[2][NBLK];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int key0 = kb + 16 * b;
      const int nvalid = min(16, k_len - key0);  // keys of this page below k_len
      const int lp = key0 >> 4;
      int pg = -1;
      if (nvalid > 0 && lp < a.pt_stride) {
        pg = pt_row[lp];
        if (pg < 0 || pg >= a.num_pages) pg = -1;
      }
      if (pg >= 0) {
        const int64_t base = ((int64_t)pg * a.num_kv_heads + kvh) * head_elems;
        const uint16_t* kp = a.k_cache + base;
        const uint16_t* vp = a.v_cache + base;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st)
          kf[b][st] = *reinterpret_cast<const u32x4*>(kp + (64 * st + lane) * 8);
#pragma unroll
        for (int n = 0; n < NBLK; ++n)
          vf[b][n] = *reinterpret_cast<const u32x2*>(vp + 256 * n + 16 * r + 4 * g4);
        // Zero-fill keys at or past k_len (never-written slots may hold NaN).
        const int nl = nvalid - 4 * g4;  // valid keys among this lane's four
        const uint32_t m0 = nl >= 2 ? 0xffffffffu : (nl == 1 ? 0x0000ffffu : 0u);
        const uint32_t m1 = nl >= 4 ? 0xffffffffu : (nl == 3 ? 0x0000ffffu : 0u);
#pragma unroll
        for (int n = 0; n < NBLK; ++n) {
          vf[b][n].x &= m0;
          vf[b][n].y &= m1;
        }
        if (r >= nvalid) {
#pragma unroll
          for (int st = 0; st < NSTEP; ++st) kf[b][st] = u32x4{0u, 0u, 0u, 0u};
        }
      } else {
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) kf[b][st] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int n = 0; n < NBLK; ++n) vf[b][n] = u32x2{0u, 0u};
      }
    }

    // Scores: lane holds keys kb + 16b + 4*g4 + i (i = 0..3) of its row.
    float x[2][4];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NSTEP; ++st) sc = mfma16x16x32(__builtin_bit_cast(bf16x8, kf[b][st]), qf[st], sc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kb + 16 * b + 4 * g4 + i;
        const bool ok = key >= rk_lo && key <= rk_hi;
        x[b][i] = ok ? sc[i] * a.qk_scale_log2 : -INFINITY;
      }
    }
    float tmax = x[0][0];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, x[b][i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const bool live = tmax != -INFINITY;  // this row sees at least one key here

    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_run == -INFINITY) ? 0.f : exp2_hw(m_run - m_new);
    __bf16 pb[2][4];
    float rs = 0.f;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = (x[b][i] != -INFINITY) ? exp2_hw(x[b][i] - m_new) : 0.f;
        pb[b][i] = (__bf16)e;
        rs += (float)pb[b][i];
      }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    const float l_new = __builtin_fmaf(alpha, l_run, rs);

    const bf16x8 pfrag = {pb[0][0], pb[0][1], pb[0][2], pb[0][3], pb[1][0], pb[1][1], pb[1][2], pb[1][3]};
#pragma unroll
    for (int n = 0; n < NBLK; ++n) {
      const u32x4 vv = {vf[0][n].x, vf[0][n].y, vf[1][n].x, vf[1][n].y};
      const f32x4 cin = acc[n] * alpha;
      const f32x4 res = mfma16x16x32(__builtin_bit_cast(bf16x8, vv), pfrag, cin);
      acc[n] = live ? res : acc[n];
    }
    m_run = live ? m_new : m_run;
    l_run = live ? l_new : l_run;
  }

  if (rk_lo <= rk_hi) {
    const int64_t row = (int64_t)(q0 + tq0 + t) * a.num_q_heads + (kvh << a.log2_group) + hh;
    const int64_t idx = row * a.ns + sigma;
    if (g4 == 0) a.ws_ml[idx] = make_float2(m_run, l_run);
    float* ap = a.ws_acc + idx * D;
#pragma unroll
    for (int n = 0; n < NBLK; ++n) *reinterpret_cast<f32x4*>(ap + 16 * n + 4 * g4) = acc[n];
  }
}

// ---------------------------------------------------------------------------
// Merge phase: one thread per (row, 4 head-dim elements).  Splits are combined
// in increasing order: m* = max m_s, w_s = 2^(m_s - m*), L = sum w_s l_s,
// N = sum w_s acc_s, o = N / L.  With a single split w = 1 exactly and the
// result is acc / l.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const AttnMergeArgs a) {
  constexpr int TPR = D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t row = gid / TPR;
  const int dq = (int)(gid % TPR);
  if (row >= (int64_t)a.num_tokens * a.num_q_heads) return;
  const int tok = (int)(row / a.num_q_heads);
  const int s = find_token_seq(a.qsl, a.num_seqs, tok);
  const int q0 = a.qsl[s];
  const int q_len = a.qsl[s + 1] - q0;
  const int k_len = a.seq_lens[s];
  const int p = k_len - q_len + (tok - q0);
  const int lo = a.window > 0 ? max(0, p - a.window + 1) : 0;
  const int sig_lo = lo / a.split;
  const int sig_hi = min(p / a.split, a.ns - 1);
  uint16_t* op = a.out + row * D + 4 * dq;
  if (p < 0 || sig_lo > sig_hi) {
    *reinterpret_cast<u32x2*>(op) = u32x2{0u, 0u};
    return;
  }
  const float2* ml = a.ws_ml + row * a.ns;
  float mstar = -INFINITY;
  for (int sg = sig_lo; sg <= sig_hi; ++sg) mstar = fmaxf(mstar, ml[sg].x);
  float L = 0.f;
  f32x4 N = {0.f, 0.f, 0.f, 0.f};
  const float* ap = a.ws_acc + row * a.ns * D + 4 * dq;
  for (int sg = sig_lo; sg <= sig_hi; ++sg) {
    const float2 v = ml[sg];
    const float w = exp2_hw(v.x - mstar);
    L = __builtin_fmaf(w, v.y, L);
    const f32x4 av = *reinterpret_cast<const f32x4*>(ap + (int64_t)sg * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) N[i] = __builtin_fmaf(w, av[i], N[i]);
  }
  bf16x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = (__bf16)(N[i] / L + 0.0f);
  *reinterpret_cast<u32x2*>(op) = __builtin_bit_cast(u32x2, o);
}

template <int D>
hipError_t split_launch(const AttnSplitArgs& a, hipStream_t stream) {
  const int tq = kRowsPerBlock >> a.log2_group;
  const int nblocks = a.num_tokens / tq + a.num_seqs;
  dim3 grid(nblocks, a.num_kv_heads, (a.ns + kSplitWaves - 1) / kSplitWaves);
  hipLaunchKernelGGL(attn_split_kernel<D>, grid, dim3(64 * kSplitWaves), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t merge_launch(const AttnMergeArgs& a, hipStream_t stream) {
  const int64_t threads = (int64_t)a.num_tokens * a.num_q_heads * (D / 4);
  dim3 grid((unsigned)((threads + 255) / 256));
  hipLaunchKernelGGL(attn_merge_kernel<D>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_split(int head_dim, const AttnSplitArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return split_launch<64>(a, stream);
    case 128: return split_launch<128>(a, stream);
    case 256: return split_launch<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_merge(int head_dim, const AttnMergeArgs& a, hipStream_t stream) {
  switch (head_dim) {
    case 64: return merge_launch<64>(a, stream);
    case 128: return merge_launch<128>(a, stream);
    case 256: return merge_launch<256>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bi
