// Per-row and elementwise glue of a decoder step: embedding gather, per-head
// q/k RMSNorm fused with rotary position embedding, residual add, gated GELU,
// and greedy sampling (argmax over a logits row).
//
// The pages define the step only as the cold causal forward Forward(W, h)
// (Vosti deep-dive blog (深入解析 Vosti), §2, Theorem 4.1); the layer details
// here are the plainest Gemma-3-style choices (pre-norm blocks, q/k norm,
// half-rotation RoPE, tanh-approximated gated GELU).  Every output element
// depends only on its own row (token) and, for RoPE, its logical position —
// never on the batch — and every reduction has a tree fixed by the row size.

#include "bi_internal.h"
#include "gelu.h"

#include <math.h>

namespace bi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// (Every sequence has at least one query row, so when there are as many
// tokens as sequences token t is sequence t's only row: no search.)
__device__ __forceinline__ int find_token_seq(const int32_t* qsl, int num_seqs, int num_tokens, int t) {
  if (num_tokens == num_seqs) return t;
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// out[t, :] = table[ids[t], :]; rows with an id outside [0, vocab) are zero.
__global__ __launch_bounds__(256) void embedding_kernel(const uint16_t* table, int64_t vocab, int64_t hidden,
                                                        const int32_t* ids, int32_t num_tokens, uint16_t* out,
                                                        int64_t ld_out) {
  const int64_t nch = hidden / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (int64_t)num_tokens * nch) return;
  const int64_t t = gid / nch, c = gid % nch;
  const int32_t id = ids[t];
  u32x4 v = {0u, 0u, 0u, 0u};
  if (id >= 0 && id < vocab) v = *reinterpret_cast<const u32x4*>(table + (int64_t)id * hidden + 8 * c);
  *reinterpret_cast<u32x4*>(out + t * ld_out + 8 * c) = v;
}

// Normalise and rotate one head row x (head_dim D) in place, one wave:
//   y = x / sqrt(sum x^2 / D + eps) * gamma         (fp32; fixed tree over D)
//   z_i       = y_i cos(a_i) - y_{i+D/2} sin(a_i)
//   z_{i+D/2} = y_i sin(a_i) + y_{i+D/2} cos(a_i),  a_i = p * theta^(-2i/D),  i < D/2
// with p the row's logical position.  The angle and its sine and cosine are
// evaluated in fp64 and rounded once to fp32; the result is rounded once to
// bf16.  This lane owns the pairs (i, i + D/2) for i = lane, lane + 64 (at most
// two for D <= 256); their results are returned in z[j] (i) and z[2 + j]
// (i + D/2), as bf16 bits.
__device__ __forceinline__ void norm_rope_row(uint16_t* x, const uint16_t* g, int head_dim, int p, float eps,
                                              double log2_theta, int lane, uint16_t (&z)[4]) {
  const int half = head_dim / 2;
  float a[2] = {0.f, 0.f}, b[2] = {0.f, 0.f};
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lane + 64 * j;
    if (i < half) {
      a[j] = bf16_to_f32(x[i]);
      b[j] = bf16_to_f32(x[i + half]);
      ss = __builtin_fmaf(a[j], a[j], ss);
      ss = __builtin_fmaf(b[j], b[j], ss);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.0f / __builtin_sqrtf(ss / (float)head_dim + eps);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = lane + 64 * j;
    z[j] = z[2 + j] = 0;
    if (i < half) {
      const float ya = (a[j] * inv) * bf16_to_f32(g[i]);
      const float yb = (b[j] * inv) * bf16_to_f32(g[i + half]);
      const double ang = (double)p * exp2(-(double)(2 * i) / (double)head_dim * log2_theta);
      const float c = (float)cos(ang), sn = (float)sin(ang);
      z[j] = f32_to_bf16(ya * c - yb * sn);
      z[2 + j] = f32_to_bf16(ya * sn + yb * c);
      x[i] = z[j];
      x[i + half] = z[2 + j];
    }
  }
}

// Element offsets, inside one (page, KV head) block of 16 tokens, of
// head-dim element d of token slot o, in the cache layouts
//   K [D/8][16][8]:          ((d / 8) * 16 + o) * 8 + d % 8
//   V [D/32][16][16][2]:     d = 32 np + 16 e + r  ->  ((np * 16 + r) * 16 + o) * 2 + e
__device__ __forceinline__ int64_t k_elem(int d, int o) { return ((int64_t)(d >> 3) * 16 + o) * 8 + (d & 7); }
__device__ __forceinline__ int64_t v_elem(int d, int o) {
  return ((int64_t)((d >> 5) * 16 + (d & 15)) * 16 + o) * 2 + ((d >> 4) & 1);
}

// One wave per (token, head) row of the q and k parts of a fused QKV row
// (norm_rope_row on each, in place).  With slots != nullptr the kernel also
// covers the v part and writes each token's k (after the rotation) and v rows
// into the paged caches at slots[t] (skipped for a negative slot or a page
// past the pool), exactly as the separate cache write does.
__global__ __launch_bounds__(256) void qk_norm_rope_kernel(uint16_t* qkv, int64_t row_stride, int32_t num_tokens,
                                                           const int32_t* seq_lens, const int32_t* qsl,
                                                           int32_t num_seqs, int32_t num_q_heads,
                                                           int32_t num_kv_heads, int32_t head_dim,
                                                           const uint16_t* gamma_q, const uint16_t* gamma_k,
                                                           float eps, double log2_theta, const int32_t* slots,
                                                           uint16_t* k_cache, uint16_t* v_cache, int32_t num_pages) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int heads = num_q_heads + num_kv_heads * (slots ? 2 : 1);
  if (row >= (int64_t)num_tokens * heads) return;
  const int t = (int)(row / heads);
  const int h = (int)(row % heads);
  uint16_t* x = qkv + (int64_t)t * row_stride + (int64_t)h * head_dim;
  int64_t base = -1;  // element offset of this token's (page, KV head) block in the caches
  if (slots && h >= num_q_heads) {
    const int slot = slots[t];
    if (slot >= 0 && (slot >> 4) < num_pages)
      base = ((int64_t)(slot >> 4) * num_kv_heads + (h - num_q_heads) % num_kv_heads) * ((int64_t)head_dim * 16);
  }
  if (h >= num_q_heads + num_kv_heads) {  // v row: copy into the cache
    if (base < 0) return;
    const int o = slots[t] & 15;
    // head dims d (e = 0) and d + 16 (e = 1) of one (np, r) are adjacent: one 4-byte store
    for (int j = lane; j < head_dim / 2; j += 64) {
      const int d = 32 * (j >> 4) + (j & 15);
      *reinterpret_cast<uint32_t*>(v_cache + base + v_elem(d, o)) = (uint32_t)x[d] | ((uint32_t)x[d + 16] << 16);
    }
    return;
  }
  const int s = find_token_seq(qsl, num_seqs, num_tokens, t);
  const int p = seq_lens[s] - (qsl[s + 1] - qsl[s]) + (t - qsl[s]);
  uint16_t z[4];
  norm_rope_row(x, h < num_q_heads ? gamma_q : gamma_k, head_dim, p, eps, log2_theta, lane, z);
  if (base >= 0) {  // k row: the rotated values into the cache
    const int o = slots[t] & 15, half = head_dim / 2;
    // head dims i and i + 1 (i even) are adjacent in a K chunk: the odd lane's
    // values travel to the even lane, which makes one 4-byte store of each pair
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int i = lane + 64 * j;
      const uint32_t lo_next = (uint32_t)__shfl_down((int)z[j], 1);
      const uint32_t hi_next = (uint32_t)__shfl_down((int)z[2 + j], 1);
      if (i < half && (lane & 1) == 0) {
        *reinterpret_cast<uint32_t*>(k_cache + base + k_elem(i, o)) = (uint32_t)z[j] | (lo_next << 16);
        *reinterpret_cast<uint32_t*>(k_cache + base + k_elem(i + half, o)) = (uint32_t)z[2 + j] | (hi_next << 16);
      }
    }
  }
}

// c = a + b elementwise in fp32, one bf16 rounding; rows of length n with strides.
__global__ __launch_bounds__(256) void add_kernel(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb,
                                                  uint16_t* c, int64_t ldc, int64_t rows, int64_t n) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= rows * n) return;
  const int64_t r = gid / n, i = gid % n;
  c[r * ldc + i] = f32_to_bf16(bf16_to_f32(a[r * lda + i]) + bf16_to_f32(b[r * ldb + i]));
}

// out[t, i] = gelu(gate[t, i]) * up[t, i], gate = in[t, 0:F], up = in[t, F:2F];
// gelu(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), fp32, one bf16 rounding.
__global__ __launch_bounds__(256) void gated_gelu_kernel(const uint16_t* in, int64_t ld_in, uint16_t* out,
                                                         int64_t ld_out, int64_t rows, int64_t F) {
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (gid >= rows * F) return;
  const int64_t r = gid / F, i = gid % F;
  const float x = bf16_to_f32(in[r * ld_in + i]);
  const float u = bf16_to_f32(in[r * ld_in + F + i]);
  out[r * ld_out + i] = f32_to_bf16(gated_gelu_f32(x, u));
}

// Greedy sampling: out[row] = the smallest index i with x[row, i] maximal
// (NaN never wins; an all-NaN row gives 0).  One workgroup of 1024 threads per
// row: each pass issues kArgUnroll independent 16-byte loads per thread before
// comparing any of them, so a single row keeps enough reads in flight to
// stream a 256K-entry vocabulary from one compute unit.  (value, index) pairs
// are combined by "larger value, else smaller index", a total order, so the
// result does not depend on which thread saw which element or on the
// combining tree.
struct ArgBest {
  float v;
  int64_t i;  // -1: nothing seen
};

__device__ __forceinline__ ArgBest arg_better(ArgBest a, ArgBest b) {
  if (a.i < 0) return b;
  if (b.i < 0) return a;
  if (a.v > b.v || (a.v == b.v && a.i < b.i)) return a;
  return b;
}

__device__ __forceinline__ void arg_consider(ArgBest& b, float v, int64_t i) {
  if (v == v && (b.i < 0 || v > b.v || (v == b.v && i < b.i))) b = ArgBest{v, i};
}

constexpr int kArgThreads = 1024;
constexpr int kArgUnroll = 8;

__global__ __launch_bounds__(kArgThreads) void argmax_kernel(const float* x, int64_t ld, int64_t n, int32_t* out) {
  __shared__ float sv[kArgThreads / 64];
  __shared__ int64_t si[kArgThreads / 64];
  const int t = threadIdx.x;
  const float* xr = x + (int64_t)blockIdx.x * ld;
  ArgBest b{0.f, -1};
  // scalar head up to the first 16-byte boundary (x is 4-byte aligned)
  int64_t head = (int64_t)(((16 - ((uintptr_t)xr & 15)) & 15) >> 2);
  if (head > n) head = n;
  if (t < head) arg_consider(b, xr[t], t);
  const float4* xv = reinterpret_cast<const float4*>(xr + head);
  const int64_t nv = (n - head) >> 2;
  constexpr int64_t kPass = (int64_t)kArgThreads * kArgUnroll;
  const int64_t full = nv / kPass * kPass;
  for (int64_t base = 0; base < full; base += kPass) {
    float4 r[kArgUnroll];
#pragma unroll
    for (int u = 0; u < kArgUnroll; ++u) r[u] = xv[base + u * kArgThreads + t];
#pragma unroll
    for (int u = 0; u < kArgUnroll; ++u) {
      const int64_t i = head + 4 * (base + u * kArgThreads + t);
      arg_consider(b, r[u].x, i);
      arg_consider(b, r[u].y, i + 1);
      arg_consider(b, r[u].z, i + 2);
      arg_consider(b, r[u].w, i + 3);
    }
  }
  for (int64_t j = full + t; j < nv; j += kArgThreads) {
    const float4 r = xv[j];
    const int64_t i = head + 4 * j;
    arg_consider(b, r.x, i);
    arg_consider(b, r.y, i + 1);
    arg_consider(b, r.z, i + 2);
    arg_consider(b, r.w, i + 3);
  }
  const int64_t tail = head + 4 * nv;  // at most three scalar entries remain
  if (tail + t < n) arg_consider(b, xr[tail + t], tail + t);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ArgBest o;
    o.v = __shfl_xor(b.v, off);
    o.i = __shfl_xor(b.i, off);
    b = arg_better(b, o);
  }
  const int wave = t >> 6;
  if ((t & 63) == 0) {
    sv[wave] = b.v;
    si[wave] = b.i;
  }
  __syncthreads();
  if (t == 0) {
    ArgBest r{sv[0], si[0]};
    for (int w = 1; w < kArgThreads / 64; ++w) r = arg_better(r, ArgBest{sv[w], si[w]});
    out[blockIdx.x] = r.i < 0 ? 0 : (int32_t)r.i;
  }
}

unsigned blocks_for(int64_t n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t launch_embedding(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* ids,
                            int32_t num_tokens, uint16_t* out, int64_t ld_out, hipStream_t stream) {
  const int64_t n = (int64_t)num_tokens * (hidden / 8);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(embedding_kernel, dim3(blocks_for(n)), dim3(256), 0, stream, table, vocab, hidden, ids,
                     num_tokens, out, ld_out);
  return hipGetLastError();
}

hipError_t launch_qk_norm_rope(uint16_t* qkv, int64_t row_stride, int32_t num_tokens, const int32_t* seq_lens,
                               const int32_t* qsl, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, const uint16_t* gamma_q, const uint16_t* gamma_k, float eps,
                               double theta, const int32_t* slots, uint16_t* k_cache, uint16_t* v_cache,
                               int32_t num_pages, hipStream_t stream) {
  const int64_t rows = (int64_t)num_tokens * (num_q_heads + num_kv_heads * (slots ? 2 : 1));
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(qk_norm_rope_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, qkv, row_stride,
                     num_tokens, seq_lens, qsl, num_seqs, num_q_heads, num_kv_heads, head_dim, gamma_q, gamma_k,
                     eps, log2(theta), slots, k_cache, v_cache, num_pages);
  return hipGetLastError();
}

hipError_t launch_add(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, uint16_t* c, int64_t ldc,
                      int64_t rows, int64_t n, hipStream_t stream) {
  if (rows * n == 0) return hipSuccess;
  hipLaunchKernelGGL(add_kernel, dim3(blocks_for(rows * n)), dim3(256), 0, stream, a, lda, b, ldb, c, ldc, rows, n);
  return hipGetLastError();
}

hipError_t launch_argmax(const float* x, int64_t ld, int64_t rows, int64_t n, int32_t* out, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(argmax_kernel, dim3((unsigned)rows), dim3(kArgThreads), 0, stream, x, ld, n, out);
  return hipGetLastError();
}

hipError_t launch_gated_gelu(const uint16_t* in, int64_t ld_in, uint16_t* out, int64_t ld_out, int64_t rows,
                             int64_t F, hipStream_t stream) {
  if (rows * F == 0) return hipSuccess;
  hipLaunchKernelGGL(gated_gelu_kernel, dim3(blocks_for(rows * F)), dim3(256), 0, stream, in, ld_in, out, ld_out,
                     rows, F);
  return hipGetLastError();
}

}  // namespace bi
