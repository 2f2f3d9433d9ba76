// Slot mapping and KV write for the paged cache.
//
// Vosti deep-dive blog (深入解析 Vosti), §3.2: invariant 1 (page tables map a
// request's prefix to allocated, in-range slots), invariant 2 and §5.1 (the
// KV value stored for position p is that logical position's value whatever
// page holds it), invariant 3 (a step writes only private, pairwise distinct
// slots; checked on the host by bi_check_write_plan).  Both kernels are pure
// integer addressing and copies, so they are bit-exact by construction.

#include "bi_internal.h"

namespace bi {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Slot of new token t: page_table[s][p / P] * P + p % P for the token's
// sequence s and logical position p = seq_lens[s] - q_len_s + j; -1 when the
// entry is outside the table row or names no page of the pool.
__device__ __forceinline__ int token_slot(const int32_t* page_table, int32_t stride, const int32_t* seq_lens,
                                          const int32_t* qsl, int32_t num_seqs, int32_t num_tokens,
                                          int32_t page_size, int32_t num_pages, int t) {
  const int s = find_token_seq(qsl, num_seqs, num_tokens, t);
  const int q0 = qsl[s];
  const int q_len = qsl[s + 1] - q0;
  const int p = seq_lens[s] - q_len + (t - q0);
  int slot = -1;
  if (p >= 0 && t < qsl[s + 1]) {
    const int lp = p / page_size;
    if (lp < stride) {
      const int pg = page_table[(int64_t)s * stride + lp];
      if (pg >= 0 && pg < num_pages) slot = pg * page_size + p % page_size;
    }
  }
  return slot;
}

__global__ __launch_bounds__(256) void slot_mapping_kernel(const int32_t* page_table, int32_t stride,
                                                           const int32_t* seq_lens, const int32_t* qsl,
                                                           int32_t num_seqs, int32_t num_tokens,
                                                           int32_t page_size, int32_t num_pages,
                                                           int32_t* slots) {
  const int t = blockIdx.x * 256 + threadIdx.x;
  if (t >= num_tokens) return;
  slots[t] = token_slot(page_table, stride, seq_lens, qsl, num_seqs, num_tokens, page_size, num_pages, t);
}

// Where the cache write finds each token's slot: a slot mapping, or the page
// table itself (the slot-mapping kernel's computation, done in place).
struct SlotSource {
  const int32_t* slots;       // non-null: slots[t]
  const int32_t* page_table;  // else token_slot over these
  int32_t stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t num_tokens;
  __device__ __forceinline__ int at(int t, int num_pages) const {
    return slots ? slots[t] : token_slot(page_table, stride, seq_lens, qsl, num_seqs, num_tokens, 16, num_pages, t);
  }
};

// One thread per (token, KV head, 8-element head-dim chunk c).
// K cache [page][h][D/8][16][8]: the chunk is one 16-byte store.
// V cache [page][h][D/32][16][16][2] (head-dim d = 32*np + 16*e + r, token o at
// ((np*16 + r)*16 + o)*2 + e): eight 2-byte stores.
template <int D>
__global__ __launch_bounds__(256) void kv_write_kernel(int num_kv_heads, const uint16_t* k_new, int64_t k_stride,
                                                       const uint16_t* v_new, int64_t v_stride,
                                                       const SlotSource slots, int32_t num_tokens,
                                                       uint16_t* k_cache, uint16_t* v_cache, int32_t num_pages) {
  constexpr int NC = D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * NC;
  if (gid >= total) return;
  const int c = (int)(gid % NC);
  const int h = (int)((gid / NC) % num_kv_heads);
  const int t = (int)(gid / ((int64_t)NC * num_kv_heads));
  const int slot = slots.at(t, num_pages);
  if (slot < 0) return;
  const int pg = slot >> 4;
  const int o = slot & 15;
  if (pg >= num_pages) return;
  const int64_t head_base = ((int64_t)pg * num_kv_heads + h) * (D * 16);
  const u32x4 kv = *reinterpret_cast<const u32x4*>(k_new + (int64_t)t * k_stride + h * D + 8 * c);
  *reinterpret_cast<u32x4*>(k_cache + head_base + (c * 16 + o) * 8) = kv;
  const u32x4 vv = *reinterpret_cast<const u32x4*>(v_new + (int64_t)t * v_stride + h * D + 8 * c);
  // d = 8c + i: np = c / 4, e = (c / 2) & 1, r = 8 * (c & 1) + i.
  const int np = c >> 2, ev = (c >> 1) & 1, r0 = 8 * (c & 1);
  uint16_t* vd = v_cache + head_base + ((int64_t)(np * 16 + r0) * 16 + o) * 2 + ev;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vd[(2 * i) * 32] = (uint16_t)(vv[i] & 0xffffu);
    vd[(2 * i + 1) * 32] = (uint16_t)(vv[i] >> 16);
  }
}

template <int D>
hipError_t kv_write_launch(int num_kv_heads, const uint16_t* k_new, int64_t k_stride, const uint16_t* v_new,
                           int64_t v_stride, const SlotSource& slots, int32_t num_tokens, uint16_t* k_cache,
                           uint16_t* v_cache, int32_t num_pages, hipStream_t stream) {
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (D / 8);
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_write_kernel<D>, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     num_kv_heads, k_new, k_stride, v_new, v_stride, slots, num_tokens, k_cache, v_cache,
                     num_pages);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_slot_mapping(const int32_t* page_table, int32_t stride, const int32_t* seq_lens,
                               const int32_t* qsl, int32_t num_seqs, int32_t num_tokens,
                               int32_t page_size, int32_t num_pages, int32_t* slots, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3((num_tokens + 255) / 256), dim3(256), 0, stream, page_table,
                     stride, seq_lens, qsl, num_seqs, num_tokens, page_size, num_pages, slots);
  return hipGetLastError();
}

hipError_t launch_kv_write(int head_dim, int num_kv_heads, const uint16_t* k_new, int64_t k_stride,
                           const uint16_t* v_new, int64_t v_stride, const int32_t* slots, int32_t num_tokens,
                           uint16_t* k_cache, uint16_t* v_cache, int32_t num_pages, hipStream_t stream) {
  const SlotSource src{slots, nullptr, 0, nullptr, nullptr, 0, 0};
  switch (head_dim) {
    case 64: return kv_write_launch<64>(num_kv_heads, k_new, k_stride, v_new, v_stride, src, num_tokens, k_cache, v_cache, num_pages, stream);
    case 128: return kv_write_launch<128>(num_kv_heads, k_new, k_stride, v_new, v_stride, src, num_tokens, k_cache, v_cache, num_pages, stream);
    case 256: return kv_write_launch<256>(num_kv_heads, k_new, k_stride, v_new, v_stride, src, num_tokens, k_cache, v_cache, num_pages, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_kv_write_paged(int head_dim, int num_kv_heads, const uint16_t* k_new, int64_t k_stride,
                                 const uint16_t* v_new, int64_t v_stride, const int32_t* page_table, int32_t stride,
                                 const int32_t* seq_lens, const int32_t* qsl, int32_t num_seqs, int32_t num_tokens,
                                 uint16_t* k_cache, uint16_t* v_cache, int32_t num_pages, hipStream_t stream) {
  const SlotSource src{nullptr, page_table, stride, seq_lens, qsl, num_seqs, num_tokens};
  switch (head_dim) {
    case 64: return kv_write_launch<64>(num_kv_heads, k_new, k_stride, v_new, v_stride, src, num_tokens, k_cache, v_cache, num_pages, stream);
    case 128: return kv_write_launch<128>(num_kv_heads, k_new, k_stride, v_new, v_stride, src, num_tokens, k_cache, v_cache, num_pages, stream);
    case 256: return kv_write_launch<256>(num_kv_heads, k_new, k_stride, v_new, v_stride, src, num_tokens, k_cache, v_cache, num_pages, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bi
