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

// One thread per (token, KV head, pair of 8-element head-dim chunks c0, c0 + 2):
// c0 = 4k or 4k + 1, so the two chunks hold head dims d and d + 16 with the
// same (np, r) of the V layout.
// K cache [page][h][D/8][16][8]: each chunk is one 16-byte store.
// V cache [page][h][D/32][16][16][2] (head-dim d = 32*np + 16*e + r, token o at
// ((np*16 + r)*16 + o)*2 + e): the e = 0 and e = 1 values of one (np, r) are
// adjacent, so the pair of chunks is eight 4-byte stores.
template <int D>
__global__ __launch_bounds__(256) void kv_write_kernel(int num_kv_heads, const uint16_t* k_new, int64_t k_stride,
                                                       const uint16_t* v_new, int64_t v_stride,
                                                       const SlotSource slots, int32_t num_tokens,
                                                       uint16_t* k_cache, uint16_t* v_cache, int32_t num_pages) {
  constexpr int NP = D / 16;  // chunk pairs per head
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)num_tokens * num_kv_heads * NP;
  if (gid >= total) return;
  const int q = (int)(gid % NP);
  const int h = (int)((gid / NP) % num_kv_heads);
  const int t = (int)(gid / ((int64_t)NP * num_kv_heads));
  const int slot = slots.at(t, num_pages);
  if (slot < 0) return;
  const int pg = slot >> 4;
  const int o = slot & 15;
  if (pg >= num_pages) return;
  const int c0 = 4 * (q >> 1) + (q & 1), c1 = c0 + 2;
  const int64_t head_base = ((int64_t)pg * num_kv_heads + h) * (D * 16);
  const uint16_t* kr = k_new + (int64_t)t * k_stride + h * D;
  const uint16_t* vr = v_new + (int64_t)t * v_stride + h * D;
  const u32x4 k0 = *reinterpret_cast<const u32x4*>(kr + 8 * c0);
  const u32x4 k1 = *reinterpret_cast<const u32x4*>(kr + 8 * c1);
  *reinterpret_cast<u32x4*>(k_cache + head_base + (c0 * 16 + o) * 8) = k0;
  *reinterpret_cast<u32x4*>(k_cache + head_base + (c1 * 16 + o) * 8) = k1;
  const u32x4 v0 = *reinterpret_cast<const u32x4*>(vr + 8 * c0);
  const u32x4 v1 = *reinterpret_cast<const u32x4*>(vr + 8 * c1);
  // d = 8 c0 + i: np = c0 / 4, r = 8 (c0 & 1) + i; its e = 1 partner d + 16 is element i of chunk c1.
  const int np = c0 >> 2, r0 = 8 * (c0 & 1);
  uint32_t* vd = reinterpret_cast<uint32_t*>(v_cache + head_base + ((int64_t)(np * 16 + r0) * 16 + o) * 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    vd[(2 * i) * 16] = (v0[i] & 0xffffu) | (v1[i] << 16);
    vd[(2 * i + 1) * 16] = (v0[i] >> 16) | (v1[i] & 0xffff0000u);
  }
}

template <int D>
hipError_t kv_write_launch(int num_kv_heads, const uint16_t* k_new, int64_t k_stride, const uint16_t* v_new,
                           int64_t v_stride, const SlotSource& slots, int32_t num_tokens, uint16_t* k_cache,
                           uint16_t* v_cache, int32_t num_pages, hipStream_t stream) {
  const int64_t total = (int64_t)num_tokens * num_kv_heads * (D / 16);
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
