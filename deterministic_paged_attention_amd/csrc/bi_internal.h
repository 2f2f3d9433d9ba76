// Internal declarations shared by the C-ABI layer (api.hip) and the kernel
// translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bi {

// Largest query-row block: the 16 columns of one 16x16 MFMA output.
constexpr int kRowsPerBlock = 16;
// Key tile: two pages of 16 tokens, the K extent of one 16x16x32 MFMA.
constexpr int kKeyTile = 32;
// Waves per attention split workgroup (each wave works through its own items).
constexpr int kSplitWaves = 4;

struct AttnSplitArgs {
  const uint16_t* q;
  int64_t q_stride;          // elements between token rows of q
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* page_table;
  int32_t pt_stride;
  int32_t num_pages;
  const int32_t* seq_lens;
  const int32_t* qsl;        // query_start_loc [num_seqs + 1]
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t log2_group;        // log2(H_q / H_kv)
  int32_t split;             // keys per split (multiple of kKeyTile)
  int32_t window;            // 0 = none
  int32_t ns;                // splits per row in the workspace
  float qk_scale_log2;       // scale * log2(e)
  float2* ws_ml;             // [R][ns]
  uint16_t* ws_acc;          // [R][ns][D] bf16
  int32_t* plan;             // [num_seqs + 1]: first work item of each sequence, total last
  int32_t qblocks;           // query-row blocks per work item (set by the launcher)
  int32_t spread;            // 1: consecutive items go to different workgroups (set by the launcher)
  uint16_t* out;             // bf16 [T][H_q][D]: written directly by the row-group decode mapping
  int32_t rg_static_rounds;  // row-group mapping: rounds of row groups dealt statically (set by the launcher)
  int32_t force_kind;        // diagnostic: 0 = choose the split-phase mapping; else 1, 4 or 8 blocks per item
};

struct AttnMergeArgs {
  const int32_t* seq_lens;
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t num_q_heads;
  int32_t split;
  int32_t window;
  int32_t ns;
  const float2* ws_ml;
  const uint16_t* ws_acc;
  uint16_t* out;             // bf16 [T][H_q][D]
};

hipError_t launch_attn_split(int head_dim, const AttnSplitArgs& a, hipStream_t stream);
// Decode batches (every q_len = 1) with enough (sequence, KV head) row groups
// to fill the GPU run split and merge in one launch that keeps the partials in
// LDS and writes only a.out (bitwise the split + merge result).  Returns true
// when this mapping applies to the arguments (needs the current device).
bool attn_rowgroup_applies(int head_dim, const AttnSplitArgs& a);
hipError_t launch_attn_rowgroup(int head_dim, const AttnSplitArgs& a, hipStream_t stream);
// Query-row blocks per work item the split launch would use for these arguments
// (1 one-block items, 4 wide items, 8 shared-tile items; needs the current
// device; 0 on failure or when a forced mapping does not exist at this head
// size, where the launch fails too).
int attn_item_blocks(int head_dim, const AttnSplitArgs& a);
hipError_t launch_attn_merge(int head_dim, const AttnMergeArgs& a, hipStream_t stream);

hipError_t launch_slot_mapping(const int32_t* page_table, int32_t stride, const int32_t* seq_lens,
                               const int32_t* qsl, int32_t num_seqs, int32_t num_tokens,
                               int32_t page_size, int32_t num_pages, int32_t* slots,
                               hipStream_t stream);

hipError_t launch_kv_write(int head_dim, int num_kv_heads, const uint16_t* k_new, int64_t k_stride,
                           const uint16_t* v_new, int64_t v_stride, const int32_t* slots,
                           int32_t num_tokens, uint16_t* k_cache, uint16_t* v_cache,
                           int32_t num_pages, hipStream_t stream);
// As launch_kv_write with each token's slot computed from the page table
// (the slot-mapping kernel's rule, page size 16).
hipError_t launch_kv_write_paged(int head_dim, int num_kv_heads, const uint16_t* k_new, int64_t k_stride,
                                 const uint16_t* v_new, int64_t v_stride, const int32_t* page_table, int32_t stride,
                                 const int32_t* seq_lens, const int32_t* qsl, int32_t num_seqs, int32_t num_tokens,
                                 uint16_t* k_cache, uint16_t* v_cache, int32_t num_pages, hipStream_t stream);

hipError_t launch_rmsnorm(const uint16_t* x, int64_t ldx, const uint16_t* gamma, float eps,
                          int64_t M, int64_t H, uint16_t* y, int64_t ldy, hipStream_t stream);
hipError_t launch_add_rmsnorm(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, uint16_t* s,
                              int64_t lds, const uint16_t* gamma, float eps, int64_t M, int64_t H, uint16_t* y,
                              int64_t ldy, hipStream_t stream);

// out_kind: 0 = bf16, 1 = fp32.  k range [k_begin, k_begin + k_len_per_split) per
// blockIdx.z when k_splits > 1 (partials to fp32 [k_splits][M][N], ldc = N).
// out[m, i] = gated_gelu((a w^T)[m, i], (a w^T)[m, F + i]) for a [gate | up]
// weight w of 2F rows, each product rounded to bf16 first: the bits of
// launch_gemm (bf16 out) followed by launch_gated_gelu, in one launch; M <= 16.
hipError_t launch_gemm_gated_gelu(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, uint16_t* out,
                                  int64_t ldo, int64_t M, int64_t F, int64_t K, hipStream_t stream);
hipError_t launch_gemm(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw, void* c,
                       int64_t ldc, int out_kind, int64_t M, int64_t N, int64_t K,
                       hipStream_t stream);
hipError_t launch_gemm_splitk(const uint16_t* a, int64_t lda, const uint16_t* w, int64_t ldw,
                              float* partial, int64_t M, int64_t N, int64_t K, int32_t k_splits,
                              hipStream_t stream);
hipError_t launch_gemm_splitk_reduce(const float* partial, int32_t k_splits, int64_t M, int64_t N,
                                     void* c, int64_t ldc, int out_kind, hipStream_t stream);

hipError_t launch_embedding(const uint16_t* table, int64_t vocab, int64_t hidden, const int32_t* ids,
                            int32_t num_tokens, uint16_t* out, int64_t ld_out, hipStream_t stream);
// slots == nullptr: q and k rows only; otherwise also the cache write of k and v.
hipError_t launch_qk_norm_rope(uint16_t* qkv, int64_t row_stride, int32_t num_tokens, const int32_t* seq_lens,
                               const int32_t* qsl, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, const uint16_t* gamma_q, const uint16_t* gamma_k, float eps,
                               double theta, const int32_t* slots, uint16_t* k_cache, uint16_t* v_cache,
                               int32_t num_pages, hipStream_t stream);
hipError_t launch_add(const uint16_t* a, int64_t lda, const uint16_t* b, int64_t ldb, uint16_t* c, int64_t ldc,
                      int64_t rows, int64_t n, hipStream_t stream);
hipError_t launch_argmax(const float* x, int64_t ld, int64_t rows, int64_t n, int32_t* out, hipStream_t stream);
// Streaming-read reference (measurement only): kStreamReadGroups workgroups,
// sink[g] = xor of the 32-bit words workgroup g read.  bytes % 16 == 0.
constexpr int kStreamReadGroups = 8192;
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t stream);
// MFMA throughput reference (measurement only): kMfmaPeakGroups workgroups of
// four waves; `rounds` (a multiple of 4) rounds of eight bf16 16x16x32 MFMAs
// per wave, fragments filled with `value`; sink[wave] = sum of element 0 of
// the wave's eight accumulators.
constexpr int kMfmaPeakGroups = 2048;
hipError_t launch_mfma_peak(float value, int32_t rounds, float* sink, hipStream_t stream);
int64_t mfma_peak_flops(int32_t rounds);
hipError_t launch_gated_gelu(const uint16_t* in, int64_t ld_in, uint16_t* out, int64_t ld_out, int64_t rows,
                             int64_t F, hipStream_t stream);

}  // namespace bi
