/*
 * bi.h — batch-invariant paged attention, RMSNorm and matrix product for
 * AMD MI355X (gfx950).  C ABI of libbi.so.
 *
 * Property.  For the same token history every output row is bitwise identical
 * whatever the batch composition, query length or chunk budget, decode versus
 * prefill, physical page layout or prefix reuse (Vosti: Specifying,
 * Implementing, and Verifying Deterministic LLM Inference, abstract; Vosti
 * deep-dive blog (深入解析 Vosti), §6.1 matmul contract and §6.2 attention
 * causal contract).  Invariance holds within one build of this library, one
 * configuration and one GPU model; nothing is claimed across dtypes, kernel
 * configurations, compiler versions or hardware (deep-dive blog, §3.5).
 *
 * Conventions for every function below.
 *  - Pointers named *_dev are device pointers (HBM); the library never
 *    allocates, frees or retains them.  Pointers named *_host are host memory.
 *  - bf16 tensors are passed as raw 16-bit storage (void*), fp32 as float*.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *    Every launch is enqueued on it; no call synchronises the device.
 *  - Arguments are validated on the host before anything is launched; an
 *    invalid call launches nothing and returns a status.  Launch failures
 *    return BI_ERR_HIP.  The text of the last error of the calling thread is
 *    available from bi_last_error_message().
 *  - Device-side data (page tables, lengths) is not read by the host.  Its
 *    validity is a precondition, checkable on host copies with
 *    bi_check_page_table / bi_check_write_plan.  The kernels stay memory-safe
 *    when it is violated (out-of-range page ids are read as zero pages,
 *    positions past the workspace bound are skipped) but the results of rows
 *    that violate it are unspecified.
 *  - No arithmetic result depends on which workgroup or wave computes it, or
 *    when.  The only atomics hand out work (the row-group mapping of
 *    bi_paged_attention claims row groups from a counter in the workspace);
 *    no kernel exchanges data between workgroups.
 */
#ifndef BI_H_
#define BI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum bi_status {
  BI_OK = 0,
  BI_ERR_INVALID_ARG = 1,         /* null pointer, negative size, inconsistent shapes  */
  BI_ERR_UNSUPPORTED_CONFIG = 2,  /* geometry this build has no kernel for: rejected  */
  BI_ERR_OUT_OF_RANGE = 3,        /* a page id / slot / length outside its bound       */
  BI_ERR_WRITE_CONFLICT = 4,      /* two writes to one slot, or a write to a shared page */
  BI_ERR_WORKSPACE_TOO_SMALL = 5, /* caller's workspace below the size query's answer  */
  BI_ERR_HIP = 6                  /* a HIP runtime call failed                          */
} bi_status;

typedef enum bi_dtype { BI_BF16 = 0, BI_F32 = 1 } bi_dtype;

/* ------------------------------------------------------------------------ */
/* Attention configuration.                                                  */
/*                                                                           */
/* Kernel choices are fixed once from the model geometry and never from the  */
/* batch, chunk or prefill-vs-decode state; a geometry with no kernel is     */
/* rejected, there is no runtime autotuning (Vosti deep-dive blog, §3.2,     */
/* "fixed kernel choices").  The key split has a fixed SIZE, not a fixed     */
/* number of splits (record "Deterministic and bit-exact inference", field   */
/* technical, Invariance).                                                   */
/* ------------------------------------------------------------------------ */
typedef struct bi_attn_desc {
  int32_t num_q_heads;   /* H_q; multiple of num_kv_heads                               */
  int32_t num_kv_heads;  /* H_kv; G = H_q / H_kv must divide 16                          */
  int32_t head_dim;      /* D in {64, 128, 256}                                          */
  int32_t page_size;     /* P, tokens per page; this build supports 16                   */
  int32_t split_size;    /* S, keys per split; a positive multiple of 32 (the key tile)  */
  int32_t window;        /* w: 0 = full causal; w >= 1 = keys [max(0, p-w+1), p]         */
  float scale;           /* softmax scale; 0 selects 1/sqrt(head_dim)                    */
} bi_attn_desc;

typedef struct bi_attn_config bi_attn_config; /* opaque, immutable after creation */

/* Create a configuration.  Returns BI_ERR_UNSUPPORTED_CONFIG for a geometry
 * this build has no kernel for and BI_ERR_INVALID_ARG for nonsense values.
 * The handle is owned by the library (free with bi_attn_config_destroy) and
 * may be shared by threads and streams. */
bi_status bi_attn_config_create(const bi_attn_desc* desc, bi_attn_config** out);
void bi_attn_config_destroy(bi_attn_config* cfg);
/* Resolved descriptor (scale filled in) and the fixed key tile (32). */
bi_status bi_attn_config_query(const bi_attn_config* cfg, bi_attn_desc* desc_out,
                               int32_t* key_tile_out);

/* ------------------------------------------------------------------------ */
/* Paged KV cache layout (one layer), bf16, owned by the caller:             */
/*   K: [num_pages][H_kv][D/8][P][8]   (8 head-dim elements of one token are */
/*       contiguous; the 16 tokens of a page follow each other per 8-chunk)  */
/*   V: [num_pages][H_kv][D/32][16][P][2]  element (np, r, o, e) holds token */
/*       o at head-dim d = 32*np + 16*e + r (two head-dim rows 16 apart are  */
/*       interleaved token by token)                                         */
/* Page table: int32 [num_seqs][page_table_stride]; entry i of sequence s is */
/* the physical page holding logical positions [i*P, (i+1)*P).  Entries past */
/* ceil(k_len/P) are never read.                                             */
/* Sequence metadata, device int32: seq_lens[s] = k_len (keys after this     */
/* step's writes); query_start_loc[0..num_seqs] = prefix sums of q_len, with */
/* 1 <= q_len <= k_len.  The new tokens of a sequence are its last q_len     */
/* positions: row i sits at p = k_len - q_len + i (Vosti deep-dive blog,     */
/* §6.2, attention causal contract).                                         */
/* ------------------------------------------------------------------------ */

/* Bytes of one layer's K (or V) cache with num_pages pages. */
bi_status bi_kv_cache_bytes(const bi_attn_config* cfg, int64_t num_pages, size_t* bytes);

/* Slot mapping (Vosti deep-dive blog, §3.2, invariant 1: page tables map the
 * prefix to allocated in-range slots).  For token t, row j of sequence s:
 *   p = seq_lens[s] - q_len_s + j,
 *   slot_mapping_dev[t] = page_table[s][p / P] * P + p % P,
 * or -1 when the page id is outside [0, num_pages) or p / P >= stride.
 * Outputs int32 [num_tokens]. */
bi_status bi_slot_mapping(const int32_t* page_table_dev, int32_t page_table_stride,
                          const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev,
                          int32_t num_seqs, int32_t num_tokens, int32_t page_size,
                          int32_t num_pages, int32_t* slot_mapping_dev, void* stream);

/* KV write (deep-dive blog, §3.2 invariant 2 and §5.1: the value stored at
 * the slot of position p is the value of that logical position).  Copies
 * k_new[t] and v_new[t] ([H_kv][D] bf16, token rows `*_row_stride` elements
 * apart) into slot slot_mapping[t] of the caches above; slots < 0 are
 * skipped.  A pure copy: bit-exact.  The slots of one call must be distinct
 * (write isolation, §3.2 invariant 3); check with bi_check_write_plan. */
bi_status bi_kv_write(const bi_attn_config* cfg,
                      const void* k_new_dev, int64_t k_row_stride,
                      const void* v_new_dev, int64_t v_row_stride,
                      const int32_t* slot_mapping_dev, int32_t num_tokens,
                      void* k_cache_dev, void* v_cache_dev, int32_t num_pages, void* stream);

/* bi_slot_mapping and bi_kv_write in one launch: each new token's slot is
 * computed from the page table as bi_slot_mapping does (page size 16; a slot
 * of -1, i.e. a position outside the table row or an entry naming no page of
 * the pool, is skipped), then its k and v rows are stored there.  The caches
 * end bitwise as after the two calls; the same write-isolation precondition
 * applies (bi_check_write_plan on the slots bi_slot_mapping would give). */
bi_status bi_kv_write_paged(const bi_attn_config* cfg, const void* k_new_dev, int64_t k_row_stride,
                            const void* v_new_dev, int64_t v_row_stride, const int32_t* page_table_dev,
                            int32_t page_table_stride, const int32_t* seq_lens_dev,
                            const int32_t* query_start_loc_dev, int32_t num_seqs, int32_t num_tokens,
                            void* k_cache_dev, void* v_cache_dev, int32_t num_pages, void* stream);

/* ------------------------------------------------------------------------ */
/* Paged attention: decode and chunked prefill through one kernel.           */
/*                                                                           */
/* For query row at position p, head h, KV head g = h / G, keys j in         */
/* [lo, p] (lo = max(0, p-w+1) if w > 0 else 0):                             */
/*   o = sum_j softmax_j(scale * <q, k_j>) v_j      (deep-dive blog, §6.2)   */
/* computed as fixed key splits [sS, (s+1)S), each a pass over 32-key tiles  */
/* in increasing order with an online softmax, and a merge of the splits in  */
/* increasing split order.  A tile in which a row has no visible key leaves  */
/* that row's state bit-for-bit unchanged (deep-dive blog, §6.2, value rules */
/* for fully masked tiles).  Output bf16 [num_tokens][H_q][D] contiguous,    */
/* round-to-nearest-even, with -0 written as +0.                             */
/*                                                                           */
/* q: bf16 [num_tokens][H_q][D], token rows q_row_stride elements apart      */
/* (>= H_q*D).  max_seq_len >= every seq_lens[s]; it sizes the grid and the  */
/* workspace only.                                                           */
/*                                                                           */
/* Workspace (caller-owned device memory, contents scratch between calls):   */
/*   NS = ceil(max_seq_len / S); R = num_tokens * H_q                        */
/*   ml  : float2 [R][NS]     (m, l) of each split, m in base-2 units:       */
/*         m = max_j y_j, l = sum_j 2^(y_j - m), y_j = scale*log2(e)*<q,k_j> */
/*   acc : bf16   [R][NS][D]  sum_j 2^(y_j - m) v_j rounded to nearest even  */
/*         (the merge reads each split's accumulator in this precision), at  */
/*         the first 256-byte boundary after ml                              */
/*   plan: int32  [num_seqs+1] the launch's own schedule (the split phase:  */
/*         first work item of each sequence; the row-group mapping: the     */
/*         sequences by visible keys and a claim counter), at the first     */
/*         256-byte boundary after acc                                       */
/* Only the splits that meet [lo, p] of a row are written and read.          */
/* BI_ERR_OUT_OF_RANGE when 16 * H_q * NS * D * 4 >= 2^31 (the partials of    */
/* one 16-column block are addressed with 32-bit offsets).                   */
/* ------------------------------------------------------------------------ */
bi_status bi_paged_attention_workspace_size(const bi_attn_config* cfg, int32_t num_seqs, int32_t num_tokens,
                                            int32_t max_seq_len, size_t* bytes);

bi_status bi_paged_attention(const bi_attn_config* cfg,
                             const void* q_dev, int64_t q_row_stride,
                             const void* k_cache_dev, const void* v_cache_dev, int32_t num_pages,
                             const int32_t* page_table_dev, int32_t page_table_stride,
                             const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev,
                             int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                             void* workspace_dev, size_t workspace_bytes,
                             void* out_dev, void* stream);

/* bi_paged_attention without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  The split partials and the work plan live in a
 * device array inside the library, 64 MiB on each GPU the library runs on,
 * held until the process ends; a call whose workspace would exceed it
 * (bi_paged_attention_workspace_size > 64 MiB) returns
 * BI_ERR_WORKSPACE_TOO_SMALL and launches nothing.  Nothing here allocates:
 * the array's device address is looked up once per device, on the first call
 * made with that device current.  Every call on one GPU shares that GPU's
 * array, and the array keeps the last call's contents (each call writes every
 * partial it reads, so no clearing is needed): calls that overlap on one GPU
 * (concurrent streams, or host threads sharing the device) race and must be
 * serialised by the caller.  Arguments, results and errors are otherwise
 * those of bi_paged_attention; the output is bitwise that of
 * bi_paged_attention for the same arguments. */
bi_status bi_paged_attention_noalloc(const bi_attn_config* cfg,
                                     const void* q_dev, int64_t q_row_stride,
                                     const void* k_cache_dev, const void* v_cache_dev, int32_t num_pages,
                                     const int32_t* page_table_dev, int32_t page_table_stride,
                                     const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev,
                                     int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                                     void* out_dev, void* stream);

/* Work mapping of the split phase (diagnostic).  A work item is one
 * (sequence, group of query-row blocks, KV head, split); *blocks receives the
 * number of 16-column query-row blocks per item the split phase would use for
 * a batch of this shape: 1 for decode-shaped batches, 4 or 8 for
 * prefill-shaped ones at head_dim <= 128, so that one loaded K/V tile serves
 * four or eight blocks.  Every mapping performs the same arithmetic for every
 * row (each block runs the same per-tile computation on its own state; tiles
 * outside a row's key range leave it unchanged), so the value affects speed
 * only.  Needs a current device (BI_ERR_HIP without one). */
bi_status bi_paged_attention_item_blocks(const bi_attn_config* cfg, int32_t num_seqs, int32_t num_tokens,
                                         int32_t max_seq_len, int32_t* blocks);

/* Work mapping of bi_paged_attention (diagnostic): *mapping = 1 when a batch of
 * this shape runs the row-group mapping — a decode batch (num_tokens ==
 * num_seqs, so every q_len is 1) of at most 2048 sequences with at least two
 * (sequence, KV head) row groups per compute unit, where a row meets few
 * enough splits (all ceil(max_seq_len / S), or with a window those of w keys)
 * that a row group's partials fit the kernel's LDS ring (up to 116 splits for
 * head_dim 128 with 4 query heads per KV head, 118 for head_dim 256 with 2).
 * There each workgroup computes the splits of whole row groups, keeps their
 * partials in LDS and merges them itself (Vosti deep-dive blog, §8.1: two
 * work mappings with the same accumulation order), writing no partials to the
 * workspace; otherwise (*mapping = 0) the split and merge phases below run.
 * Both mappings give every row the same bits.  Needs a current device. */
bi_status bi_paged_attention_mapping(const bi_attn_config* cfg, int32_t num_seqs, int32_t num_tokens,
                                    int32_t max_seq_len, int32_t* mapping);

/* Force the work mapping of the attention calls made afterwards on the calling
 * thread (diagnostic; Vosti deep-dive blog, §8.1: work mappings with the same
 * accumulation order must agree bit for bit, and forcing lets one batch run
 * through each).  mapping: 0 = chosen per call (the default); otherwise the
 * split phase takes items of that many query-row blocks: 1 = one-block items,
 * one wave each; 4 = wide items; 8 = shared-tile items.  While a
 * mapping is forced, bi_paged_attention and its no-allocation form never take
 * the row-group mapping, and the split phase of every call (the split-K
 * comparator's too) uses the forced one; 4 and 8 exist only for head_dim <=
 * 128 (calls at 256 then fail with BI_ERR_UNSUPPORTED_CONFIG).  No forced
 * mapping changes any result bit.  BI_ERR_INVALID_ARG for other values. */
bi_status bi_paged_attention_force_mapping(int32_t mapping);

/* The two phases of bi_paged_attention, separately: the split phase writes the
 * workspace partials described above; the merge phase reads them and writes
 * the output.  bi_paged_attention == split then merge on the same stream. */
bi_status bi_paged_attention_split(const bi_attn_config* cfg,
                                   const void* q_dev, int64_t q_row_stride,
                                   const void* k_cache_dev, const void* v_cache_dev, int32_t num_pages,
                                   const int32_t* page_table_dev, int32_t page_table_stride,
                                   const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev,
                                   int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                                   void* workspace_dev, size_t workspace_bytes, void* stream);

bi_status bi_paged_attention_merge(const bi_attn_config* cfg,
                                   const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev,
                                   int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                                   const void* workspace_dev, size_t workspace_bytes,
                                   void* out_dev, void* stream);

/* ------------------------------------------------------------------------ */
/* RMSNorm, one row at a time (record "Deterministic and bit-exact           */
/* inference", field technical, Invariance).                                 */
/*   y[m,:] = x[m,:] * (sum_k x[m,k]^2 / H + eps)^(-1/2) * gamma             */
/* fp32 sum of squares in a reduction tree fixed by H alone, fp32 scaling,   */
/* one bf16 rounding.  x, y bf16 with row strides ld_x, ld_y (elements);     */
/* gamma bf16 [H].  H must be a positive multiple of 8; in-place (x == y,    */
/* same stride) is allowed.                                                  */
/* ------------------------------------------------------------------------ */
bi_status bi_rmsnorm(const void* x_dev, int64_t ld_x, const void* gamma_dev, float eps,
                     int64_t M, int64_t H, void* y_dev, int64_t ld_y, void* stream);

/* ------------------------------------------------------------------------ */
/* Matrix product with a K path fixed independently of M (Vosti deep-dive    */
/* blog, §6.1, matmul contract and its obligations: zero-initialised         */
/* accumulator, same-order iteration and reduction over a shared K).         */
/*   c[m,n] = sum_k a[m,k] * w[n,k]                                          */
/* a bf16 [M][K] (row stride lda), w bf16 [N][K] (row stride ldw), c [M][N]  */
/* (row stride ldc) in bf16 or fp32.  bf16 MFMA, fp32 accumulation in one    */
/* accumulator per output element, K visited in increasing 32-wide steps, no */
/* split of K.  K must be a multiple of 32; lda, ldw multiples of 8 and     */
/* below 2^23 (BI_ERR_OUT_OF_RANGE otherwise).  The result does not depend   */
/* on M, on the row's position, or on the tile configuration chosen.         */
/* ------------------------------------------------------------------------ */
bi_status bi_gemm(const void* a_dev, int64_t lda, const void* w_dev, int64_t ldw,
                  void* c_dev, int64_t ldc, bi_dtype c_dtype,
                  int64_t M, int64_t N, int64_t K, void* stream);

/* ------------------------------------------------------------------------ */
/* Decoder-step glue.  The pages define the step only as the cold causal     */
/* forward Forward(W, h) (Vosti deep-dive blog, §2, Theorem 4.1); the layer  */
/* details are the plainest Gemma-3-style choices.  Each output element      */
/* depends on its own row (token) only, and on the row's logical position    */
/* for RoPE, so all of these are batch-invariant by construction.            */
/* ------------------------------------------------------------------------ */

/* out[t, :] = table[ids[t], :] (bf16 copy; rows with an id outside
 * [0, vocab) are zero).  table [vocab][hidden], hidden a multiple of 8;
 * out rows ld_out elements apart. */
bi_status bi_embedding(const void* table_dev, int64_t vocab, int64_t hidden, const int32_t* ids_dev,
                       int32_t num_tokens, void* out_dev, int64_t ld_out, void* stream);

/* In place on the q and k parts of fused QKV rows (token t's row starts at
 * qkv + t*row_stride: H_q heads of q, then H_kv heads of k, each head_dim
 * long).  Each head row x is normalised, y = x / sqrt(mean(x^2) + eps) *
 * gamma (gamma_q for q heads, gamma_k for k heads, bf16 [head_dim]), then
 * rotated in half-split pairs (i, i + D/2) by the angle p * theta^(-2i/D),
 * p = seq_lens[s] - q_len_s + j the row's logical position.  fp32
 * arithmetic, angle and sin/cos in fp64, one bf16 rounding.
 * head_dim in {64, 128, 256}. */
bi_status bi_qk_norm_rope(void* qkv_dev, int64_t row_stride, int32_t num_tokens, const int32_t* seq_lens_dev,
                          const int32_t* query_start_loc_dev, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, const void* gamma_q_dev,
                          const void* gamma_k_dev, float eps, double rope_theta, void* stream);

/* bi_qk_norm_rope on the q and k parts of fused QKV rows [q | k | v] (head
 * geometry from cfg; row_stride >= (H_q + 2 H_kv) D) fused with the cache
 * write of bi_kv_write: each token's rotated k heads and its v heads are
 * stored at slot_mapping[t] in the paged caches (negative slots and pages
 * past the pool skipped).  The qkv rows and the caches end bitwise as after
 * bi_qk_norm_rope followed by bi_kv_write of qkv's k and v parts. */
bi_status bi_qk_norm_rope_kv_write(const bi_attn_config* cfg, void* qkv_dev, int64_t row_stride, int32_t num_tokens,
                                   const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev, int32_t num_seqs,
                                   const void* gamma_q_dev, const void* gamma_k_dev, float eps, double rope_theta,
                                   const int32_t* slot_mapping_dev, void* k_cache_dev, void* v_cache_dev,
                                   int32_t num_pages, void* stream);

/* Residual add fused with the RMSNorm that follows it in a pre-norm block:
 * s = a + b (as bi_add) and y = rmsnorm(s, gamma, eps) (as bi_rmsnorm on s),
 * in one launch; s and y are bitwise those of the two calls.  All bf16,
 * rows of H (a positive multiple of 8) with row strides lda, ldb, ld_s, ld_y
 * (multiples of 8); pointers 16-byte aligned.  s may alias a or b; y must not
 * overlap a, b or s. */
bi_status bi_add_rmsnorm(const void* a_dev, int64_t lda, const void* b_dev, int64_t ldb, void* s_dev, int64_t ld_s,
                         const void* gamma_dev, float eps, int64_t M, int64_t H, void* y_dev, int64_t ld_y,
                         void* stream);

/* c = a + b elementwise (fp32 add, one bf16 rounding); rows x n with row
 * strides lda, ldb, ldc.  c may alias a or b. */
bi_status bi_add(const void* a_dev, int64_t lda, const void* b_dev, int64_t ldb, void* c_dev, int64_t ldc,
                 int64_t rows, int64_t n, void* stream);

/* out[r, i] = gelu(in[r, i]) * in[r, ffn + i] for i < ffn, with the tanh
 * form gelu(x) = 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), fp32, one
 * bf16 rounding. */
bi_status bi_gated_gelu(const void* in_dev, int64_t ld_in, void* out_dev, int64_t ld_out, int64_t rows,
                        int64_t ffn, void* stream);

/* bi_gemm (bf16 output) of a [gate | up] weight followed by bi_gated_gelu, in
 * one launch, for M <= 16 rows of a: out[m, i] = gelu(g) * u with g, u the
 * bf16 products of row m of a with rows i and ffn + i of w (w bf16 [2 ffn][K],
 * row stride ldw; out bf16 [M][ffn], row stride ldo >= ffn).  Every output
 * bit equals that of the two calls (each product runs bi_gemm's own K path
 * and is rounded to bf16 before the activation).  The shape rules of bi_gemm
 * apply, and (ffn + 16) * ldw * 2 < 2^32 (BI_ERR_OUT_OF_RANGE otherwise);
 * BI_ERR_UNSUPPORTED_CONFIG for M > 16. */
bi_status bi_gemm_gated_gelu(const void* a_dev, int64_t lda, const void* w_dev, int64_t ldw, void* out_dev,
                             int64_t ldo, int64_t M, int64_t ffn, int64_t K, void* stream);

/* ------------------------------------------------------------------------ */
/* Host-side plan checks (host arrays; nothing is launched).                 */
/* ------------------------------------------------------------------------ */

/* Every entry a sequence uses (indices < ceil(seq_lens[s]/P)) lies in
 * [0, num_pages) and fits in the row (ceil(k_len/P) <= stride); also
 * 1 <= q_len <= k_len when query_start_loc_host is non-NULL.
 * BI_ERR_OUT_OF_RANGE otherwise (deep-dive blog, §3.2 invariant 1). */
bi_status bi_check_page_table(const int32_t* page_table_host, int32_t page_table_stride,
                              const int32_t* seq_lens_host, const int32_t* query_start_loc_host,
                              int32_t num_seqs, int32_t page_size, int32_t num_pages);

/* Slots in range and distinct, and none inside a page whose
 * page_writable_host[page] is 0 (a shared prefix page is immutable; writable
 * suffix slots are private; one plan's slots are disjoint: deep-dive blog,
 * §3.2 invariant 3).  Negative slots are ignored.  BI_ERR_OUT_OF_RANGE or
 * BI_ERR_WRITE_CONFLICT otherwise. */
bi_status bi_check_write_plan(const int32_t* slot_mapping_host, int32_t num_tokens,
                              const uint8_t* page_writable_host, int32_t num_pages,
                              int32_t page_size);

/* ------------------------------------------------------------------------ */
/* Greedy sampling: out[t] = the smallest index i with x[t, i] maximal over  */
/* the row (NaN entries never win; a row of NaN gives 0).  x fp32 [rows][n]  */
/* with row stride ld; out int32 [rows].  Deterministic for any row count.   */
/* x_dev must be 4-byte aligned; rows and n below 2^31 (BI_ERR_OUT_OF_RANGE  */
/* otherwise).  One 1024-thread workgroup per row.                           */
/* ------------------------------------------------------------------------ */
bi_status bi_argmax(const float* x_dev, int64_t ld, int64_t rows, int64_t n, int32_t* out_dev, void* stream);

/* ------------------------------------------------------------------------ */
/* Prefix cache of KV pages (host side; Vosti deep-dive blog, §3.2           */
/* engineering constraints "exact prefix matching" and "separate cache reuse */
/* from generation", §5.4).  Tracks which physical page holds the KV of      */
/* which token prefix.  A rolling hash over the prefix only nominates        */
/* candidates; a page is reused only if its tokens, its depth and its parent */
/* page match exactly.  Registered pages are immutable and shared; new KV    */
/* goes to private pages, registered once the step that fills them is done.  */
/* Under memory pressure only unreferenced leaves are evicted (least         */
/* recently used first), so a parent cannot be recycled while a retained    */
/* child names it.  All arrays are host arrays.  Not thread-safe.            */
/* ------------------------------------------------------------------------ */
typedef struct bi_prefix_cache bi_prefix_cache; /* opaque */

/* hash_bits in [0, 64]: bits of the rolling hash kept (fewer force
 * collisions, for testing; 64 in normal use). */
bi_status bi_prefix_cache_create(int32_t num_pages, int32_t page_size, int32_t hash_bits, bi_prefix_cache** out);
void      bi_prefix_cache_destroy(bi_prefix_cache* cache);

/* Longest run of cached pages holding tokens[0 : page_size*k) exactly, k <=
 * max_pages; pages_out[0..k) receive them, each acquired (one reference).
 * A caller that must still compute the last prompt position passes
 * max_pages = (num_tokens - 1) / page_size. */
bi_status bi_prefix_cache_match(bi_prefix_cache* cache, const int32_t* tokens, int64_t num_tokens,
                                int32_t* pages_out, int32_t max_pages, int32_t* num_matched);

/* n private pages (one reference each, writable), from free pages first,
 * then by evicting unreferenced leaves.  All or nothing: BI_ERR_OUT_OF_RANGE
 * and no change if n pages cannot be provided. */
bi_status bi_prefix_cache_alloc(bi_prefix_cache* cache, int32_t n, int32_t* pages_out);

/* Registers private page `page` (held by exactly one reference) as the
 * cached page of tokens[0 : page_size) at `depth` below `parent` (-1 at
 * depth 0; a parent must be registered, at depth - 1).  Call only after the
 * writes that fill the page have completed.  If an identical entry already
 * exists, *existing receives its page id and `page` stays private
 * (*existing = -1 otherwise).  BI_ERR_WRITE_CONFLICT if `page` is shared or
 * already registered, BI_ERR_INVALID_ARG on a bad parent or depth. */
bi_status bi_prefix_cache_register(bi_prefix_cache* cache, int32_t page, int32_t parent, int32_t depth,
                                   const int32_t* tokens, int32_t* existing);

/* Drops one reference from each listed page (negative ids are skipped).
 * BI_ERR_INVALID_ARG, with no change, if a page would drop below zero. */
bi_status bi_prefix_cache_release(bi_prefix_cache* cache, const int32_t* pages, int32_t n);

/* mask_out[p] = 1 iff page p may be written (private and unregistered):
 * the page_writable argument of bi_check_write_plan. */
bi_status bi_prefix_cache_writable(const bi_prefix_cache* cache, uint8_t* mask_out, int32_t num_pages);

/* stats_out[0..4) = free pages, registered pages, evictable pages, evictions. */
bi_status bi_prefix_cache_stats(const bi_prefix_cache* cache, int64_t* stats_out);

/* ------------------------------------------------------------------------ */
/* Non-invariant comparators, for measurement only (never used by the        */
/* invariant path).  The pages name split-K, whose reduction tree follows    */
/* the shape, as what batch invariance gives up (LLM-42 summary, §1-§2).     */
/* ------------------------------------------------------------------------ */

/* Split count a batch-aware split-KV kernel would pick: enough work items to
 * give every compute unit `waves_per_cu` of them.  The split length that
 * follows, ceil(max_seq_len / num_splits) rounded up to the key tile, changes
 * with the batch, and so does each row's reduction order. */
bi_status bi_splitk_attention_heuristic(const bi_attn_config* cfg, int32_t num_seqs,
                                        int32_t max_seq_len, int32_t num_compute_units,
                                        int32_t waves_per_cu, int32_t* num_splits_out);

bi_status bi_paged_attention_splitk_workspace_size(const bi_attn_config* cfg, int32_t num_seqs,
                                                   int32_t num_tokens, int32_t max_seq_len,
                                                   int32_t num_splits, size_t* bytes);

/* Same kernels as bi_paged_attention, with the split length derived from
 * num_splits and max_seq_len instead of the configuration's fixed size. */
bi_status bi_paged_attention_splitk(const bi_attn_config* cfg,
                                    const void* q_dev, int64_t q_row_stride,
                                    const void* k_cache_dev, const void* v_cache_dev, int32_t num_pages,
                                    const int32_t* page_table_dev, int32_t page_table_stride,
                                    const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev,
                                    int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                                    int32_t num_splits,
                                    void* workspace_dev, size_t workspace_bytes,
                                    void* out_dev, void* stream);

/* k-splits a shape-aware GEMM would pick from M: 8 for M <= 16, 4 for
 * M <= 128, else 1. */
int32_t bi_gemm_splitk_heuristic(int64_t M);
/* fp32 partial buffer [k_splits][M][N]. */
bi_status bi_gemm_splitk_workspace_size(int64_t M, int64_t N, int32_t k_splits, size_t* bytes);
/* K cut into k_splits equal 32-aligned ranges, each reduced separately, then
 * summed in split order into c.  (K / 32) must be divisible by k_splits. */
bi_status bi_gemm_splitk(const void* a_dev, int64_t lda, const void* w_dev, int64_t ldw,
                         void* c_dev, int64_t ldc, bi_dtype c_dtype,
                         int64_t M, int64_t N, int64_t K, int32_t k_splits,
                         void* workspace_dev, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Streaming-read reference, for measurement only: the bandwidth a plain     */
/* read of one contiguous buffer reaches on this GPU, quoted beside the      */
/* published HBM peak for the bandwidth-bound split phase (the pages report  */
/* decode as memory-bound; BASELINE's metric is HBM GB/s against peak).      */
/* ------------------------------------------------------------------------ */

/* Number of uint32 words bi_bench_stream_read writes to its sink. */
int32_t bi_bench_stream_read_sink_words(void);
/* Reads every byte of src_dev[0 .. bytes) once (non-temporal 16-byte loads)
 * and writes to sink_dev[g], g < bi_bench_stream_read_sink_words(), the xor
 * of the 32-bit words workgroup g read, so the xor of all sink words is the
 * xor of every 32-bit word of the buffer.  src_dev: device memory, 16-byte
 * aligned, bytes a multiple of 16 (BI_ERR_INVALID_ARG otherwise; bytes == 0
 * still writes the sink, all zeros).  Caller owns both buffers. */
bi_status bi_bench_stream_read(const void* src_dev, size_t bytes, uint32_t* sink_dev, void* stream);

/* MFMA throughput reference, for measurement only: the bf16 rate the       */
/* matrix cores sustain on this GPU with the GEMM's own instruction          */
/* (v_mfma_f32_16x16x32_bf16), quoted beside the published dense peak.       */
/* Launches a fixed grid whose every wave runs `rounds` rounds of eight      */
/* independent MFMAs on fragments filled with bf16(value) and writes, per    */
/* wave, the sum of element 0 of its eight accumulators to sink_dev (float,  */
/* bi_bench_mfma_peak_sink_words() entries; with value 1 and rounds r each   */
/* entry is 8 * 32 * r when that is exact in fp32).  rounds: a positive      */
/* multiple of 4 (BI_ERR_INVALID_ARG otherwise).  *flops receives the        */
/* launch's floating-point operation count (2 per multiply-add).            */
int32_t bi_bench_mfma_peak_sink_words(void);
bi_status bi_bench_mfma_peak(float value, int32_t rounds, float* sink_dev, int64_t* flops, void* stream);

/* ------------------------------------------------------------------------ */
/* Diagnostics.                                                              */
/* ------------------------------------------------------------------------ */
const char* bi_status_string(bi_status status);
/* Message of the last failed call on this thread ("" if none). */
const char* bi_last_error_message(void);
/* Library ABI version (major*10000 + minor*100 + patch). */
int32_t bi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BI_H_ */
