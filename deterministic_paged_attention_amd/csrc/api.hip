// C-ABI layer of libbi.so: argument validation, configuration objects,
// workspace sizing and launches.  Every check here looks at scalar arguments
// and pointer values only; nothing reads device memory and nothing
// synchronises, so a rejected call has launched nothing.

#include "../../include/bi.h"
#include "bi_internal.h"
#include "prefix_cache.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

struct bi_attn_config {
  bi_attn_desc desc;     // resolved (scale filled in)
  int log2_group;
  float qk_scale_log2;   // scale * log2(e), rounded once to fp32
};

namespace {

thread_local std::string g_last_error;
// Split-phase mapping forced by bi_paged_attention_force_mapping (0: chosen
// per launch).
thread_local int32_t g_force_kind = 0;

bi_status fail(bi_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bi_status fail(bi_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bi_status ok() {
  g_last_error.clear();
  return BI_OK;
}

bi_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int ilog2_exact(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return (1 << l) == v ? l : -1;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct WsLayout {
  size_t ml_bytes = 0, acc_offset = 0, plan_offset = 0, total = 0;
};

// ml float2 [R][ns] | pad to 256 | acc bf16 [R][ns][D] | pad to 256 | plan int32 [num_seqs + 1]
WsLayout ws_layout(int head_dim, int64_t rows, int64_t ns, int64_t num_seqs) {
  WsLayout w;
  w.ml_bytes = (size_t)rows * (size_t)ns * sizeof(float) * 2;
  w.acc_offset = round_up(w.ml_bytes, kAlign);
  w.plan_offset = round_up(w.acc_offset + (size_t)rows * (size_t)ns * (size_t)head_dim * sizeof(uint16_t), kAlign);
  w.total = w.plan_offset + (size_t)(num_seqs + 1) * sizeof(int32_t);
  return w;
}

bi_status check_cfg(const bi_attn_config* cfg) {
  if (!cfg) return fail(BI_ERR_INVALID_ARG, "config is NULL");
  return BI_OK;
}

struct AttnCall {
  const void* q;
  int64_t q_row_stride;
  const void* k_cache;
  const void* v_cache;
  int32_t num_pages;
  const int32_t* page_table;
  int32_t pt_stride;
  const int32_t* seq_lens;
  const int32_t* qsl;
  int32_t num_seqs;
  int32_t num_tokens;
  int32_t max_seq_len;
};

bi_status check_attn_call(const bi_attn_config* cfg, const AttnCall& c) {
  if (bi_status st = check_cfg(cfg)) return st;
  const bi_attn_desc& d = cfg->desc;
  if (c.num_seqs < 1 || c.num_tokens < 0 || c.max_seq_len < 1)
    return fail(BI_ERR_INVALID_ARG, "num_seqs (%d) must be >= 1, num_tokens (%d) >= 0, max_seq_len (%d) >= 1",
                c.num_seqs, c.num_tokens, c.max_seq_len);
  if (c.num_tokens < c.num_seqs && c.num_tokens != 0)
    return fail(BI_ERR_INVALID_ARG, "num_tokens (%d) < num_seqs (%d): every sequence needs q_len >= 1",
                c.num_tokens, c.num_seqs);
  if (!c.q || !c.k_cache || !c.v_cache || !c.page_table || !c.seq_lens || !c.qsl)
    return fail(BI_ERR_INVALID_ARG, "null device pointer");
  if (c.q_row_stride < (int64_t)d.num_q_heads * d.head_dim || c.q_row_stride % 8 != 0)
    return fail(BI_ERR_INVALID_ARG, "q_row_stride %lld must be >= H_q*D = %d and a multiple of 8",
                (long long)c.q_row_stride, d.num_q_heads * d.head_dim);
  if (!aligned(c.q, 16) || !aligned(c.k_cache, 16) || !aligned(c.v_cache, 16))
    return fail(BI_ERR_INVALID_ARG, "q, k_cache and v_cache must be 16-byte aligned");
  if (c.num_pages < 1) return fail(BI_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (c.pt_stride < 1) return fail(BI_ERR_INVALID_ARG, "page_table_stride must be >= 1");
  if ((int64_t)c.pt_stride * d.page_size < c.max_seq_len)
    return fail(BI_ERR_OUT_OF_RANGE, "page table row (%d pages) cannot hold max_seq_len %d", c.pt_stride,
                c.max_seq_len);
  const int64_t tq = 16 >> cfg->log2_group;
  if ((int64_t)c.num_tokens / tq + c.num_seqs > 0x7fffffffLL)
    return fail(BI_ERR_OUT_OF_RANGE, "too many query blocks");
  if (d.num_kv_heads > 65535) return fail(BI_ERR_OUT_OF_RANGE, "too many KV heads");
  return BI_OK;
}

}  // namespace

extern "C" {

const char* bi_status_string(bi_status s) {
  switch (s) {
    case BI_OK: return "BI_OK";
    case BI_ERR_INVALID_ARG: return "BI_ERR_INVALID_ARG";
    case BI_ERR_UNSUPPORTED_CONFIG: return "BI_ERR_UNSUPPORTED_CONFIG";
    case BI_ERR_OUT_OF_RANGE: return "BI_ERR_OUT_OF_RANGE";
    case BI_ERR_WRITE_CONFLICT: return "BI_ERR_WRITE_CONFLICT";
    case BI_ERR_WORKSPACE_TOO_SMALL: return "BI_ERR_WORKSPACE_TOO_SMALL";
    case BI_ERR_HIP: return "BI_ERR_HIP";
  }
  return "BI_ERR_UNKNOWN";
}

const char* bi_last_error_message(void) { return g_last_error.c_str(); }

int32_t bi_version(void) { return 100; }

bi_status bi_attn_config_create(const bi_attn_desc* desc, bi_attn_config** out) {
  if (!desc || !out) return fail(BI_ERR_INVALID_ARG, "desc and out must be non-NULL");
  *out = nullptr;
  const bi_attn_desc& d = *desc;
  if (d.num_q_heads < 1 || d.num_kv_heads < 1 || d.head_dim < 1 || d.page_size < 1 || d.split_size < 1 ||
      d.window < 0 || !(d.scale >= 0.f) || std::isinf(d.scale))
    return fail(BI_ERR_INVALID_ARG, "descriptor has a non-positive size, a negative window or a bad scale");
  if (d.num_q_heads % d.num_kv_heads != 0)
    return fail(BI_ERR_INVALID_ARG, "num_q_heads %d is not a multiple of num_kv_heads %d", d.num_q_heads,
                d.num_kv_heads);
  const int G = d.num_q_heads / d.num_kv_heads;
  const int lg = ilog2_exact(G);
  if (lg < 0 || G > 16)
    return fail(BI_ERR_UNSUPPORTED_CONFIG, "GQA group %d: this build needs a power of two <= 16", G);
  if (d.head_dim != 64 && d.head_dim != 128 && d.head_dim != 256)
    return fail(BI_ERR_UNSUPPORTED_CONFIG, "head_dim %d: this build supports 64, 128, 256", d.head_dim);
  if (d.page_size != 16)
    return fail(BI_ERR_UNSUPPORTED_CONFIG, "page_size %d: this build supports 16", d.page_size);
  if (d.split_size % bi::kKeyTile != 0)
    return fail(BI_ERR_UNSUPPORTED_CONFIG, "split_size %d must be a multiple of the key tile %d", d.split_size,
                bi::kKeyTile);
  bi_attn_config* c = new (std::nothrow) bi_attn_config;
  if (!c) return fail(BI_ERR_INVALID_ARG, "out of host memory");
  c->desc = d;
  const double scale = d.scale == 0.f ? 1.0 / std::sqrt((double)d.head_dim) : (double)d.scale;
  c->desc.scale = (float)scale;
  c->log2_group = lg;
  c->qk_scale_log2 = (float)(scale * 1.4426950408889634);
  *out = c;
  return ok();
}

void bi_attn_config_destroy(bi_attn_config* cfg) { delete cfg; }

bi_status bi_attn_config_query(const bi_attn_config* cfg, bi_attn_desc* desc_out, int32_t* key_tile_out) {
  if (bi_status st = check_cfg(cfg)) return st;
  if (desc_out) *desc_out = cfg->desc;
  if (key_tile_out) *key_tile_out = bi::kKeyTile;
  return ok();
}

bi_status bi_kv_cache_bytes(const bi_attn_config* cfg, int64_t num_pages, size_t* bytes) {
  if (bi_status st = check_cfg(cfg)) return st;
  if (!bytes || num_pages < 0) return fail(BI_ERR_INVALID_ARG, "bytes NULL or num_pages < 0");
  *bytes = (size_t)num_pages * cfg->desc.num_kv_heads * cfg->desc.head_dim * cfg->desc.page_size * 2;
  return ok();
}

bi_status bi_slot_mapping(const int32_t* page_table_dev, int32_t page_table_stride, const int32_t* seq_lens_dev,
                          const int32_t* query_start_loc_dev, int32_t num_seqs, int32_t num_tokens,
                          int32_t page_size, int32_t num_pages, int32_t* slot_mapping_dev, void* stream) {
  if (num_seqs < 1 || num_tokens < 0 || page_table_stride < 1 || num_pages < 1)
    return fail(BI_ERR_INVALID_ARG, "num_seqs >= 1, num_tokens >= 0, stride >= 1, num_pages >= 1 required");
  if (page_size != 16) return fail(BI_ERR_UNSUPPORTED_CONFIG, "page_size %d: this build supports 16", page_size);
  if ((int64_t)num_pages * page_size > 0x7fffffffLL)
    return fail(BI_ERR_OUT_OF_RANGE, "num_pages * page_size overflows a 32-bit slot index");
  if (num_tokens == 0) return ok();
  if (!page_table_dev || !seq_lens_dev || !query_start_loc_dev || !slot_mapping_dev)
    return fail(BI_ERR_INVALID_ARG, "null device pointer");
  return hip_status(bi::launch_slot_mapping(page_table_dev, page_table_stride, seq_lens_dev, query_start_loc_dev,
                                            num_seqs, num_tokens, page_size, num_pages, slot_mapping_dev,
                                            (hipStream_t)stream),
                    "slot_mapping launch");
}

bi_status bi_kv_write(const bi_attn_config* cfg, const void* k_new_dev, int64_t k_row_stride, const void* v_new_dev,
                      int64_t v_row_stride, const int32_t* slot_mapping_dev, int32_t num_tokens, void* k_cache_dev,
                      void* v_cache_dev, int32_t num_pages, void* stream) {
  if (bi_status st = check_cfg(cfg)) return st;
  const bi_attn_desc& d = cfg->desc;
  if (num_tokens < 0 || num_pages < 1) return fail(BI_ERR_INVALID_ARG, "num_tokens >= 0 and num_pages >= 1 required");
  const int64_t row = (int64_t)d.num_kv_heads * d.head_dim;
  if (k_row_stride < row || v_row_stride < row || k_row_stride % 8 || v_row_stride % 8)
    return fail(BI_ERR_INVALID_ARG, "k/v row strides must be >= H_kv*D = %lld and multiples of 8", (long long)row);
  if (num_tokens == 0) return ok();
  if (!k_new_dev || !v_new_dev || !slot_mapping_dev || !k_cache_dev || !v_cache_dev)
    return fail(BI_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(k_new_dev, 16) || !aligned(v_new_dev, 16) || !aligned(k_cache_dev, 16) || !aligned(v_cache_dev, 16))
    return fail(BI_ERR_INVALID_ARG, "k_new, v_new and the caches must be 16-byte aligned");
  return hip_status(bi::launch_kv_write(d.head_dim, d.num_kv_heads, (const uint16_t*)k_new_dev, k_row_stride,
                                        (const uint16_t*)v_new_dev, v_row_stride, slot_mapping_dev, num_tokens,
                                        (uint16_t*)k_cache_dev, (uint16_t*)v_cache_dev, num_pages,
                                        (hipStream_t)stream),
                    "kv_write launch");
}

bi_status bi_kv_write_paged(const bi_attn_config* cfg, const void* k_new_dev, int64_t k_row_stride,
                            const void* v_new_dev, int64_t v_row_stride, const int32_t* page_table_dev,
                            int32_t page_table_stride, const int32_t* seq_lens_dev,
                            const int32_t* query_start_loc_dev, int32_t num_seqs, int32_t num_tokens,
                            void* k_cache_dev, void* v_cache_dev, int32_t num_pages, void* stream) {
  if (bi_status st = check_cfg(cfg)) return st;
  const bi_attn_desc& d = cfg->desc;
  if (num_seqs < 1 || num_tokens < 0 || page_table_stride < 1 || num_pages < 1)
    return fail(BI_ERR_INVALID_ARG, "num_seqs >= 1, num_tokens >= 0, stride >= 1, num_pages >= 1 required");
  if ((int64_t)num_pages * d.page_size > 0x7fffffffLL)
    return fail(BI_ERR_OUT_OF_RANGE, "num_pages * page_size overflows a 32-bit slot index");
  const int64_t row = (int64_t)d.num_kv_heads * d.head_dim;
  if (k_row_stride < row || v_row_stride < row || k_row_stride % 8 || v_row_stride % 8)
    return fail(BI_ERR_INVALID_ARG, "k/v row strides must be >= H_kv*D = %lld and multiples of 8", (long long)row);
  if (num_tokens == 0) return ok();
  if (!k_new_dev || !v_new_dev || !page_table_dev || !seq_lens_dev || !query_start_loc_dev || !k_cache_dev ||
      !v_cache_dev)
    return fail(BI_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(k_new_dev, 16) || !aligned(v_new_dev, 16) || !aligned(k_cache_dev, 16) || !aligned(v_cache_dev, 16))
    return fail(BI_ERR_INVALID_ARG, "k_new, v_new and the caches must be 16-byte aligned");
  return hip_status(bi::launch_kv_write_paged(d.head_dim, d.num_kv_heads, (const uint16_t*)k_new_dev, k_row_stride,
                                              (const uint16_t*)v_new_dev, v_row_stride, page_table_dev,
                                              page_table_stride, seq_lens_dev, query_start_loc_dev, num_seqs,
                                              num_tokens, (uint16_t*)k_cache_dev, (uint16_t*)v_cache_dev, num_pages,
                                              (hipStream_t)stream),
                    "kv_write_paged launch");
}

bi_status bi_paged_attention_workspace_size(const bi_attn_config* cfg, int32_t num_seqs, int32_t num_tokens,
                                            int32_t max_seq_len, size_t* bytes) {
  if (bi_status st = check_cfg(cfg)) return st;
  if (!bytes || num_seqs < 1 || num_tokens < 0 || max_seq_len < 1)
    return fail(BI_ERR_INVALID_ARG, "bytes NULL, num_seqs < 1, num_tokens < 0 or max_seq_len < 1");
  const int64_t ns = (max_seq_len + (int64_t)cfg->desc.split_size - 1) / cfg->desc.split_size;
  *bytes = ws_layout(cfg->desc.head_dim, (int64_t)num_tokens * cfg->desc.num_q_heads, ns, num_seqs).total;
  return ok();
}

bi_status bi_paged_attention_item_blocks(const bi_attn_config* cfg, int32_t num_seqs, int32_t num_tokens,
                                         int32_t max_seq_len, int32_t* blocks) {
  if (bi_status st = check_cfg(cfg)) return st;
  if (!blocks || num_seqs < 1 || num_tokens < 0 || max_seq_len < 1)
    return fail(BI_ERR_INVALID_ARG, "blocks NULL, num_seqs < 1, num_tokens < 0 or max_seq_len < 1");
  bi::AttnSplitArgs a{};
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = cfg->desc.num_q_heads;
  a.num_kv_heads = cfg->desc.num_kv_heads;
  a.log2_group = cfg->log2_group;
  a.split = cfg->desc.split_size;
  a.window = cfg->desc.window;
  a.ns = (int32_t)((max_seq_len + (int64_t)cfg->desc.split_size - 1) / cfg->desc.split_size);
  a.force_kind = g_force_kind;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(BI_ERR_HIP, "no usable device to size the launch");
  const int qb = bi::attn_item_blocks(cfg->desc.head_dim, a);
  if (qb <= 0)
    return fail(BI_ERR_UNSUPPORTED_CONFIG, "the forced mapping does not exist at head_dim %d", cfg->desc.head_dim);
  *blocks = qb;
  return ok();
}

bi_status bi_paged_attention_mapping(const bi_attn_config* cfg, int32_t num_seqs, int32_t num_tokens,
                                    int32_t max_seq_len, int32_t* mapping) {
  if (bi_status st = check_cfg(cfg)) return st;
  if (!mapping || num_seqs < 1 || num_tokens < 0 || max_seq_len < 1)
    return fail(BI_ERR_INVALID_ARG, "mapping NULL, num_seqs < 1, num_tokens < 0 or max_seq_len < 1");
  bi::AttnSplitArgs a{};
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = cfg->desc.num_q_heads;
  a.num_kv_heads = cfg->desc.num_kv_heads;
  a.log2_group = cfg->log2_group;
  a.split = cfg->desc.split_size;
  a.window = cfg->desc.window;
  a.ns = (int32_t)((max_seq_len + (int64_t)cfg->desc.split_size - 1) / cfg->desc.split_size);
  a.force_kind = g_force_kind;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(BI_ERR_HIP, "no usable device to size the launch");
  *mapping = g_force_kind == 0 && bi::attn_rowgroup_applies(cfg->desc.head_dim, a) ? 1 : 0;
  return ok();
}

bi_status bi_paged_attention_force_mapping(int32_t mapping) {
  if (mapping != 0 && mapping != 1 && mapping != 4 && mapping != 8)
    return fail(BI_ERR_INVALID_ARG, "mapping must be 0, 1, 4 or 8 (got %d)", mapping);
  g_force_kind = mapping;
  return ok();
}

bi_status bi_paged_attention_splitk_workspace_size(const bi_attn_config* cfg, int32_t num_seqs, int32_t num_tokens,
                                                   int32_t max_seq_len, int32_t num_splits, size_t* bytes) {
  if (bi_status st = check_cfg(cfg)) return st;
  if (!bytes || num_seqs < 1 || num_tokens < 0 || max_seq_len < 1 || num_splits < 1)
    return fail(BI_ERR_INVALID_ARG, "bytes NULL, num_seqs < 1, num_tokens < 0, max_seq_len < 1 or num_splits < 1");
  *bytes = ws_layout(cfg->desc.head_dim, (int64_t)num_tokens * cfg->desc.num_q_heads, num_splits, num_seqs).total;
  return ok();
}

}  // extern "C"

namespace {

// The split phase; with `fused` non-null (the invariant path of
// bi_paged_attention, output `out`), a decode batch that the row-group mapping
// covers runs split and merge in one launch instead, and *fused is set.
bi_status run_split(const bi_attn_config* cfg, const AttnCall& c, int32_t split, int32_t ns, void* ws, size_t ws_bytes,
                    hipStream_t stream, void* out = nullptr, bool* fused = nullptr) {
  if (fused) *fused = false;
  const WsLayout L = ws_layout(cfg->desc.head_dim, (int64_t)c.num_tokens * cfg->desc.num_q_heads, ns, c.num_seqs);
  if (!ws && L.total) return fail(BI_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < L.total)
    return fail(BI_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (!aligned(ws, 16)) return fail(BI_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (c.num_tokens == 0) return ok();
  // Work items are counted in 32-bit integers: bound their number.
  const int64_t tq = 16 >> cfg->log2_group;
  if (((int64_t)c.num_tokens / tq + c.num_seqs) * cfg->desc.num_kv_heads * ns > 0x7fffffffLL)
    return fail(BI_ERR_OUT_OF_RANGE, "too many work items");
  if ((int64_t)c.num_tokens * cfg->desc.num_q_heads * ns > 0x7fffffffffffLL)
    return fail(BI_ERR_OUT_OF_RANGE, "workspace index overflow");
  // The partials of one query-row block are written with 32-bit byte offsets
  // from the block's first partial: bound their span.
  if ((int64_t)16 * cfg->desc.num_q_heads * ns * cfg->desc.head_dim * 4 > 0x7fffffffLL)
    return fail(BI_ERR_OUT_OF_RANGE, "H_q * ceil(max_seq_len / split) * D too large");
  bi::AttnSplitArgs a;
  a.q = (const uint16_t*)c.q;
  a.q_stride = c.q_row_stride;
  a.k_cache = (const uint16_t*)c.k_cache;
  a.v_cache = (const uint16_t*)c.v_cache;
  a.page_table = c.page_table;
  a.pt_stride = c.pt_stride;
  a.num_pages = c.num_pages;
  a.seq_lens = c.seq_lens;
  a.qsl = c.qsl;
  a.num_seqs = c.num_seqs;
  a.num_tokens = c.num_tokens;
  a.num_q_heads = cfg->desc.num_q_heads;
  a.num_kv_heads = cfg->desc.num_kv_heads;
  a.log2_group = cfg->log2_group;
  a.split = split;
  a.window = cfg->desc.window;
  a.ns = ns;
  a.qk_scale_log2 = cfg->qk_scale_log2;
  a.ws_ml = (float2*)ws;
  a.ws_acc = (uint16_t*)((char*)ws + L.acc_offset);
  a.plan = (int32_t*)((char*)ws + L.plan_offset);
  a.out = (uint16_t*)out;
  a.rg_static_rounds = 0;
  a.force_kind = g_force_kind;
  if ((g_force_kind == 4 || g_force_kind == 8) && cfg->desc.head_dim > 128)
    return fail(BI_ERR_UNSUPPORTED_CONFIG, "the forced mapping %d does not exist at head_dim %d", g_force_kind,
                cfg->desc.head_dim);
  if (g_force_kind == 0 && fused && out && aligned(out, 8) && bi::attn_rowgroup_applies(cfg->desc.head_dim, a)) {
    *fused = true;
    return hip_status(bi::launch_attn_rowgroup(cfg->desc.head_dim, a, stream), "attention row-group launch");
  }
  return hip_status(bi::launch_attn_split(cfg->desc.head_dim, a, stream), "attention split launch");
}

bi_status run_merge(const bi_attn_config* cfg, const int32_t* seq_lens, const int32_t* qsl, int32_t num_seqs,
                    int32_t num_tokens, int32_t split, int32_t ns, const void* ws, size_t ws_bytes, void* out,
                    hipStream_t stream) {
  const WsLayout L = ws_layout(cfg->desc.head_dim, (int64_t)num_tokens * cfg->desc.num_q_heads, ns, num_seqs);
  if (!ws && L.total) return fail(BI_ERR_INVALID_ARG, "workspace is NULL");
  if (ws_bytes < L.total)
    return fail(BI_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", ws_bytes, L.total);
  if (num_tokens == 0) return ok();
  if (!out || !seq_lens || !qsl) return fail(BI_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(out, 8)) return fail(BI_ERR_INVALID_ARG, "out must be 8-byte aligned");
  bi::AttnMergeArgs a;
  a.seq_lens = seq_lens;
  a.qsl = qsl;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = cfg->desc.num_q_heads;
  a.split = split;
  a.window = cfg->desc.window;
  a.ns = ns;
  a.ws_ml = (const float2*)ws;
  a.ws_acc = (const uint16_t*)((const char*)ws + L.acc_offset);
  a.out = (uint16_t*)out;
  return hip_status(bi::launch_attn_merge(cfg->desc.head_dim, a, stream), "attention merge launch");
}

int32_t fixed_ns(const bi_attn_config* cfg, int32_t max_seq_len) {
  return (int32_t)((max_seq_len + (int64_t)cfg->desc.split_size - 1) / cfg->desc.split_size);
}

// Split length of the batch-aware comparator: ceil(max_seq_len / num_splits)
// rounded up to the key tile.
int32_t splitk_len(int32_t max_seq_len, int32_t num_splits) {
  int64_t len = (max_seq_len + (int64_t)num_splits - 1) / num_splits;
  len = (len + bi::kKeyTile - 1) / bi::kKeyTile * bi::kKeyTile;
  return (int32_t)len;
}

}  // namespace

extern "C" {

bi_status bi_paged_attention_split(const bi_attn_config* cfg, const void* q_dev, int64_t q_row_stride,
                                   const void* k_cache_dev, const void* v_cache_dev, int32_t num_pages,
                                   const int32_t* page_table_dev, int32_t page_table_stride,
                                   const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev,
                                   int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len, void* workspace_dev,
                                   size_t workspace_bytes, void* stream) {
  const AttnCall c{q_dev, q_row_stride, k_cache_dev, v_cache_dev, num_pages, page_table_dev, page_table_stride,
                   seq_lens_dev, query_start_loc_dev, num_seqs, num_tokens, max_seq_len};
  if (bi_status st = check_attn_call(cfg, c)) return st;
  return run_split(cfg, c, cfg->desc.split_size, fixed_ns(cfg, max_seq_len), workspace_dev, workspace_bytes,
                   (hipStream_t)stream);
}

bi_status bi_paged_attention_merge(const bi_attn_config* cfg, const int32_t* seq_lens_dev,
                                   const int32_t* query_start_loc_dev, int32_t num_seqs, int32_t num_tokens,
                                   int32_t max_seq_len, const void* workspace_dev, size_t workspace_bytes,
                                   void* out_dev, void* stream) {
  if (bi_status st = check_cfg(cfg)) return st;
  if (num_seqs < 1 || num_tokens < 0 || max_seq_len < 1)
    return fail(BI_ERR_INVALID_ARG, "num_seqs >= 1, num_tokens >= 0, max_seq_len >= 1 required");
  return run_merge(cfg, seq_lens_dev, query_start_loc_dev, num_seqs, num_tokens, cfg->desc.split_size,
                   fixed_ns(cfg, max_seq_len), workspace_dev, workspace_bytes, out_dev, (hipStream_t)stream);
}

bi_status bi_paged_attention(const bi_attn_config* cfg, const void* q_dev, int64_t q_row_stride,
                             const void* k_cache_dev, const void* v_cache_dev, int32_t num_pages,
                             const int32_t* page_table_dev, int32_t page_table_stride, const int32_t* seq_lens_dev,
                             const int32_t* query_start_loc_dev, int32_t num_seqs, int32_t num_tokens,
                             int32_t max_seq_len, void* workspace_dev, size_t workspace_bytes, void* out_dev,
                             void* stream) {
  const AttnCall c{q_dev, q_row_stride, k_cache_dev, v_cache_dev, num_pages, page_table_dev, page_table_stride,
                   seq_lens_dev, query_start_loc_dev, num_seqs, num_tokens, max_seq_len};
  if (bi_status st = check_attn_call(cfg, c)) return st;
  if (num_tokens > 0 && !out_dev) return fail(BI_ERR_INVALID_ARG, "out is NULL");
  const int32_t ns = fixed_ns(cfg, max_seq_len);
  bool fused = false;
  if (bi_status st = run_split(cfg, c, cfg->desc.split_size, ns, workspace_dev, workspace_bytes, (hipStream_t)stream,
                               out_dev, &fused))
    return st;
  if (fused) return ok();
  return run_merge(cfg, seq_lens_dev, query_start_loc_dev, num_seqs, num_tokens, cfg->desc.split_size, ns,
                   workspace_dev, workspace_bytes, out_dev, (hipStream_t)stream);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free paged attention: the partials live in a file-scope device
// array instead of a caller workspace.  Each GPU the library runs on holds its
// own copy of the array (kNoallocScratchBytes, until the process ends); the
// host name `scratch` is only a stand-in for it, so the device address is
// looked up once per device (with that device current) and only that address
// is ever handed to a kernel.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of this device's scratch array (nullptr with the HIP error on failure).
void* device_scratch(int dev, hipError_t* err) {
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

bi_status bi_paged_attention_noalloc(const bi_attn_config* cfg, const void* q_dev, int64_t q_row_stride,
                                     const void* k_cache_dev, const void* v_cache_dev, int32_t num_pages,
                                     const int32_t* page_table_dev, int32_t page_table_stride,
                                     const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev,
                                     int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len, void* out_dev,
                                     void* stream) {
  const AttnCall c{q_dev, q_row_stride, k_cache_dev, v_cache_dev, num_pages, page_table_dev, page_table_stride,
                   seq_lens_dev, query_start_loc_dev, num_seqs, num_tokens, max_seq_len};
  if (bi_status st = check_attn_call(cfg, c)) return st;
  if (num_tokens > 0 && !out_dev) return fail(BI_ERR_INVALID_ARG, "out is NULL");
  const int32_t ns = fixed_ns(cfg, max_seq_len);
  const size_t need =
      ws_layout(cfg->desc.head_dim, (int64_t)num_tokens * cfg->desc.num_q_heads, ns, num_seqs).total;
  if (need > kNoallocScratchBytes)
    return fail(BI_ERR_WORKSPACE_TOO_SMALL,
                "this call needs %zu bytes of partials; the allocation-free entry point holds at most %zu "
                "(use bi_paged_attention with a workspace)",
                need, kNoallocScratchBytes);
  if (num_tokens == 0) return ok();
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(BI_ERR_HIP, "no usable current device");
  hipError_t e = hipSuccess;
  void* ws = device_scratch(dev, &e);
  if (!ws) return hip_status(e == hipSuccess ? hipErrorInvalidSymbol : e, "scratch symbol lookup");
  bool fused = false;
  if (bi_status st =
          run_split(cfg, c, cfg->desc.split_size, ns, ws, kNoallocScratchBytes, (hipStream_t)stream, out_dev, &fused))
    return st;
  if (fused) return ok();
  return run_merge(cfg, seq_lens_dev, query_start_loc_dev, num_seqs, num_tokens, cfg->desc.split_size, ns, ws,
                   kNoallocScratchBytes, out_dev, (hipStream_t)stream);
}

bi_status bi_splitk_attention_heuristic(const bi_attn_config* cfg, int32_t num_seqs, int32_t max_seq_len,
                                        int32_t num_compute_units, int32_t waves_per_cu, int32_t* num_splits_out) {
  if (bi_status st = check_cfg(cfg)) return st;
  if (num_seqs < 1 || max_seq_len < 1 || num_compute_units < 1 || waves_per_cu < 1 || !num_splits_out)
    return fail(BI_ERR_INVALID_ARG, "bad heuristic arguments");
  const int64_t units = (int64_t)num_seqs * cfg->desc.num_kv_heads;
  const int64_t target = (int64_t)num_compute_units * waves_per_cu;
  int64_t n = (target + units - 1) / units;
  const int64_t nmax = (max_seq_len + bi::kKeyTile - 1) / bi::kKeyTile;
  if (n < 1) n = 1;
  if (n > nmax) n = nmax;
  *num_splits_out = (int32_t)n;
  return ok();
}

bi_status bi_paged_attention_splitk(const bi_attn_config* cfg, const void* q_dev, int64_t q_row_stride,
                                    const void* k_cache_dev, const void* v_cache_dev, int32_t num_pages,
                                    const int32_t* page_table_dev, int32_t page_table_stride,
                                    const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev,
                                    int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len, int32_t num_splits,
                                    void* workspace_dev, size_t workspace_bytes, void* out_dev, void* stream) {
  const AttnCall c{q_dev, q_row_stride, k_cache_dev, v_cache_dev, num_pages, page_table_dev, page_table_stride,
                   seq_lens_dev, query_start_loc_dev, num_seqs, num_tokens, max_seq_len};
  if (bi_status st = check_attn_call(cfg, c)) return st;
  if (num_splits < 1) return fail(BI_ERR_INVALID_ARG, "num_splits must be >= 1");
  if (num_tokens > 0 && !out_dev) return fail(BI_ERR_INVALID_ARG, "out is NULL");
  const int32_t len = splitk_len(max_seq_len, num_splits);
  const int32_t ns = (max_seq_len + len - 1) / len;
  if (bi_status st = run_split(cfg, c, len, ns, workspace_dev, workspace_bytes, (hipStream_t)stream)) return st;
  return run_merge(cfg, seq_lens_dev, query_start_loc_dev, num_seqs, num_tokens, len, ns, workspace_dev,
                   workspace_bytes, out_dev, (hipStream_t)stream);
}

bi_status bi_rmsnorm(const void* x_dev, int64_t ld_x, const void* gamma_dev, float eps, int64_t M, int64_t H,
                     void* y_dev, int64_t ld_y, void* stream) {
  if (M < 0 || H < 8 || H % 8 != 0)
    return fail(BI_ERR_INVALID_ARG, "M must be >= 0 and H a positive multiple of 8 (M=%lld H=%lld)", (long long)M,
                (long long)H);
  if (ld_x < H || ld_y < H || ld_x % 8 || ld_y % 8)
    return fail(BI_ERR_INVALID_ARG, "row strides must be >= H and multiples of 8");
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(BI_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (M > 0x7fffffffLL) return fail(BI_ERR_OUT_OF_RANGE, "M too large");
  if (M == 0) return ok();
  if (!x_dev || !gamma_dev || !y_dev) return fail(BI_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(x_dev, 16) || !aligned(gamma_dev, 16) || !aligned(y_dev, 16))
    return fail(BI_ERR_INVALID_ARG, "x, gamma and y must be 16-byte aligned");
  return hip_status(bi::launch_rmsnorm((const uint16_t*)x_dev, ld_x, (const uint16_t*)gamma_dev, eps, M, H,
                                       (uint16_t*)y_dev, ld_y, (hipStream_t)stream),
                    "rmsnorm launch");
}

namespace {
bi_status check_gemm(const void* a, int64_t lda, const void* w, int64_t ldw, const void* c, int64_t ldc, bi_dtype dt,
                     int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 32 || K % 32 != 0)
    return fail(BI_ERR_INVALID_ARG, "M, N >= 0 and K a positive multiple of 32 required (K=%lld)", (long long)K);
  if (dt != BI_BF16 && dt != BI_F32) return fail(BI_ERR_INVALID_ARG, "unknown output dtype");
  if (lda < K || ldw < K || ldc < N || lda % 8 || ldw % 8)
    return fail(BI_ERR_INVALID_ARG, "lda, ldw must be >= K and multiples of 8; ldc >= N");
  if ((M + 15) / 16 > 65535 || N > 0x7fffffffLL) return fail(BI_ERR_OUT_OF_RANGE, "M or N too large");
  // Each workgroup addresses at most 256 rows of a or w through 32-bit byte offsets.
  if (lda >= (1LL << 23) || ldw >= (1LL << 23)) return fail(BI_ERR_OUT_OF_RANGE, "lda, ldw must be below 2^23");
  if (M == 0 || N == 0) return BI_OK;
  if (!a || !w || !c) return fail(BI_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(a, 16) || !aligned(w, 16)) return fail(BI_ERR_INVALID_ARG, "a and w must be 16-byte aligned");
  return BI_OK;
}
}  // namespace

bi_status bi_gemm(const void* a_dev, int64_t lda, const void* w_dev, int64_t ldw, void* c_dev, int64_t ldc,
                  bi_dtype c_dtype, int64_t M, int64_t N, int64_t K, void* stream) {
  if (bi_status st = check_gemm(a_dev, lda, w_dev, ldw, c_dev, ldc, c_dtype, M, N, K)) return st;
  if (M == 0 || N == 0) return ok();
  return hip_status(bi::launch_gemm((const uint16_t*)a_dev, lda, (const uint16_t*)w_dev, ldw, c_dev, ldc,
                                    c_dtype == BI_F32 ? 1 : 0, M, N, K, (hipStream_t)stream),
                    "gemm launch");
}

bi_status bi_gemm_gated_gelu(const void* a_dev, int64_t lda, const void* w_dev, int64_t ldw, void* out_dev,
                             int64_t ldo, int64_t M, int64_t ffn, int64_t K, void* stream) {
  if (M > 16) return fail(BI_ERR_UNSUPPORTED_CONFIG, "bi_gemm_gated_gelu takes at most 16 rows (M=%lld)", (long long)M);
  if (ffn < 1 || ldo < ffn) return fail(BI_ERR_INVALID_ARG, "ffn >= 1 and ldo >= ffn required");
  if (bi_status st = check_gemm(a_dev, lda, w_dev, ldw, out_dev, 2 * ffn, BI_BF16, M, 2 * ffn, K)) return st;
  // The up rows are addressed ffn rows past the gate rows with 32-bit byte offsets.
  if ((ffn + 16) * ldw * 2 >= (1LL << 32)) return fail(BI_ERR_OUT_OF_RANGE, "ffn * ldw too large");
  if (M == 0) return ok();
  return hip_status(bi::launch_gemm_gated_gelu((const uint16_t*)a_dev, lda, (const uint16_t*)w_dev, ldw,
                                               (uint16_t*)out_dev, ldo, M, ffn, K, (hipStream_t)stream),
                    "gemm_gated_gelu launch");
}

bi_status bi_embedding(const void* table_dev, int64_t vocab, int64_t hidden, const int32_t* ids_dev,
                       int32_t num_tokens, void* out_dev, int64_t ld_out, void* stream) {
  if (vocab < 1 || hidden < 8 || hidden % 8 || num_tokens < 0 || ld_out < hidden || ld_out % 8)
    return fail(BI_ERR_INVALID_ARG, "vocab >= 1, hidden a positive multiple of 8, ld_out >= hidden (multiple of 8)");
  if (num_tokens == 0) return ok();
  if (!table_dev || !ids_dev || !out_dev) return fail(BI_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(table_dev, 16) || !aligned(out_dev, 16)) return fail(BI_ERR_INVALID_ARG, "table and out must be 16-byte aligned");
  return hip_status(bi::launch_embedding((const uint16_t*)table_dev, vocab, hidden, ids_dev, num_tokens,
                                         (uint16_t*)out_dev, ld_out, (hipStream_t)stream),
                    "embedding launch");
}

bi_status bi_qk_norm_rope(void* qkv_dev, int64_t row_stride, int32_t num_tokens, const int32_t* seq_lens_dev,
                          const int32_t* query_start_loc_dev, int32_t num_seqs, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, const void* gamma_q_dev, const void* gamma_k_dev,
                          float eps, double rope_theta, void* stream) {
  if (num_seqs < 1 || num_tokens < 0 || num_q_heads < 1 || num_kv_heads < 1)
    return fail(BI_ERR_INVALID_ARG, "num_seqs, num_q_heads, num_kv_heads >= 1 and num_tokens >= 0 required");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(BI_ERR_UNSUPPORTED_CONFIG, "head_dim %d: this build supports 64, 128, 256", head_dim);
  if (row_stride < (int64_t)(num_q_heads + num_kv_heads) * head_dim)
    return fail(BI_ERR_INVALID_ARG, "row_stride smaller than the q and k parts of a row");
  if (!(eps >= 0.f) || std::isinf(eps) || !(rope_theta > 1.0) || std::isinf(rope_theta))
    return fail(BI_ERR_INVALID_ARG, "eps must be finite and >= 0, rope_theta finite and > 1");
  if (num_tokens == 0) return ok();
  if (!qkv_dev || !seq_lens_dev || !query_start_loc_dev || !gamma_q_dev || !gamma_k_dev)
    return fail(BI_ERR_INVALID_ARG, "null device pointer");
  return hip_status(bi::launch_qk_norm_rope((uint16_t*)qkv_dev, row_stride, num_tokens, seq_lens_dev,
                                            query_start_loc_dev, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                            (const uint16_t*)gamma_q_dev, (const uint16_t*)gamma_k_dev, eps,
                                            rope_theta, nullptr, nullptr, nullptr, 0, (hipStream_t)stream),
                    "qk_norm_rope launch");
}

bi_status bi_qk_norm_rope_kv_write(const bi_attn_config* cfg, void* qkv_dev, int64_t row_stride, int32_t num_tokens,
                                   const int32_t* seq_lens_dev, const int32_t* query_start_loc_dev, int32_t num_seqs,
                                   const void* gamma_q_dev, const void* gamma_k_dev, float eps, double rope_theta,
                                   const int32_t* slot_mapping_dev, void* k_cache_dev, void* v_cache_dev,
                                   int32_t num_pages, void* stream) {
  if (bi_status st = check_cfg(cfg)) return st;
  const bi_attn_desc& d = cfg->desc;
  if (num_seqs < 1 || num_tokens < 0 || num_pages < 1)
    return fail(BI_ERR_INVALID_ARG, "num_seqs >= 1, num_tokens >= 0 and num_pages >= 1 required");
  if (row_stride < (int64_t)(d.num_q_heads + 2 * d.num_kv_heads) * d.head_dim)
    return fail(BI_ERR_INVALID_ARG, "row_stride smaller than the q, k and v parts of a row");
  if (!(eps >= 0.f) || std::isinf(eps) || !(rope_theta > 1.0) || std::isinf(rope_theta))
    return fail(BI_ERR_INVALID_ARG, "eps must be finite and >= 0, rope_theta finite and > 1");
  if (num_tokens == 0) return ok();
  if (!qkv_dev || !seq_lens_dev || !query_start_loc_dev || !gamma_q_dev || !gamma_k_dev || !slot_mapping_dev ||
      !k_cache_dev || !v_cache_dev)
    return fail(BI_ERR_INVALID_ARG, "null device pointer");
  return hip_status(bi::launch_qk_norm_rope((uint16_t*)qkv_dev, row_stride, num_tokens, seq_lens_dev,
                                            query_start_loc_dev, num_seqs, d.num_q_heads, d.num_kv_heads, d.head_dim,
                                            (const uint16_t*)gamma_q_dev, (const uint16_t*)gamma_k_dev, eps,
                                            rope_theta, slot_mapping_dev, (uint16_t*)k_cache_dev,
                                            (uint16_t*)v_cache_dev, num_pages, (hipStream_t)stream),
                    "qk_norm_rope_kv_write launch");
}

bi_status bi_add_rmsnorm(const void* a_dev, int64_t lda, const void* b_dev, int64_t ldb, void* s_dev, int64_t ld_s,
                         const void* gamma_dev, float eps, int64_t M, int64_t H, void* y_dev, int64_t ld_y,
                         void* stream) {
  if (M < 0 || H < 8 || H % 8 != 0)
    return fail(BI_ERR_INVALID_ARG, "M must be >= 0 and H a positive multiple of 8 (M=%lld H=%lld)", (long long)M,
                (long long)H);
  if (lda < H || ldb < H || ld_s < H || ld_y < H || lda % 8 || ldb % 8 || ld_s % 8 || ld_y % 8)
    return fail(BI_ERR_INVALID_ARG, "row strides must be >= H and multiples of 8");
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(BI_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (M > 0x7fffffffLL) return fail(BI_ERR_OUT_OF_RANGE, "M too large");
  if (M == 0) return ok();
  if (!a_dev || !b_dev || !s_dev || !gamma_dev || !y_dev) return fail(BI_ERR_INVALID_ARG, "null device pointer");
  if (!aligned(a_dev, 16) || !aligned(b_dev, 16) || !aligned(s_dev, 16) || !aligned(gamma_dev, 16) ||
      !aligned(y_dev, 16))
    return fail(BI_ERR_INVALID_ARG, "a, b, s, gamma and y must be 16-byte aligned");
  return hip_status(bi::launch_add_rmsnorm((const uint16_t*)a_dev, lda, (const uint16_t*)b_dev, ldb,
                                           (uint16_t*)s_dev, ld_s, (const uint16_t*)gamma_dev, eps, M, H,
                                           (uint16_t*)y_dev, ld_y, (hipStream_t)stream),
                    "add_rmsnorm launch");
}

bi_status bi_add(const void* a_dev, int64_t lda, const void* b_dev, int64_t ldb, void* c_dev, int64_t ldc,
                 int64_t rows, int64_t n, void* stream) {
  if (rows < 0 || n < 0 || lda < n || ldb < n || ldc < n) return fail(BI_ERR_INVALID_ARG, "bad add shape");
  if (rows * n == 0) return ok();
  if (!a_dev || !b_dev || !c_dev) return fail(BI_ERR_INVALID_ARG, "null device pointer");
  return hip_status(bi::launch_add((const uint16_t*)a_dev, lda, (const uint16_t*)b_dev, ldb, (uint16_t*)c_dev, ldc,
                                   rows, n, (hipStream_t)stream),
                    "add launch");
}

bi_status bi_gated_gelu(const void* in_dev, int64_t ld_in, void* out_dev, int64_t ld_out, int64_t rows, int64_t ffn,
                        void* stream) {
  if (rows < 0 || ffn < 1 || ld_in < 2 * ffn || ld_out < ffn) return fail(BI_ERR_INVALID_ARG, "bad gated_gelu shape");
  if (rows == 0) return ok();
  if (!in_dev || !out_dev) return fail(BI_ERR_INVALID_ARG, "null device pointer");
  return hip_status(bi::launch_gated_gelu((const uint16_t*)in_dev, ld_in, (uint16_t*)out_dev, ld_out, rows, ffn,
                                          (hipStream_t)stream),
                    "gated_gelu launch");
}

int32_t bi_gemm_splitk_heuristic(int64_t M) { return M <= 16 ? 8 : (M <= 128 ? 4 : 1); }

bi_status bi_gemm_splitk_workspace_size(int64_t M, int64_t N, int32_t k_splits, size_t* bytes) {
  if (!bytes || M < 0 || N < 0 || k_splits < 1) return fail(BI_ERR_INVALID_ARG, "bad workspace-size arguments");
  *bytes = (size_t)k_splits * (size_t)M * (size_t)N * sizeof(float);
  return ok();
}

bi_status bi_gemm_splitk(const void* a_dev, int64_t lda, const void* w_dev, int64_t ldw, void* c_dev, int64_t ldc,
                         bi_dtype c_dtype, int64_t M, int64_t N, int64_t K, int32_t k_splits, void* workspace_dev,
                         size_t workspace_bytes, void* stream) {
  if (bi_status st = check_gemm(a_dev, lda, w_dev, ldw, c_dev, ldc, c_dtype, M, N, K)) return st;
  if (k_splits < 1 || (K / 32) % k_splits != 0)
    return fail(BI_ERR_INVALID_ARG, "k_splits %d must divide K/32 = %lld", k_splits, (long long)(K / 32));
  if (M == 0 || N == 0) return ok();
  const size_t need = (size_t)k_splits * (size_t)M * (size_t)N * sizeof(float);
  if (workspace_bytes < need)
    return fail(BI_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < required %zu", workspace_bytes, need);
  if (!workspace_dev || !aligned(workspace_dev, 16))
    return fail(BI_ERR_INVALID_ARG, "workspace NULL or not 16-byte aligned");
  hipError_t e = bi::launch_gemm_splitk((const uint16_t*)a_dev, lda, (const uint16_t*)w_dev, ldw,
                                        (float*)workspace_dev, M, N, K, k_splits, (hipStream_t)stream);
  if (e != hipSuccess) return hip_status(e, "gemm split-K launch");
  return hip_status(bi::launch_gemm_splitk_reduce((const float*)workspace_dev, k_splits, M, N, c_dev, ldc,
                                                  c_dtype == BI_F32 ? 1 : 0, (hipStream_t)stream),
                    "gemm split-K reduce launch");
}

int32_t bi_bench_mfma_peak_sink_words(void) { return bi::kMfmaPeakGroups * 4; }

bi_status bi_bench_mfma_peak(float value, int32_t rounds, float* sink_dev, int64_t* flops, void* stream) {
  if (!sink_dev || !aligned(sink_dev, 4)) return fail(BI_ERR_INVALID_ARG, "sink NULL or not 4-byte aligned");
  if (!flops) return fail(BI_ERR_INVALID_ARG, "flops NULL");
  if (rounds < 4 || rounds % 4 != 0) return fail(BI_ERR_INVALID_ARG, "rounds %d not a positive multiple of 4", rounds);
  *flops = bi::mfma_peak_flops(rounds);
  return hip_status(bi::launch_mfma_peak(value, rounds, sink_dev, (hipStream_t)stream), "mfma peak launch");
}

int32_t bi_bench_stream_read_sink_words(void) { return bi::kStreamReadGroups; }

bi_status bi_bench_stream_read(const void* src_dev, size_t bytes, uint32_t* sink_dev, void* stream) {
  if (!sink_dev || !aligned(sink_dev, 4)) return fail(BI_ERR_INVALID_ARG, "sink NULL or not 4-byte aligned");
  if (bytes % 16 != 0) return fail(BI_ERR_INVALID_ARG, "bytes %zu not a multiple of 16", bytes);
  if (bytes > 0 && (!src_dev || !aligned(src_dev, 16)))
    return fail(BI_ERR_INVALID_ARG, "src NULL or not 16-byte aligned");
  if (bytes > (size_t)0x7fffffffffffffffULL) return fail(BI_ERR_OUT_OF_RANGE, "bytes too large");
  return hip_status(bi::launch_stream_read(src_dev, (int64_t)bytes, sink_dev, (hipStream_t)stream),
                    "stream read launch");
}

bi_status bi_check_page_table(const int32_t* page_table_host, int32_t page_table_stride, const int32_t* seq_lens_host,
                              const int32_t* query_start_loc_host, int32_t num_seqs, int32_t page_size,
                              int32_t num_pages) {
  if (!page_table_host || !seq_lens_host || num_seqs < 0 || page_table_stride < 1 || page_size < 1 || num_pages < 0)
    return fail(BI_ERR_INVALID_ARG, "bad arguments to bi_check_page_table");
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t k_len = seq_lens_host[s];
    if (k_len < 0) return fail(BI_ERR_OUT_OF_RANGE, "sequence %d: negative length %d", s, k_len);
    const int64_t need = ((int64_t)k_len + page_size - 1) / page_size;
    if (need > page_table_stride)
      return fail(BI_ERR_OUT_OF_RANGE, "sequence %d: k_len %d needs %lld pages, row holds %d", s, k_len,
                  (long long)need, page_table_stride);
    for (int64_t i = 0; i < need; ++i) {
      const int32_t pg = page_table_host[(int64_t)s * page_table_stride + i];
      if (pg < 0 || pg >= num_pages)
        return fail(BI_ERR_OUT_OF_RANGE, "sequence %d: page-table entry %lld = %d outside [0, %d)", s, (long long)i,
                    pg, num_pages);
    }
    if (query_start_loc_host) {
      const int32_t q_len = query_start_loc_host[s + 1] - query_start_loc_host[s];
      if (q_len < 1 || q_len > k_len)
        return fail(BI_ERR_OUT_OF_RANGE, "sequence %d: q_len %d outside [1, k_len = %d]", s, q_len, k_len);
    }
  }
  return ok();
}

bi_status bi_argmax(const float* x_dev, int64_t ld, int64_t rows, int64_t n, int32_t* out_dev, void* stream) {
  if (rows < 0 || n < 1 || ld < n) return fail(BI_ERR_INVALID_ARG, "rows >= 0, n >= 1 and ld >= n required");
  if (rows > 0x7fffffffLL || n > 0x7fffffffLL) return fail(BI_ERR_OUT_OF_RANGE, "rows and n must fit in int32");
  if (rows == 0) return ok();
  if (!x_dev || !out_dev || ((uintptr_t)x_dev & 3)) return fail(BI_ERR_INVALID_ARG, "null or misaligned device pointer");
  return hip_status(bi::launch_argmax(x_dev, ld, rows, n, out_dev, (hipStream_t)stream), "argmax launch");
}

}  // extern "C"

struct bi_prefix_cache {
  bi::PrefixCache impl;
  bi_prefix_cache(int32_t n, int32_t p, int32_t bits) : impl(n, p, bits) {}
};

extern "C" {

bi_status bi_prefix_cache_create(int32_t num_pages, int32_t page_size, int32_t hash_bits, bi_prefix_cache** out) {
  if (!out || num_pages < 1 || page_size < 1 || hash_bits < 0 || hash_bits > 64)
    return fail(BI_ERR_INVALID_ARG, "num_pages >= 1, page_size >= 1, hash_bits in [0, 64] and out required");
  *out = nullptr;
  bi_prefix_cache* c = new (std::nothrow) bi_prefix_cache(num_pages, page_size, hash_bits);
  if (!c) return fail(BI_ERR_OUT_OF_RANGE, "out of host memory");
  *out = c;
  return ok();
}

void bi_prefix_cache_destroy(bi_prefix_cache* cache) { delete cache; }

bi_status bi_prefix_cache_match(bi_prefix_cache* cache, const int32_t* tokens, int64_t num_tokens,
                                int32_t* pages_out, int32_t max_pages, int32_t* num_matched) {
  if (!cache || !num_matched || num_tokens < 0 || max_pages < 0 || (num_tokens > 0 && !tokens) ||
      (max_pages > 0 && !pages_out))
    return fail(BI_ERR_INVALID_ARG, "bad arguments to bi_prefix_cache_match");
  *num_matched = cache->impl.match(tokens, num_tokens, pages_out, max_pages);
  return ok();
}

bi_status bi_prefix_cache_alloc(bi_prefix_cache* cache, int32_t n, int32_t* pages_out) {
  if (!cache || n < 0 || (n > 0 && !pages_out)) return fail(BI_ERR_INVALID_ARG, "bad arguments to bi_prefix_cache_alloc");
  if (!cache->impl.alloc(n, pages_out))
    return fail(BI_ERR_OUT_OF_RANGE, "cannot provide %d pages (all others referenced)", n);
  return ok();
}

bi_status bi_prefix_cache_register(bi_prefix_cache* cache, int32_t page, int32_t parent, int32_t depth,
                                   const int32_t* tokens, int32_t* existing) {
  if (!cache || !tokens || !existing || page < 0 || page >= cache->impl.num_pages() || parent < -1 ||
      parent >= cache->impl.num_pages())
    return fail(BI_ERR_INVALID_ARG, "bad arguments to bi_prefix_cache_register");
  const int r = cache->impl.register_page(page, parent, depth, tokens, existing);
  if (r == -1) return fail(BI_ERR_WRITE_CONFLICT, "page %d is shared or already registered", page);
  if (r == -2) return fail(BI_ERR_INVALID_ARG, "page %d: parent %d / depth %d inconsistent", page, parent, depth);
  return ok();
}

bi_status bi_prefix_cache_release(bi_prefix_cache* cache, const int32_t* pages, int32_t n) {
  if (!cache || n < 0 || (n > 0 && !pages)) return fail(BI_ERR_INVALID_ARG, "bad arguments to bi_prefix_cache_release");
  if (!cache->impl.release(pages, n)) return fail(BI_ERR_INVALID_ARG, "a page would lose a reference it does not hold");
  return ok();
}

bi_status bi_prefix_cache_writable(const bi_prefix_cache* cache, uint8_t* mask_out, int32_t num_pages) {
  if (!cache || !mask_out || num_pages != cache->impl.num_pages())
    return fail(BI_ERR_INVALID_ARG, "mask must cover exactly the cache's pages");
  for (int32_t p = 0; p < num_pages; ++p) mask_out[p] = cache->impl.writable(p) ? 1 : 0;
  return ok();
}

bi_status bi_prefix_cache_stats(const bi_prefix_cache* cache, int64_t* stats_out) {
  if (!cache || !stats_out) return fail(BI_ERR_INVALID_ARG, "bad arguments to bi_prefix_cache_stats");
  cache->impl.stats(stats_out);
  return ok();
}

bi_status bi_check_write_plan(const int32_t* slot_mapping_host, int32_t num_tokens, const uint8_t* page_writable_host,
                              int32_t num_pages, int32_t page_size) {
  if ((!slot_mapping_host && num_tokens > 0) || num_tokens < 0 || num_pages < 0 || page_size < 1)
    return fail(BI_ERR_INVALID_ARG, "bad arguments to bi_check_write_plan");
  std::vector<uint8_t> seen((size_t)num_pages * page_size, 0);
  for (int32_t t = 0; t < num_tokens; ++t) {
    const int32_t slot = slot_mapping_host[t];
    if (slot < 0) continue;
    if ((int64_t)slot >= (int64_t)num_pages * page_size)
      return fail(BI_ERR_OUT_OF_RANGE, "token %d: slot %d outside the %d-page pool", t, slot, num_pages);
    if (page_writable_host && !page_writable_host[slot / page_size])
      return fail(BI_ERR_WRITE_CONFLICT, "token %d: slot %d lies in read-only (shared) page %d", t, slot,
                  slot / page_size);
    if (seen[slot]) return fail(BI_ERR_WRITE_CONFLICT, "token %d: slot %d written twice in one plan", t, slot);
    seen[slot] = 1;
  }
  return ok();
}

}  // extern "C"
