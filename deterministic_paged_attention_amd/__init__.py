"""Python binding of libbi.so (batch-invariant paged attention, RMSNorm, GEMM).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libbi.so.  Functions carry the names of the C entry points in
``include/bi.h``; tensors are torch tensors on the GPU (torch provides device
memory and the current stream, nothing else).  Importing this package fails
loudly when the library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbi.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "bi.h")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it first with "
                      "`python deterministic_paged_attention_amd/build.py` (or __graft_entry__.build())")

# torch is imported first so that its HIP runtime is the one loaded into the
# process: libbi.so then binds to that same libamdhip64 (same soname) instead of
# bringing a second runtime in from the system ROCm install.  One process, one
# HIP runtime, shared with the tensors and streams torch hands us.
import torch as _torch_runtime  # noqa: E402,F401

lib = ctypes.CDLL(LIB_PATH)

c_i32, c_i64, c_f32, c_sz, c_vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
P_i32 = ctypes.POINTER(ctypes.c_int32)

BI_OK = 0
STATUS_NAMES = {0: "BI_OK", 1: "BI_ERR_INVALID_ARG", 2: "BI_ERR_UNSUPPORTED_CONFIG", 3: "BI_ERR_OUT_OF_RANGE",
                4: "BI_ERR_WRITE_CONFLICT", 5: "BI_ERR_WORKSPACE_TOO_SMALL", 6: "BI_ERR_HIP"}
BI_BF16, BI_F32 = 0, 1


class bi_attn_desc(ctypes.Structure):
    _fields_ = [("num_q_heads", c_i32), ("num_kv_heads", c_i32), ("head_dim", c_i32), ("page_size", c_i32),
                ("split_size", c_i32), ("window", c_i32), ("scale", c_f32)]


class BiError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = STATUS_NAMES.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


def _sig(name, restype, *argtypes):
    f = getattr(lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_sig("bi_attn_config_create", c_i32, ctypes.POINTER(bi_attn_desc), ctypes.POINTER(c_vp))
_sig("bi_attn_config_destroy", None, c_vp)
_sig("bi_attn_config_query", c_i32, c_vp, ctypes.POINTER(bi_attn_desc), P_i32)
_sig("bi_kv_cache_bytes", c_i32, c_vp, c_i64, ctypes.POINTER(c_sz))
_sig("bi_slot_mapping", c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp)
_sig("bi_kv_write", c_i32, c_vp, c_vp, c_i64, c_vp, c_i64, c_vp, c_i32, c_vp, c_vp, c_i32, c_vp)
_sig("bi_kv_write_paged", c_i32, c_vp, c_vp, c_i64, c_vp, c_i64, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_vp, c_vp, c_i32,
     c_vp)
_sig("bi_paged_attention_workspace_size", c_i32, c_vp, c_i32, c_i32, c_i32, ctypes.POINTER(c_sz))
_sig("bi_paged_attention_item_blocks", c_i32, c_vp, c_i32, c_i32, c_i32, P_i32)
_sig("bi_paged_attention_mapping", c_i32, c_vp, c_i32, c_i32, c_i32, P_i32)
_sig("bi_paged_attention_force_mapping", c_i32, c_i32)
_ATTN_ARGS = (c_vp, c_vp, c_i64, c_vp, c_vp, c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32)
_sig("bi_paged_attention", c_i32, *_ATTN_ARGS, c_vp, c_sz, c_vp, c_vp)
_sig("bi_paged_attention_split", c_i32, *_ATTN_ARGS, c_vp, c_sz, c_vp)
_sig("bi_paged_attention_noalloc", c_i32, *_ATTN_ARGS, c_vp, c_vp)
_sig("bi_paged_attention_merge", c_i32, c_vp, c_vp, c_vp, c_i32, c_i32, c_i32, c_vp, c_sz, c_vp, c_vp)
_sig("bi_rmsnorm", c_i32, c_vp, c_i64, c_vp, c_f32, c_i64, c_i64, c_vp, c_i64, c_vp)
_sig("bi_gemm", c_i32, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_i32, c_i64, c_i64, c_i64, c_vp)
_sig("bi_check_page_table", c_i32, c_vp, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32)
_sig("bi_check_write_plan", c_i32, c_vp, c_i32, c_vp, c_i32, c_i32)
_sig("bi_argmax", c_i32, c_vp, c_i64, c_i64, c_i64, c_vp, c_vp)
_sig("bi_prefix_cache_create", c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_vp))
_sig("bi_prefix_cache_destroy", None, c_vp)
_sig("bi_prefix_cache_match", c_i32, c_vp, c_vp, c_i64, c_vp, c_i32, P_i32)
_sig("bi_prefix_cache_alloc", c_i32, c_vp, c_i32, c_vp)
_sig("bi_prefix_cache_register", c_i32, c_vp, c_i32, c_i32, c_i32, c_vp, P_i32)
_sig("bi_prefix_cache_release", c_i32, c_vp, c_vp, c_i32)
_sig("bi_prefix_cache_writable", c_i32, c_vp, c_vp, c_i32)
_sig("bi_prefix_cache_stats", c_i32, c_vp, c_vp)
_sig("bi_splitk_attention_heuristic", c_i32, c_vp, c_i32, c_i32, c_i32, c_i32, P_i32)
_sig("bi_paged_attention_splitk_workspace_size", c_i32, c_vp, c_i32, c_i32, c_i32, c_i32, ctypes.POINTER(c_sz))
_sig("bi_paged_attention_splitk", c_i32, *_ATTN_ARGS, c_i32, c_vp, c_sz, c_vp, c_vp)
_sig("bi_bench_mfma_peak_sink_words", c_i32)
_sig("bi_bench_mfma_peak", c_i32, c_f32, c_i32, c_vp, ctypes.POINTER(c_i64), c_vp)
_sig("bi_bench_stream_read_sink_words", c_i32)
_sig("bi_bench_stream_read", c_i32, c_vp, c_sz, c_vp, c_vp)
_sig("bi_gemm_splitk_heuristic", c_i32, c_i64)
_sig("bi_gemm_splitk_workspace_size", c_i32, c_i64, c_i64, c_i32, ctypes.POINTER(c_sz))
_sig("bi_gemm_splitk", c_i32, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_i32, c_i64, c_i64, c_i64, c_i32, c_vp, c_sz,
     c_vp)
_sig("bi_embedding", c_i32, c_vp, c_i64, c_i64, c_vp, c_i32, c_vp, c_i64, c_vp)
_sig("bi_qk_norm_rope", c_i32, c_vp, c_i64, c_i32, c_vp, c_vp, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp, c_f32,
     ctypes.c_double, c_vp)
_sig("bi_qk_norm_rope_kv_write", c_i32, c_vp, c_vp, c_i64, c_i32, c_vp, c_vp, c_i32, c_vp, c_vp, c_f32, ctypes.c_double,
     c_vp, c_vp, c_vp, c_i32, c_vp)
_sig("bi_add", c_i32, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_vp)
_sig("bi_add_rmsnorm", c_i32, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_f32, c_i64, c_i64, c_vp, c_i64, c_vp)
_sig("bi_gated_gelu", c_i32, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_vp)
_sig("bi_gemm_gated_gelu", c_i32, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_i64, c_vp)
_sig("bi_status_string", ctypes.c_char_p, c_i32)
_sig("bi_last_error_message", ctypes.c_char_p)
_sig("bi_version", c_i32)


def _check(status: int) -> None:
    if status != BI_OK:
        raise BiError(status, lib.bi_last_error_message().decode())


def declared_functions(header: str = HEADER_PATH):
    """Names of the functions include/bi.h declares (used by the export test)."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z0-9_]+)\s*\(", text)))


# ---------------------------------------------------------------------------
# torch marshalling helpers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _stream(stream=None) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t, dtype, name, device=True):
    torch = _torch()
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if device and t.device.type != "cuda":
        raise TypeError(f"{name} must be a GPU tensor")


def _row_stride(t, name):
    """Element stride between rows of a [rows, ...] view whose trailing dims are contiguous."""
    inner = 1
    for d in range(t.dim() - 1, 0, -1):
        if t.stride(d) != inner:
            raise ValueError(f"{name}: trailing dimensions must be contiguous")
        inner *= t.shape[d]
    return t.stride(0) if t.shape[0] > 1 else max(inner, t.stride(0))


class AttnConfig:
    """Owns a bi_attn_config handle (bi_attn_config_create / _destroy)."""

    def __init__(self, num_q_heads, num_kv_heads, head_dim, page_size=16, split_size=256, window=0, scale=0.0):
        d = bi_attn_desc(num_q_heads, num_kv_heads, head_dim, page_size, split_size, window, float(scale))
        h = c_vp()
        _check(lib.bi_attn_config_create(ctypes.byref(d), ctypes.byref(h)))
        self.handle = h
        q = bi_attn_desc()
        tile = c_i32()
        _check(lib.bi_attn_config_query(self.handle, ctypes.byref(q), ctypes.byref(tile)))
        self.desc = q
        self.key_tile = tile.value
        self.num_q_heads, self.num_kv_heads, self.head_dim = num_q_heads, num_kv_heads, head_dim
        self.page_size, self.split_size, self.window, self.scale = page_size, split_size, window, q.scale

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value and lib is not None:  # lib may be gone at interpreter exit
            lib.bi_attn_config_destroy(h)
            self.handle = None

    def k_cache_shape(self, num_pages) -> Tuple[int, ...]:
        return (num_pages, self.num_kv_heads, self.head_dim // 8, self.page_size, 8)

    def v_cache_shape(self, num_pages) -> Tuple[int, ...]:
        return (num_pages, self.num_kv_heads, self.head_dim // 32, 16, self.page_size, 2)


def bi_attn_config_create(num_q_heads, num_kv_heads, head_dim, page_size=16, split_size=256, window=0, scale=0.0):
    return AttnConfig(num_q_heads, num_kv_heads, head_dim, page_size, split_size, window, scale)


def bi_kv_cache_bytes(cfg: AttnConfig, num_pages: int) -> int:
    b = c_sz()
    _check(lib.bi_kv_cache_bytes(cfg.handle, num_pages, ctypes.byref(b)))
    return b.value


def bi_slot_mapping(page_table, seq_lens, query_start_loc, num_tokens, page_size, num_pages, out=None, stream=None):
    torch = _torch()
    for t, n in ((page_table, "page_table"), (seq_lens, "seq_lens"), (query_start_loc, "query_start_loc")):
        _need(t, torch.int32, n)
    if out is None:
        out = torch.empty(num_tokens, dtype=torch.int32, device=page_table.device)
    _need(out, torch.int32, "out")
    assert page_table.is_contiguous()
    _check(lib.bi_slot_mapping(_ptr(page_table), page_table.shape[1], _ptr(seq_lens), _ptr(query_start_loc),
                               seq_lens.shape[0], num_tokens, page_size, num_pages, _ptr(out), _stream(stream)))
    return out


def bi_kv_write(cfg: AttnConfig, k_new, v_new, slot_mapping, k_cache, v_cache, stream=None):
    torch = _torch()
    _need(k_new, torch.bfloat16, "k_new")
    _need(v_new, torch.bfloat16, "v_new")
    _need(slot_mapping, torch.int32, "slot_mapping")
    n = k_new.shape[0]
    _check(lib.bi_kv_write(cfg.handle, _ptr(k_new), _row_stride(k_new, "k_new") if n else cfg.num_kv_heads * cfg.head_dim,
                           _ptr(v_new), _row_stride(v_new, "v_new") if n else cfg.num_kv_heads * cfg.head_dim,
                           _ptr(slot_mapping), n, _ptr(k_cache), _ptr(v_cache), k_cache.shape[0], _stream(stream)))


def bi_kv_write_paged(cfg: AttnConfig, k_new, v_new, page_table, seq_lens, query_start_loc, k_cache, v_cache,
                      stream=None):
    """bi_slot_mapping + bi_kv_write in one launch (slots from the page table)."""
    torch = _torch()
    _need(k_new, torch.bfloat16, "k_new")
    _need(v_new, torch.bfloat16, "v_new")
    for t, nm in ((page_table, "page_table"), (seq_lens, "seq_lens"), (query_start_loc, "query_start_loc")):
        _need(t, torch.int32, nm)
    if not page_table.is_contiguous():
        raise ValueError("page_table must be contiguous")
    n = k_new.shape[0]
    row = cfg.num_kv_heads * cfg.head_dim
    _check(lib.bi_kv_write_paged(cfg.handle, _ptr(k_new), _row_stride(k_new, "k_new") if n else row,
                                 _ptr(v_new), _row_stride(v_new, "v_new") if n else row, _ptr(page_table),
                                 page_table.shape[1], _ptr(seq_lens), _ptr(query_start_loc), seq_lens.shape[0], n,
                                 _ptr(k_cache), _ptr(v_cache), k_cache.shape[0], _stream(stream)))


def bi_paged_attention_workspace_size(cfg: AttnConfig, num_seqs: int, num_tokens: int, max_seq_len: int) -> int:
    b = c_sz()
    _check(lib.bi_paged_attention_workspace_size(cfg.handle, num_seqs, num_tokens, max_seq_len, ctypes.byref(b)))
    return b.value


def bi_paged_attention_splitk_workspace_size(cfg: AttnConfig, num_seqs: int, num_tokens: int, max_seq_len: int,
                                             num_splits: int):
    b = c_sz()
    _check(lib.bi_paged_attention_splitk_workspace_size(cfg.handle, num_seqs, num_tokens, max_seq_len, num_splits,
                                                        ctypes.byref(b)))
    return b.value


def alloc_workspace(nbytes: int, device="cuda"):
    torch = _torch()
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def _attn_common(cfg, q, k_cache, v_cache, page_table, seq_lens, query_start_loc):
    torch = _torch()
    _need(q, torch.bfloat16, "q")
    _need(k_cache, torch.bfloat16, "k_cache")
    _need(v_cache, torch.bfloat16, "v_cache")
    for t, nm in ((page_table, "page_table"), (seq_lens, "seq_lens"), (query_start_loc, "query_start_loc")):
        _need(t, torch.int32, nm)
    if not (page_table.is_contiguous() and k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("page_table and caches must be contiguous")
    T = q.shape[0]
    qs = _row_stride(q, "q") if T else cfg.num_q_heads * cfg.head_dim
    return (cfg.handle, _ptr(q), qs, _ptr(k_cache), _ptr(v_cache), k_cache.shape[0], _ptr(page_table),
            page_table.shape[1], _ptr(seq_lens), _ptr(query_start_loc), seq_lens.shape[0], T)


def bi_paged_attention(cfg: AttnConfig, q, k_cache, v_cache, page_table, seq_lens, query_start_loc, max_seq_len,
                       workspace=None, out=None, stream=None):
    torch = _torch()
    args = _attn_common(cfg, q, k_cache, v_cache, page_table, seq_lens, query_start_loc)
    T = q.shape[0]
    if workspace is None:
        workspace = alloc_workspace(bi_paged_attention_workspace_size(cfg, seq_lens.shape[0], T, max_seq_len),
                                    q.device)
    if out is None:
        out = torch.empty((T, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device=q.device)
    _check(lib.bi_paged_attention(*args, max_seq_len, _ptr(workspace), workspace.numel() * workspace.element_size(),
                                  _ptr(out), _stream(stream)))
    return out


def bi_paged_attention_noalloc(cfg: AttnConfig, q, k_cache, v_cache, page_table, seq_lens, query_start_loc,
                               max_seq_len, out=None, stream=None):
    """bi_paged_attention with the partials in the library's own device array
    (no workspace; the caller passes inputs and the output)."""
    torch = _torch()
    args = _attn_common(cfg, q, k_cache, v_cache, page_table, seq_lens, query_start_loc)
    T = q.shape[0]
    if out is None:
        out = torch.empty((T, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device=q.device)
    _check(lib.bi_paged_attention_noalloc(*args, max_seq_len, _ptr(out), _stream(stream)))
    return out


def bi_paged_attention_split(cfg: AttnConfig, q, k_cache, v_cache, page_table, seq_lens, query_start_loc,
                             max_seq_len, workspace, stream=None):
    args = _attn_common(cfg, q, k_cache, v_cache, page_table, seq_lens, query_start_loc)
    _check(lib.bi_paged_attention_split(*args, max_seq_len, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))


def bi_paged_attention_merge(cfg: AttnConfig, seq_lens, query_start_loc, num_tokens, max_seq_len, workspace,
                             out=None, stream=None):
    torch = _torch()
    if out is None:
        out = torch.empty((num_tokens, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device=seq_lens.device)
    _check(lib.bi_paged_attention_merge(cfg.handle, _ptr(seq_lens), _ptr(query_start_loc), seq_lens.shape[0],
                                        num_tokens, max_seq_len, _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)))
    return out


def workspace_views(cfg: AttnConfig, workspace, num_tokens: int, num_splits: int):
    """(ml [R, NS, 2] fp32, acc [R, NS, D] bf16) views of a workspace, per the layout in bi.h."""
    torch = _torch()
    R = num_tokens * cfg.num_q_heads
    ml_bytes = R * num_splits * 8
    acc_off = (ml_bytes + 255) // 256 * 256
    f = workspace.view(torch.uint8)
    ml = f[:ml_bytes].view(torch.float32).view(R, num_splits, 2)
    acc = f[acc_off: acc_off + R * num_splits * cfg.head_dim * 2].view(torch.bfloat16).view(R, num_splits, cfg.head_dim)
    return ml, acc


def bi_paged_attention_item_blocks(cfg: AttnConfig, num_seqs: int, num_tokens: int, max_seq_len: int) -> int:
    v = c_i32()
    _check(lib.bi_paged_attention_item_blocks(cfg.handle, num_seqs, num_tokens, max_seq_len, ctypes.byref(v)))
    return v.value


def bi_paged_attention_mapping(cfg: AttnConfig, num_seqs: int, num_tokens: int, max_seq_len: int) -> int:
    """1 when bi_paged_attention runs the row-group mapping for this batch shape, else 0."""
    v = c_i32()
    _check(lib.bi_paged_attention_mapping(cfg.handle, num_seqs, num_tokens, max_seq_len, ctypes.byref(v)))
    return v.value


def bi_paged_attention_force_mapping(mapping: int) -> None:
    """Force the attention work mapping on this thread (0 = chosen per call)."""
    _check(lib.bi_paged_attention_force_mapping(mapping))


class forced_mapping:
    """Context manager: attention calls inside use the given work mapping."""

    def __init__(self, mapping: int):
        self.mapping = mapping

    def __enter__(self):
        bi_paged_attention_force_mapping(self.mapping)
        return self

    def __exit__(self, *exc):
        bi_paged_attention_force_mapping(0)
        return False


def bi_splitk_attention_heuristic(cfg: AttnConfig, num_seqs, max_seq_len, num_compute_units, waves_per_cu=8):
    n = c_i32()
    _check(lib.bi_splitk_attention_heuristic(cfg.handle, num_seqs, max_seq_len, num_compute_units, waves_per_cu,
                                             ctypes.byref(n)))
    return n.value


def bi_paged_attention_splitk(cfg: AttnConfig, q, k_cache, v_cache, page_table, seq_lens, query_start_loc,
                              max_seq_len, num_splits, workspace=None, out=None, stream=None):
    torch = _torch()
    args = _attn_common(cfg, q, k_cache, v_cache, page_table, seq_lens, query_start_loc)
    T = q.shape[0]
    if workspace is None:
        workspace = alloc_workspace(bi_paged_attention_splitk_workspace_size(cfg, seq_lens.shape[0], T, max_seq_len,
                                                                             num_splits), q.device)
    if out is None:
        out = torch.empty((T, cfg.num_q_heads, cfg.head_dim), dtype=torch.bfloat16, device=q.device)
    _check(lib.bi_paged_attention_splitk(*args, max_seq_len, num_splits, _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _ptr(out), _stream(stream)))
    return out


def bi_rmsnorm(x, gamma, eps, out=None, stream=None):
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    _need(gamma, torch.bfloat16, "gamma")
    M, H = x.shape
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=x.device)
    ldx = x.stride(0) if M > 1 else H
    ldy = out.stride(0) if M > 1 else H
    if x.stride(1) != 1 or out.stride(1) != 1 or not gamma.is_contiguous():
        raise ValueError("rows of x / out and gamma must be contiguous")
    _check(lib.bi_rmsnorm(_ptr(x), ldx, _ptr(gamma), float(eps), M, H, _ptr(out), ldy, _stream(stream)))
    return out


def _gemm_args(a, w, out, out_dtype):
    torch = _torch()
    _need(a, torch.bfloat16, "a")
    _need(w, torch.bfloat16, "w")
    M, K = a.shape
    N = w.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a.device)
    if a.stride(1) != 1 or w.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("a, w and out need contiguous rows")
    dt = BI_F32 if out.dtype == torch.float32 else BI_BF16
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be bf16 or fp32")
    lda = a.stride(0) if M > 1 else K
    ldw = w.stride(0) if N > 1 else K
    ldc = out.stride(0) if M > 1 else N
    return out, (_ptr(a), lda, _ptr(w), ldw, _ptr(out), ldc, dt, M, N, K)


def bi_gemm(a, w, out_dtype=None, out=None, stream=None):
    torch = _torch()
    out, args = _gemm_args(a, w, out, out_dtype or torch.bfloat16)
    _check(lib.bi_gemm(*args, _stream(stream)))
    return out


def bi_gemm_splitk_heuristic(M: int) -> int:
    return lib.bi_gemm_splitk_heuristic(M)


def bi_gemm_splitk(a, w, k_splits, out_dtype=None, out=None, workspace=None, stream=None):
    torch = _torch()
    out, args = _gemm_args(a, w, out, out_dtype or torch.bfloat16)
    M, N = out.shape
    need = c_sz()
    _check(lib.bi_gemm_splitk_workspace_size(M, N, k_splits, ctypes.byref(need)))
    if workspace is None:
        workspace = alloc_workspace(need.value, a.device)
    _check(lib.bi_gemm_splitk(*args, k_splits, _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _stream(stream)))
    return out


def bi_bench_stream_read(src, sink=None, stream=None):
    """Streaming-read reference (measurement only): reads every byte of the
    contiguous device tensor src once; returns the uint32 sink (one xor word
    per workgroup; their xor is the xor of src's 32-bit words)."""
    torch = _torch()
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    nbytes = src.numel() * src.element_size()
    if sink is None:
        sink = torch.empty(lib.bi_bench_stream_read_sink_words(), dtype=torch.int32, device=src.device)
    _check(lib.bi_bench_stream_read(_ptr(src), nbytes, _ptr(sink), _stream(stream)))
    return sink


def bi_bench_mfma_peak(rounds, value=0.0, sink=None, stream=None):
    """MFMA throughput reference (measurement only): one launch of `rounds`
    rounds of eight bf16 MFMAs per wave over a full grid.  Returns (sink,
    flops) — the per-wave float sink and the launch's flop count."""
    torch = _torch()
    if sink is None:
        sink = torch.empty(lib.bi_bench_mfma_peak_sink_words(), dtype=torch.float32, device="cuda")
    flops = c_i64()
    _check(lib.bi_bench_mfma_peak(float(value), int(rounds), _ptr(sink), ctypes.byref(flops), _stream(stream)))
    return sink, flops.value


def bi_embedding(table, ids, out=None, stream=None):
    torch = _torch()
    _need(table, torch.bfloat16, "table")
    _need(ids, torch.int32, "ids")
    V, H = table.shape
    T = ids.shape[0]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=table.device)
    ld = out.stride(0) if T > 1 else H
    _check(lib.bi_embedding(_ptr(table), V, H, _ptr(ids), T, _ptr(out), ld, _stream(stream)))
    return out


def bi_qk_norm_rope(qkv, seq_lens, query_start_loc, num_q_heads, num_kv_heads, head_dim, gamma_q, gamma_k, eps,
                    rope_theta, stream=None):
    """In place on the q and k parts of qkv [T, row] (bf16)."""
    torch = _torch()
    _need(qkv, torch.bfloat16, "qkv")
    T = qkv.shape[0]
    rs = qkv.stride(0) if T > 1 else qkv.shape[1]
    _check(lib.bi_qk_norm_rope(_ptr(qkv), rs, T, _ptr(seq_lens), _ptr(query_start_loc), seq_lens.shape[0],
                               num_q_heads, num_kv_heads, head_dim, _ptr(gamma_q), _ptr(gamma_k), float(eps),
                               float(rope_theta), _stream(stream)))
    return qkv


def bi_qk_norm_rope_kv_write(cfg: AttnConfig, qkv, seq_lens, query_start_loc, gamma_q, gamma_k, eps, rope_theta,
                             slot_mapping, k_cache, v_cache, stream=None):
    """bi_qk_norm_rope on qkv [T, (H_q + 2 H_kv) D] in place, fused with the cache
    write of its k and v parts at slot_mapping (one launch)."""
    torch = _torch()
    _need(qkv, torch.bfloat16, "qkv")
    _need(k_cache, torch.bfloat16, "k_cache")
    _need(v_cache, torch.bfloat16, "v_cache")
    _need(slot_mapping, torch.int32, "slot_mapping")
    T = qkv.shape[0]
    rs = qkv.stride(0) if T > 1 else qkv.shape[1]
    if qkv.stride(1) != 1 or not (k_cache.is_contiguous() and v_cache.is_contiguous()):
        raise ValueError("qkv rows and the caches must be contiguous")
    _check(lib.bi_qk_norm_rope_kv_write(cfg.handle, _ptr(qkv), rs, T, _ptr(seq_lens), _ptr(query_start_loc),
                                        seq_lens.shape[0], _ptr(gamma_q), _ptr(gamma_k), float(eps), float(rope_theta),
                                        _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache), k_cache.shape[0],
                                        _stream(stream)))
    return qkv


def bi_add(a, b, out=None, stream=None):
    torch = _torch()
    _need(a, torch.bfloat16, "a")
    _need(b, torch.bfloat16, "b")
    R, N = a.shape
    if out is None:
        out = torch.empty((R, N), dtype=torch.bfloat16, device=a.device)
    ld = lambda t: t.stride(0) if R > 1 else N  # noqa: E731
    _check(lib.bi_add(_ptr(a), ld(a), _ptr(b), ld(b), _ptr(out), ld(out), R, N, _stream(stream)))
    return out


def bi_add_rmsnorm(a, b, gamma, eps, sum_out=None, out=None, stream=None):
    """(s, y) with s = a + b and y = rmsnorm(s): one launch, bitwise equal to
    bi_add followed by bi_rmsnorm.  sum_out may be a or b (in place)."""
    torch = _torch()
    _need(a, torch.bfloat16, "a")
    _need(b, torch.bfloat16, "b")
    _need(gamma, torch.bfloat16, "gamma")
    M, H = a.shape
    if sum_out is None:
        sum_out = torch.empty((M, H), dtype=torch.bfloat16, device=a.device)
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=a.device)
    for t, nm in ((a, "a"), (b, "b"), (sum_out, "sum_out"), (out, "out")):
        if t.stride(1) != 1:
            raise ValueError(f"rows of {nm} must be contiguous")
    if not gamma.is_contiguous():
        raise ValueError("gamma must be contiguous")
    ld = lambda t: t.stride(0) if M > 1 else H  # noqa: E731
    _check(lib.bi_add_rmsnorm(_ptr(a), ld(a), _ptr(b), ld(b), _ptr(sum_out), ld(sum_out), _ptr(gamma), float(eps), M, H,
                              _ptr(out), ld(out), _stream(stream)))
    return sum_out, out


def bi_gated_gelu(x, out=None, stream=None):
    torch = _torch()
    _need(x, torch.bfloat16, "x")
    R, F2 = x.shape
    F = F2 // 2
    if out is None:
        out = torch.empty((R, F), dtype=torch.bfloat16, device=x.device)
    _check(lib.bi_gated_gelu(_ptr(x), x.stride(0) if R > 1 else F2, _ptr(out), out.stride(0) if R > 1 else F, R, F,
                             _stream(stream)))
    return out


def bi_gemm_gated_gelu(a, w_gu, out=None, stream=None):
    """gated_gelu(a w_gu^T) for a [gate | up] weight of 2F rows, M <= 16 rows of a."""
    torch = _torch()
    _need(a, torch.bfloat16, "a")
    _need(w_gu, torch.bfloat16, "w_gu")
    M, K = a.shape
    F = w_gu.shape[0] // 2
    if out is None:
        out = torch.empty((M, F), dtype=torch.bfloat16, device=a.device)
    if a.stride(1) != 1 or w_gu.stride(1) != 1 or out.stride(1) != 1:
        raise ValueError("a, w_gu and out need contiguous rows")
    _check(lib.bi_gemm_gated_gelu(_ptr(a), a.stride(0) if M > 1 else K, _ptr(w_gu), w_gu.stride(0), _ptr(out),
                                  out.stride(0) if M > 1 else F, M, F, K, _stream(stream)))
    return out


def bi_check_page_table(page_table, seq_lens, query_start_loc, page_size, num_pages):
    """Host check of a page table (numpy / list inputs); raises BiError."""
    pt = np.ascontiguousarray(np.asarray(page_table, dtype=np.int32))
    sl = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    qsl = None if query_start_loc is None else np.ascontiguousarray(np.asarray(query_start_loc, dtype=np.int32))
    _check(lib.bi_check_page_table(pt.ctypes.data, pt.shape[1], sl.ctypes.data,
                                   None if qsl is None else qsl.ctypes.data, sl.shape[0], page_size, num_pages))


def bi_check_write_plan(slot_mapping, page_writable, num_pages, page_size):
    """Host check of a write plan (numpy / list inputs); raises BiError."""
    sm = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int32))
    pw = None if page_writable is None else np.ascontiguousarray(np.asarray(page_writable, dtype=np.uint8))
    _check(lib.bi_check_write_plan(sm.ctypes.data if sm.size else None, sm.shape[0],
                                   None if pw is None else pw.ctypes.data, num_pages, page_size))


def bi_argmax(x, out=None, stream=None):
    """Greedy sampling over fp32 rows: smallest index of the row maximum."""
    torch = _torch()
    _need(x, torch.float32, "x")
    R, n = x.shape
    if out is None:
        out = torch.empty((R,), dtype=torch.int32, device=x.device)
    if x.stride(1) != 1:
        raise ValueError("rows of x must be contiguous")
    _check(lib.bi_argmax(_ptr(x), x.stride(0) if R > 1 else n, R, n, _ptr(out), _stream(stream)))
    return out


class PrefixCache:
    """Host-side prefix cache of KV pages (the C ABI's bi_prefix_cache_*);
    arguments and results are Python lists of ints."""

    def __init__(self, num_pages: int, page_size: int = 16, hash_bits: int = 64):
        h = c_vp()
        _check(lib.bi_prefix_cache_create(num_pages, page_size, hash_bits, ctypes.byref(h)))
        self.handle = h
        self.num_pages = num_pages
        self.page_size = page_size

    def __del__(self):
        if getattr(self, "handle", None) and lib is not None:
            lib.bi_prefix_cache_destroy(self.handle)
            self.handle = None

    @staticmethod
    def _arr(values, dtype=np.int32):
        return np.ascontiguousarray(np.asarray(values, dtype=dtype))

    def match(self, tokens, max_pages: int):
        t = self._arr(tokens)
        out = np.zeros(max(max_pages, 1), dtype=np.int32)
        k = c_i32()
        _check(lib.bi_prefix_cache_match(self.handle, t.ctypes.data if t.size else None, t.size, out.ctypes.data,
                                         max_pages, ctypes.byref(k)))
        return out[:k.value].tolist()

    def alloc(self, n: int):
        out = np.zeros(max(n, 1), dtype=np.int32)
        _check(lib.bi_prefix_cache_alloc(self.handle, n, out.ctypes.data))
        return out[:n].tolist()

    def register(self, page: int, parent: int, depth: int, tokens):
        """Returns the id of an identical cached page (page stays private), or -1."""
        t = self._arr(tokens)
        if t.size != self.page_size:
            raise ValueError("a page holds exactly page_size tokens")
        ex = c_i32()
        _check(lib.bi_prefix_cache_register(self.handle, page, parent, depth, t.ctypes.data, ctypes.byref(ex)))
        return ex.value

    def release(self, pages):
        p = self._arr(pages)
        _check(lib.bi_prefix_cache_release(self.handle, p.ctypes.data if p.size else None, p.size))

    def writable(self):
        m = np.zeros(self.num_pages, dtype=np.uint8)
        _check(lib.bi_prefix_cache_writable(self.handle, m.ctypes.data, self.num_pages))
        return m

    def stats(self):
        """(free pages, registered pages, evictable pages, evictions so far)"""
        s = np.zeros(4, dtype=np.int64)
        _check(lib.bi_prefix_cache_stats(self.handle, s.ctypes.data))
        return tuple(int(v) for v in s)


def bi_version() -> int:
    return lib.bi_version()
