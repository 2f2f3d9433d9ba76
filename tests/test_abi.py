"""C-ABI tests that need no GPU: the library loads, exports every declared
symbol, rejects unsupported configurations and bad arguments before any
launch, and the host-side plan checkers return the documented statuses."""
import ctypes

import numpy as np
import pytest

import deterministic_paged_attention_amd as bi


def test_exports_every_declared_symbol():
    names = bi.declared_functions()
    assert len(names) >= 20
    missing = [n for n in names if not hasattr(bi.lib, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert bi.bi_version() == 100
    for code, name in bi.STATUS_NAMES.items():
        assert bi.lib.bi_status_string(code).decode() == name


@pytest.mark.parametrize("geom,status", [
    (dict(num_q_heads=32, num_kv_heads=8, head_dim=128), 0),
    (dict(num_q_heads=8, num_kv_heads=4, head_dim=256, window=1024), 0),
    (dict(num_q_heads=4, num_kv_heads=2, head_dim=64, split_size=32), 0),
    (dict(num_q_heads=12, num_kv_heads=4, head_dim=128), 2),      # G = 3
    (dict(num_q_heads=64, num_kv_heads=2, head_dim=128), 2),      # G = 32
    (dict(num_q_heads=32, num_kv_heads=8, head_dim=96), 2),       # D = 96
    (dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=32), 2),
    (dict(num_q_heads=32, num_kv_heads=8, head_dim=128, split_size=48), 2),
    (dict(num_q_heads=30, num_kv_heads=8, head_dim=128), 1),      # not a multiple
    (dict(num_q_heads=32, num_kv_heads=8, head_dim=128, window=-1), 1),
    (dict(num_q_heads=0, num_kv_heads=8, head_dim=128), 1),
])
def test_config_create(geom, status):
    if status == 0:
        cfg = bi.AttnConfig(**geom)
        assert cfg.key_tile == 32
        assert cfg.scale == pytest.approx(1.0 / np.sqrt(geom["head_dim"]), rel=1e-7)
    else:
        with pytest.raises(bi.BiError) as e:
            bi.AttnConfig(**geom)
        assert e.value.status == status


def test_workspace_size_matches_documented_layout():
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    B, T, L = 3, 7, 1000
    ns = -(-L // 256)
    R = T * 32
    ml = R * ns * 8
    acc_end = (ml + 255) // 256 * 256 + R * ns * 128 * 2  # acc is bf16
    expect = (acc_end + 255) // 256 * 256 + (B + 1) * 4
    assert bi.bi_paged_attention_workspace_size(cfg, B, T, L) == expect
    assert bi.bi_kv_cache_bytes(cfg, 10) == 10 * 8 * 128 * 16 * 2


def test_splitk_heuristic_depends_on_batch():
    cfg = bi.AttnConfig(32, 8, 128)
    n1 = bi.bi_splitk_attention_heuristic(cfg, 1, 8192, 256, 8)
    n64 = bi.bi_splitk_attention_heuristic(cfg, 64, 8192, 256, 8)
    n256 = bi.bi_splitk_attention_heuristic(cfg, 256, 8192, 256, 8)
    assert n1 == 256 and n64 == 4 and n256 == 1
    assert bi.bi_splitk_attention_heuristic(cfg, 1, 100, 256, 8) == 4   # capped by ceil(100/32)
    assert [bi.bi_gemm_splitk_heuristic(m) for m in (1, 16, 17, 128, 129, 1024)] == [8, 8, 4, 4, 1, 1]


# ---------------------------------------------------------------- plan checkers

def test_check_page_table():
    pt = np.array([[3, 1, -1], [0, 2, 4]], dtype=np.int32)
    bi.bi_check_page_table(pt, [20, 48], [0, 1, 3], 16, 5)
    with pytest.raises(bi.BiError) as e:
        bi.bi_check_page_table(pt, [40, 48], [0, 1, 3], 16, 5)     # third entry of row 0 is -1
    assert e.value.status == 3
    with pytest.raises(bi.BiError) as e:
        bi.bi_check_page_table(pt, [20, 48], None, 16, 4)          # page 4 outside a 4-page pool
    assert e.value.status == 3
    with pytest.raises(bi.BiError) as e:
        bi.bi_check_page_table(pt, [20, 49], None, 16, 5)          # 4 pages needed, row holds 3
    assert e.value.status == 3
    with pytest.raises(bi.BiError) as e:
        bi.bi_check_page_table(pt, [20, 48], [0, 1, 50], 16, 5)    # q_len 49 > k_len 48
    assert e.value.status == 3


def test_check_write_plan():
    writable = np.array([1, 0, 1, 1], dtype=np.uint8)
    bi.bi_check_write_plan([0, 1, 33, 48, -1], writable, 4, 16)
    with pytest.raises(bi.BiError) as e:
        bi.bi_check_write_plan([0, 17], writable, 4, 16)           # page 1 is shared
    assert e.value.status == 4
    with pytest.raises(bi.BiError) as e:
        bi.bi_check_write_plan([5, 40, 5], writable, 4, 16)        # slot 5 twice
    assert e.value.status == 4
    with pytest.raises(bi.BiError) as e:
        bi.bi_check_write_plan([64], writable, 4, 16)              # outside the pool
    assert e.value.status == 3
    bi.bi_check_write_plan([], None, 4, 16)


# ---------------------------------------------------------------- argument validation (nothing launched)

FAKE = 0x10000  # aligned non-null stand-in; every call below is rejected before any HIP call


def _attn(cfg, **kw):
    a = dict(q=FAKE, qs=32 * 128, k=FAKE, v=FAKE, np=10, pt=FAKE, pts=4, sl=FAKE, qsl=FAKE, ns=2, nt=2,
             msl=64, ws=FAKE, wsb=1 << 30, out=FAKE)
    a.update(kw)
    return bi.lib.bi_paged_attention(cfg.handle, a["q"], a["qs"], a["k"], a["v"], a["np"], a["pt"], a["pts"],
                                     a["sl"], a["qsl"], a["ns"], a["nt"], a["msl"], a["ws"], a["wsb"], a["out"],
                                     None)


@pytest.mark.parametrize("kw,status", [
    (dict(ns=0), 1),
    (dict(nt=1, ns=2), 1),
    (dict(q=None), 1),
    (dict(qs=100), 1),
    (dict(q=FAKE + 8), 1),
    (dict(pts=3, msl=64), 3),      # 3 pages of 16 cannot hold 64 keys
    (dict(wsb=100), 5),
    (dict(np=0), 1),
    (dict(msl=0), 1),
])
def test_attention_rejects_bad_arguments(kw, status):
    cfg = bi.AttnConfig(32, 8, 128)
    assert _attn(cfg, **kw) == status
    assert bi.lib.bi_last_error_message().decode() != ""


def test_noalloc_attention_rejects_before_any_launch():
    """The allocation-free entry point refuses a call whose partials exceed its
    64 MiB device array (the 8B decode at 256 sequences of up to 8192 keys needs
    about 69 MB) and bad arguments, before touching the device."""
    cfg = bi.AttnConfig(32, 8, 128)
    L = bi.lib
    args = (cfg.handle, FAKE, 32 * 128, FAKE, FAKE, 10, FAKE, 512, FAKE, FAKE)
    assert bi.bi_paged_attention_workspace_size(cfg, 256, 256, 8192) > 64 << 20
    assert L.bi_paged_attention_noalloc(*args, 256, 256, 8192, FAKE, None) == 5
    assert "64" in bi.lib.bi_last_error_message().decode() or "67108864" in bi.lib.bi_last_error_message().decode()
    assert L.bi_paged_attention_noalloc(*args, 2, 2, 64, None, None) == 1            # no output
    assert L.bi_paged_attention_noalloc(*args, 0, 2, 64, FAKE, None) == 1            # no sequences
    assert L.bi_paged_attention_noalloc(cfg.handle, FAKE, 100, FAKE, FAKE, 10, FAKE, 512, FAKE, FAKE, 2, 2, 64, FAKE,
                                        None) == 1                                    # q row stride < H_q * D
    assert L.bi_paged_attention_noalloc(*args, 2, 0, 64, None, None) == 0             # no tokens: nothing to do


def test_other_entry_points_reject_bad_arguments():
    L = bi.lib
    assert L.bi_rmsnorm(FAKE, 4096, FAKE, 1e-5, 4, 4100, FAKE, 4096, None) == 1      # H not multiple of 8
    assert L.bi_rmsnorm(FAKE, 4000, FAKE, 1e-5, 4, 4096, FAKE, 4096, None) == 1      # ld < H
    assert L.bi_rmsnorm(FAKE, 4096, FAKE, -1.0, 4, 4096, FAKE, 4096, None) == 1      # eps < 0
    assert L.bi_rmsnorm(None, 4096, None, 1e-5, 0, 4096, None, 4096, None) == 0      # M = 0: nothing to do
    assert L.bi_add_rmsnorm(FAKE, 4096, FAKE, 4096, FAKE, 4096, FAKE, 1e-5, 4, 4100, FAKE, 4096, None) == 1
    assert L.bi_add_rmsnorm(FAKE, 4096, FAKE, 4000, FAKE, 4096, FAKE, 1e-5, 4, 4096, FAKE, 4096, None) == 1
    assert L.bi_add_rmsnorm(FAKE, 4096, FAKE, 4096, FAKE, 4096, FAKE, -1.0, 4, 4096, FAKE, 4096, None) == 1
    assert L.bi_add_rmsnorm(None, 4096, None, 4096, None, 4096, None, 1e-5, 0, 4096, None, 4096, None) == 0
    assert L.bi_gemm(None, 4096, None, 4096, None, 14336, 0, 0, 14336, 4096, None) == 0   # M = 0: nothing to do
    assert L.bi_gemm(None, 4096, None, 4096, None, 0, 1, 5, 0, 4096, None) == 0           # N = 0: nothing to do
    assert L.bi_gemm(FAKE, 4096, FAKE, 4096, FAKE, 14336, 0, 4, 14336, 4010, None) == 1   # K % 32
    assert L.bi_gemm(FAKE, 4096, FAKE, 4096, FAKE, 14336, 7, 4, 14336, 4096, None) == 1   # dtype
    assert L.bi_gemm(FAKE, 100, FAKE, 4096, FAKE, 14336, 0, 4, 14336, 4096, None) == 1    # lda < K
    assert L.bi_gemm(FAKE, 1 << 23, FAKE, 4096, FAKE, 14336, 0, 4, 14336, 4096, None) == 3  # lda too large
    assert L.bi_gemm_gated_gelu(FAKE, 2560, FAKE, 2560, FAKE, 10240, 17, 10240, 2560, None) == 2   # M > 16
    assert L.bi_gemm_gated_gelu(FAKE, 2560, FAKE, 2560, FAKE, 100, 4, 10240, 2560, None) == 1      # ldo < ffn
    assert L.bi_gemm_gated_gelu(FAKE, 2560, FAKE, 2560, FAKE, 10240, 4, 10240, 2550, None) == 1    # K % 32
    assert L.bi_gemm_gated_gelu(None, 2560, None, 2560, None, 10240, 0, 10240, 2560, None) == 0    # M = 0
    assert L.bi_gemm_splitk(FAKE, 4096, FAKE, 4096, FAKE, 256, 0, 4, 256, 4096, 3, FAKE, 1 << 30, None) == 1
    assert L.bi_gemm_splitk(FAKE, 4096, FAKE, 4096, FAKE, 256, 0, 4, 256, 4096, 4, FAKE, 16, None) == 5
    cfg = bi.AttnConfig(32, 8, 128)
    out = ctypes.c_int32(-1)
    assert L.bi_paged_attention_item_blocks(cfg.handle, 0, 16, 64, ctypes.byref(out)) == 1   # no sequences
    assert L.bi_paged_attention_item_blocks(cfg.handle, 1, 16, 64, None) == 1                # no result slot
    assert out.value == -1
    assert L.bi_paged_attention_mapping(cfg.handle, 0, 16, 64, ctypes.byref(out)) == 1       # no sequences
    assert L.bi_paged_attention_mapping(cfg.handle, 4, 4, 64, None) == 1                    # no result slot
    assert out.value == -1
    for bad in (-1, 2, 3, 5, 16):
        assert L.bi_paged_attention_force_mapping(bad) == 1                                  # no such mapping
    assert L.bi_paged_attention_force_mapping(0) == 0
    assert L.bi_kv_write(cfg.handle, FAKE, 100, FAKE, 1024, FAKE, 3, FAKE, FAKE, 10, None) == 1
    assert L.bi_kv_write(cfg.handle, FAKE, 1024, FAKE, 1024, FAKE, 3, FAKE + 4, FAKE, 10, None) == 1
    assert L.bi_slot_mapping(FAKE, 4, FAKE, FAKE, 2, 3, 32, 10, FAKE, None) == 2      # page size 32
    assert L.bi_slot_mapping(FAKE, 4, FAKE, FAKE, 0, 3, 16, 10, FAKE, None) == 1
    assert L.bi_paged_attention_merge(cfg.handle, FAKE, FAKE, 2, 2, 64, FAKE, 16, FAKE, None) == 5
    assert L.bi_attn_config_create(None, None) == 1


def test_qk_norm_rope_kv_write_rejects_bad_arguments():
    cfg = bi.AttnConfig(8, 4, 256)
    L = bi.lib
    row = (8 + 2 * 4) * 256

    def call(**kw):
        a = dict(qkv=FAKE, rs=row, nt=3, sl=FAKE, qsl=FAKE, ns=1, gq=FAKE, gk=FAKE, eps=1e-6, theta=1e4, slots=FAKE,
                 k=FAKE, v=FAKE, np=4)
        a.update(kw)
        return L.bi_qk_norm_rope_kv_write(cfg.handle, a["qkv"], a["rs"], a["nt"], a["sl"], a["qsl"], a["ns"], a["gq"],
                                          a["gk"], a["eps"], a["theta"], a["slots"], a["k"], a["v"], a["np"], None)

    assert call(rs=row - 256) == 1             # the v part must fit in a row
    assert call(ns=0) == 1
    assert call(np=0) == 1
    assert call(eps=-1.0) == 1
    assert call(theta=1.0) == 1
    assert call(slots=None) == 1
    assert call(nt=0) == 0                     # nothing to do


def test_kv_write_paged_rejects_bad_arguments():
    cfg = bi.AttnConfig(32, 8, 128)
    L = bi.lib

    def call(**kw):
        a = dict(k=FAKE, ks=1024, v=FAKE, vs=1024, pt=FAKE, pts=4, sl=FAKE, qsl=FAKE, ns=2, nt=3, kc=FAKE, vc=FAKE,
                 np=10)
        a.update(kw)
        return L.bi_kv_write_paged(cfg.handle, a["k"], a["ks"], a["v"], a["vs"], a["pt"], a["pts"], a["sl"],
                                   a["qsl"], a["ns"], a["nt"], a["kc"], a["vc"], a["np"], None)

    assert call(ks=1000) == 1                 # row stride below H_kv * D
    assert call(pts=0) == 1
    assert call(ns=0) == 1
    assert call(np=0) == 1
    assert call(np=1 << 28) == 3              # slot index would overflow 32 bits
    assert call(pt=None) == 1
    assert call(k=FAKE + 8) == 1              # misaligned
    assert call(nt=0) == 0                    # nothing to do


def test_stream_read_rejects_bad_arguments_before_any_launch():
    """The streaming-read reference validates on the host: a size that is not
    a multiple of 16, a misaligned or NULL source, or a NULL sink launch nothing."""
    assert bi.lib.bi_bench_stream_read_sink_words() == 8192
    sink = ctypes.c_void_p(4096)          # never dereferenced on these paths
    assert bi.lib.bi_bench_stream_read(ctypes.c_void_p(4096), 24, sink, None) == 1
    assert bi.lib.bi_bench_stream_read(ctypes.c_void_p(4104), 32, sink, None) == 1
    assert bi.lib.bi_bench_stream_read(None, 32, sink, None) == 1
    assert bi.lib.bi_bench_stream_read(ctypes.c_void_p(4096), 32, None, None) == 1


def test_mfma_peak_rejects_bad_arguments_before_any_launch():
    flops = ctypes.c_int64(0)
    sink = ctypes.c_void_p(4096)          # never dereferenced on these paths
    assert bi.lib.bi_bench_mfma_peak_sink_words() == 8192
    for rounds in (0, 3, -4, 6):
        assert bi.lib.bi_bench_mfma_peak(1.0, rounds, sink, ctypes.byref(flops), None) == 1
    assert bi.lib.bi_bench_mfma_peak(1.0, 8, None, ctypes.byref(flops), None) == 1
    assert bi.lib.bi_bench_mfma_peak(1.0, 8, sink, None, None) == 1
