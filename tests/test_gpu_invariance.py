"""Bitwise invariance harness (GPU vs GPU).

The same requests (Q/K/V a function of request seed and position only) are run
under execution variants; every (request, position) row produced by more than
one variant must be bit-identical.  Variant classes follow the evaluation of
the Vosti deep-dive blog (深入解析 Vosti), §7.1 (batch composition, chunked
prefill, prefill vs decode, prefix reuse) and the failure modes of §4
(batch-wide specialisation, page-table width, prefill/decode algorithm split,
query partitioning that visits different fully masked tiles).  A passing run
is evidence, not proof (§4, scope note).

Positive control: the split-K comparators, whose split count follows the
batch, must show mismatches under the same variants — otherwise the harness
could not see a violation.
"""
import numpy as np
import pytest
import torch

import deterministic_paged_attention_amd as bi
import synth
from harness import DEV, PagedKV, Request, first_mismatch, run_step

pytestmark = pytest.mark.gpu

LLAMA = synth.Geometry(32, 8, 128, 16)
GEMMA = synth.Geometry(8, 4, 256, 16)


def _pool(geom, n, seed, lo, hi, prefix=None):
    lens = synth.uniform_ints(n, lo, hi, seed)
    reqs = {}
    for i, L in enumerate(lens):
        if prefix:
            reqs[i] = Request(seed * 1000 + i, prefix + L, geom, prefix_seed=seed * 1000 + 999, prefix_len=prefix)
        else:
            reqs[i] = Request(seed * 1000 + i, L, geom)
    return reqs


def _pages_for(reqs, slack=40):
    return sum(synth.pages_needed(r.length, 16) for r in reqs.values()) + slack


def _assert_same(a: dict, b: dict, what: str):
    common = sorted(set(a) & set(b))
    assert common, f"{what}: no common rows"
    for k in common:
        mm = first_mismatch(a[k], b[k])
        assert mm is None, f"{what}: row {k} differs: {mm}"
    return len(common)


def _decode_last(cfg, reqs, groups, page_seed, stride_extra=0, table_fill=-1, splitk=None):
    """Fill every request up to its last position, then decode that position,
    with the requests grouped into batches as given."""
    kv = PagedKV(cfg, _pages_for(reqs), page_seed)
    for g in groups:
        run_step(kv, reqs, [(i, reqs[i].length - 1) for i in g], attention=False)
    out = {}
    for g in groups:
        ns = None
        if splitk is not None:
            ns = bi.bi_splitk_attention_heuristic(cfg, len(g), max(reqs[i].length for i in g), 256, 8)
        out.update(run_step(kv, reqs, [(i, 1) for i in g], stride_extra=stride_extra, table_fill=table_fill,
                            splitk=ns))
    return out


# ---------------------------------------------------------------- batch composition + physical layout

def test_decode_batch_composition_order_and_page_layout():
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    reqs = _pool(LLAMA, 24, seed=31, lo=100, hi=3000)
    ids = list(range(24))
    ref = _decode_last(cfg, reqs, [[i] for i in ids], page_seed=1)              # each request alone
    variants = {
        "one batch": ([ids], 2, 0, -1),
        "one batch reversed, wide table, garbage fill": ([ids[::-1]], 3, 7, 123456),
        "batches of 4": ([ids[i:i + 4] for i in range(0, 24, 4)], 4, 0, -1),
        "random groups": ([[5, 17, 2], [0, 23, 11, 8, 9, 1], [3, 4, 6, 7, 10, 12, 13, 14, 15, 16, 18, 19, 20, 21,
                                                              22]], 5, 1, 0),
    }
    for name, (groups, pseed, sx, fill) in variants.items():
        got = _decode_last(cfg, reqs, groups, page_seed=pseed, stride_extra=sx, table_fill=fill)
        assert _assert_same(ref, got, name) == 24


def test_plan_in_lds_and_in_workspace_agree():
    """Above 2048 sequences the split phase reads its work plan from the
    workspace (written by a separate launch); below, each workgroup builds it
    in LDS.  The same decode rows through both paths are bitwise equal."""
    geom = synth.Geometry(4, 2, 64, 16)
    cfg = bi.AttnConfig(4, 2, 64, split_size=32)
    n = 2100
    reqs = _pool(geom, n, seed=41, lo=1, hi=90)
    ids = list(range(n))
    ref = _decode_last(cfg, reqs, [ids[i:i + 700] for i in range(0, n, 700)], page_seed=3)
    got = _decode_last(cfg, reqs, [ids[::-1]], page_seed=4)
    assert _assert_same(ref, got, "plan in workspace vs in LDS") == n


def test_decode_mixed_short_and_long_contexts_under_window():
    """Window 1024 with contexts below and above it in one batch (a batch-wide
    K-length bound must not change any row)."""
    cfg = bi.AttnConfig(8, 4, 256, split_size=256, window=1024)
    lens = [300, 1024, 1025, 2500, 40, 4000]
    reqs = {i: Request(70 + i, L, GEMMA) for i, L in enumerate(lens)}
    ref = _decode_last(cfg, reqs, [[i] for i in range(6)], page_seed=1)
    got = _decode_last(cfg, reqs, [[5, 0, 3, 1, 4, 2]], page_seed=9, stride_extra=2)
    _assert_same(ref, got, "mixed window batch")


# ---------------------------------------------------------------- prefill vs decode, chunk budgets

def _run_schedule(cfg, reqs, schedule, page_seed, stride_extra=0):
    kv = PagedKV(cfg, _pages_for(reqs), page_seed)
    out = {}
    for step in schedule:
        out.update(run_step(kv, reqs, step, stride_extra=stride_extra))
    return out


def _chunked(reqs, budget, offset=0):
    """Per-request chunk lists, interleaved across requests step by step."""
    per = {i: synth.chunk_schedule(r.length, budget, offset) for i, r in reqs.items()}
    steps = []
    k = 0
    while any(k < len(v) for v in per.values()):
        steps.append([(i, v[k]) for i, v in per.items() if k < len(v)])
        k += 1
    return steps


@pytest.mark.parametrize("geom,window", [(LLAMA, 0), (GEMMA, 1024)])
def test_prefill_chunks_and_token_by_token_agree(geom, window):
    cfg = bi.AttnConfig(geom.num_q_heads, geom.num_kv_heads, geom.head_dim, split_size=256, window=window)
    lens = [700, 1300] if window == 0 else [1300, 600]
    reqs = {i: Request(500 + i + window, L, geom) for i, L in enumerate(lens)}
    if geom is LLAMA:
        # the one-shot prefill runs workgroup-shared tiles (eight blocks per item), token by
        # token runs one-block items: the comparison below is then also a cross-mapping check
        assert bi.bi_paged_attention_item_blocks(cfg, 2, sum(lens), max(lens)) == 8
        assert bi.bi_paged_attention_item_blocks(cfg, 2, 2, max(lens)) == 1
    one_shot = _run_schedule(cfg, reqs, [[(i, r.length) for i, r in reqs.items()]], page_seed=3)
    assert len(one_shot) == sum(lens)
    for budget, offset, pseed in [(16, 0, 4), (128, 37, 5), (512, 5, 6), (1, 0, 7)]:
        sched = _chunked(reqs, budget, offset)
        got = _run_schedule(cfg, reqs, sched, page_seed=pseed, stride_extra=budget % 3)
        n = _assert_same(one_shot, got, f"budget {budget} offset {offset}")
        assert n == sum(lens)


def test_wide_and_shared_items_agree_with_one_block_items():
    """48 requests prefilled in 40-token chunks through four-block wide items
    (forced: the launcher takes shared tiles wherever both apply), in 24-token
    chunks (six query blocks, padded into eight-block shared-tile items), in one
    shot (shared-tile items) and token by token (one-block items): every row
    bitwise equal."""
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    reqs = _pool(LLAMA, 48, seed=61, lo=520, hi=700)
    assert bi.bi_paged_attention_item_blocks(cfg, 48, 24 * 48, 700) == 8
    T = sum(r.length for r in reqs.values())
    assert bi.bi_paged_attention_item_blocks(cfg, 48, T, 700) == 8
    one_shot = _run_schedule(cfg, reqs, [[(i, r.length) for i, r in reqs.items()]], page_seed=8)
    bi.bi_paged_attention_force_mapping(4)
    try:
        assert bi.bi_paged_attention_item_blocks(cfg, 48, 40 * 48, 700) == 4
        chunked = _run_schedule(cfg, reqs, _chunked(reqs, 40), page_seed=9)
    finally:
        bi.bi_paged_attention_force_mapping(0)
    assert _assert_same(one_shot, chunked, "40-token chunks (wide items) vs one shot") == T
    chunked = _run_schedule(cfg, reqs, _chunked(reqs, 24), page_seed=13)
    assert _assert_same(one_shot, chunked, "24-token chunks vs one shot") == T
    sample = {i: reqs[i] for i in (0, 17, 47)}
    by_token = _run_schedule(cfg, sample, _chunked(sample, 1), page_seed=10)
    assert _assert_same(one_shot, by_token, "token by token vs one shot") == sum(r.length for r in sample.values())


def test_shared_items_head_dim_64_agree_with_one_block_items():
    """Head dim 64 (GQA group 2): one-shot prefill on the shared-tile kernel against the same
    rows token by token, bitwise."""
    geom = synth.Geometry(4, 2, 64, 16)
    cfg = bi.AttnConfig(4, 2, 64, split_size=256)
    reqs = _pool(geom, 48, seed=71, lo=560, hi=640)
    T = sum(r.length for r in reqs.values())
    assert bi.bi_paged_attention_item_blocks(cfg, 48, T, 640) == 8
    one_shot = _run_schedule(cfg, reqs, [[(i, r.length) for i, r in reqs.items()]], page_seed=11)
    sample = {i: reqs[i] for i in (0, 9, 47)}
    by_token = _run_schedule(cfg, sample, _chunked(sample, 1), page_seed=12)
    assert _assert_same(one_shot, by_token, "token by token vs one shot") == sum(r.length for r in sample.values())


def test_continuous_batching_mixed_prefill_and_decode_steps():
    """One request decodes token by token while others prefill in chunks in the
    same steps; compare with each request run alone in one shot."""
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    reqs = {0: Request(811, 900, LLAMA), 1: Request(812, 333, LLAMA), 2: Request(813, 600, LLAMA)}
    alone = {}
    for i in reqs:
        alone.update(_run_schedule(cfg, {i: reqs[i]}, [[(i, reqs[i].length)]], page_seed=10 + i))
    kv = PagedKV(cfg, _pages_for(reqs), 77)
    got = {}
    got.update(run_step(kv, reqs, [(0, 500)]))
    while any(kv.lens.get(i, 0) < reqs[i].length for i in reqs):
        batch = []
        for i, n in ((2, 97), (0, 1), (1, 64)):
            rem = reqs[i].length - kv.lens.get(i, 0)
            if rem > 0:
                batch.append((i, min(n, rem)))
        got.update(run_step(kv, reqs, batch))
    assert _assert_same(alone, got, "continuous batching") == sum(r.length for r in reqs.values())


# ---------------------------------------------------------------- prefix reuse

def test_shared_private_and_recomputed_prefix():
    """4 requests share a 1024-token prefix (64 full pages) plus a unique suffix."""
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    P = 1024
    reqs = _pool(LLAMA, 4, seed=41, lo=256, hi=700, prefix=P)
    # (a) private: each request writes its own copy of the prefix, one shot
    private = _run_schedule(cfg, reqs, [[(i, r.length) for i, r in reqs.items()]], page_seed=1)
    # (b) shared: request 0 prefills the prefix; the others start on its pages
    kv = PagedKV(cfg, _pages_for(reqs), 2)
    shared = run_step(kv, reqs, [(0, P)])
    for i in (1, 2, 3):
        kv.share(i, kv.tables[0][: P // 16], P)
    for step in _chunked({i: reqs[i] for i in reqs}, 128, 0):
        batch = []
        for i, n in step:
            rem = reqs[i].length - kv.lens[i]
            if rem > 0:
                batch.append((i, min(n, rem)))
        if batch:
            shared.update(run_step(kv, reqs, batch))
    # (c) recomputed: the prefix is rebuilt into fresh pages with another chunking, then decoded token by token
    kv2 = PagedKV(cfg, _pages_for(reqs), 3)
    recomputed = {}
    for step in _chunked({i: reqs[i] for i in reqs}, 512, 100):
        batch = [(i, min(n, P - kv2.lens.get(i, 0))) for i, n in step if kv2.lens.get(i, 0) < P]
        if batch:
            recomputed.update(run_step(kv2, reqs, batch))
    for i in reqs:
        while kv2.lens[i] < reqs[i].length:
            recomputed.update(run_step(kv2, reqs, [(i, 1)]))
    n1 = _assert_same(private, shared, "private vs shared prefix")
    n2 = _assert_same(private, recomputed, "private vs recomputed prefix")
    assert n1 >= sum(r.length - P for r in reqs.values())
    assert n2 == sum(r.length for r in reqs.values())
    finals = [(i, r.length - 1) for i, r in reqs.items()]
    assert all(k in shared and k in recomputed for k in finals)


def test_generated_prefix_reuse():
    """A request's first 800 tokens (prompt + 'generated' tail) become the prefix
    of a second request that diverges afterwards."""
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    a = Request(901, 1200, LLAMA)
    b = Request(902, 1500, LLAMA, prefix_seed=901, prefix_len=800)
    reqs = {0: a, 1: b}
    kv = PagedKV(cfg, 300, 5)
    out = run_step(kv, reqs, [(0, 800)])
    kv.share(1, kv.tables[0][:50], 800)
    out.update(run_step(kv, reqs, [(0, 400), (1, 700)]))
    alone_b = _run_schedule(cfg, {1: b}, [[(1, 1500)]], page_seed=8)
    alone_a = _run_schedule(cfg, {0: a}, [[(0, 1200)]], page_seed=9)
    _assert_same(alone_b, {k: v for k, v in out.items() if k[0] == 1}, "generated-prefix reuse (b)")
    _assert_same(alone_a, {k: v for k, v in out.items() if k[0] == 0}, "generated-prefix reuse (a)")


# ---------------------------------------------------------------- run to run

def test_run_to_run_identical():
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    from synth.workloads import build_decode_workload
    wl = build_decode_workload(32, 8, 128, batch=64, seed=2000)
    outs = [bi.bi_paged_attention(cfg, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.qsl,
                                  wl.max_seq_len) for _ in range(3)]
    for o in outs[1:]:
        assert first_mismatch(outs[0], o) is None


# ---------------------------------------------------------------- RMSNorm + GEMM rows vs M

@pytest.mark.parametrize("N,out_dtype", [(14336, torch.bfloat16), (8192, torch.float32), (128256, torch.float32)])
def test_rmsnorm_gemm_rows_independent_of_M(N, out_dtype):
    """Each M (1, 7, 64, 256, 1024) selects another kernel or tile bracket at
    these widths, including the 128256-wide fp32 logits: every sampled row
    equals that row computed alone, also with the rows permuted."""
    H = 4096
    x = synth.normal_bf16_device((1024, H), 601)
    g = synth.normal_bf16_device((H,), 602, std=0.1, mean=1.0)
    w = synth.normal_bf16_device((N, H), 603, std=0.02)
    single = {}
    rows = [0, 5, 63, 255, 1023]
    for r in rows:
        y1 = bi.bi_rmsnorm(x[r:r + 1], g, 1e-5)
        single[r] = (y1, bi.bi_gemm(y1, w, out_dtype=out_dtype))
    for M in (7, 64, 256, 1024):
        perm = torch.tensor(synth.permutation(M, 600 + M), device=DEV)
        for order in (None, perm):
            xs = x[:M] if order is None else x[:M][order]
            y = bi.bi_rmsnorm(xs, g, 1e-5)
            c = bi.bi_gemm(y, w, out_dtype=out_dtype)
            for r in rows:
                if r >= M:
                    continue
                pos = r if order is None else int((order == r).nonzero()[0])
                assert first_mismatch(y[pos:pos + 1], single[r][0]) is None, (M, r)
                assert first_mismatch(c[pos:pos + 1], single[r][1]) is None, (M, r)


@pytest.mark.parametrize("N,K", [(20480, 2560), (2560, 10240), (2560, 2048), (4096, 2560)])
def test_decoder_projection_rows_independent_of_M(N, K):
    """The Gemma-shaped projections, whose tile configuration changes with M
    (skinny, 32 x 80, 64 x 64, 128 x 160, 256 x 128 ...): every row of every M
    equals that row computed alone, bit for bit."""
    a = synth.normal_bf16_device((512, K), 611 + N % 97)
    w = synth.normal_bf16_device((N, K), 612 + N % 89, std=0.02)
    rows = [0, 3, 130, 255, 511]
    single = {r: bi.bi_gemm(a[r:r + 1], w) for r in rows}
    for M in (4, 16, 129, 200, 256, 300, 512):
        c = bi.bi_gemm(a[:M], w)
        for r in rows:
            if r < M:
                assert first_mismatch(c[r:r + 1], single[r]) is None, (N, K, M, r)


# ---------------------------------------------------------------- positive controls

def test_positive_control_splitk_attention_varies_with_batch():
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    reqs = _pool(LLAMA, 16, seed=51, lo=1500, hi=4000)
    ids = list(range(16))
    alone = _decode_last(cfg, reqs, [[i] for i in ids], page_seed=1, splitk=True)
    batched = _decode_last(cfg, reqs, [ids], page_seed=1, splitk=True)
    diffs = sum(first_mismatch(alone[k], batched[k]) is not None for k in alone)
    assert diffs > 0, "split-K comparator showed no batch dependence: the harness would be blind"
    inv_alone = _decode_last(cfg, reqs, [[i] for i in ids], page_seed=1)
    inv_batched = _decode_last(cfg, reqs, [ids], page_seed=1)
    assert _assert_same(inv_alone, inv_batched, "invariant path") == 16


def test_positive_control_splitk_gemm_varies_with_M():
    x = synth.normal_bf16_device((256, 4096), 611)
    w = synth.normal_bf16_device((2048, 4096), 612, std=0.02)
    c1 = bi.bi_gemm_splitk(x[:1], w, bi.bi_gemm_splitk_heuristic(1), out_dtype=torch.float32)
    c256 = bi.bi_gemm_splitk(x, w, bi.bi_gemm_splitk_heuristic(256), out_dtype=torch.float32)
    assert first_mismatch(c1, c256[:1]) is not None
    i1 = bi.bi_gemm(x[:1], w, out_dtype=torch.float32)
    i256 = bi.bi_gemm(x, w, out_dtype=torch.float32)
    assert first_mismatch(i1, i256[:1]) is None
