"""The workload configurations at their stated sizes (GPU).

* The headline 8B-shaped decode pool (256 requests, contexts U{512..8192}):
  every row bitwise equal whether its request runs alone, in batches of 8, 64
  or all 256, in any order, on relocated pages with wider page tables; and
  every one of the 256 rows against the oracle.
* The workgroup-shared (eight query blocks per item) and wide (four blocks)
  prefill mappings against the oracle, row by row.
* Chunked prefill with a shared 1024-token prefix: 8 requests with U{256..2048}
  unique tokens, per-step budgets 16 / 128 / 512 in request order, one-shot and
  token by token, shared and private prefix pages: every row produced by more
  than one schedule, the final positions included, bitwise equal.
* A length past the max_seq_len a call was sized for stays inside the
  workspace.

Variant classes follow the evaluation of the Vosti deep-dive blog
(深入解析 Vosti), §7.1 (batch composition, chunking, prefill vs decode,
prefix reuse); the fixed split size follows the record "Deterministic and
bit-exact inference" (field technical, Invariance).
"""
import numpy as np
import pytest
import torch

import deterministic_paged_attention_amd as bi
import oracle
import synth
from harness import DEV, PagedKV, Request, first_mismatch, oracle_rows, page_table_tensor, run_step

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2
LLAMA = synth.Geometry(32, 8, 128, 16)


def _max_err(gpu_rows, ref_rows):
    return max(float(np.max(np.abs(synth.to_f64(gpu_rows[k]) - ref_rows[k]))) for k in ref_rows)


def _assert_same(a: dict, b: dict, what: str):
    common = sorted(set(a) & set(b))
    assert common, f"{what}: no common rows"
    for k in common:
        mm = first_mismatch(a[k], b[k])
        assert mm is None, f"{what}: row {k} differs: {mm}"
    return len(common)


# ---------------------------------------------------------------- the headline decode pool

@pytest.fixture(scope="module")
def headline():
    from synth.workloads import build_decode_workload
    wl = build_decode_workload(32, 8, 128, batch=256, seed=2000)
    torch.cuda.synchronize()
    return wl


def _relocate(wl, seed):
    """The pool's pages moved to other physical pages: page p goes to pos[p] of a
    fresh pool (an exact copy), and the page lists are rewritten accordingly."""
    pos = synth.permutation(wl.num_pages, seed)
    idx = torch.tensor(pos, dtype=torch.long, device=DEV)
    k = torch.empty_like(wl.k_cache)
    k.index_copy_(0, idx, wl.k_cache)
    v = torch.empty_like(wl.v_cache)
    v.index_copy_(0, idx, wl.v_cache)
    return k, v, [[pos[p] for p in row] for row in wl.pages]


def _decode_group(cfg, wl, k, v, pages, ids, stride_extra=0, fill=-1):
    """One decode launch over the requests `ids` (in that order); {request: row}."""
    sel = torch.tensor(ids, dtype=torch.long, device=DEV)
    q = wl.q.index_select(0, sel).contiguous()
    lens = [wl.lengths[i] for i in ids]
    pt = page_table_tensor([pages[i] for i in ids], max(len(pages[i]) for i in ids) + stride_extra, fill).to(DEV)
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    qsl = torch.arange(len(ids) + 1, dtype=torch.int32, device=DEV)
    out = bi.bi_paged_attention(cfg, q, k, v, pt, sl, qsl, max(lens))
    return {i: out[j] for j, i in enumerate(ids)}


def test_headline_pool_rows_bitwise_across_batch_sizes(headline):
    """Batch 256 against batches of 64 and 8 (random compositions and orders),
    32 requests alone, and batch 256 reversed: relocated pages, page tables
    wider than needed with garbage past the used entries."""
    wl = headline
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    ids = list(range(256))
    ref = _decode_group(cfg, wl, wl.k_cache, wl.v_cache, wl.pages, ids)
    k2, v2, pages2 = _relocate(wl, 7001)
    n = _assert_same(ref, _decode_group(cfg, wl, k2, v2, pages2, ids[::-1], stride_extra=3, fill=10 ** 9),
                     "batch 256 reversed, relocated")
    assert n == 256
    perm = synth.permutation(256, 7002)
    for B, sx, fill in ((64, 1, -1), (8, 2, 123456)):
        got = {}
        for g in range(0, 256, B):
            got.update(_decode_group(cfg, wl, k2, v2, pages2, perm[g:g + B], stride_extra=sx, fill=fill))
        assert _assert_same(ref, got, f"batches of {B}") == 256
    del k2, v2
    # alone: the 16 longest, the 8 shortest and 8 others
    by_len = sorted(ids, key=lambda i: wl.lengths[i])
    alone_ids = by_len[-16:] + by_len[:8] + perm[:8]
    got = {}
    for i in dict.fromkeys(alone_ids):
        got.update(_decode_group(cfg, wl, wl.k_cache, wl.v_cache, wl.pages, [i], stride_extra=1, fill=-5))
    assert _assert_same(ref, got, "batch 1") >= 30


def test_headline_pool_every_row_against_the_oracle(headline):
    """All 256 rows of the batch-256 launch against the oracle (the launch the
    bench times)."""
    wl = headline
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    out = bi.bi_paged_attention(cfg, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.qsl,
                                wl.max_seq_len).cpu()
    q_all = synth.to_f64(wl.q.cpu())
    worst = 0.0
    for s in range(256):
        kk, vv, table, L = wl.host_sequence(s)
        ref = oracle.attention_ref(q_all[s:s + 1], kk, vv, table, [L], [0, 1], 8, 16)
        worst = max(worst, float(np.max(np.abs(synth.to_f64(out[s:s + 1]) - ref))))
    assert worst <= BF16_TOL, worst


# ---------------------------------------------------------------- row-group vs split mapping (cross-kernel)

def _phases(cfg, q, k, v, pt, sl, qsl, msl):
    """The split and merge phases as separate launches (always the split mapping)."""
    ws = bi.alloc_workspace(bi.bi_paged_attention_workspace_size(cfg, sl.shape[0], q.shape[0], msl))
    bi.bi_paged_attention_split(cfg, q, k, v, pt, sl, qsl, msl, ws)
    return bi.bi_paged_attention_merge(cfg, sl, qsl, q.shape[0], msl, ws)


@pytest.mark.parametrize("B,window", [(1, 0), (8, 0), (32, 0), (64, 0), (256, 0), (256, 1000)])
def test_row_group_mapping_matches_split_and_merge_bitwise(headline, B, window):
    """Decode batches of the headline pool: bi_paged_attention (the row-group
    mapping once a batch fills the GPU, the split mapping below) against the
    split and merge phases launched separately, every row bitwise."""
    wl = headline
    cfg = bi.AttnConfig(32, 8, 128, split_size=256, window=window)
    lens = wl.lengths[:B]
    q, pt, sl = wl.q[:B], wl.page_table[:B], wl.seq_lens[:B]
    qsl = torch.arange(B + 1, dtype=torch.int32, device=DEV)
    mapping = bi.bi_paged_attention_mapping(cfg, B, B, max(lens))
    if B >= 64:
        assert mapping == 1
    if B <= 8:
        assert mapping == 0
    got = bi.bi_paged_attention(cfg, q, wl.k_cache, wl.v_cache, pt, sl, qsl, max(lens))
    ref = _phases(cfg, q, wl.k_cache, wl.v_cache, pt, sl, qsl, max(lens))
    assert first_mismatch(got, ref) is None


@pytest.mark.parametrize("Hq,Hk,D,lo,hi,window", [(4, 2, 64, 17, 3000, 0), (32, 4, 128, 300, 4096, 0),
                                                  (8, 8, 128, 100, 2000, 0), (16, 1, 64, 50, 1500, 0),
                                                  (8, 4, 256, 512, 4096, 0), (8, 4, 256, 100, 20000, 1024)])
def test_row_group_mapping_other_head_geometries(Hq, Hk, D, lo, hi, window):
    """GQA groups of 2, 8, 1 and 16, head dims 64 and 256 (the Gemma-shaped
    layers: global, and local with a 1024 window over contexts up to 20000,
    more splits than the ring holds but a window that meets at most five): the
    row-group mapping against the separate phases bitwise, and the oracle on
    sampled rows."""
    cfg = bi.AttnConfig(Hq, Hk, D, split_size=256, window=window)
    B = max(1, 2048 // Hk) if Hk < 8 else 300
    B = min(B, 600 if hi <= 4096 else 256)
    lengths = synth.uniform_ints(B, lo, hi, 3000 + Hq + Hk + D)
    need = [synth.pages_needed(L, 16) for L in lengths]
    num_pages = sum(need) + 11
    perm = synth.permutation(num_pages, 3001)
    pages, cur = [], 0
    for n in need:
        pages.append(perm[cur:cur + n])
        cur += n
    k = synth.normal_bf16_device(cfg.k_cache_shape(num_pages), 3002)
    v = synth.normal_bf16_device(cfg.v_cache_shape(num_pages), 3003)
    q = synth.normal_bf16_device((B, Hq, D), 3004)
    pt = page_table_tensor(pages, max(need) + 1).to(DEV)
    sl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    qsl = torch.arange(B + 1, dtype=torch.int32, device=DEV)
    mapping = bi.bi_paged_attention_mapping(cfg, B, B, max(lengths))
    got = bi.bi_paged_attention(cfg, q, k, v, pt, sl, qsl, max(lengths))
    ref = _phases(cfg, q, k, v, pt, sl, qsl, max(lengths))
    assert first_mismatch(got, ref) is None, mapping
    if Hk in (2, 4, 8) and Hq // Hk <= 8:
        assert mapping == 1, (Hq, Hk, D)
    for s in (0, B // 2, B - 1):
        idx = torch.tensor(pages[s], dtype=torch.long, device=DEV)
        kk = k.index_select(0, idx).cpu().permute(0, 3, 1, 2, 4).reshape(len(pages[s]), 16, Hk, D)
        vv = v.index_select(0, idx).cpu().permute(0, 4, 1, 2, 5, 3).reshape(len(pages[s]), 16, Hk, D)
        ref_o = oracle.attention_ref(synth.to_f64(q[s:s + 1].cpu()), synth.to_f64(kk), synth.to_f64(vv),
                                     np.arange(len(pages[s]))[None, :], [lengths[s]], [0, 1], Hk, 16, window=window)
        assert float(np.max(np.abs(synth.to_f64(got[s:s + 1].cpu()) - ref_o))) <= BF16_TOL


def test_row_group_mapping_lengths_past_max_seq_len():
    """Lengths past max_seq_len in a batch the row-group mapping takes: rows are
    truncated at the workspace's splits exactly as the split mapping truncates
    them (bitwise), and a zero-length row is written as zeros."""
    geom = synth.Geometry(4, 2, 64, 16)
    cfg = bi.AttnConfig(4, 2, 64, split_size=32)
    B = 300
    lengths = synth.uniform_ints(B, 1, 200, 3100)
    need = [synth.pages_needed(L, 16) for L in lengths]
    num_pages = sum(need) + 3
    perm = synth.permutation(num_pages, 3101)
    pages, cur = [], 0
    for n in need:
        pages.append(perm[cur:cur + n])
        cur += n
    k = synth.normal_bf16_device(cfg.k_cache_shape(num_pages), 3102)
    v = synth.normal_bf16_device(cfg.v_cache_shape(num_pages), 3103)
    q = synth.normal_bf16_device((B, 4, 64), 3104)
    pt = page_table_tensor(pages, 13).to(DEV)
    dev_lens = list(lengths)
    dev_lens[7] = 0
    sl = torch.tensor(dev_lens, dtype=torch.int32, device=DEV)
    qsl = torch.arange(B + 1, dtype=torch.int32, device=DEV)
    msl = 96                                  # three splits of 32; many rows are longer
    assert bi.bi_paged_attention_mapping(cfg, B, B, msl) == 1
    got = bi.bi_paged_attention(cfg, q, k, v, pt, sl, qsl, msl)
    ref = _phases(cfg, q, k, v, pt, sl, qsl, msl)
    assert first_mismatch(got, ref) is None
    assert bool((got[7].float() == 0).all())


# ---------------------------------------------------------------- every split-phase mapping on one batch

def _random_batch(Hq, Hk, D, q_lens, k_lens, seed, window=0):
    """Queries of q_lens[s] tokens at the end of k_lens[s]-token sequences over
    a randomly permuted page pool (K/V ~ N(0,1)); returns the call arguments
    and the per-sequence page lists."""
    cfg = bi.AttnConfig(Hq, Hk, D, split_size=256, window=window)
    need = [synth.pages_needed(L, 16) for L in k_lens]
    num_pages = sum(need) + 7
    perm = synth.permutation(num_pages, seed)
    pages, cur = [], 0
    for n in need:
        pages.append(perm[cur:cur + n])
        cur += n
    T = sum(q_lens)
    k = synth.normal_bf16_device(cfg.k_cache_shape(num_pages), seed + 1)
    v = synth.normal_bf16_device(cfg.v_cache_shape(num_pages), seed + 2)
    q = synth.normal_bf16_device((T, Hq, D), seed + 3)
    pt = page_table_tensor(pages, max(need) + 2, fill=-3).to(DEV)
    sl = torch.tensor(k_lens, dtype=torch.int32, device=DEV)
    qsl = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32, device=DEV)
    return cfg, (q, k, v, pt, sl, qsl, max(k_lens)), pages


@pytest.mark.parametrize("Hq,Hk,D,B,lo,hi,window", [
    (32, 8, 128, 1, 8000, 8192, 0),        # the headline layer, one sequence
    (32, 8, 128, 8, 512, 1500, 0),
    (8, 4, 256, 4, 15000, 17000, 1024),    # Gemma-shaped local layer at the agentic batch
    (4, 2, 64, 16, 17, 3000, 0),
    (16, 1, 64, 3, 50, 1500, 100)])
def test_small_decode_batches_through_every_split_mapping(Hq, Hk, D, B, lo, hi, window):
    """Small decode batches forced through one-block, wide and shared-tile
    items (the last two exist at head_dim <= 128): every row bitwise equal to
    the launcher's own choice, and every row against the oracle."""
    k_lens = synth.uniform_ints(B, lo, hi, 3200 + B + D + window)
    cfg, args, pages = _random_batch(Hq, Hk, D, [1] * B, k_lens, 3210 + B + D, window)
    auto = bi.bi_paged_attention(cfg, *args)
    assert bi.bi_paged_attention_mapping(cfg, B, B, max(k_lens)) == 0
    for kind in ((1, 4, 8) if D <= 128 else (1,)):
        with bi.forced_mapping(kind):
            assert first_mismatch(bi.bi_paged_attention(cfg, *args), auto) is None, kind
    q = args[0]
    for s in range(B):
        idx = torch.tensor(pages[s], dtype=torch.long, device=DEV)
        kk = args[1].index_select(0, idx).cpu().permute(0, 3, 1, 2, 4).reshape(len(pages[s]), 16, Hk, D)
        vv = args[2].index_select(0, idx).cpu().permute(0, 4, 1, 2, 5, 3).reshape(len(pages[s]), 16, Hk, D)
        ref_o = oracle.attention_ref(synth.to_f64(q[s:s + 1].cpu()), synth.to_f64(kk), synth.to_f64(vv),
                                     np.arange(len(pages[s]))[None, :], [k_lens[s]], [0, 1], Hk, 16, window=window)
        assert float(np.max(np.abs(synth.to_f64(auto[s:s + 1].cpu()) - ref_o))) <= BF16_TOL, s


@pytest.mark.parametrize("D,window", [(128, 0), (64, 100), (256, 1024)])
def test_prefill_batch_through_every_split_mapping(D, window):
    """A mixed step (prefill chunks of 1..300 tokens and decode tokens) forced
    through each split-phase mapping: every row bitwise equal (and a forced
    mapping that does not exist at head_dim 256 is refused)."""
    Hq, Hk = (32, 8) if D == 128 else ((4, 2) if D == 64 else (8, 4))
    q_lens = [300, 1, 37, 1, 128, 5]
    k_lens = [900, 2100, 600, 45, 1400, 5]
    cfg, args, _ = _random_batch(Hq, Hk, D, q_lens, k_lens, 3300 + D, window)
    kinds = (1, 4, 8) if D <= 128 else (1,)
    outs = {}
    for kind in kinds:
        with bi.forced_mapping(kind):
            outs[kind] = bi.bi_paged_attention(cfg, *args)
    for kind in kinds:
        assert first_mismatch(outs[kind], outs[1]) is None, kind
    assert first_mismatch(bi.bi_paged_attention(cfg, *args), outs[1]) is None
    if D == 256:
        with bi.forced_mapping(8):
            with pytest.raises(bi.BiError):
                bi.bi_paged_attention(cfg, *args)


# ---------------------------------------------------------------- prefill mappings against the oracle

@pytest.mark.parametrize("window", [0, 100])
def test_shared_tile_items_against_the_oracle(window):
    """A prefill step the launcher maps to workgroup-shared tiles (eight query
    blocks per item): 300-token chunks at the end of four long requests."""
    cfg = bi.AttnConfig(32, 8, 128, split_size=256, window=window)
    lengths = [900, 1100, 700, 1300]
    reqs = {i: Request(1200 + i + window, L, LLAMA) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, sum(synth.pages_needed(L, 16) for L in lengths) + 9, seed=21)
    run_step(kv, reqs, [(i, L - 300) for i, L in enumerate(lengths)], attention=False)
    assert bi.bi_paged_attention_item_blocks(cfg, 4, 1200, max(lengths)) == 8
    out = run_step(kv, reqs, [(i, 300) for i in range(4)])
    assert len(out) == 1200
    ref = oracle_rows(reqs, list(out.keys()), LLAMA, window)
    assert _max_err(out, ref) <= BF16_TOL


def test_shared_tile_items_head_dim_64_against_the_oracle():
    geom = synth.Geometry(4, 2, 64, 16)
    cfg = bi.AttnConfig(4, 2, 64, split_size=256)
    lengths = synth.uniform_ints(48, 560, 640, 1301)
    reqs = {i: Request(1300 + i, L, geom) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, sum(synth.pages_needed(L, 16) for L in lengths) + 9, seed=22)
    assert bi.bi_paged_attention_item_blocks(cfg, 48, sum(lengths), max(lengths)) == 8
    out = run_step(kv, reqs, [(i, L) for i, L in enumerate(lengths)])
    # every row of three requests, and every request's last row
    keys = [k for k in out if k[0] in (0, 17, 47) or k[1] == lengths[k[0]] - 1]
    ref = oracle_rows(reqs, keys, geom, 0)
    assert _max_err(out, ref) <= BF16_TOL


def test_wide_items_against_the_oracle():
    """Four-block items (a mapping the launcher leaves to forced use: shared-tile
    items win wherever both apply) against the oracle: 40-token chunks at the
    end of 48 requests of 520..700 tokens."""
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    lengths = synth.uniform_ints(48, 520, 700, 1401)
    reqs = {i: Request(1400 + i, L, LLAMA) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, sum(synth.pages_needed(L, 16) for L in lengths) + 9, seed=23)
    run_step(kv, reqs, [(i, L - 40) for i, L in enumerate(lengths)], attention=False)
    assert bi.bi_paged_attention_item_blocks(cfg, 48, 40 * 48, max(lengths)) == 8
    bi.bi_paged_attention_force_mapping(4)
    try:
        assert bi.bi_paged_attention_item_blocks(cfg, 48, 40 * 48, max(lengths)) == 4
        out = run_step(kv, reqs, [(i, 40) for i in range(48)])
    finally:
        bi.bi_paged_attention_force_mapping(0)
    ref = oracle_rows(reqs, list(out.keys()), LLAMA, 0)
    assert _max_err(out, ref) <= BF16_TOL


# ---------------------------------------------------------------- chunked prefill with a shared prefix

PREFIX = 1024
DECODE_TAIL = 16


def _prefix_pool():
    unique = synth.uniform_ints(8, 256, 2048, 2060)
    return {i: Request(2061 + i, PREFIX + u, LLAMA, prefix_seed=2099, prefix_len=PREFIX) for i, u in enumerate(unique)}


def _schedule_run(cfg, reqs, budget, shared, page_seed, stride_extra=0, fill=-1):
    """Prompts (all but the last DECODE_TAIL tokens) under a per-step token
    budget taken in request order (budget None: every prompt whole in one step;
    budget 1: one token per live request per step), then DECODE_TAIL decode
    steps of every request.  Shared: request 0 computes the prefix alone first
    and the others start on its pages."""
    n = len(reqs)
    kv = PagedKV(cfg, sum(synth.pages_needed(r.length, 16) for r in reqs.values()) + 64, page_seed)
    out = {}

    def step(batch):
        out.update(run_step(kv, reqs, batch, stride_extra=stride_extra, table_fill=fill))

    if shared:
        while kv.lens.get(0, 0) < PREFIX:
            done = kv.lens.get(0, 0)
            step([(0, PREFIX - done if budget is None else min(budget, PREFIX - done))])
        for i in range(1, n):
            kv.share(i, kv.tables[0][: PREFIX // 16], PREFIX)
    prompt = {i: r.length - DECODE_TAIL for i, r in reqs.items()}
    while True:
        batch, left = [], budget
        for i in range(n):
            rem = prompt[i] - kv.lens.get(i, 0)
            if rem <= 0:
                continue
            if budget is None:
                batch.append((i, rem))
            elif budget == 1:
                batch.append((i, 1))
            elif left > 0:
                batch.append((i, min(left, rem)))
                left -= batch[-1][1]
        if not batch:
            break
        step(batch)
    for _ in range(DECODE_TAIL):
        step([(i, 1) for i in range(n)])
    return out


def test_prefix_sharing_schedules_at_full_size():
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    reqs = _prefix_pool()
    total = sum(r.length for r in reqs.values())
    ref = _schedule_run(cfg, reqs, None, shared=False, page_seed=1)            # private prefixes, one shot
    assert len(ref) == total
    finals = [(i, r.length - 1) for i, r in reqs.items()]
    variants = [("budget 16, shared", 16, True, 2, 0, -1), ("budget 128, shared", 128, True, 3, 2, 77777),
                ("budget 512, shared", 512, True, 4, 5, -1), ("token by token, private", 1, False, 5, 1, -1)]
    for name, budget, shared, pseed, sx, fill in variants:
        got = _schedule_run(cfg, reqs, budget, shared, pseed, sx, fill)
        n = _assert_same(ref, got, name)
        # shared schedules produce the prefix rows of request 0 only
        assert n == (total - (len(reqs) - 1) * PREFIX if shared else total), name
        assert all(k in got for k in finals), name


# ---------------------------------------------------------------- precondition violation stays in bounds

def test_length_past_max_seq_len_stays_inside_the_workspace():
    """max_seq_len is documented as an upper bound of every length; a device
    length past it (here 100 against 64) must still keep every partial store
    inside the workspace (the split phase caps each row at the workspace's
    splits, as the merge does), and rows within the bound are unaffected."""
    geom = synth.Geometry(4, 2, 64, 16)
    cfg = bi.AttnConfig(4, 2, 64, split_size=32)
    lengths = [100, 60]
    reqs = {i: Request(1500 + i, L, geom) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, 16, seed=24)
    run_step(kv, reqs, [(0, 100), (1, 60)], attention=False)
    pt = page_table_tensor([kv.tables[0], kv.tables[1]], 7).to(DEV)
    sl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    qsl = torch.tensor([0, 1, 2], dtype=torch.int32, device=DEV)
    q = torch.stack([reqs[0].q[99], reqs[1].q[59]]).to(DEV)
    need = bi.bi_paged_attention_workspace_size(cfg, 2, 2, 64)
    guard = 1 << 16
    buf = torch.full((need + guard,), 0xA5, dtype=torch.uint8, device=DEV)
    out = torch.empty((2, 4, 64), dtype=torch.bfloat16, device=DEV)
    lib = bi.lib
    args = bi._attn_common(cfg, q, kv.k, kv.v, pt, sl, qsl)
    bi._check(lib.bi_paged_attention(*args, 64, bi._ptr(buf), need, bi._ptr(out), bi._stream()))
    torch.cuda.synchronize()
    assert bool((buf[need:] == 0xA5).all()), "a store landed past the workspace"
    alone = bi.bi_paged_attention(cfg, q[1:], kv.k, kv.v, pt[1:], sl[1:], torch.tensor([0, 1], dtype=torch.int32,
                                                                                          device=DEV), 60)
    assert first_mismatch(out[1:], alone) is None
