"""The allocation-free paged attention entry point (GPU), through the C ABI.

bi_paged_attention_noalloc keeps the split partials in a device array inside
the library instead of a caller workspace; its output must be bitwise that of
bi_paged_attention on the same arguments.  Two calls in a row, the second
smaller (the array keeps the first call's contents), then a prefill-shaped
call, each against bi_paged_attention with a fresh workspace.
"""
import pytest
import torch

import deterministic_paged_attention_amd as bi
import synth
from harness import DEV, PagedKV, Request, first_mismatch, page_table_tensor, run_step

pytestmark = pytest.mark.gpu


def _both(cfg, q, k, v, pt, sl, qsl, msl):
    ref = bi.bi_paged_attention(cfg, q, k, v, pt, sl, qsl, msl)
    args = bi._attn_common(cfg, q, k, v, pt, sl, qsl)
    out = torch.full_like(ref, float("nan"))
    status = bi.lib.bi_paged_attention_noalloc(*args, msl, bi._ptr(out), bi._stream())
    assert status == 0, bi.lib.bi_last_error_message().decode()
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_matches_workspace_entry_point_on_consecutive_calls():
    from synth.workloads import build_decode_workload
    cfg = bi.AttnConfig(32, 8, 128, split_size=256)
    # call 1: 48 sequences of the 8B-shaped decode pool (contexts up to 8192)
    wl = build_decode_workload(32, 8, 128, batch=48, seed=2000)
    need = bi.bi_paged_attention_workspace_size(cfg, 48, 48, wl.max_seq_len)
    assert need <= 64 << 20
    ref, out = _both(cfg, wl.q, wl.k_cache, wl.v_cache, wl.page_table, wl.seq_lens, wl.qsl, wl.max_seq_len)
    assert first_mismatch(out, ref) is None
    # call 2: a smaller batch of shorter sequences, right after (the array still
    # holds call 1's partials)
    idx = torch.tensor([5, 1, 30], dtype=torch.long, device=DEV)
    lens = [min(wl.lengths[i], 700) for i in (5, 1, 30)]
    sl = torch.tensor(lens, dtype=torch.int32, device=DEV)
    qsl = torch.arange(4, dtype=torch.int32, device=DEV)
    pt = wl.page_table.index_select(0, idx).contiguous()
    q = wl.q.index_select(0, idx).contiguous()
    ref2, out2 = _both(cfg, q, wl.k_cache, wl.v_cache, pt, sl, qsl, max(lens))
    assert first_mismatch(out2, ref2) is None
    # the same through the Python binding
    out3 = bi.bi_paged_attention_noalloc(cfg, q, wl.k_cache, wl.v_cache, pt, sl, qsl, max(lens))
    assert first_mismatch(out3, ref2) is None


def test_noalloc_prefill_chunk_and_rejection():
    geom = synth.Geometry(8, 4, 256, 16)
    cfg = bi.AttnConfig(8, 4, 256, split_size=256, window=1024)
    lengths = [1500, 300]
    reqs = {i: Request(3100 + i, L, geom) for i, L in enumerate(lengths)}
    kv = PagedKV(cfg, 120, seed=31)
    run_step(kv, reqs, [(0, 1400), (1, 250)], attention=False)
    run_step(kv, reqs, [(0, 100), (1, 50)], attention=False)
    tabs = [kv.tables[0], kv.tables[1]]
    pt = page_table_tensor(tabs, max(len(t) for t in tabs)).to(DEV)
    sl = torch.tensor(lengths, dtype=torch.int32, device=DEV)
    qsl = torch.tensor([0, 100, 150], dtype=torch.int32, device=DEV)
    q = torch.cat([reqs[0].q[1400:1500], reqs[1].q[250:300]]).to(DEV)
    ref, out = _both(cfg, q, kv.k, kv.v, pt, sl, qsl, 1500)
    assert first_mismatch(out, ref) is None
    # a call needing more than the array holds is refused and writes nothing
    big = torch.full((2, 8, 256), 7.0, dtype=torch.bfloat16, device=DEV)
    assert bi.bi_paged_attention_workspace_size(cfg, 2, 150, 1 << 20) > 64 << 20
    ptw = page_table_tensor(tabs, (1 << 20) // 16).to(DEV)
    args = bi._attn_common(cfg, q, kv.k, kv.v, ptw, sl, qsl)
    assert bi.lib.bi_paged_attention_noalloc(*args, 1 << 20, bi._ptr(big), bi._stream()) == 5
    torch.cuda.synchronize()
    assert bool((big.float() == 7.0).all())
