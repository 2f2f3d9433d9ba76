"""End-to-end determinism of the engine on the Gemma-3-4B-shaped decoder
(Definition 2.1, Vosti deep-dive blog §2): for requests with the same prompt
and the same (greedy) sampler, the per-request views — every sampled token and
the bits of the logits row it was sampled from — must agree across executions
that differ in arrival order, batch composition, chunk budget, page pool,
prefix-cache hits and evictions.  Also: greedy sampling against the oracle.
"""
import numpy as np
import pytest
import torch

import deterministic_paged_attention_amd as bi
import oracle
import synth
from deterministic_paged_attention_amd.decoder import Decoder, DecoderShape
from deterministic_paged_attention_amd.engine import Engine
from synth.workloads import decoder_weights

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_argmax_parity_ties_nan_and_full_vocab():
    x = torch.tensor([[1.0, 3.0, 3.0, -1.0],
                      [float("nan"), float("-inf"), float("-inf"), float("nan")],
                      [float("nan")] * 4,
                      [-5.0, float("inf"), 2.0, float("inf")]], device=DEV)
    assert bi.bi_argmax(x).cpu().tolist() == oracle.argmax_ref(x.cpu().numpy()).tolist() == [1, 1, 0, 1]
    g = torch.Generator(device=DEV)
    g.manual_seed(91)
    big = torch.randn((37, 262144), generator=g, device=DEV)
    big[5, 1000] = big[5, 77] = big[5].max() + 1.0          # a tie: the first index wins
    got = bi.bi_argmax(big).cpu().numpy()
    ref = oracle.argmax_ref(big.cpu().numpy())
    assert np.array_equal(got, ref)
    assert got[5] == 77
    sub = big[:, :100003]                                   # strided rows, odd length
    assert np.array_equal(bi.bi_argmax(sub).cpu().numpy(), oracle.argmax_ref(sub.cpu().numpy()))
    # rows starting off a 16-byte boundary (scalar head), short rows, ties across the
    # head / vector body / scalar tail boundaries
    for start, n in [(1, 100003), (3, 262141), (2, 1), (1, 2), (3, 5), (1, 8195), (2, 65536 + 7)]:
        v = big[:12, start:start + n]
        if n >= 8:
            v[7, n - 1] = v[7, 0] = v[7].max() + 2.0         # first (head) and last (tail) tie
        got = bi.bi_argmax(v).cpu().numpy()
        assert np.array_equal(got, oracle.argmax_ref(v.cpu().numpy())), (start, n)
        if n >= 8:
            assert got[7] == 0
    big[9, :] = float("-inf")
    big[9, 123456] = float("nan")
    got = bi.bi_argmax(big[:12]).cpu().numpy()
    assert got[9] == 0 and np.array_equal(got, oracle.argmax_ref(big[:12].cpu().numpy()))


@pytest.fixture(scope="module")
def decoder():
    s = DecoderShape()
    w = decoder_weights(s.layers, s.hidden, s.q_heads, s.kv_heads, s.head_dim, s.ffn, s.vocab, seed=7000)
    torch.cuda.synchronize()
    return Decoder(s, w)


def _prompts():
    V = DecoderShape().vocab
    system = synth.uniform_ints(80, 0, V - 1, 201)          # 5 full pages shared by requests 0-4
    p = {}
    for i, n in enumerate([40, 150, 7, 260, 96]):
        p[i] = system + synth.uniform_ints(n, 0, V - 1, 210 + i)
    p[5] = list(p[1])                                       # an exact duplicate of request 1
    p[6] = synth.uniform_ints(333, 0, V - 1, 230)
    p[7] = synth.uniform_ints(16, 0, V - 1, 231)            # exactly one page
    return p


def _arrivals(order, gaps, prompts, max_new):
    out, s = {}, 0
    for rid, gap in zip(order, gaps):
        s += gap
        out.setdefault(s, []).append((rid, prompts[rid], max_new))
    return out


def test_per_request_views_agree_across_schedules_pools_and_cache_hits(decoder):
    prompts = _prompts()
    max_new = 6
    runs = {}
    # A: staggered arrivals (later requests hit the cached system prefix), budget 256
    eA = Engine(decoder, num_pages=600, budget=256)
    runs["A"] = eA.run(arrivals=_arrivals([0, 6, 1, 2, 3, 7, 4, 5], [0, 0, 4, 0, 0, 0, 5, 0], prompts, max_new))
    # B: reversed order, small budget (many chunks, mixed prefill/decode steps), another pool size
    eB = Engine(decoder, num_pages=450, budget=48)
    runs["B"] = eB.run(arrivals=_arrivals([5, 4, 7, 3, 2, 6, 1, 0], [0, 2, 0, 3, 1, 0, 6, 2], prompts, max_new))
    # C: one request at a time on a pool so small that cached pages must be evicted
    eC = Engine(decoder, num_pages=40, budget=512)
    runs["C"] = eC.run(arrivals=_arrivals([2, 0, 3, 1, 4, 5, 6, 7], [0, 8, 8, 8, 8, 8, 8, 8], prompts, max_new))
    # E: as A, with decode steps replayed from captured HIP graphs (many replays per graph,
    # eager prefill steps between them)
    eE = Engine(decoder, num_pages=600, budget=256, graphs=True)
    runs["E"] = eE.run(arrivals=_arrivals([0, 6, 1, 2, 3, 7, 4, 5], [0, 0, 4, 0, 0, 0, 5, 0], prompts, max_new))
    assert len(eE._graphs) >= 1 and eE.graph_replays >= 3
    # D: every request alone, no sharing possible (fresh engine each)
    runs["D"] = {}
    for rid in prompts:
        e = Engine(decoder, num_pages=40, budget=100)
        runs["D"].update(e.run(arrivals={0: [(rid, prompts[rid], max_new)]}))

    for name, fin in runs.items():
        assert sorted(fin) == sorted(prompts), name
        for rid, r in fin.items():
            assert len(r.tokens) == max_new, (name, rid)
    ref = runs["D"]
    for name in ("A", "B", "C", "E"):
        for rid in prompts:
            assert runs[name][rid].view() == ref[rid].view(), (name, rid)
    for name in runs:
        assert runs[name][5].view() == runs[name][1].view(), name     # same prompt, same sampler
    # the variants really differed: prefix hits in A and B, evictions in C
    assert sum(r.reused_pages for r in runs["A"].values()) >= 5
    assert sum(r.reused_pages for r in runs["B"].values()) >= 5
    assert eC.cache.stats()[3] > 0
    assert eA.steps != eB.steps
