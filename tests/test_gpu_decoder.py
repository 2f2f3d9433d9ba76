"""Decoder step (Gemma-3-4B-shaped, 34 layers, vocab 262144): per-op parity
against the oracle, chained from the GPU's own inputs to each op, and bitwise
logits across execution variants (GPU vs GPU).

End-to-end fp64 parity over 34 bf16 layers is not a meaningful target (rounding
drift compounds), so the oracle checks each operation on the bf16 input the
GPU gave it; the end-to-end property is bitwise invariance.
"""
import numpy as np
import pytest
import torch

import deterministic_paged_attention_amd as bi
import oracle
import synth
from deterministic_paged_attention_amd.decoder import Decoder, DecoderShape
from harness import DEV, first_mismatch, page_table_tensor
from synth.workloads import decoder_weights

pytestmark = pytest.mark.gpu
BF16_TOL = 2e-2
SHAPE = DecoderShape()


def bf16_tol(ref):
    """Tolerance for a bf16 output whose exact value is ref.

    The GPU result is bf16(y32): one round-to-nearest of an fp32 value, so its
    error is at most half the bf16 spacing at the result plus the fp32
    arithmetic error before the rounding.  bf16 keeps 8 significant bits, so the
    spacing in [2^e, 2^(e+1)) is 2^(e-7): half of it is at most 2^-6 = 0.0156
    below |x| = 8, and the absolute bound 2e-2 holds there as stated.  From
    |x| = 8 on, half the spacing (2^-5 and up) alone exceeds 2e-2, so there the
    bound is one spacing at |ref|: half for the rounding, half for the fp32
    error (orders of magnitude smaller) and for a result that rounds up into
    the next binade."""
    a = np.abs(ref)
    _, e = np.frexp(a)                       # a = m 2^e, m in [0.5, 1): spacing 2^(e - 8)
    return np.where(a < 8.0, BF16_TOL, np.ldexp(1.0, e - 8))


def within_bf16_tol(got, ref):
    return bool(np.all(np.abs(got - ref) <= bf16_tol(ref)))


@pytest.fixture(scope="module")
def decoder():
    s = SHAPE
    w = decoder_weights(s.layers, s.hidden, s.q_heads, s.kv_heads, s.head_dim, s.ffn, s.vocab, seed=5000)
    torch.cuda.synchronize()
    return Decoder(s, w)


class Session:
    """Pages shared by all layers; per request a token list and a page list."""

    def __init__(self, dec: Decoder, tokens: dict, num_pages: int, page_seed: int):
        self.dec = dec
        self.tokens = tokens
        self.caches = dec.new_caches(num_pages, fill_nan=True)
        self.num_pages = num_pages
        self.free = synth.permutation(num_pages, page_seed)
        self.tables = {}
        self.lens = {}

    def share(self, rid, src, n_tokens):
        assert n_tokens % 16 == 0
        self.tables[rid] = list(self.tables[src][: n_tokens // 16])
        self.lens[rid] = n_tokens

    def step(self, batch, last_only=False, capture=None):
        ids, qls, sls, tabs, keys = [], [], [], [], []
        for rid, n in batch:
            start = self.lens.get(rid, 0)
            end = start + n
            tab = self.tables.setdefault(rid, [])
            need = -(-end // 16)
            while len(tab) < need:
                tab.append(self.free.pop(0))
            ids.extend(self.tokens[rid][start:end])
            qls.append(n)
            sls.append(end)
            tabs.append(tab)
            keys.extend((rid, p) for p in range(start, end))
        T = len(ids)
        rows = [sum(qls[: i + 1]) - 1 for i in range(len(qls))] if last_only else list(range(T))
        pt = page_table_tensor(tabs, max(len(t) for t in tabs)).to(DEV)
        sl = torch.tensor(sls, dtype=torch.int32, device=DEV)
        qsl = torch.tensor(np.concatenate([[0], np.cumsum(qls)]), dtype=torch.int32, device=DEV)
        logits = self.dec.step(torch.tensor(ids, dtype=torch.int32, device=DEV), self.caches, pt, sl, qsl,
                               max(sls), capture=capture,
                               logit_rows=torch.tensor(rows, dtype=torch.int32, device=DEV)).cpu()
        for rid, n in batch:
            self.lens[rid] = self.lens.get(rid, 0) + n
        return {keys[r]: logits[i] for i, r in enumerate(rows)}


def _f64(t):
    return t.detach().cpu().double().numpy() if t.dtype == torch.float32 else synth.to_f64(t.cpu())


def test_per_op_parity_chain(decoder):
    s = SHAPE
    toks = {0: synth.uniform_ints(40, 0, s.vocab - 1, 71), 1: synth.uniform_ints(25, 0, s.vocab - 1, 72)}
    sess = Session(decoder, toks, 16, 3)
    cap = {"layers": {0, 5}}
    sess.step([(0, 40), (1, 25)], capture=cap)
    ids = toks[0] + toks[1]
    positions = list(range(40)) + list(range(25))
    # embedding: a bit-exact gather of weight rows
    assert first_mismatch(cap["embed.out"], decoder.w["embed"][torch.tensor(ids, device=DEV)]) is None
    for layer in (0, 5):
        W = {k: _f64(v) for k, v in decoder.w["layers"][layer].items()}
        p = f"l{layer}."
        def ok(got, ref):
            return within_bf16_tol(_f64(got), ref)
        assert ok(cap[p + "xn"], oracle.rmsnorm_ref(_f64(cap[p + "h_in"]), W["g_attn"], s.eps))
        assert ok(cap[p + "qkv_raw"], oracle.gemm_ref(_f64(cap[p + "xn"]), W["w_qkv"]))
        raw = _f64(cap[p + "qkv_raw"])
        Hq, Hk, D = s.q_heads, s.kv_heads, s.head_dim
        theta = s.theta_global if s.is_global(layer) else s.theta_local
        qr, kr = oracle.qk_norm_rope_ref(raw[:, : Hq * D].reshape(-1, Hq, D), raw[:, Hq * D:(Hq + Hk) * D].reshape(-1, Hk, D),
                                         W["g_q"], W["g_k"], s.eps, positions, theta)
        got = _f64(cap[p + "qkv"])
        assert within_bf16_tol(got[:, : Hq * D], qr.reshape(65, -1))
        assert within_bf16_tol(got[:, Hq * D:(Hq + Hk) * D], kr.reshape(65, -1))
        assert first_mismatch(cap[p + "qkv"][:, (Hq + Hk) * D:], cap[p + "qkv_raw"][:, (Hq + Hk) * D:]) is None
        # attention over each request's own (post-RoPE) keys and values, from the captured qkv
        kv = got[:, Hq * D:].reshape(65, 2, Hk, D)
        out_ref = np.zeros((65, Hq, D))
        for r, (lo, n) in enumerate(((0, 40), (40, 25))):
            kc = kv[lo:lo + n, 0].reshape(n, 1, Hk, D).transpose(1, 0, 2, 3).reshape(1, n, Hk, D)
            vc = kv[lo:lo + n, 1].reshape(1, n, Hk, D)
            window = 0 if s.is_global(layer) else s.window
            out_ref[lo:lo + n] = oracle.attention_ref(got[lo:lo + n, : Hq * D].reshape(n, Hq, D), kc, vc, [[0]], [n],
                                                      [0, n], Hk, n, window=window)
        assert ok(cap[p + "attn"], out_ref)
        assert ok(cap[p + "o"], oracle.gemm_ref(_f64(cap[p + "attn"]).reshape(65, -1), W["w_o"]))
        assert ok(cap[p + "h_mid"], oracle.add_ref(_f64(cap[p + "h_in"]), _f64(cap[p + "o"])))
        assert ok(cap[p + "xn2"], oracle.rmsnorm_ref(_f64(cap[p + "h_mid"]), W["g_mlp"], s.eps))
        assert ok(cap[p + "gu"], oracle.gemm_ref(_f64(cap[p + "xn2"]), W["w_gu"]))
        assert ok(cap[p + "act"], oracle.gated_gelu_ref(_f64(cap[p + "gu"])))
        assert ok(cap[p + "down"], oracle.gemm_ref(_f64(cap[p + "act"]), W["w_down"]))
        assert ok(cap[p + "h_out"], oracle.add_ref(_f64(cap[p + "h_mid"]), _f64(cap[p + "down"])))
    g_final = _f64(decoder.w["g_final"])
    xf_ref = oracle.rmsnorm_ref(_f64(cap["final.h"]), g_final, s.eps)
    assert within_bf16_tol(_f64(cap["final.xn"]), xf_ref)
    cols = torch.tensor(synth.uniform_ints(512, 0, s.vocab - 1, 73))
    E = _f64(decoder.w["embed"][cols.to(DEV)])
    xn = _f64(cap["final.xn"])
    got = cap["final.logits"][:, cols.to(DEV)].cpu().double().numpy()
    assert np.all(np.abs(got - oracle.gemm_ref(xn, E)) <= 1e-3 * oracle.gemm_abs_ref(xn, E))


def test_per_op_parity_chain_long_context(decoder):
    """The chain inside a long context: request 0 has 1250 cached tokens and adds
    30, so local layers read a 1024-key window and global layers merge five
    splits; the attention oracle reads each layer's cache (logical layout)."""
    from harness import logical_k, logical_v
    s = SHAPE
    toks = {0: synth.uniform_ints(1280, 0, s.vocab - 1, 74), 1: synth.uniform_ints(25, 0, s.vocab - 1, 75)}
    sess = Session(decoder, toks, 100, 4)
    sess.step([(0, 1250), (1, 20)])
    cap = {"layers": {0, 5}}
    sess.step([(0, 30), (1, 5)], capture=cap)
    n = 35
    positions = list(range(1250, 1280)) + list(range(20, 25))
    Hq, Hk, D = s.q_heads, s.kv_heads, s.head_dim
    tables = [sess.tables[0], sess.tables[1]]
    pt = page_table_tensor(tables, max(len(t) for t in tables)).numpy()
    for layer in (0, 5):
        W = {k: _f64(v) for k, v in decoder.w["layers"][layer].items()}
        p = f"l{layer}."
        assert within_bf16_tol(_f64(cap[p + "xn"]), oracle.rmsnorm_ref(_f64(cap[p + "h_in"]), W["g_attn"], s.eps))
        assert within_bf16_tol(_f64(cap[p + "qkv_raw"]), oracle.gemm_ref(_f64(cap[p + "xn"]), W["w_qkv"]))
        raw = _f64(cap[p + "qkv_raw"])
        theta = s.theta_global if s.is_global(layer) else s.theta_local
        qr, kr = oracle.qk_norm_rope_ref(raw[:, : Hq * D].reshape(n, Hq, D), raw[:, Hq * D:(Hq + Hk) * D].reshape(n, Hk, D),
                                         W["g_q"], W["g_k"], s.eps, positions, theta)
        got = _f64(cap[p + "qkv"])
        assert within_bf16_tol(got[:, : Hq * D], qr.reshape(n, -1))
        assert within_bf16_tol(got[:, Hq * D:(Hq + Hk) * D], kr.reshape(n, -1))
        k_cache, v_cache = sess.caches[layer]
        window = 0 if s.is_global(layer) else s.window
        out_ref = oracle.attention_ref(got[:, : Hq * D].reshape(n, Hq, D), logical_k(k_cache), logical_v(v_cache), pt,
                                       [1280, 25], [0, 30, 35], Hk, 16, window=window)
        assert within_bf16_tol(_f64(cap[p + "attn"]), out_ref)
        assert within_bf16_tol(_f64(cap[p + "o"]), oracle.gemm_ref(_f64(cap[p + "attn"]).reshape(n, -1), W["w_o"]))
        assert within_bf16_tol(_f64(cap[p + "down"]), oracle.gemm_ref(_f64(cap[p + "act"]), W["w_down"]))


def _run(decoder, toks, schedule, page_seed, num_pages=400, shared=None):
    sess = Session(decoder, toks, num_pages, page_seed)
    out = {}
    for step in schedule:
        if isinstance(step, tuple) and step[0] == "share":
            sess.share(*step[1:])
            continue
        out.update(sess.step(step, last_only=True))
    return out


def test_logits_bitwise_across_batch_chunking_layout_and_prefix_reuse(decoder):
    """Three requests crossing the 1024-token window of the local layers; two of
    them share a 512-token prompt prefix.  Logits of every step's last rows and
    of four decode steps must agree bitwise across the schedules."""
    s = SHAPE
    prefix = synth.uniform_ints(512, 0, s.vocab - 1, 81)
    toks = {0: prefix + synth.uniform_ints(700, 0, s.vocab - 1, 82),
            1: prefix + synth.uniform_ints(620, 0, s.vocab - 1, 83),
            2: synth.uniform_ints(1100, 0, s.vocab - 1, 84)}
    lens = {r: len(t) for r, t in toks.items()}
    prompt = {r: lens[r] - 4 for r in toks}
    # A: each request alone, one-shot prompt, then 4 single-token steps
    alone = {}
    for r in toks:
        alone.update(_run(decoder, {r: toks[r]}, [[(r, prompt[r])]] + [[(r, 1)]] * 4, page_seed=10 + r))
    # B: batched; prompts in chunks of 300 interleaved; request 1 reuses request 0's prefix pages
    sched_b = [[(0, 512)], ("share", 1, 0, 512)]
    rem = {0: prompt[0] - 512, 1: prompt[1] - 512, 2: prompt[2]}
    while any(rem.values()):
        st = [(r, min(300, n)) for r, n in rem.items() if n > 0]
        for r, n in st:
            rem[r] -= n
        sched_b.append(st)
    sched_b += [[(2, 1), (0, 1), (1, 1)]] * 4
    batched = _run(decoder, toks, sched_b, page_seed=20)
    # C: chunk budget 512 with a shifted first chunk, private prefix copies, decodes in a different order
    sched_c = []
    rem = dict(prompt)
    first = True
    while any(rem.values()):
        st = [(r, min(200 if first else 512, n)) for r, n in sorted(rem.items(), reverse=True) if n > 0]
        first = False
        for r, n in st:
            rem[r] -= n
        sched_c.append(st)
    sched_c += [[(1, 1), (2, 1), (0, 1)]] * 4
    chunked = _run(decoder, toks, sched_c, page_seed=30)
    decode_keys = [(r, p) for r in toks for p in range(prompt[r], lens[r])]
    for k in decode_keys:
        assert first_mismatch(alone[k], batched[k]) is None, ("batched", k)
        assert first_mismatch(alone[k], chunked[k]) is None, ("chunked", k)
    # the prompt's last row as well (produced by a final prefill chunk in each schedule)
    for r in toks:
        k = (r, prompt[r] - 1)
        assert first_mismatch(alone[k], batched[k]) is None and first_mismatch(alone[k], chunked[k]) is None, k


def test_decode_step_logits_bitwise_at_batch_256(decoder):
    """The decode step at batch 256 over synthetic caches (contexts U{64..600}
    plus one of 32767 tokens), against the same sequences in batches of 64 in
    another order on relocated pages with wider tables, alone, and as a batch
    of 255 without the long one: every logits row bitwise.  At 256 the local
    layers take the row-group attention mapping and the global ones (128 splits
    per row) the split mapping; at 255 every layer takes the row-group mapping;
    below, the split mapping."""
    s = SHAPE
    B = 256
    ctx = synth.uniform_ints(B, 64, 600, 5100)
    ctx[7] = 32767
    k_lens = [L + 1 for L in ctx]
    need = [synth.pages_needed(L, 16) for L in k_lens]
    num_pages = sum(need) + 8
    perm = synth.permutation(num_pages, 5101)
    tables, cur = [], 0
    for n in need:
        tables.append(perm[cur:cur + n])
        cur += n
    caches = decoder.new_caches(num_pages)
    g = torch.Generator(device=DEV)
    g.manual_seed(5102)
    for k, v in caches:
        k.normal_(generator=g)
        v.normal_(generator=g)
    ids = synth.uniform_ints(B, 0, s.vocab - 1, 5103)

    def run(group, cch, tabs, stride_extra=0, fill=-1):
        pt = page_table_tensor([tabs[i] for i in group], max(len(tabs[i]) for i in group) + stride_extra, fill).to(DEV)
        sl = torch.tensor([k_lens[i] for i in group], dtype=torch.int32, device=DEV)
        qsl = torch.arange(len(group) + 1, dtype=torch.int32, device=DEV)
        ii = torch.tensor([ids[i] for i in group], dtype=torch.int32, device=DEV)
        logits = decoder.step(ii, cch, pt, sl, qsl, max(k_lens[i] for i in group))
        return {i: logits[j] for j, i in enumerate(group)}

    full = run(list(range(B)), caches, tables)
    c_local = decoder.cfg(0)
    assert bi.bi_paged_attention_mapping(c_local, B, B, max(k_lens)) == 1
    assert bi.bi_paged_attention_mapping(decoder.cfg(5), B, B, max(k_lens)) == 0
    # batch of 255 (no long context): row-group mapping in every layer
    rest = [i for i in range(B) if i != 7]
    assert bi.bi_paged_attention_mapping(decoder.cfg(5), 255, 255, max(k_lens[i] for i in rest)) == 1
    got = run(rest[::-1], caches, tables)
    for i in rest:
        assert first_mismatch(got[i], full[i]) is None, ("batch 255", i)
    # batches of 64 in another order, pages relocated, tables wider than needed
    pos = synth.permutation(num_pages, 5104)
    idx = torch.tensor(pos, dtype=torch.long, device=DEV)
    moved = []
    for k, v in caches:
        k2, v2 = torch.empty_like(k), torch.empty_like(v)
        k2.index_copy_(0, idx, k)
        v2.index_copy_(0, idx, v)
        moved.append((k2, v2))
    tables2 = [[pos[p] for p in t] for t in tables]
    order = synth.permutation(B, 5105)
    for b0 in range(0, B, 64):
        got = run(order[b0:b0 + 64], moved, tables2, stride_extra=3, fill=77777)
        for i, row in got.items():
            assert first_mismatch(row, full[i]) is None, ("batches of 64", i)
    del moved
    # alone: the long context, the shortest and two others
    for i in (7, min(range(B), key=lambda j: ctx[j]), 100, 255):
        got = run([i], caches, tables, stride_extra=1)
        assert first_mismatch(got[i], full[i]) is None, ("alone", i)


@pytest.mark.parametrize("Hq,Hk,D", [(8, 4, 256), (32, 8, 128), (4, 2, 64)])
def test_qk_norm_rope_kv_write_is_the_two_launches(Hq, Hk, D):
    """The fused q/k norm + RoPE + cache write leaves qkv and both caches bitwise
    as bi_qk_norm_rope followed by bi_kv_write (including a skipped negative slot
    and rows of sequences at different positions)."""
    cfg = bi.AttnConfig(Hq, Hk, D)
    T, num_pages = 11, 9
    qkv0 = synth.normal_bf16((T, (Hq + 2 * Hk) * D + 8), 610, std=2.0).to(DEV)[:, : (Hq + 2 * Hk) * D]
    gq = synth.normal_bf16((D,), 611, std=0.1, mean=1.0).to(DEV)
    gk = synth.normal_bf16((D,), 612, std=0.1, mean=1.0).to(DEV)
    seq_lens = torch.tensor([40, 7, 300], dtype=torch.int32, device=DEV)
    qsl = torch.tensor([0, 5, 6, 11], dtype=torch.int32, device=DEV)
    slots = torch.tensor([3, 17, 18, 19, 140, 70, -1, 5, 127, 128, 2], dtype=torch.int32, device=DEV)
    caches = []
    for _ in range(2):
        k = torch.full(cfg.k_cache_shape(num_pages), float("nan"), dtype=torch.bfloat16, device=DEV)
        v = torch.full(cfg.v_cache_shape(num_pages), float("nan"), dtype=torch.bfloat16, device=DEV)
        caches.append((k, v))
    a = qkv0.clone()
    bi.bi_qk_norm_rope(a, seq_lens, qsl, Hq, Hk, D, gq, gk, 1e-6, 10000.0)
    bi.bi_kv_write(cfg, a[:, Hq * D:(Hq + Hk) * D].view(T, Hk, D), a[:, (Hq + Hk) * D:].view(T, Hk, D), slots,
                   caches[0][0], caches[0][1])
    b = qkv0.clone()
    bi.bi_qk_norm_rope_kv_write(cfg, b, seq_lens, qsl, gq, gk, 1e-6, 10000.0, slots, caches[1][0], caches[1][1])
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for x, y in zip(caches[0], caches[1]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert torch.equal(b[:, (Hq + Hk) * D:].view(torch.int16), qkv0[:, (Hq + Hk) * D:].view(torch.int16))
