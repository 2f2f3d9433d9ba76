"""Pins of the attention oracle against hand-worked values, brute force, a library
special case, closed forms and the causal/window invariants.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import load_golden

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _paged_case(geom, lengths, q_lens, seed, slack=3, window=0, stride_extra=0):
    """Random paged case: logical caches in the oracle layout with NaN in unused slots."""
    P = geom.page_size
    plan = synth.random_page_plan(lengths, P, seed, slack=slack)
    kc = np.full((plan.num_pages, P, geom.num_kv_heads, geom.head_dim), np.nan)
    vc = np.full_like(kc, np.nan)
    qs = []
    for s, L in enumerate(lengths):
        k, v = synth.token_kv(geom, seed * 31 + s, L)
        q = synth.token_q(geom, seed * 37 + s, L)
        for j in range(L):
            pg = plan.pages[s][j // P]
            kc[pg, j % P] = synth.to_f64(k[j])
            vc[pg, j % P] = synth.to_f64(v[j])
        qs.append(synth.to_f64(q[L - q_lens[s]:L]))
    table = plan.table(stride=max(len(p) for p in plan.pages) + stride_extra).numpy()
    qsl = np.concatenate([[0], np.cumsum(q_lens)])
    return np.concatenate(qs, 0), kc, vc, table, np.asarray(lengths), qsl


# ---------------------------------------------------------------- hand-worked values

@pytest.mark.parametrize("case", load_golden("attention_hand.json")["cases"], ids=lambda c: c["name"])
def test_golden_attention(case):
    g = load_golden("attention_hand.json")
    P = g["page_size"]
    kc = np.full((g["num_pages"], P, 1, 2), np.nan)
    vc = np.full_like(kc, np.nan)
    for j, (k, v) in enumerate(zip(g["keys"], g["values"])):
        pg = g["page_table"][0][j // P]
        kc[pg, j % P, 0] = k
        vc[pg, j % P, 0] = v
    q = np.asarray(case["q"], dtype=np.float64)[:, None, :]
    out = oracle.attention_ref(q, kc, vc, g["page_table"], [case["seq_len"]], [0, q.shape[0]],
                               1, P, scale=g["scale"], window=case["window"])
    np.testing.assert_allclose(out[:, 0, :], np.asarray(case["expected"]), rtol=0, atol=1e-13)


def test_golden_merge():
    g = load_golden("merge_hand.json")
    m = np.asarray(g["m"])[None, None, :]
    l = np.asarray(g["l"])[None, None, :]
    acc = np.asarray(g["acc"])[None, None, :, :]
    valid = np.ones_like(m, dtype=bool)
    out = oracle.merge_ref(m, l, acc, valid)
    np.testing.assert_allclose(out[0, 0], g["expected"], rtol=0, atol=1e-15)


# ---------------------------------------------------------------- brute force

CONFIG1 = synth.Geometry(num_q_heads=4, num_kv_heads=2, head_dim=64, page_size=16)


@pytest.mark.parametrize("window", [0, 5, 40])
@pytest.mark.parametrize("q_lens", [[1, 1, 1, 1], [3, 17, 1, 30]])
def test_paged_equals_dense_bruteforce(window, q_lens):
    lengths = [17, 33, 64, 100]
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, lengths, q_lens, seed=11, window=window)
    out = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16, window=window)
    t0 = 0
    for s, L in enumerate(lengths):
        k, v = synth.token_kv(CONFIG1, 11 * 31 + s, L)
        pos = list(range(L - q_lens[s], L))
        ref = oracle.dense_attention_bruteforce(q[t0:t0 + q_lens[s]], synth.to_f64(k), synth.to_f64(v),
                                                pos, 2, window=window)
        np.testing.assert_allclose(out[t0:t0 + q_lens[s]], ref, rtol=0, atol=1e-12)
        t0 += q_lens[s]
    assert np.isfinite(out).all()


@pytest.mark.parametrize("window", [0, 7])
def test_matches_torch_sdpa_float64(window):
    """Library special case: torch's SDPA in float64 on the CPU with an explicit mask."""
    geom = synth.Geometry(4, 2, 32, 16)
    lengths, q_lens = [21, 50], [21, 5]
    q, kc, vc, pt, sl, qsl = _paged_case(geom, lengths, q_lens, seed=5, window=window)
    out = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16, window=window)
    t0 = 0
    for s, L in enumerate(lengths):
        k, v = synth.token_kv(geom, 5 * 31 + s, L)
        qq = torch.from_numpy(q[t0:t0 + q_lens[s]]).permute(1, 0, 2)          # [Hq, n, D]
        kk = torch.from_numpy(synth.to_f64(k)).permute(1, 0, 2).repeat_interleave(2, dim=0)
        vv = torch.from_numpy(synth.to_f64(v)).permute(1, 0, 2).repeat_interleave(2, dim=0)
        pos = torch.arange(L - q_lens[s], L)[:, None]
        j = torch.arange(L)[None, :]
        mask = j <= pos
        if window:
            mask &= j >= pos - window + 1
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        np.testing.assert_allclose(out[t0:t0 + q_lens[s]], ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
        t0 += q_lens[s]


# ---------------------------------------------------------------- softmax weights

def test_probs_rowsum_nonneg_and_support():
    lengths, q_lens, window = [17, 33, 64, 100], [2, 3, 1, 9], 20
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, lengths, q_lens, seed=3, window=window)
    probs = oracle.attention_probs_ref(q, kc, vc, pt, sl, qsl, 2, 16, window=window)
    for (s, p), W in zip(oracle.row_positions(sl, qsl), probs):
        assert (W >= 0).all()
        np.testing.assert_allclose(W.sum(axis=1), 1.0, rtol=0, atol=1e-12)
        lo = max(0, p - window + 1)
        assert (W[:, :lo] == 0).all() and (W[:, p + 1:] == 0).all()
        assert (W[:, lo:p + 1] > 0).all()


# ---------------------------------------------------------------- closed forms

def test_single_key_returns_v0():
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, [1, 1], [1, 1], seed=9)
    out = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16)
    for s in range(2):
        v0 = vc[pt[s][0], 0]                       # [H_kv, D]
        np.testing.assert_array_equal(out[s], np.repeat(v0, 2, axis=0))


def test_zero_query_gives_mean_of_visible_values():
    lengths, q_lens, window = [33, 100], [4, 1], 9
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, lengths, q_lens, seed=4, window=window)
    q[:] = 0.0
    out = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16, window=window)
    for t, (s, p) in enumerate(oracle.row_positions(sl, qsl)):
        V = oracle.gather_prefix(vc, pt[s], int(sl[s]), 16)
        lo = max(0, p - window + 1)
        for h in range(4):
            np.testing.assert_allclose(out[t, h], V[lo:p + 1, h // 2].mean(axis=0), rtol=0, atol=1e-12)


def test_constant_values_and_identical_keys():
    lengths, q_lens = [40, 70], [3, 2]
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, lengths, q_lens, seed=8)
    vconst = vc.copy()
    vconst[np.isfinite(vconst)] = 0.375
    out = oracle.attention_ref(q, kc, vconst, pt, sl, qsl, 2, 16)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-14)
    ksame = kc.copy()
    ksame[np.isfinite(ksame)] = 0.5
    probs = oracle.attention_probs_ref(q, ksame, vc, pt, sl, qsl, 2, 16)
    for (s, p), W in zip(oracle.row_positions(sl, qsl), probs):
        np.testing.assert_allclose(W[:, :p + 1], 1.0 / (p + 1), rtol=1e-13)


# ---------------------------------------------------------------- causal / window invariants

def test_future_keys_do_not_matter():
    lengths, q_lens = [64, 100], [10, 20]
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, lengths, q_lens, seed=21)
    base = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16)
    # overwrite every key/value at positions > p of the first prefill row of sequence 1
    s, p = oracle.row_positions(sl, qsl)[q_lens[0]]
    kc2, vc2 = kc.copy(), vc.copy()
    for j in range(p + 1, int(sl[s])):
        kc2[pt[s][j // 16], j % 16] = 1e3
        vc2[pt[s][j // 16], j % 16] = -7.0
    out = oracle.attention_ref(q, kc2, vc2, pt, sl, qsl, 2, 16)
    np.testing.assert_array_equal(out[q_lens[0]], base[q_lens[0]])


def test_prefill_row_equals_decode_exactly():
    L, n = 77, 12
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, [L], [n], seed=13)
    pre = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16)
    for i in range(n):
        p = L - n + i
        dec = oracle.attention_ref(q[i:i + 1], kc, vc, pt, [p + 1], [0, 1], 2, 16)
        np.testing.assert_array_equal(dec[0], pre[i])


def test_wide_window_is_no_window_and_mha_and_gqa_rows():
    lengths, q_lens = [30, 64], [5, 1]
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, lengths, q_lens, seed=17)
    a = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16, window=0)
    b = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16, window=64)
    np.testing.assert_array_equal(a, b)
    # identical query rows in one GQA group give identical outputs
    q2 = q.copy()
    q2[:, 1] = q2[:, 0]
    o2 = oracle.attention_ref(q2, kc, vc, pt, sl, qsl, 2, 16)
    np.testing.assert_array_equal(o2[:, 0], o2[:, 1])
    # H_q = H_kv: each head reads its own KV head
    o3 = oracle.attention_ref(q[:, 0:4:2], kc, vc, pt, sl, qsl, 2, 16)
    np.testing.assert_array_equal(o3[:, 0], a[:, 0])
    np.testing.assert_array_equal(o3[:, 1], a[:, 2])


def test_gqa_head_map_against_bruteforce_per_head():
    """Head h must read KV head h // G: check one head at a time with an MHA brute force."""
    geom = synth.Geometry(4, 2, 16, 16)
    q, kc, vc, pt, sl, qsl = _paged_case(geom, [45], [3], seed=23)
    out = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16)
    k, v = synth.token_kv(geom, 23 * 31, 45)
    for h in range(4):
        g = h // 2
        ref = oracle.dense_attention_bruteforce(q[:, h:h + 1], synth.to_f64(k)[:, g:g + 1],
                                                synth.to_f64(v)[:, g:g + 1], [42, 43, 44], 1)
        np.testing.assert_allclose(out[:, h], ref[:, 0], rtol=0, atol=1e-12)


# ---------------------------------------------------------------- split + merge model

@pytest.mark.parametrize("S", [16, 32, 256])
@pytest.mark.parametrize("window", [0, 23])
def test_split_merge_equals_softmax(S, window):
    lengths, q_lens = [17, 33, 64, 100], [1, 7, 16, 35]
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, lengths, q_lens, seed=29, window=window)
    ref = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16, window=window)
    m, l, acc, valid = oracle.split_partials_ref(q, kc, vc, pt, sl, qsl, 2, 16, S, window=window)
    out = oracle.merge_ref(m, l, acc, valid)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # the splits that carry a partial are exactly those meeting [lo, p]
    for t, (s, p) in enumerate(oracle.row_positions(sl, qsl)):
        lo = max(0, p - window + 1) if window else 0
        expect = [lo // S <= sp <= p // S for sp in range(valid.shape[2])]
        assert list(valid[t, 0]) == expect


def test_single_split_partial_is_plain_softmax_numerator():
    """With one split the partial is (max, sum of 2^(y-m), weighted sum): acc/l = output."""
    q, kc, vc, pt, sl, qsl = _paged_case(CONFIG1, [100], [1], seed=31)
    m, l, acc, valid = oracle.split_partials_ref(q, kc, vc, pt, sl, qsl, 2, 16, 128)
    ref = oracle.attention_ref(q, kc, vc, pt, sl, qsl, 2, 16)
    np.testing.assert_allclose(acc[:, :, 0] / l[:, :, 0, None], ref, rtol=0, atol=1e-12)
    probs = oracle.attention_probs_ref(q, kc, vc, pt, sl, qsl, 2, 16)[0]
    # l = sum 2^(y - m) and the largest weight is 1/l
    np.testing.assert_allclose(probs.max(axis=1), 1.0 / l[0, :, 0], rtol=1e-12)
