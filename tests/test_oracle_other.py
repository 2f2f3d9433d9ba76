"""Pins of the paging, RMSNorm and matrix-product oracles.  CPU only."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth
from conftest import load_golden


# ---------------------------------------------------------------- paging

def test_golden_slot_mapping():
    g = load_golden("slot_mapping_hand.json")
    got = oracle.slot_mapping_ref(g["page_table"], g["seq_lens"], g["query_start_loc"], g["page_size"])
    assert got.tolist() == g["expected"]


def test_write_then_gather_roundtrip_and_untouched_slots():
    geom = synth.Geometry(4, 2, 8, 4)
    lengths, q_lens = [9, 14, 3], [9, 5, 2]
    plan = synth.random_page_plan(lengths, 4, seed=2, slack=4)
    pt = plan.table(stride=6).numpy()
    qsl = np.concatenate([[0], np.cumsum(q_lens)])
    kc = np.full((plan.num_pages, 4, 2, 8), np.nan)
    vc = kc.copy()
    # pre-fill the cached part of every sequence
    for s, L in enumerate(lengths):
        k, v = synth.token_kv(geom, 100 + s, L)
        for j in range(L - q_lens[s]):
            kc[pt[s][j // 4], j % 4] = synth.to_f64(k[j])
            vc[pt[s][j // 4], j % 4] = synth.to_f64(v[j])
    kn = np.concatenate([synth.to_f64(synth.token_kv(geom, 100 + s, L)[0][L - q_lens[s]:]) for s, L in enumerate(lengths)])
    vn = np.concatenate([synth.to_f64(synth.token_kv(geom, 100 + s, L)[1][L - q_lens[s]:]) for s, L in enumerate(lengths)])
    slots = oracle.slot_mapping_ref(pt, lengths, qsl, 4)
    assert len(set(slots.tolist())) == len(slots)
    k2, v2 = oracle.kv_write_ref(kc, vc, kn, vn, slots, 4)
    for s, L in enumerate(lengths):
        k, v = synth.token_kv(geom, 100 + s, L)
        np.testing.assert_array_equal(oracle.gather_prefix(k2, pt[s], L, 4), synth.to_f64(k))
        np.testing.assert_array_equal(oracle.gather_prefix(v2, pt[s], L, 4), synth.to_f64(v))
    # every slot outside the used prefixes is still NaN
    used = {(pt[s][j // 4], j % 4) for s, L in enumerate(lengths) for j in range(L)}
    for pg in range(plan.num_pages):
        for o in range(4):
            if (pg, o) not in used:
                assert np.isnan(k2[pg, o]).all() and np.isnan(v2[pg, o]).all()


def test_identity_table_slot_is_position():
    pt = np.arange(10)[None, :]
    slots = oracle.slot_mapping_ref(pt, [37], [0, 37], 4)
    assert slots.tolist() == list(range(37))


# ---------------------------------------------------------------- RMSNorm

@pytest.mark.parametrize("i", [0, 1])
def test_golden_rmsnorm(i):
    c = load_golden("rmsnorm_hand.json")["cases"][i]
    y = oracle.rmsnorm_ref(np.asarray([c["x"]]), np.asarray(c["gamma"]), c["eps"])
    np.testing.assert_allclose(y[0], c["expected"], rtol=1e-15, atol=0)


def test_rmsnorm_closed_forms():
    H, eps = 4096, 1e-5
    gamma = synth.to_f64(synth.normal_bf16((H,), 7, std=0.1, mean=1.0))
    for c in [0.5, -3.0, 1e-3]:
        y = oracle.rmsnorm_ref(np.full((1, H), c), gamma, eps)
        np.testing.assert_allclose(y[0], c / math.sqrt(c * c + eps) * gamma, rtol=1e-14)
    sign = np.where(synth.to_f64(synth.normal_bf16((H,), 8)) >= 0, 1.0, -1.0)
    y = oracle.rmsnorm_ref(sign[None, :], gamma, eps)
    np.testing.assert_allclose(y[0], sign * gamma / math.sqrt(1 + eps), rtol=1e-14)


def test_rmsnorm_scale_invariance_and_rows_independent():
    H = 512
    x = synth.to_f64(synth.normal_bf16((5, H), 9))
    g = synth.to_f64(synth.normal_bf16((H,), 10, std=0.1, mean=1.0))
    y = oracle.rmsnorm_ref(x, g, 0.0)
    np.testing.assert_allclose(oracle.rmsnorm_ref(8.0 * x, g, 0.0), y, rtol=1e-14)
    # unit RMS after dividing by gamma
    np.testing.assert_allclose(np.sqrt(np.mean((y / g) ** 2, axis=1)), 1.0, rtol=1e-13)
    np.testing.assert_array_equal(oracle.rmsnorm_ref(x[3:4], g, 0.0)[0], y[3])


# ---------------------------------------------------------------- GEMM

def test_golden_gemm():
    g = load_golden("gemm_hand.json")
    np.testing.assert_array_equal(oracle.gemm_ref(np.asarray(g["a"]), np.asarray(g["w"])),
                                  np.asarray(g["expected"], dtype=np.float64))


def test_golden_gemm_abs_mixed_signs():
    """Hand-worked sum_k |a w| with mixed signs: the signed product, or an
    absolute value on one factor only, fails it."""
    g = load_golden("gemm_abs_hand.json")
    a, w = np.asarray(g["a"], dtype=np.float64), np.asarray(g["w"], dtype=np.float64)
    np.testing.assert_array_equal(oracle.gemm_abs_ref(a, w), np.asarray(g["expected"], dtype=np.float64))
    np.testing.assert_array_equal(oracle.gemm_ref(a, w), np.asarray(g["signed_product"], dtype=np.float64))


def test_gemm_small_integers_exact_against_python_ints():
    a = synth.small_int_bf16((7, 40), 1)
    w = synth.small_int_bf16((9, 40), 2)
    A = [[int(x) for x in row] for row in a.float().tolist()]
    W = [[int(x) for x in row] for row in w.float().tolist()]
    ref = [[sum(A[m][k] * W[n][k] for k in range(40)) for n in range(9)] for m in range(7)]
    np.testing.assert_array_equal(oracle.gemm_ref(synth.to_f64(a), synth.to_f64(w)), np.asarray(ref, dtype=np.float64))


def test_gemm_random_bf16_against_exact_rational_sum():
    a = synth.to_f64(synth.normal_bf16((3, 64), 3))
    w = synth.to_f64(synth.normal_bf16((5, 64), 4, std=0.02))
    c = oracle.gemm_ref(a, w)
    for m in range(3):
        for n in range(5):
            exact = sum(Fraction(a[m, k]) * Fraction(w[n, k]) for k in range(64))
            assert abs(c[m, n] - float(exact)) <= 1e-15 * float(sum(abs(Fraction(a[m, k]) * Fraction(w[n, k])) for k in range(64)))
    np.testing.assert_allclose(oracle.gemm_abs_ref(a, w), np.abs(a) @ np.abs(w).T, rtol=1e-15)
