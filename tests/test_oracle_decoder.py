"""Pins of the decoder-step glue oracles.  CPU only."""
import math

import numpy as np
import pytest

import oracle
import synth
from conftest import load_golden


@pytest.mark.parametrize("i", [0, 1, 2])
def test_golden_rope(i):
    g = load_golden("rope_hand.json")
    c = g["cases"][i]
    out = oracle.rope_ref(np.asarray([c["x"]]), [c["p"]], g["theta"])
    np.testing.assert_allclose(out[0], c["expected"], rtol=0, atol=1e-15)


def test_rope_preserves_pair_norms_and_adds_angles():
    x = synth.to_f64(synth.normal_bf16((3, 2, 16), 5))
    p = [0, 7, 1000]
    y = oracle.rope_ref(x, p, 10000.0)
    for t in range(3):
        n0 = x[t, :, :8] ** 2 + x[t, :, 8:] ** 2
        n1 = y[t, :, :8] ** 2 + y[t, :, 8:] ** 2
        np.testing.assert_allclose(n1, n0, rtol=1e-12)
    np.testing.assert_array_equal(y[0], x[0])
    # rotating by p1 then by p2 equals rotating by p1 + p2
    two = oracle.rope_ref(oracle.rope_ref(x, [3, 5, 11], 1e6), [4, 9, 13], 1e6)
    one = oracle.rope_ref(x, [7, 14, 24], 1e6)
    np.testing.assert_allclose(two, one, rtol=0, atol=1e-12)


def test_qk_norm_rope_at_position_zero_is_rmsnorm():
    q = synth.to_f64(synth.normal_bf16((2, 8, 256), 6))
    k = synth.to_f64(synth.normal_bf16((2, 4, 256), 7))
    gq = synth.to_f64(synth.normal_bf16((256,), 8, std=0.1, mean=1.0))
    gk = synth.to_f64(synth.normal_bf16((256,), 9, std=0.1, mean=1.0))
    qo, ko = oracle.qk_norm_rope_ref(q, k, gq, gk, 1e-6, [0, 0], 10000.0)
    np.testing.assert_array_equal(qo.reshape(16, 256), oracle.rmsnorm_ref(q.reshape(16, 256), gq, 1e-6))
    np.testing.assert_array_equal(ko.reshape(8, 256), oracle.rmsnorm_ref(k.reshape(8, 256), gk, 1e-6))


def test_golden_qk_norm_rope_norm_before_rotation():
    """Hand-worked at p >= 1 with a non-uniform gain: rotating before the norm
    (or dropping the norm, or the gain) fails it."""
    g = load_golden("qk_norm_rope_hand.json")
    q, k = g["q"], g["k"]
    # two tokens: the q case at its position, the k case at its own
    xq = np.asarray([[q["x"]], [q["x"]]])
    xk = np.asarray([[k["x"]], [k["x"]]])
    qo, ko = oracle.qk_norm_rope_ref(xq, xk, np.asarray(q["gamma"]), np.asarray(k["gamma"]), g["eps"],
                                     [q["p"], k["p"]], g["theta"])
    qo, ko = qo[:1], ko[1:]
    np.testing.assert_allclose(qo[0, 0], q["expected"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(ko[0, 0], k["expected"], rtol=0, atol=1e-14)
    # the swapped order is really distinguishable at these inputs
    assert np.max(np.abs(np.asarray(q["expected"]) - q["rope_first"])) > 1e-2
    assert np.max(np.abs(np.asarray(k["expected"]) - k["rope_first"])) > 1e-2


def test_gelu_odd_part_limits_and_erf_form():
    x = np.linspace(-8, 8, 1601)
    g = oracle.gelu_tanh(x)
    np.testing.assert_allclose(g - oracle.gelu_tanh(-x), x, rtol=0, atol=1e-12)   # exact identity of the tanh form
    assert oracle.gelu_tanh(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(oracle.gelu_tanh(np.array([20.0, -20.0])), [20.0, 0.0], atol=1e-12)
    erf_form = np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in x])
    assert np.max(np.abs(g - erf_form)) < 1e-3    # the tanh form approximates x * Phi(x)


def test_gated_gelu_and_add_and_embedding():
    x = synth.to_f64(synth.normal_bf16((3, 10), 10))
    out = oracle.gated_gelu_ref(x)
    np.testing.assert_array_equal(out, oracle.gelu_tanh(x[:, :5]) * x[:, 5:])
    x[:, 5:] = 1.0
    np.testing.assert_array_equal(oracle.gated_gelu_ref(x), oracle.gelu_tanh(x[:, :5]))
    a, b = synth.to_f64(synth.normal_bf16((2, 4), 11)), synth.to_f64(synth.normal_bf16((2, 4), 12))
    np.testing.assert_array_equal(oracle.add_ref(a, b), a + b)
    table = synth.to_f64(synth.normal_bf16((7, 16), 13))
    e = oracle.embedding_ref(table, [3, 0, 6, 9, -1])
    np.testing.assert_array_equal(e[:3], table[[3, 0, 6]])
    assert (e[3:] == 0).all()


def test_argmax_ref_ties_nan_and_infinities():
    x = np.array([[1.0, 3.0, 3.0, -1.0],          # tie: first index
                  [np.nan, -np.inf, -np.inf, np.nan],   # NaN never wins; tie of -inf: first
                  [np.nan, np.nan, np.nan, np.nan],     # all NaN: 0
                  [-5.0, np.inf, 2.0, np.inf]])
    assert oracle.argmax_ref(x).tolist() == [1, 1, 0, 1]
    r = np.random.default_rng(7).standard_normal((5, 100))
    assert oracle.argmax_ref(r).tolist() == np.argmax(r, axis=1).tolist()
