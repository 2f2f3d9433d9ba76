"""Decoder-step glue in float64: embedding gather, rotary position embedding,
per-head q/k RMSNorm, residual add, gated GELU.

The pages define the decoder step only as the cold causal forward
Forward(W, h) (Vosti deep-dive blog (深入解析 Vosti), §2, Theorem 4.1).  The
layer details are the plainest Gemma-3-style reading, listed in the design
notes: pre-norm residual blocks, q/k RMSNorm per head, rotary embedding on
half-split pairs (i, i + D/2) with angle p * theta^(-2i/D), and a gated GELU in
its tanh form.  Each function is the plain definition.
"""
from __future__ import annotations

import math

import numpy as np

from .rmsnorm import rmsnorm_ref


def embedding_ref(table, ids):
    """Rows table[ids[t]]; ids outside [0, vocab) give zero rows."""
    table = np.asarray(table, dtype=np.float64)
    out = np.zeros((len(ids), table.shape[1]))
    for t, i in enumerate(ids):
        if 0 <= int(i) < table.shape[0]:
            out[t] = table[int(i)]
    return out


def rope_ref(x, positions, theta):
    """Rotate the last axis of x [T, ..., D] in pairs (i, i + D/2) by p * theta^(-2i/D)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    out = np.empty_like(x)
    for t, p in enumerate(positions):
        for i in range(half):
            a = p * theta ** (-2.0 * i / D)
            c, s = math.cos(a), math.sin(a)
            xi, xj = x[t, ..., i], x[t, ..., i + half]
            out[t, ..., i] = xi * c - xj * s
            out[t, ..., i + half] = xi * s + xj * c
    return out


def qk_norm_rope_ref(q, k, gamma_q, gamma_k, eps, positions, theta):
    """q [T, Hq, D], k [T, Hkv, D]: RMSNorm of every head row, then rotary embedding."""
    T, Hq, D = q.shape
    Hk = k.shape[1]
    qn = rmsnorm_ref(np.asarray(q).reshape(T * Hq, D), gamma_q, eps).reshape(T, Hq, D)
    kn = rmsnorm_ref(np.asarray(k).reshape(T * Hk, D), gamma_k, eps).reshape(T, Hk, D)
    return rope_ref(qn, positions, theta), rope_ref(kn, positions, theta)


def add_ref(a, b):
    return np.asarray(a, dtype=np.float64) + np.asarray(b, dtype=np.float64)


def gelu_tanh(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def gated_gelu_ref(x):
    """x [R, 2F] = [gate | up] -> gelu(gate) * up."""
    x = np.asarray(x, dtype=np.float64)
    F = x.shape[1] // 2
    return gelu_tanh(x[:, :F]) * x[:, F:]


def argmax_ref(x):
    """Greedy sampling over rows of x [R, n]: the smallest index of a row's
    maximum, ignoring NaN entries; 0 for a row that is all NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape[0], dtype=np.int64)
    for r in range(x.shape[0]):
        best = None
        for i, v in enumerate(x[r]):
            if v == v and (best is None or v > x[r, best]):
                best = i
        out[r] = 0 if best is None else best
    return out
