"""Matrix product c = a b in float64, with the weight stored as w = b^T ([N, K]).

Vosti deep-dive blog (深入解析 Vosti), §6.1, matmul relational contract:
c[x, 0:N] is determined by a[x, 0:K] and b[0:K, 0:N].  Here b[k, n] = w[n, k]
(the nn.Linear storage, K contiguous), so c[m, n] = sum_k a[m, k] * w[n, k].
"""
from __future__ import annotations

import numpy as np


def gemm_ref(a, w):
    """a: [M, K], w: [N, K] (float64) -> [M, N] float64."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def gemm_abs_ref(a, w):
    """sum_k |a[m,k] * w[n,k]|: the scale of the componentwise error bound."""
    return np.abs(np.asarray(a, dtype=np.float64)) @ np.abs(np.asarray(w, dtype=np.float64)).T
