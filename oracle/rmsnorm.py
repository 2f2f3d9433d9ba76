"""Per-row RMSNorm in float64.

The record "Deterministic and bit-exact inference" (field "technical",
Invariance) names RMSNorm among the kernels made batch-invariant.  The pages do
not spell out its formula; the plain reading used here (listed in the design
notes): y = x / sqrt(mean_k x_k^2 + eps) * gamma, mean over the hidden size,
eps inside the square root, multiplied by gamma (not 1 + gamma).
"""
from __future__ import annotations

import numpy as np


def rmsnorm_ref(x, gamma, eps):
    """x: [M, H] float64, gamma: [H] float64 -> [M, H] float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(gamma, dtype=np.float64)[None, :]
