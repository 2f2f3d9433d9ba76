"""Seeded synthetic inputs shared by the tests, the bench and the oracle timing.

This module draws random numbers and builds index structures (page pools, page
tables, length mixes, chunk schedules).  It holds none of the arithmetic of the
method itself: no attention, no normalisation, no matrix product.  Both the HIP
path and the CPU oracle receive exactly the tensors produced here, so they see
identical bf16 bits.

Every draw comes from its own ``torch.Generator`` (CPU) seeded explicitly, so a
(seed, shape) pair always yields the same bits on any machine.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence

import numpy as np
import torch


def gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def normal_bf16(shape: Sequence[int], seed: int, std: float = 1.0, mean: float = 0.0) -> torch.Tensor:
    """fp32 N(mean, std) draw rounded once to bf16 (round-to-nearest-even), on the CPU."""
    x = torch.randn(tuple(shape), generator=gen(seed), dtype=torch.float32)
    if std != 1.0:
        x = x * std
    if mean != 0.0:
        x = x + mean
    return x.to(torch.bfloat16)


def small_int_bf16(shape: Sequence[int], seed: int, lo: int = -3, hi: int = 3) -> torch.Tensor:
    """Integers in [lo, hi] stored as bf16 (exactly representable)."""
    x = torch.randint(lo, hi + 1, tuple(shape), generator=gen(seed), dtype=torch.int32)
    return x.to(torch.bfloat16)


def uniform_ints(n: int, lo: int, hi: int, seed: int) -> List[int]:
    """n integers uniform in [lo, hi] (inclusive)."""
    x = torch.randint(lo, hi + 1, (n,), generator=gen(seed), dtype=torch.int64)
    return [int(v) for v in x.tolist()]


def permutation(n: int, seed: int) -> List[int]:
    return [int(v) for v in torch.randperm(n, generator=gen(seed)).tolist()]


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a CPU tensor (bf16/fp32) to a float64 numpy array."""
    return t.detach().to("cpu").to(torch.float64).numpy()


# ----------------------------------------------------------------------------
# Paged KV-cache layouts used by the harness (index structures only)
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class PagePlan:
    """Physical page assignment for a set of sequences.

    ``pages[s]`` lists the physical page ids backing the logical pages of
    sequence ``s`` in order.  ``num_pages`` is the pool size.
    """
    pages: List[List[int]]
    num_pages: int

    def table(self, stride: Optional[int] = None, fill: int = -1) -> torch.Tensor:
        """int32 page table [num_seqs, stride]; unused entries hold ``fill``."""
        width = max([len(p) for p in self.pages] + [1])
        stride = width if stride is None else stride
        assert stride >= width
        t = torch.full((len(self.pages), stride), fill, dtype=torch.int32)
        for s, row in enumerate(self.pages):
            if row:
                t[s, : len(row)] = torch.tensor(row, dtype=torch.int32)
        return t


def pages_needed(length: int, page_size: int) -> int:
    return (length + page_size - 1) // page_size


def random_page_plan(lengths: Sequence[int], page_size: int, seed: int, slack: int = 0,
                     shared_prefix_pages: int = 0) -> PagePlan:
    """Randomly permuted physical pages for sequences of the given lengths.

    With ``shared_prefix_pages = n`` every sequence maps its first n logical pages
    to the same n physical pages (a shared prefix); the rest are private.
    """
    need = [pages_needed(L, page_size) for L in lengths]
    private = [max(0, n - shared_prefix_pages) for n in need]
    total = shared_prefix_pages + sum(private) + slack
    perm = permutation(max(total, 1), seed)
    shared = perm[:shared_prefix_pages]
    cur = shared_prefix_pages
    pages = []
    for n, pv in zip(need, private):
        row = shared[: min(n, shared_prefix_pages)] + perm[cur: cur + pv]
        cur += pv
        pages.append(row)
    return PagePlan(pages=pages, num_pages=max(total, 1))


# ----------------------------------------------------------------------------
# Request content: the K/V/Q of a token is a function of (seed, request, position)
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Geometry:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int = 16


def token_kv(geom: Geometry, seed: int, length: int, std: float = 1.0):
    """K and V rows for positions [0, length) of one logical token history.

    Returns two bf16 tensors [length, H_kv, D].  The value at position j depends
    only on (seed, j), so two histories with the same seed and a common prefix
    share bit-identical K/V on that prefix (a stand-in for the canonical-prefix
    property of a cached KV entry).
    """
    H, D = geom.num_kv_heads, geom.head_dim
    k = torch.empty((length, H, D), dtype=torch.bfloat16)
    v = torch.empty((length, H, D), dtype=torch.bfloat16)
    block = 256
    for b0 in range(0, length, block):
        n = min(block, length - b0)
        k[b0:b0 + n] = normal_bf16((block, H, D), seed * 7919 + 2 * (b0 // block) + 1, std)[:n]
        v[b0:b0 + n] = normal_bf16((block, H, D), seed * 7919 + 2 * (b0 // block) + 2, std)[:n]
    return k, v


def token_q(geom: Geometry, seed: int, length: int, std: float = 1.0) -> torch.Tensor:
    """Q rows [length, H_q, D] for positions [0, length) of one token history."""
    Hq, D = geom.num_q_heads, geom.head_dim
    q = torch.empty((length, Hq, D), dtype=torch.bfloat16)
    block = 256
    for b0 in range(0, length, block):
        n = min(block, length - b0)
        q[b0:b0 + n] = normal_bf16((block, Hq, D), seed * 104729 + (b0 // block) + 7, std)[:n]
    return q


def chunk_schedule(total: int, budget: int, offset: int = 0) -> List[int]:
    """Chunk sizes covering ``total`` tokens with a per-step budget.

    ``offset`` shortens the first chunk (shifted chunk boundaries).
    """
    out = []
    rem = total
    first = budget - (offset % budget) if offset else budget
    while rem > 0:
        n = min(first if not out else budget, rem)
        out.append(n)
        rem -= n
    return out


def normal_bf16_device(shape: Sequence[int], seed: int, device="cuda", std: float = 1.0,
                       mean: float = 0.0) -> torch.Tensor:
    """N(mean, std) bf16 drawn by torch's generator on the GPU (for full-size inputs
    too large to draw on the host).  The bits are a fixed function of (seed, shape)
    on a given device; a test that needs them on the host copies this tensor back
    before any kernel under test has touched it."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(torch.bfloat16)


def llama8b_decode_lengths(batch: int, seed: int = 2000) -> List[int]:
    """Context lengths of the 8B-shaped decode workload: k_len ~ U{512..8192}."""
    return uniform_ints(batch, 512, 8192, seed)
