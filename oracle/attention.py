"""Causal (optionally windowed) GQA attention over a paged KV cache, in float64.

What is computed follows the Vosti deep-dive blog (深入解析 Vosti):
  * §2 (Theorem 4.1): attention is part of ``Forward(W, h)``, a cold forward
    over the causal prefix of the token history;
  * §6.2, attention causal contract: query row i of a q_len-row block has
    position p = k_len - q_len + i and sees keys K[0 : p+1];
  * §6.2, sliding-window traversal: with window w > 0 the keys start at
    max(0, p - w + 1).
The split partials and their merge model the fixed key-split *size* (not a
fixed split count) of the Thinking Machines recipe as summarised in the record
"Deterministic and bit-exact inference" (field "technical", Invariance).

Readings where the pages are silent (each is listed in the design notes):
  * softmax scale defaults to 1/sqrt(D);
  * query head h uses KV head h // (H_q / H_kv) (contiguous GQA groups);
  * partials are kept in base 2: m = max_j z_j*log2(e), l = sum_j 2^(z_j*log2(e) - m),
    acc = sum_j 2^(z_j*log2(e) - m) v_j, with z_j = scale * <q, k_j>.
"""
from __future__ import annotations

import math

import numpy as np

from .paging import gather_prefix, row_positions

LOG2E = 1.4426950408889634  # log2(e)


def _default_scale(head_dim, scale):
    return 1.0 / math.sqrt(head_dim) if (scale is None or scale == 0.0) else float(scale)


def key_range(p, window):
    """Visible keys of the row at position p: [lo, p] (inclusive)."""
    lo = max(0, p - window + 1) if window and window > 0 else 0
    return lo, p


def _check(q, k_cache, num_kv_heads):
    Hq = q.shape[1]
    assert Hq % num_kv_heads == 0, "H_q must be a multiple of H_kv"
    assert k_cache.shape[2] == num_kv_heads
    return Hq // num_kv_heads


def attention_probs_ref(q, k_cache, v_cache, page_table, seq_lens, query_start_loc,
                        num_kv_heads, page_size, scale=None, window=0):
    """Softmax weights of every query row over all k_len positions of its sequence.

    Returns a list with one float64 array [H_q, k_len] per query token; weights
    outside [lo, p] are exactly 0.
    """
    G = _check(q, k_cache, num_kv_heads)
    D = q.shape[2]
    sc = _default_scale(D, scale)
    pt = np.asarray(page_table)
    out = []
    for t, (s, p) in enumerate(row_positions(seq_lens, query_start_loc)):
        k_len = int(seq_lens[s])
        K = gather_prefix(k_cache, pt[s], k_len, page_size)
        lo, hi = key_range(p, window)
        W = np.zeros((q.shape[1], k_len))
        for h in range(q.shape[1]):
            z = sc * (K[lo:hi + 1, h // G, :] @ q[t, h, :])
            e = np.exp(z - z.max())
            W[h, lo:hi + 1] = e / e.sum()
        out.append(W)
    return out


def attention_ref(q, k_cache, v_cache, page_table, seq_lens, query_start_loc,
                  num_kv_heads, page_size, scale=None, window=0):
    """o[t, h] = sum_j softmax_j(scale * <q[t,h], K[j, g]>) V[j, g], j in [lo, p].

    q: [T, H_q, D] float64; caches: [num_pages, P, H_kv, D] float64 (logical layout);
    page_table: [B, stride] ints; seq_lens: [B] (k_len, this step's tokens included);
    query_start_loc: [B+1].  Returns [T, H_q, D] float64.
    """
    G = _check(q, k_cache, num_kv_heads)
    T, Hq, D = q.shape
    sc = _default_scale(D, scale)
    pt = np.asarray(page_table)
    out = np.zeros((T, Hq, D))
    for t, (s, p) in enumerate(row_positions(seq_lens, query_start_loc)):
        k_len = int(seq_lens[s])
        K = gather_prefix(k_cache, pt[s], k_len, page_size)
        V = gather_prefix(v_cache, pt[s], k_len, page_size)
        lo, hi = key_range(p, window)
        for h in range(Hq):
            g = h // G
            z = sc * (K[lo:hi + 1, g, :] @ q[t, h, :])
            e = np.exp(z - z.max())
            out[t, h] = (e @ V[lo:hi + 1, g, :]) / e.sum()
    return out


def split_partials_ref(q, k_cache, v_cache, page_table, seq_lens, query_start_loc,
                       num_kv_heads, page_size, split_size, scale=None, window=0):
    """Per-(row, split) softmax partials over the fixed key ranges [sS, (s+1)S).

    For each query row and each split s whose key range meets [lo, p]:
      m_s   = max_j y_j,      y_j = scale * <q, k_j> * log2(e)
      l_s   = sum_j 2^(y_j - m_s)
      acc_s = sum_j 2^(y_j - m_s) v_j
    over j in [lo, p] intersected with the split.  Returns (m, l, acc, valid)
    with shapes [T, H_q, NS], [T, H_q, NS], [T, H_q, NS, D], [T, H_q, NS] where
    NS = ceil(max k_len / S); entries with valid == False are NaN.
    """
    G = _check(q, k_cache, num_kv_heads)
    T, Hq, D = q.shape
    sc = _default_scale(D, scale)
    S = int(split_size)
    NS = max(1, -(-max(int(x) for x in seq_lens) // S)) if len(seq_lens) else 1
    m = np.full((T, Hq, NS), np.nan)
    l = np.full((T, Hq, NS), np.nan)
    acc = np.full((T, Hq, NS, D), np.nan)
    valid = np.zeros((T, Hq, NS), dtype=bool)
    pt = np.asarray(page_table)
    for t, (s, p) in enumerate(row_positions(seq_lens, query_start_loc)):
        k_len = int(seq_lens[s])
        K = gather_prefix(k_cache, pt[s], k_len, page_size)
        V = gather_prefix(v_cache, pt[s], k_len, page_size)
        lo, hi = key_range(p, window)
        for sp in range(lo // S, hi // S + 1):
            a, b = max(lo, sp * S), min(hi, sp * S + S - 1)
            for h in range(Hq):
                g = h // G
                y = sc * (K[a:b + 1, g, :] @ q[t, h, :]) * LOG2E
                mx = y.max()
                e = np.exp2(y - mx)
                m[t, h, sp] = mx
                l[t, h, sp] = e.sum()
                acc[t, h, sp] = e @ V[a:b + 1, g, :]
                valid[t, h, sp] = True
    return m, l, acc, valid


def merge_ref(m, l, acc, valid):
    """Combine split partials in increasing split order into the attention output.

    m* = max over present splits, w_s = 2^(m_s - m*), o = (sum_s w_s acc_s) / (sum_s w_s l_s).
    Arguments as returned by ``split_partials_ref``; returns [T, H_q, D].
    """
    T, Hq, NS, D = acc.shape
    out = np.zeros((T, Hq, D))
    for t in range(T):
        for h in range(Hq):
            idx = [s for s in range(NS) if valid[t, h, s]]
            mstar = max(m[t, h, s] for s in idx)
            L = 0.0
            N = np.zeros(D)
            for s in idx:
                w = 2.0 ** (m[t, h, s] - mstar)
                L += w * l[t, h, s]
                N += w * acc[t, h, s]
            out[t, h] = N / L
    return out


def dense_attention_bruteforce(q_rows, K, V, positions, num_kv_heads, scale=None, window=0):
    """Dense attention with an explicit boolean mask matrix, for pinning the oracle.

    q_rows: [n, H_q, D]; K, V: [k_len, H_kv, D] contiguous (no paging);
    positions: [n] logical positions of the query rows.  Builds the full score
    matrix over all k_len keys, sets masked entries to -inf, and takes a plain
    row softmax.
    """
    n, Hq, D = q_rows.shape
    k_len = K.shape[0]
    G = Hq // num_kv_heads
    sc = _default_scale(D, scale)
    mask = np.zeros((n, k_len), dtype=bool)
    for i, p in enumerate(positions):
        for j in range(k_len):
            mask[i, j] = (j <= p) and (not window or window <= 0 or j >= p - window + 1)
    out = np.zeros((n, Hq, D))
    for h in range(Hq):
        g = h // G
        scores = sc * (q_rows[:, h, :] @ K[:, g, :].T)
        scores = np.where(mask, scores, -np.inf)
        mx = scores.max(axis=1, keepdims=True)
        e = np.exp(scores - mx)
        probs = e / e.sum(axis=1, keepdims=True)
        out[:, h, :] = probs @ V[:, g, :]
    return out
