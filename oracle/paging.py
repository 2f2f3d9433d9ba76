"""Paged KV-cache addressing, written out plainly.

Follows the Vosti deep-dive blog (深入解析 Vosti), §3.2: invariant 1 (page
tables map a request's prefix to allocated, in-range slots) and invariant 2
(the KV value stored at the slot of position p is the value of that logical
position, whatever the physical page), and §5.1 (canonical prefix).  The
mapping position -> (page, slot-in-page) is the plain reading of a page table:
logical page ``p // P`` of the sequence, entry ``p % P`` inside it.
"""
from __future__ import annotations

import numpy as np


def row_positions(seq_lens, query_start_loc):
    """For each query token t: (sequence index, logical position p).

    The query rows of a sequence are its last q_len positions, so row i of a
    sequence with k_len keys sits at p = k_len - q_len + i (Vosti deep-dive,
    §6.2, attention causal contract).
    """
    seq_lens = [int(x) for x in seq_lens]
    qsl = [int(x) for x in query_start_loc]
    out = []
    for s in range(len(seq_lens)):
        q_len = qsl[s + 1] - qsl[s]
        for i in range(q_len):
            out.append((s, seq_lens[s] - q_len + i))
    return out


def slot_mapping_ref(page_table, seq_lens, query_start_loc, page_size):
    """Flat slot index (page * P + offset) of every new token of this step."""
    pt = np.asarray(page_table)
    slots = []
    for s, p in row_positions(seq_lens, query_start_loc):
        page = int(pt[s, p // page_size])
        slots.append(page * page_size + p % page_size)
    return np.asarray(slots, dtype=np.int64)


def kv_write_ref(k_cache, v_cache, k_new, v_new, slots, page_size):
    """Copy token rows k_new[t], v_new[t] ([H_kv, D]) into their slots.

    Caches use the oracle's logical layout [num_pages, P, H_kv, D].  Returns new
    arrays; the inputs are not modified.
    """
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    for t, slot in enumerate(np.asarray(slots).tolist()):
        k_out[slot // page_size, slot % page_size] = k_new[t]
        v_out[slot // page_size, slot % page_size] = v_new[t]
    return k_out, v_out


def gather_prefix(cache, page_row, length, page_size):
    """Logical rows [0, length) of one sequence: out[j] = cache[page_row[j // P], j % P]."""
    rows = [cache[int(page_row[j // page_size]), j % page_size] for j in range(length)]
    if not rows:
        return np.zeros((0,) + tuple(cache.shape[2:]), dtype=cache.dtype)
    return np.stack(rows, axis=0)
