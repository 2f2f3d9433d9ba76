"""GPU-side test harness: a small paged-KV "engine" that drives the product path
(slot mapping -> KV write -> paged attention) through the C ABI, plus the glue
that turns the documented cache layout back into the oracle's logical layout.

Nothing here computes attention: outputs come from libbi.so, expected values
from the oracle.  The request content (Q/K/V of every position) comes from
``synth`` and is a function of (request seed, position) only.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import deterministic_paged_attention_amd as bi
import synth

DEV = "cuda"
BF16_NAN = 0x7FC0


def nan_cache(shape) -> torch.Tensor:
    """bf16 tensor on the GPU filled with NaN (poisons never-written slots)."""
    t = torch.full(shape, BF16_NAN, dtype=torch.int16, device=DEV)
    return t.view(torch.bfloat16)


def logical_k(k_cache: torch.Tensor) -> np.ndarray:
    """[pages][H][D/8][16][8] -> [pages][16][H][D] float64 (documented K layout)."""
    pg, H, c, P, e = k_cache.shape
    return synth.to_f64(k_cache.cpu().permute(0, 3, 1, 2, 4).reshape(pg, P, H, c * e))


def logical_v(v_cache: torch.Tensor) -> np.ndarray:
    """[pages][H][D/32][16 r][16 tok][2 e] -> [pages][16][H][D] float64, d = 32*np + 16*e + r
    (documented V layout)."""
    pg, H, nq, R, P, E = v_cache.shape
    return synth.to_f64(v_cache.cpu().permute(0, 4, 1, 2, 5, 3).reshape(pg, P, H, nq * E * R))


@dataclasses.dataclass
class Request:
    """A token history: Q/K/V of position j depend only on (seed, j)."""
    seed: int
    length: int
    geom: synth.Geometry
    prefix_seed: Optional[int] = None   # positions < prefix_len come from prefix_seed
    prefix_len: int = 0

    def __post_init__(self):
        k, v = synth.token_kv(self.geom, self.seed, self.length)
        q = synth.token_q(self.geom, self.seed, self.length)
        if self.prefix_seed is not None and self.prefix_len:
            pk, pv = synth.token_kv(self.geom, self.prefix_seed, self.prefix_len)
            k[: self.prefix_len] = pk
            v[: self.prefix_len] = pv
        self.k, self.v, self.q = k, v, q   # CPU bf16 [L, H, D]


class PagedKV:
    """One layer's paged cache on the GPU with a seeded random page allocator."""

    def __init__(self, cfg: bi.AttnConfig, num_pages: int, seed: int):
        self.cfg = cfg
        self.num_pages = num_pages
        self.k = nan_cache(cfg.k_cache_shape(num_pages))
        self.v = nan_cache(cfg.v_cache_shape(num_pages))
        self.free = synth.permutation(num_pages, seed)
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    def alloc(self, n: int) -> List[int]:
        assert len(self.free) >= n, "page pool exhausted"
        out, self.free = self.free[:n], self.free[n:]
        return out

    def ensure(self, rid: int, length: int):
        tab = self.tables.setdefault(rid, [])
        need = synth.pages_needed(length, self.cfg.page_size)
        if need > len(tab):
            tab.extend(self.alloc(need - len(tab)))

    def share(self, rid: int, pages: Sequence[int], length: int):
        """Start request rid on already-filled pages (a shared prefix)."""
        self.tables[rid] = list(pages)
        self.lens[rid] = length


def page_table_tensor(tables: List[List[int]], stride: int, fill: int = -1) -> torch.Tensor:
    t = torch.full((len(tables), stride), fill, dtype=torch.int32)
    for i, row in enumerate(tables):
        if row:
            t[i, : len(row)] = torch.tensor(row, dtype=torch.int32)
    return t


def run_step(kv: PagedKV, reqs: Dict[int, Request], batch: List[Tuple[int, int]], stride_extra: int = 0,
             table_fill: int = -1, attention: bool = True, splitk: Optional[int] = None,
             max_seq_len: Optional[int] = None):
    """One engine step: for each (request id, n new tokens), write the n new
    tokens' K/V into the cache, then run attention for those n query rows.

    Returns {(rid, position): bf16 output row [H_q, D] (CPU)}.
    """
    cfg = kv.cfg
    ids, q_lens, seq_lens = [], [], []
    qs, ks, vs = [], [], []
    for rid, n in batch:
        r = reqs[rid]
        start = kv.lens.get(rid, 0)
        end = start + n
        assert end <= r.length
        kv.ensure(rid, end)
        ids.append(rid)
        q_lens.append(n)
        seq_lens.append(end)
        qs.append(r.q[start:end])
        ks.append(r.k[start:end])
        vs.append(r.v[start:end])
    stride = max(len(kv.tables[i]) for i in ids) + stride_extra
    pt = page_table_tensor([kv.tables[i] for i in ids], stride, table_fill).to(DEV)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=DEV)
    qsl = torch.tensor(np.concatenate([[0], np.cumsum(q_lens)]), dtype=torch.int32, device=DEV)
    T = int(sum(q_lens))
    q = torch.cat(qs).to(DEV)
    k_new = torch.cat(ks).to(DEV)
    v_new = torch.cat(vs).to(DEV)
    slots = bi.bi_slot_mapping(pt, sl, qsl, T, cfg.page_size, kv.num_pages)
    bi.bi_kv_write(cfg, k_new, v_new, slots, kv.k, kv.v)
    for rid, n in batch:
        kv.lens[rid] = kv.lens.get(rid, 0) + n
    if not attention:
        return {}
    msl = max(seq_lens) if max_seq_len is None else max_seq_len
    if splitk is None:
        out = bi.bi_paged_attention(cfg, q, kv.k, kv.v, pt, sl, qsl, msl)
    else:
        out = bi.bi_paged_attention_splitk(cfg, q, kv.k, kv.v, pt, sl, qsl, msl, splitk)
    out = out.cpu()
    res = {}
    t = 0
    for (rid, n), end in zip(batch, seq_lens):
        for j in range(n):
            res[(rid, end - n + j)] = out[t]
            t += 1
    return res


def oracle_rows(reqs: Dict[int, Request], keys: Sequence[Tuple[int, int]], geom: synth.Geometry, window: int,
                scale=None):
    """Oracle output for (request, position) rows, from the logical token history."""
    import oracle
    out = {}
    by_req: Dict[int, List[int]] = {}
    for rid, p in keys:
        by_req.setdefault(rid, []).append(p)
    P = geom.page_size
    for rid, ps in by_req.items():
        r = reqs[rid]
        L = max(ps) + 1
        npg = synth.pages_needed(L, P)
        kc = np.zeros((npg, P, geom.num_kv_heads, geom.head_dim))
        vc = np.zeros_like(kc)
        kk = synth.to_f64(r.k[:L])
        vv = synth.to_f64(r.v[:L])
        for j in range(L):
            kc[j // P, j % P] = kk[j]
            vc[j // P, j % P] = vv[j]
        table = np.arange(npg)[None, :]
        for p in ps:
            q = synth.to_f64(r.q[p:p + 1])
            o = oracle.attention_ref(q, kc, vc, table, [p + 1], [0, 1], geom.num_kv_heads, P, scale=scale,
                                     window=window)
            out[(rid, p)] = o[0]
    return out


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.contiguous().view(torch.int16)


def first_mismatch(a: torch.Tensor, b: torch.Tensor) -> Optional[str]:
    ba, bb = bits(a), bits(b)
    if torch.equal(ba, bb):
        return None
    idx = (ba != bb).nonzero()[0].tolist()
    return f"first differing element {idx}: {a[tuple(idx)].item()} vs {b[tuple(idx)].item()}"
