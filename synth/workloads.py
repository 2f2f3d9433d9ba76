"""Full-size synthetic workloads, built directly on the GPU.

The 8B-shaped decode workload: 32 query / 8 KV heads, head_dim 128, pages of
16 tokens, context lengths ~ U{512..8192}, K/V ~ N(0, 1) bf16, pages randomly
permuted in a pool with slack.  K/V are drawn straight into the cache tensors
by torch's GPU generator (random bits are random in any layout); the host copy
of a sequence is read back from those tensors before any kernel under test has
written to them.  Index structures only — no attention arithmetic here.
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np
import torch

from . import llama8b_decode_lengths, normal_bf16_device, pages_needed, permutation, to_f64


@dataclasses.dataclass
class DecodeWorkload:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    lengths: List[int]
    pages: List[List[int]]
    num_pages: int
    q: torch.Tensor           # [B, H_q, D] bf16
    k_new: torch.Tensor       # [B, H_kv, D] bf16 (this step's token)
    v_new: torch.Tensor
    k_cache: torch.Tensor     # [pages, H_kv, D/8, 16, 8] bf16
    v_cache: torch.Tensor     # [pages, H_kv, D/32, 16, 16, 2] bf16
    page_table: torch.Tensor  # [B, stride] int32
    seq_lens: torch.Tensor    # [B] int32
    qsl: torch.Tensor         # [B+1] int32
    max_seq_len: int
    workspace: torch.Tensor = None

    @property
    def batch(self) -> int:
        return len(self.lengths)

    def host_sequence(self, s: int):
        """Logical K, V [npg, 16, H_kv, D] (float64), identity table, k_len of sequence s,
        decoded from the documented cache layout."""
        idx = torch.tensor(self.pages[s], dtype=torch.long, device=self.k_cache.device)
        kp = self.k_cache.index_select(0, idx).cpu()
        vp = self.v_cache.index_select(0, idx).cpu()
        npg = len(self.pages[s])
        k = kp.permute(0, 3, 1, 2, 4).reshape(npg, self.page_size, self.num_kv_heads, self.head_dim)
        v = vp.permute(0, 4, 1, 2, 5, 3).reshape(npg, self.page_size, self.num_kv_heads, self.head_dim)
        return to_f64(k), to_f64(v), np.arange(npg)[None, :], self.lengths[s]

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one decode pass reads: 2 * k_len * H_kv * D * 2 per sequence."""
        return sum(2 * L * self.num_kv_heads * self.head_dim * 2 for L in self.lengths)


def build_decode_workload(num_q_heads: int, num_kv_heads: int, head_dim: int, batch: int, seed: int,
                          page_size: int = 16, device: str = "cuda", slack_pages: int = 64,
                          lengths: List[int] = None) -> DecodeWorkload:
    lengths = llama8b_decode_lengths(batch, seed) if lengths is None else list(lengths)
    need = [pages_needed(L, page_size) for L in lengths]
    num_pages = sum(need) + slack_pages
    perm = permutation(num_pages, seed + 1)
    pages, cur = [], 0
    for n in need:
        pages.append(perm[cur:cur + n])
        cur += n
    stride = max(need)
    pt = torch.full((batch, stride), -1, dtype=torch.int32)
    for s, row in enumerate(pages):
        pt[s, :len(row)] = torch.tensor(row, dtype=torch.int32)
    H, D = num_kv_heads, head_dim
    k_cache = normal_bf16_device((num_pages, H, D // 8, page_size, 8), seed + 2, device)
    v_cache = normal_bf16_device((num_pages, H, D // 32, 16, page_size, 2), seed + 3, device)
    q = normal_bf16_device((batch, num_q_heads, D), seed + 4, device)
    k_new = normal_bf16_device((batch, H, D), seed + 5, device)
    v_new = normal_bf16_device((batch, H, D), seed + 6, device)
    return DecodeWorkload(
        num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim, page_size=page_size,
        lengths=lengths, pages=pages, num_pages=num_pages, q=q, k_new=k_new, v_new=v_new,
        k_cache=k_cache, v_cache=v_cache, page_table=pt.to(device),
        seq_lens=torch.tensor(lengths, dtype=torch.int32, device=device),
        qsl=torch.arange(batch + 1, dtype=torch.int32, device=device),
        max_seq_len=max(lengths))


def decoder_weights(layers: int, hidden: int, q_heads: int, kv_heads: int, head_dim: int, ffn: int, vocab: int,
                    seed: int, device: str = "cuda") -> dict:
    """Random-init weights of a pre-norm decoder stack: matrices ~ N(0, 0.02) stored
    [out, in], norm gains ~ N(1, 0.1), tied embedding [vocab, hidden] ~ N(0, 0.02)."""
    qkv = (q_heads + 2 * kv_heads) * head_dim
    out = {"embed": normal_bf16_device((vocab, hidden), seed, device, std=0.02),
           "g_final": normal_bf16_device((hidden,), seed + 1, device, std=0.1, mean=1.0), "layers": []}
    for l in range(layers):
        b = seed + 100 * (l + 1)
        out["layers"].append({
            "w_qkv": normal_bf16_device((qkv, hidden), b + 1, device, std=0.02),
            "w_o": normal_bf16_device((hidden, q_heads * head_dim), b + 2, device, std=0.02),
            "w_gu": normal_bf16_device((2 * ffn, hidden), b + 3, device, std=0.02),
            "w_down": normal_bf16_device((hidden, ffn), b + 4, device, std=0.02),
            "g_attn": normal_bf16_device((hidden,), b + 5, device, std=0.1, mean=1.0),
            "g_mlp": normal_bf16_device((hidden,), b + 6, device, std=0.1, mean=1.0),
            "g_q": normal_bf16_device((head_dim,), b + 7, device, std=0.1, mean=1.0),
            "g_k": normal_bf16_device((head_dim,), b + 8, device, std=0.1, mean=1.0),
        })
    return out
