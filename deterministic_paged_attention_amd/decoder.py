"""Decoder-step composition over the libbi kernels (Gemma-3-4B-shaped stack).

Python only sequences launches; every operation runs in a libbi kernel.  One
call processes one engine step: any mix of prefill chunks and decode tokens,
given as the rows of a paged-attention batch (token ids, page table, k_len per
sequence, query start offsets).  The same page table serves every layer; each
layer owns its own K and V cache tensors.

Layer (pre-norm):  h += O(attn(rope(qk_norm(QKV(norm(h))))));
                   h += Down(gelu(Gate(norm(h))) * Up(norm(h)))
then logits = Embed^T norm(h) in fp32 (tied embedding).  Local layers attend
inside a sliding window; every `global_every`-th layer is global.  These are
the plainest choices for the layers, which the pages do not describe; they
define the step only as the cold causal forward Forward(W, h) (Vosti deep-dive
blog (深入解析 Vosti), §2, Theorem 4.1).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional

import torch

from . import (AttnConfig, alloc_workspace, bi_add, bi_add_rmsnorm, bi_embedding, bi_gated_gelu, bi_gemm,
               bi_gemm_gated_gelu, bi_paged_attention, bi_paged_attention_workspace_size, bi_qk_norm_rope_kv_write,
               bi_rmsnorm, bi_slot_mapping)


@dataclasses.dataclass(frozen=True)
class DecoderShape:
    layers: int = 34
    hidden: int = 2560
    q_heads: int = 8
    kv_heads: int = 4
    head_dim: int = 256
    ffn: int = 10240
    vocab: int = 262144
    window: int = 1024
    global_every: int = 6
    theta_local: float = 10000.0
    theta_global: float = 1000000.0
    eps: float = 1e-6
    page_size: int = 16
    split_size: int = 256
    split_size_local: int = 128  # windowed layers: their own fixed split size

    def is_global(self, layer: int) -> bool:
        return (layer + 1) % self.global_every == 0

    @property
    def qkv_width(self) -> int:
        return (self.q_heads + 2 * self.kv_heads) * self.head_dim


def weight_shapes(shape: DecoderShape) -> Dict[str, tuple]:
    """Shapes of the per-layer tensors (all bf16; matrices stored [out, in])."""
    H, D, F = shape.hidden, shape.head_dim, shape.ffn
    return {"w_qkv": (shape.qkv_width, H), "w_o": (H, shape.q_heads * D), "w_gu": (2 * F, H), "w_down": (H, F),
            "g_attn": (H,), "g_mlp": (H,), "g_q": (D,), "g_k": (D,)}


class Decoder:
    """Runs decoder steps for given weights:
    weights = {"embed": [V, H], "g_final": [H], "layers": [{name: tensor} per layer]}."""

    def __init__(self, shape: DecoderShape, weights: dict):
        self.shape = shape
        self.w = weights
        s = shape
        self.cfg_local = AttnConfig(s.q_heads, s.kv_heads, s.head_dim, s.page_size, s.split_size_local,
                                    window=s.window)
        self.cfg_global = AttnConfig(s.q_heads, s.kv_heads, s.head_dim, s.page_size, s.split_size, window=0)

    def cfg(self, layer: int) -> AttnConfig:
        return self.cfg_global if self.shape.is_global(layer) else self.cfg_local

    def new_caches(self, num_pages: int, fill_nan: bool = False) -> List[tuple]:
        caches = []
        for layer in range(self.shape.layers):
            c = self.cfg(layer)
            if fill_nan:
                k = torch.full(c.k_cache_shape(num_pages), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
                v = torch.full(c.v_cache_shape(num_pages), 0x7FC0, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            else:
                k = torch.empty(c.k_cache_shape(num_pages), dtype=torch.bfloat16, device="cuda")
                v = torch.empty(c.v_cache_shape(num_pages), dtype=torch.bfloat16, device="cuda")
            caches.append((k, v))
        return caches

    def step(self, ids, caches, page_table, seq_lens, query_start_loc, max_seq_len: int,
             capture: Optional[dict] = None, layers: Optional[int] = None, logit_rows=None):
        """One step over T = ids.shape[0] new tokens.  Writes their K/V into every
        layer's cache and returns fp32 logits [T, vocab] (or [len(logit_rows), vocab]
        for the rows of this step listed in the int32 tensor logit_rows).

        capture: if a dict with key "layers" (a set of layer indices), the inputs
        and outputs of every operation of those layers and of the final norm and
        head are stored in it (as clones)."""
        s = self.shape
        T = ids.shape[0]
        nl = s.layers if layers is None else layers
        num_pages = caches[0][0].shape[0]
        D, Hq, Hk = s.head_dim, s.q_heads, s.kv_heads
        cap_layers = capture.get("layers", set()) if capture is not None else set()

        def keep(name, t):
            capture[name] = t.clone()

        slots = bi_slot_mapping(page_table, seq_lens, query_start_loc, T, s.page_size, num_pages)
        ws = alloc_workspace(max(bi_paged_attention_workspace_size(c, seq_lens.shape[0], T, max_seq_len)
                                 for c in (self.cfg_local, self.cfg_global)))
        h = bi_embedding(self.w["embed"], ids)
        if capture is not None:
            keep("embed.out", h)
        # Each residual add is fused with the RMSNorm that follows it (the next
        # block's input norm); the values are those of the separate add and norm.
        xn = bi_rmsnorm(h, self.w["layers"][0]["g_attn"], s.eps) if nl > 0 else None
        for layer in range(nl):
            W = self.w["layers"][layer]
            c = self.cfg(layer)
            k_cache, v_cache = caches[layer]
            cap = layer in cap_layers
            pre = f"l{layer}."
            qkv = bi_gemm(xn, W["w_qkv"])
            if cap:
                keep(pre + "h_in", h); keep(pre + "xn", xn); keep(pre + "qkv_raw", qkv)
            theta = s.theta_global if s.is_global(layer) else s.theta_local
            # q/k norm and RoPE in place, fused with the cache write of k and v
            bi_qk_norm_rope_kv_write(c, qkv, seq_lens, query_start_loc, W["g_q"], W["g_k"], s.eps, theta, slots,
                                     k_cache, v_cache)
            q = qkv[:, : Hq * D].view(T, Hq, D)
            attn = bi_paged_attention(c, q, k_cache, v_cache, page_table, seq_lens, query_start_loc, max_seq_len,
                                      workspace=ws)
            o = bi_gemm(attn.view(T, Hq * D), W["w_o"])
            h2, xn2 = bi_add_rmsnorm(h, o, W["g_mlp"], s.eps)
            if T <= 16 and not cap:
                # one launch for the gate/up product and the activation (the same bits)
                gu = None
                act = bi_gemm_gated_gelu(xn2, W["w_gu"])
            else:
                gu = bi_gemm(xn2, W["w_gu"])
                act = bi_gated_gelu(gu)
            dn = bi_gemm(act, W["w_down"])
            if layer + 1 < nl:
                h3, xn = bi_add_rmsnorm(h2, dn, self.w["layers"][layer + 1]["g_attn"], s.eps)
            else:
                h3 = bi_add(h2, dn)
            if cap:
                keep(pre + "qkv", qkv); keep(pre + "attn", attn); keep(pre + "o", o); keep(pre + "h_mid", h2)
                keep(pre + "xn2", xn2); keep(pre + "gu", gu); keep(pre + "act", act); keep(pre + "down", dn)
                keep(pre + "h_out", h3)
            h = h3
        if logit_rows is not None:
            h = bi_embedding(h, logit_rows)  # row gather
        xf = bi_rmsnorm(h, self.w["g_final"], s.eps)
        logits = bi_gemm(xf, self.w["embed"], out_dtype=torch.float32)
        if capture is not None:
            keep("final.h", h); keep("final.xn", xf); keep("final.logits", logits)
        return logits
