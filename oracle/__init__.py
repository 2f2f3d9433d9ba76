"""CPU oracle for batch-invariant paged attention, RMSNorm and the matrix product.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or tables) and imports nothing from it.

Everything here is plain numpy in float64 over the exact widening of the bf16
input bits.  Each function is the plain definition of what the GPU path
computes; none of the blocking, splitting or fusion of the GPU kernels is
reproduced, except where a function's docstring says it models one on purpose
(``split_partials_ref`` / ``merge_ref`` model the fixed-size key split and the
fixed-order log-sum-exp merge, so the split phase can be checked on its own).

Logical KV-cache layout used by the oracle (independent of the GPU layout):
``cache[page, slot_in_page, kv_head, d]``.
"""
from .paging import slot_mapping_ref, kv_write_ref, gather_prefix, row_positions
from .attention import (attention_ref, attention_probs_ref, split_partials_ref, merge_ref,
                        dense_attention_bruteforce, LOG2E)
from .rmsnorm import rmsnorm_ref
from .gemm import gemm_ref, gemm_abs_ref
from .decoder import embedding_ref, rope_ref, qk_norm_rope_ref, add_ref, gated_gelu_ref, gelu_tanh, argmax_ref
from .prefix_cache import PrefixCacheRef

__all__ = [
    "slot_mapping_ref", "kv_write_ref", "gather_prefix", "row_positions",
    "attention_ref", "attention_probs_ref", "split_partials_ref", "merge_ref",
    "dense_attention_bruteforce", "LOG2E", "rmsnorm_ref", "gemm_ref", "gemm_abs_ref",
    "embedding_ref", "rope_ref", "qk_norm_rope_ref", "add_ref", "gated_gelu_ref", "gelu_tanh",
    "PrefixCacheRef", "argmax_ref",
]
