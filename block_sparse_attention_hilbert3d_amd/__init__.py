"""MI355X-native dynamic block-sparse attention over Hilbert-reordered video tokens.

The computation lives in libhsa.so (hand-written gfx950 HIP kernels behind a C
ABI, declared in include/hsa.h); this package only marshals arguments to it.
"""
from .binding import (HsaError, hsa_attn, hsa_attn_bwd, hsa_attn_tokens, hsa_attn_order, hsa_block_mass, hsa_perm, hsa_plan, hsa_plan_size,
                      hsa_score, hsa_select, hsa_select_list_width, hsa_select_noalloc, hsa_unperm, lib,
                      make_params)
from .layer import SparseAttentionLayer, layer_for_workload, vmoba_order

__all__ = ["HsaError", "hsa_attn", "hsa_attn_bwd", "hsa_attn_tokens", "hsa_attn_order", "hsa_block_mass", "hsa_perm", "hsa_plan", "hsa_plan_size", "hsa_score",
           "hsa_select", "hsa_select_list_width", "hsa_select_noalloc", "hsa_unperm", "lib", "make_params", "SparseAttentionLayer",
           "layer_for_workload", "vmoba_order"]
