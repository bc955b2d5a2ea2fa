"""One attention layer of the path, end to end (oracle; test infrastructure only).

Order of steps: reorder (DFSAttn design 1) -> score (design 2) -> select
(design 3 / LVSA section 2 / VMoBA abstract) -> block-sparse attention ->
restore the original order. Mask caching (DFSAttn design 3): the mask is
recomputed only on refresh steps and reused in between, while attention is
recomputed every step on that step's Q/K/V; pass ``mask=(kv_idx, kv_cnt)`` to
reuse one.
"""
from __future__ import annotations

import numpy as np

from .attn import attn_blocks
from .gather import gather, scatter
from .plan import inverse_perm, plan
from .score import score
from .select import select_lvsa, select_thresh_global, select_topk


def run_layer(T, H, W, order, B, q, k, v, *, select, s=0, agg="mass", k_top=0, tau=0.0,
              ratio=0.0, C=0, T_per=1, step=0, mask=None, rows_tokens=None, max_kv=None):
    """q, k, v: [1, N, heads, D] (torch or numpy). rows_tokens: optional
    per-head arrays of original token indices to evaluate attention on.

    Returns a dict with perm, blk_len, S (or None), kv_idx, kv_cnt, op, lse and o.
    """
    perm, blk_len = plan(T, H, W, order, B)
    N = T * H * W
    qp, kp, vp = gather(q, perm), gather(k, perm), gather(v, perm)
    nh = qp.shape[0]
    S = None
    if mask is not None:
        kv_idx, kv_cnt = mask
    elif select == "lvsa":
        tiles = perm.size // B // T
        kv_idx, kv_cnt = select_lvsa(T, tiles, C, T_per, step, max_kv)
    else:
        S = score(qp, kp, perm, B, s, agg)
        if select == "topk":
            kv_idx, kv_cnt = select_topk(S, k_top, max_kv)
        elif select == "thresh_global":
            kv_idx, kv_cnt = select_thresh_global(S, tau, ratio, max_kv)
        else:
            raise ValueError(select)
    rows = None
    if rows_tokens is not None:
        inv = inverse_perm(perm, N)
        rows = [inv[np.asarray(r, dtype=np.int64)] for r in rows_tokens]
    op, lse = attn_blocks(qp, kp, vp, perm, B, kv_idx, kv_cnt, rows=rows)
    o = scatter(op, perm, N)
    return dict(perm=perm, blk_len=blk_len, S=S, kv_idx=kv_idx, kv_cnt=kv_cnt,
                op=op, lse=lse, o=o, nh=nh)
