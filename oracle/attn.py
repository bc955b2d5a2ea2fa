"""Block-sparse attention (oracle; test infrastructure only).

DFSAttn, Significance (block-wise execution over reordered tokens) and
DynamicRad, section 2.2 (block-wise aggregation over a shared candidate set):
each query block attends only to the real tokens of the key blocks in its
list; everything else is skipped. Non-causal softmax attention with scale
1/sqrt(D) (reading: the pages state no scale or causality); the log-sum-exp
uses the natural logarithm.

Computed in float64 as the plain two-pass formula: logits, subtract the row
maximum, exponentiate, normalise, weight the values.
"""
from __future__ import annotations

import numpy as np


def attn_blocks(qp: np.ndarray, kp: np.ndarray, vp: np.ndarray, perm: np.ndarray, B: int,
                kv_idx: np.ndarray, kv_cnt: np.ndarray, scale: float | None = None,
                rows: list | None = None):
    """qp, kp, vp [heads, N_pad, D] float64; kv_idx [G, nb, max_kv] with G = heads or 1.

    rows: optional per-head arrays of slot indices to evaluate (others are left 0).
    Returns (op [heads, N_pad, D], lse [heads, N_pad]); pad query rows stay 0.
    """
    nh, n_pad, D = qp.shape
    nb = n_pad // B
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    real = perm >= 0
    op = np.zeros_like(qp)
    lse = np.zeros((nh, n_pad), dtype=np.float64)
    for h in range(nh):
        g = h if kv_idx.shape[0] > 1 else 0
        if rows is None:
            want = np.nonzero(real)[0]
        else:
            want = np.asarray(rows[h], dtype=np.int64)
            want = want[real[want]]
        blocks = want // B
        for I in np.unique(blocks):
            qi = want[blocks == I]
            sel = kv_idx[g, I, :kv_cnt[g, I]].astype(np.int64)
            if sel.size == 0:
                continue
            keys = (sel[:, None] * B + np.arange(B)[None, :]).ravel()
            keys = keys[real[keys]]
            logits = (qp[h, qi] @ kp[h, keys].T) * scale
            m = logits.max(axis=1, keepdims=True)
            e = np.exp(logits - m)
            l = e.sum(axis=1, keepdims=True)
            op[h, qi] = (e @ vp[h, keys]) / l
            lse[h, qi] = (m + np.log(l))[:, 0]
    return op, lse


def attn_dense(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float | None = None):
    """Dense softmax attention on token-major [1, N, heads, D] float64 arrays."""
    _, N, nh, D = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros_like(q)
    for h in range(nh):
        logits = (q[0, :, h] @ k[0, :, h].T) * scale
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        out[0, :, h] = (e @ v[0, :, h]) / e.sum(axis=1, keepdims=True)
    return out


def block_mass(qp: np.ndarray, kp: np.ndarray, perm: np.ndarray, B: int, rows: list,
               scale: float | None = None) -> np.ndarray:
    """Exact attention mass of query rows on key blocks (the quantity block
    selection tries to keep: DFSAttn, Methodology, designs 2-3 estimate it from
    pooled scores). For each head h and slot r = rows[h][i]: the dense softmax
    over every real key, summed over the real keys of each block J.
    Returns [heads, len(rows[h]), nb] float64."""
    nh, n_pad, D = qp.shape
    nb = n_pad // B
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    real = perm >= 0
    keys = np.nonzero(real)[0]
    out = np.zeros((nh, len(rows[0]), nb), dtype=np.float64)
    for h in range(nh):
        r = np.asarray(rows[h], dtype=np.int64)
        logits = (qp[h, r] @ kp[h, keys].T) * scale
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        np.add.at(out[h].T, keys // B, p.T)
    return out


def recall(mass: np.ndarray, rows: list, B: int, kv_idx: np.ndarray, kv_cnt: np.ndarray) -> np.ndarray:
    """Attention recall of a selection: for each sampled row, the share of its
    exact attention mass that falls on the key blocks listed for its query
    block. [heads, rows]."""
    nh = mass.shape[0]
    out = np.zeros((nh, mass.shape[1]), dtype=np.float64)
    for h in range(nh):
        g = h if kv_idx.shape[0] > 1 else 0
        for i, r in enumerate(np.asarray(rows[h], dtype=np.int64)):
            I = r // B
            out[h, i] = mass[h, i, kv_idx[g, I, :kv_cnt[g, I]]].sum()
    return out


def attn_blocks_bwd(qp: np.ndarray, kp: np.ndarray, vp: np.ndarray, dop: np.ndarray, perm: np.ndarray,
                    B: int, kv_idx: np.ndarray, kv_cnt: np.ndarray, scale: float | None = None):
    """Gradients of the block-sparse attention of attn_blocks (the same
    attended key set per query block) with respect to Q, K and V, given the
    output gradient dO. Plain softmax calculus per query row over its
    attended keys, in float64:
        P = softmax(scale * q K^T),  dV += P^T dO,  dP = dO V^T,
        dS = P * (dP - rowsum(dP * P)),  dQ = scale * dS K,  dK += scale * dS^T Q.
    Pad query rows and pad keys carry no gradient.
    Returns (dq, dk, dv), each [heads, N_pad, D]."""
    nh, n_pad, D = qp.shape
    nb = n_pad // B
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    real = perm >= 0
    dq, dk, dv = np.zeros_like(qp), np.zeros_like(kp), np.zeros_like(vp)
    for h in range(nh):
        g = h if kv_idx.shape[0] > 1 else 0
        for I in range(nb):
            qi = np.arange(I * B, (I + 1) * B)
            qi = qi[real[qi]]
            sel = kv_idx[g, I, :kv_cnt[g, I]].astype(np.int64)
            if qi.size == 0 or sel.size == 0:
                continue
            keys = (sel[:, None] * B + np.arange(B)[None, :]).ravel()
            keys = keys[real[keys]]
            logits = (qp[h, qi] @ kp[h, keys].T) * scale
            P = np.exp(logits - logits.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dO = dop[h, qi]
            dv[h, keys] += P.T @ dO
            dP = dO @ vp[h, keys].T
            dS = P * (dP - (dP * P).sum(axis=1, keepdims=True))
            dq[h, qi] += scale * (dS @ kp[h, keys])
            dk[h, keys] += scale * (dS.T @ qp[h, qi])
    return dq, dk, dv
