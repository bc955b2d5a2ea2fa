"""Hierarchical block scoring (oracle; test infrastructure only).

DFSAttn, Methodology, design 2: instead of pooling whole blocks, each block is
split into smaller sub-blocks, attention scores are computed between
sub-block summaries, and those scores are aggregated into a block-to-block
importance.

Readings (the page gives no formula):
* pooling is the arithmetic mean over a sub-block's real (non-pad) tokens;
* the logit scale is 1/sqrt(D), as in attention;
* MASS aggregation: for each query sub-block u, a softmax over all key
  sub-blocks v weighted by their token counts c_v estimates how attention
  mass spreads over keys; a block score S[I, J] is the token-weighted mean
  over u in I of the mass u sends to the sub-blocks of J. Rows of S sum to 1.
  (Averaging raw sub-block logits would equal coarse block pooling by
  bilinearity, so it could not be the refinement the page describes.)
  With sub-block size 1 this is exactly the block attention mass of dense
  attention; with sub-block size B it is the count-weighted softmax of
  block-pooled logits.
* MAX aggregation (alternative): the largest sub-block logit between I and J.
"""
from __future__ import annotations

import numpy as np


def pool(xp: np.ndarray, perm: np.ndarray, s: int):
    """Sub-block means. xp [heads, N_pad, D] -> (means [heads, nsub, D], counts int64[nsub])."""
    nh, n_pad, D = xp.shape
    if n_pad % s:
        raise ValueError("sub-block size must divide the padded length")
    nsub = n_pad // s
    real = (perm >= 0).reshape(nsub, s)
    counts = real.sum(axis=1).astype(np.int64)
    sums = (xp.reshape(nh, nsub, s, D) * real[None, :, :, None]).sum(axis=2)
    means = np.zeros_like(sums)
    nz = counts > 0
    means[:, nz, :] = sums[:, nz, :] / counts[nz][None, :, None]
    return means, counts


def _subblock_logits(qp, kp, perm, s, scale):
    qbar, counts = pool(qp, perm, s)
    kbar, _ = pool(kp, perm, s)
    z = np.matmul(qbar, np.transpose(kbar, (0, 2, 1))) * scale
    return z, counts


def score_mass(qp: np.ndarray, kp: np.ndarray, perm: np.ndarray, B: int, s: int,
               scale: float | None = None) -> np.ndarray:
    """MASS block scores S [heads, nb, nb] (float64)."""
    nh, n_pad, D = qp.shape
    if B % s:
        raise ValueError("sub-block size must divide the block size")
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    nb, r = n_pad // B, B // s
    z, c = _subblock_logits(qp, kp, perm, s, scale)
    live = c > 0
    z = np.where(live[None, None, :], z, -np.inf)
    m = z.max(axis=2, keepdims=True)
    e = c[None, None, :] * np.exp(z - m)
    p = e / e.sum(axis=2, keepdims=True)
    p[:, ~live, :] = 0.0                               # empty query sub-blocks carry no weight
    to_block = p.reshape(nh, nb * r, nb, r).sum(axis=3)    # mass of u onto each key block
    weighted = c[None, :, None] * to_block
    num = weighted.reshape(nh, nb, r, nb).sum(axis=2)
    den = c.reshape(nb, r).sum(axis=1).astype(np.float64)
    out = np.zeros_like(num)
    ok = den > 0
    out[:, ok, :] = num[:, ok, :] / den[ok][None, :, None]
    return out


def score_max(qp: np.ndarray, kp: np.ndarray, perm: np.ndarray, B: int, s: int,
              scale: float | None = None) -> np.ndarray:
    """MAX block scores: largest sub-block logit between blocks (-inf if a block is empty)."""
    nh, n_pad, D = qp.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    nb, r = n_pad // B, B // s
    z, c = _subblock_logits(qp, kp, perm, s, scale)
    live = c > 0
    z = np.where(live[None, :, None] & live[None, None, :], z, -np.inf)
    return z.reshape(nh, nb, r, nb, r).max(axis=(2, 4))


def score(qp, kp, perm, B, s, agg="mass", scale=None):
    if agg == "mass":
        return score_mass(qp, kp, perm, B, s, scale)
    if agg == "max":
        return score_max(qp, kp, perm, B, s, scale)
    raise ValueError(agg)
