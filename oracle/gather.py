"""Gather into / scatter out of the reordered layout (oracle; test infrastructure only).

DFSAttn, Methodology, design 1: tokens are reordered before attention; the
inverse reorder restores the original token order afterwards.

Layouts: token-major x[1, N, heads, D] <-> head-major slots xp[heads, N_pad, D]
with ``xp[h, i] = x[0, perm[i], h]`` and zero rows at pad slots.
"""
from __future__ import annotations

import numpy as np


def _as_f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def gather(x, perm: np.ndarray) -> np.ndarray:
    """x [1, N, heads, D] -> xp [heads, N_pad, D] (float64, pads zero)."""
    x = _as_f64(x)
    if x.ndim != 4 or x.shape[0] != 1:
        raise ValueError("expected [1, N, heads, D]")
    _, N, nh, D = x.shape
    out = np.zeros((nh, perm.size, D), dtype=np.float64)
    real = np.nonzero(perm >= 0)[0]
    out[:, real, :] = np.transpose(x[0, perm[real], :, :], (1, 0, 2))
    return out


def scatter(xp: np.ndarray, perm: np.ndarray, N: int) -> np.ndarray:
    """xp [heads, N_pad, D] -> x [1, N, heads, D]; pad slots are dropped."""
    nh, n_pad, D = xp.shape
    out = np.zeros((1, int(N), nh, D), dtype=xp.dtype)
    real = np.nonzero(perm >= 0)[0]
    out[0, perm[real], :, :] = np.transpose(xp[:, real, :], (1, 0, 2))
    return out
