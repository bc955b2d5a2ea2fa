"""3D Hilbert curve index (oracle; test infrastructure only).

DFSAttn, Methodology, design 1: all video tokens are reordered along one
global 3D Hilbert curve before attention, so that runs of consecutive tokens
(blocks) are compact spatiotemporal neighbourhoods.

The pages name no particular Hilbert construction. This oracle uses John
Skilling's transpose formulation ("Programming the Hilbert curve", AIP Conf.
Proc. 707, 2004): the axes are mapped to a "transposed" index by undoing the
excess work of the curve level by level and then Gray-encoding; the integer
index interleaves the transposed words most-significant bit first, axis 0
most significant. Axes are (t, y, x) -> (X0, X1, X2).

Only the encoding direction (coordinates -> index) is implemented here; the
HIP plan kernel implements the decoding direction, so the two sides share no
arithmetic and agreement is a real check.
"""
from __future__ import annotations

import numpy as np


def hilbert_order_bits(T: int, H: int, W: int) -> int:
    """Bits per axis of the enclosing cube: the smallest b >= 1 with
    2**b >= max(T, H, W)."""
    m = max(int(T), int(H), int(W))
    return max(1, (m - 1).bit_length())


def hilbert_index(t, y, x, b: int) -> np.ndarray:
    """Hilbert index of cells (t, y, x) on the (2**b)**3 cube (vectorised)."""
    X0 = np.array(t, dtype=np.int64, copy=True)
    X1 = np.array(y, dtype=np.int64, copy=True)
    X2 = np.array(x, dtype=np.int64, copy=True)
    if b < 1:
        raise ValueError("b must be >= 1")
    lim = 1 << b
    for a in (X0, X1, X2):
        if a.size and (a.min() < 0 or a.max() >= lim):
            raise ValueError("coordinate outside the cube")
    X = [X0, X1, X2]
    top = 1 << (b - 1)

    # Undo the curve's excess work, from the top level down: at level Q, if
    # axis i has the level bit set, the lower bits of axis 0 are inverted;
    # otherwise the lower bits of axes 0 and i are swapped.
    q = top
    while q > 1:
        low = q - 1
        for i in range(3):
            set_i = (X[i] & q) != 0
            if i == 0:
                X[0] = np.where(set_i, X[0] ^ low, X[0])
            else:
                swap = (X[0] ^ X[i]) & low
                swap = np.where(set_i, 0, swap)
                inv = np.where(set_i, low, 0)
                X[0] = X[0] ^ inv ^ swap
                X[i] = X[i] ^ swap
        q >>= 1

    # Gray encode across the axes.
    X[1] = X[1] ^ X[0]
    X[2] = X[2] ^ X[1]
    flip = np.zeros_like(X[0])
    q = top
    while q > 1:
        flip = np.where((X[2] & q) != 0, flip ^ (q - 1), flip)
        q >>= 1
    X = [a ^ flip for a in X]

    # Interleave: at each level (most significant first) the bits of X0, X1,
    # X2 become three consecutive index bits, X0's the most significant.
    h = np.zeros_like(X[0])
    for level in range(b - 1, -1, -1):
        for i in range(3):
            h = (h << 1) | ((X[i] >> level) & 1)
    return h


def hilbert_index_2d(y, x, b: int) -> np.ndarray:
    """Hilbert index of cells (y, x) on the (2**b)**2 square (vectorised), by
    the same transpose construction in two dimensions: undo the excess work
    level by level, Gray-encode, interleave the two words, y most significant."""
    X = [np.array(y, dtype=np.int64, copy=True), np.array(x, dtype=np.int64, copy=True)]
    if b < 1:
        raise ValueError("b must be >= 1")
    lim = 1 << b
    for a in X:
        if a.size and (a.min() < 0 or a.max() >= lim):
            raise ValueError("coordinate outside the square")
    top = 1 << (b - 1)
    q = top
    while q > 1:
        low = q - 1
        X[0] = np.where((X[0] & q) != 0, X[0] ^ low, X[0])
        set_1 = (X[1] & q) != 0
        swap = np.where(set_1, 0, (X[0] ^ X[1]) & low)
        X[0] = X[0] ^ np.where(set_1, low, 0) ^ swap
        X[1] = X[1] ^ swap
        q >>= 1
    X[1] = X[1] ^ X[0]
    flip = np.zeros_like(X[0])
    q = top
    while q > 1:
        flip = np.where((X[1] & q) != 0, flip ^ (q - 1), flip)
        q >>= 1
    X = [a ^ flip for a in X]
    h = np.zeros_like(X[0])
    for level in range(b - 1, -1, -1):
        for i in range(2):
            h = (h << 1) | ((X[i] >> level) & 1)
    return h
