"""Token order plan (oracle; test infrastructure only).

A plan maps slots of the reordered, padded sequence to original tokens:
``perm[i]`` is the row-major token index n = (t*H + y)*W + x held by slot i,
or -1 for a pad slot. Blocks are runs of B consecutive slots
(DFSAttn, Methodology, designs 1-2: blocks are contiguous runs of the
reordered 1D sequence); ``blk_len[I]`` counts the real tokens of block I.

Orders:
* "row": row-major flattening, the baseline the pages compare against
  (DFSAttn, Experimental results, ablations).
* "hilbert": in-grid cells sorted by their index on the enclosing
  (2**b)**3 Hilbert cube; out-of-grid cells are skipped. Pads go at the tail.
* "frame": frame-major; each frame's H*W tokens in row-major order, padded up
  to whole tiles of B so no tile straddles two frames (LVSA, section 2: the
  attention unit is the frame).
* "hilbert2d": frame-major; inside each frame the cells follow the 2D Hilbert
  curve of the enclosing (2**b)**2 square (b from max(H, W)), out-of-grid
  cells skipped; pads at the tail of the sequence. The per-frame curve the
  3D curve is compared against (DFSAttn, Methodology, design 1, argues for a
  global 3D curve).
* "tile2d" / "cube3d": the 2D and 3D block partitions of VMoBA (abstract:
  layer-wise recurrent 1D-2D-3D partitions, "row" being the 1D one). The grid
  is cut into tiles of 1 x 8 x B/8 (2D) or B/64 x 8 x 8 (3D) cells, tiles at
  the far edges clipped to the grid; every tile is one block: its cells in
  row-major order, then pads up to B. Tiles (blocks) are taken in row-major
  order of their tile coordinates. (Reading: the pages name the partitions
  only; the tile shapes are the ones whose volume is the block size B.)
"""
from __future__ import annotations

import numpy as np

from .hilbert import hilbert_index, hilbert_index_2d, hilbert_order_bits


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def plan(T: int, H: int, W: int, order: str, B: int):
    """Return (perm int64[N_pad], blk_len int64[nb])."""
    T, H, W, B = int(T), int(H), int(W), int(B)
    if min(T, H, W, B) < 1:
        raise ValueError("empty grid or block")
    N = T * H * W
    if order == "row":
        n_pad = _ceil_div(N, B) * B
        perm = np.full(n_pad, -1, dtype=np.int64)
        perm[:N] = np.arange(N)
    elif order == "hilbert":
        b = hilbert_order_bits(T, H, W)
        t, y, x = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
        h = hilbert_index(t.ravel(), y.ravel(), x.ravel(), b)
        # cells were enumerated in row-major order, so the argsort is the
        # list of row-major token indices in curve order (h is unique).
        cells = np.argsort(h, kind="stable")
        n_pad = _ceil_div(N, B) * B
        perm = np.full(n_pad, -1, dtype=np.int64)
        perm[:N] = cells
    elif order == "hilbert2d":
        b = max(1, (max(H, W) - 1).bit_length())
        y, x = np.meshgrid(np.arange(H), np.arange(W), indexing="ij")
        h2 = hilbert_index_2d(y.ravel(), x.ravel(), b)
        frame_cells = np.argsort(h2, kind="stable")      # row-major cell ids in curve order
        n_pad = _ceil_div(N, B) * B
        perm = np.full(n_pad, -1, dtype=np.int64)
        perm[:N] = (np.arange(T)[:, None] * (H * W) + frame_cells[None, :]).ravel()
    elif order == "frame":
        P = H * W
        tiles = _ceil_div(P, B)
        per = tiles * B
        perm = np.full(T * per, -1, dtype=np.int64)
        for f in range(T):
            perm[f * per: f * per + P] = np.arange(f * P, (f + 1) * P)
    elif order in ("tile2d", "cube3d"):
        if order == "tile2d":
            if B % 8:
                raise ValueError("tile2d needs B a multiple of 8")
            tT, tH, tW = 1, 8, B // 8
        else:
            if B % 64:
                raise ValueError("cube3d needs B a multiple of 64")
            tT, tH, tW = B // 64, 8, 8
        slots = []
        for a in range(0, T, tT):
            for b in range(0, H, tH):
                for c in range(0, W, tW):
                    tile = [(t * H + y) * W + x
                            for t in range(a, min(a + tT, T))
                            for y in range(b, min(b + tH, H))
                            for x in range(c, min(c + tW, W))]
                    slots.extend(tile + [-1] * (B - len(tile)))
        perm = np.asarray(slots, dtype=np.int64)
    else:
        raise ValueError(f"unknown order {order!r}")
    nb = perm.size // B
    blk_len = (perm.reshape(nb, B) >= 0).sum(axis=1).astype(np.int64)
    return perm, blk_len


def inverse_perm(perm: np.ndarray, N: int) -> np.ndarray:
    """slot of each original token (inverse of the plan on real tokens)."""
    inv = np.full(int(N), -1, dtype=np.int64)
    idx = np.nonzero(perm >= 0)[0]
    inv[perm[idx]] = idx
    return inv
