"""Block selection (oracle; test infrastructure only).

Three rules, each producing per-query-block lists of key blocks in ascending
order (the shared candidate-set format of DynamicRad, section 2.2: one list
per query block, consumed block-wise by the attention kernel). Lists are
returned densely as (kv_idx int32[G, nb, max_kv] filled with -1 past the
count, kv_cnt int32[G, nb]) where G is the number of heads, or 1 for a
head-shared mask.

Ranking ties: equal scores are ordered by the lower block index (lower
linear pair index for the global ranking).
"""
from __future__ import annotations

import math

import numpy as np

FIXED_ONE = 1 << 62   # fixed-point unit for exact, order-independent prefix sums


def _pack(lists, nb, max_kv):
    G = len(lists)
    kv_idx = np.full((G, nb, max_kv), -1, dtype=np.int32)
    kv_cnt = np.zeros((G, nb), dtype=np.int32)
    for g, rows in enumerate(lists):
        for i, row in enumerate(rows):
            row = np.sort(np.asarray(row, dtype=np.int64))
            if row.size > max_kv:
                raise ValueError("max_kv too small for the selection")
            kv_idx[g, i, :row.size] = row
            kv_cnt[g, i] = row.size
    return kv_idx, kv_cnt


def _rank_desc(row: np.ndarray) -> np.ndarray:
    """Indices of a score row, highest score first, ties to the lower index."""
    return np.argsort(-np.asarray(row), kind="stable")


def select_topk(S: np.ndarray, k: int, max_kv: int | None = None):
    """DFSAttn, Methodology, designs 2-3: keep the k most important key blocks
    of every query block under a sparsity budget (pure ranking; the diagonal
    block is not forced)."""
    nh, nb, nb2 = S.shape
    if nb != nb2:
        raise ValueError("square block grid expected")
    k = int(k)
    if not 1 <= k <= nb:
        raise ValueError("k out of range")
    max_kv = k if max_kv is None else int(max_kv)
    lists = [[_rank_desc(S[h, i])[:k] for i in range(nb)] for h in range(nh)]
    return _pack(lists, nb, max_kv)


def thresh_fixed_point(x) -> np.ndarray:
    """floor(x * 2**62) for 0 <= x (exact: a power-of-two scaling then floor)."""
    a = np.asarray(x, dtype=np.float64)
    if np.any(a < 0) or np.any(~np.isfinite(a)):
        raise ValueError("threshold scores must be finite and non-negative")
    return np.floor(a * float(FIXED_ONE)).astype(np.uint64)


def budget_pairs(ratio: float, nb: int) -> int:
    """Global budget in block pairs: ratio * nb**2, rounded half up."""
    return int(math.floor(float(ratio) * float(nb * nb) + 0.5))


def select_thresh_global(S: np.ndarray, tau: float, ratio: float, max_kv: int | None = None):
    """VMoBA abstract: threshold selection (the number of key blocks a query
    block attends to is set by cumulative similarity) combined with global
    selection over the whole head; DFSAttn, Methodology, design 3: a budget
    that shrinks over the denoising steps.

    Reading: per query block I, T_I is the shortest prefix of its key blocks
    ranked by score whose summed score reaches tau (at least one block; sums
    in 2**-62 fixed point so they are exact and order-free). Then, per head,
    all (I, J) pairs are ranked by score (ties: lower I*nb + J) and pairs not
    yet chosen are added in rank order until the head holds
    K = round(ratio * nb**2) pairs. T is never trimmed, so a head holds
    max(|T|, K) pairs.
    """
    nh, nb, _ = S.shape
    max_kv = nb if max_kv is None else int(max_kv)
    target = int(math.floor(float(tau) * float(FIXED_ONE)))
    K = budget_pairs(ratio, nb)
    fixed = thresh_fixed_point(S)
    lists = []
    for h in range(nh):
        chosen = np.zeros((nb, nb), dtype=bool)
        for i in range(nb):
            order = _rank_desc(S[h, i])
            total = 0
            n = nb
            for pos, j in enumerate(order):
                total += int(fixed[h, i, j])
                if total >= target:
                    n = pos + 1
                    break
            chosen[i, order[:max(1, n)]] = True
        need = K - int(chosen.sum())
        if need > 0:
            ranked = _rank_desc(S[h].ravel())
            free = ranked[~chosen.ravel()[ranked]]
            chosen.ravel()[free[:need]] = True
        lists.append([np.nonzero(chosen[i])[0] for i in range(nb)])
    return _pack(lists, nb, max_kv)


def lvsa_frame_sets(T: int, C: int, T_per: int, step: int):
    """LVSA, section 2: the frames a query frame t attends to,
    A(t) = G_s u W(t).

    * G_s, rotating global anchors: the frames f with f = step (mod T_per),
      so over T_per consecutive steps every frame is an anchor exactly once.
    * W(t), expanded local window: the nominal window has C - |G_s| frames;
      where it would overlap anchors it extends further, so W(t) is the
      C - |G_s| non-anchor frames nearest to t (ties: the earlier frame), at
      least one, capped by the number of non-anchor frames. Hence
      |A(t)| = C whenever T >= C > |G_s|, and t is always in A(t).
    Returns a list of sorted frame arrays, one per query frame.
    """
    T, C, T_per = int(T), int(C), int(T_per)
    if T < 1 or C < 1 or T_per < 1:
        raise ValueError("T, C and T_per must be positive")
    r = int(step) % T_per
    anchors = [f for f in range(T) if f % T_per == r]
    others = [f for f in range(T) if f % T_per != r]
    nw = min(max(C - len(anchors), 1), len(others))
    sets = []
    for t in range(T):
        window = sorted(others, key=lambda f: (abs(f - t), f))[:nw]
        sets.append(np.array(sorted(set(anchors) | set(window)), dtype=np.int64))
    return sets


def select_lvsa(T: int, tiles_per_frame: int, C: int, T_per: int, step: int,
                max_kv: int | None = None):
    """Head-shared tile lists for the LVSA frame mask: every tile of query
    frame t lists every tile of every frame in A(t), ascending."""
    sets = lvsa_frame_sets(T, C, T_per, step)
    n = int(tiles_per_frame)
    rows = []
    for t in range(T):
        tiles = np.concatenate([np.arange(f * n, (f + 1) * n) for f in sets[t]])
        rows.extend([tiles] * n)
    width = max(len(r) for r in rows)
    max_kv = width if max_kv is None else int(max_kv)
    return _pack([rows], T * n, max_kv)


def radial_width(d: int, tiles_per_frame: int, lam: float) -> int:
    """DynamicRad, section 2 item 2: a logarithmic radial window whose size
    decays exponentially with temporal distance, with a long-range factor.

    Reading: at temporal distance d the window keeps ceil(P / 2**k) of the
    P tiles of the key frame, k = floor(log2(d + 1)) (the window halves each
    time the distance doubles: d = 0 keeps the whole frame, d = 1..2 half,
    d = 3..6 a quarter, ...); the long-range factor lam in [0, 1] is a floor,
    at least ceil(lam * P) tiles of every frame, so distant (for example
    periodic) frames keep a share; at least one tile, at most P."""
    P = int(tiles_per_frame)
    k = int(d + 1).bit_length() - 1
    w = max(-(-P // (1 << k)), int(math.ceil(float(lam) * P)), 1)
    return min(w, P)


def radial_window(j: int, d: int, tiles_per_frame: int, lam: float):
    """Tile indices (within a key frame) kept for query tile j at distance d:
    the radial_width nearest tiles to position j, nearest first with ties to
    the lower index (a tile's row-major position in its frame stands for its
    spatial place)."""
    P = int(tiles_per_frame)
    w = radial_width(d, P, lam)
    return np.array(sorted(sorted(range(P), key=lambda x: (abs(x - j), x))[:w]), dtype=np.int64)


def select_radial(T: int, tiles_per_frame: int, lam: float, max_kv: int | None = None):
    """DynamicRad static-ratio mode (section 2 item 1): every query tile keeps,
    in every frame, the radial window around its own position for that
    frame's temporal distance. Geometry only, so one list set for all heads
    (the shared candidate set of section 2 item 2). Blocks are frame tiles:
    block t*P + j is tile j of frame t."""
    T, P = int(T), int(tiles_per_frame)
    rows = []
    for t in range(T):
        for j in range(P):
            rows.append(np.concatenate([f * P + radial_window(j, abs(t - f), P, lam) for f in range(T)]))
    width = max(len(r) for r in rows)
    max_kv = width if max_kv is None else int(max_kv)
    return _pack([rows], T * P, max_kv)


def select_radial_dynamic(S32: np.ndarray, T: int, tiles_per_frame: int, lam: float, delta: float,
                          max_kv: int | None = None):
    """DynamicRad dynamic-threshold mode (section 2 item 1): pre-softmax logits
    serve as importance and a pair outside the radial window is kept when its
    logit clears a threshold.

    Reading: S32 holds float32 block logits (MAX aggregation of sub-block
    logits, [nh][nb][nb]); the threshold of row I is its best logit minus
    delta (weights within a factor e**-delta of the row's strongest block),
    formed and compared in float32; each head keeps the union of the radial
    window and the blocks at or above the threshold."""
    T, P = int(T), int(tiles_per_frame)
    nb = T * P
    S32 = np.asarray(S32, dtype=np.float32)
    base, _ = select_radial(T, P, lam)
    lists = []
    for h in range(S32.shape[0]):
        rows = []
        for i in range(nb):
            thr = np.float32(S32[h, i].max()) - np.float32(delta)
            strong = np.nonzero(S32[h, i] >= thr)[0]
            rows.append(np.union1d(base[0, i][base[0, i] >= 0], strong))
        lists.append(rows)
    max_kv = nb if max_kv is None else int(max_kv)
    return _pack(lists, nb, max_kv)
