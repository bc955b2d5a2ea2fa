"""Pins for the oracle's block selection rules (CPU only).

Pinned against: brute-force ranking with exact Python integers, the
minimality/sufficiency definition of a threshold prefix, the anchor
partition and budget properties stated on the LVSA page, and hand-derived
frame sets (tests/golden/lvsa_T10_C5_P4.txt).
"""
import math
import os

import numpy as np
import pytest

import oracle

ONE = 1 << 62


def _rank(row, j):
    """Position of entry j in the ranking (score desc, index asc), brute force."""
    return sum(1 for i, x in enumerate(row) if x > row[j] or (x == row[j] and i < j))


def _lists(kv_idx, kv_cnt):
    return [[list(kv_idx[g, i, :kv_cnt[g, i]]) for i in range(kv_idx.shape[1])]
            for g in range(kv_idx.shape[0])]


@pytest.mark.parametrize("k", [1, 3, 7, 12])
def test_topk_matches_brute_force_rank(k):
    rng = np.random.default_rng(5)
    S = rng.random((2, 12, 12)).astype(np.float32)
    S[0, 3, :] = 0.5                       # a row of exact ties
    S[1, 4, ::3] = S[1, 4, 1]              # partial ties
    kv_idx, kv_cnt = oracle.select_topk(S, k, max_kv=12)
    for h in range(2):
        for i in range(12):
            row = [float(x) for x in S[h, i]]
            want = sorted(j for j in range(12) if _rank(row, j) < k)
            assert list(kv_idx[h, i, :k]) == want
            assert kv_cnt[h, i] == k
            assert np.all(kv_idx[h, i, k:] == -1)
    assert list(kv_idx[0, 3, :k]) == list(range(k))      # ties go to the lowest index


def test_topk_all_blocks():
    S = np.random.default_rng(6).random((1, 5, 5))
    kv_idx, kv_cnt = oracle.select_topk(S, 5)
    assert np.all(kv_idx == np.arange(5)) and np.all(kv_cnt == 5)


def test_fixed_point():
    assert int(oracle.thresh_fixed_point(0.25)) == 1 << 60
    assert int(oracle.thresh_fixed_point(1.0)) == 1 << 62
    assert int(oracle.thresh_fixed_point(np.float32(3.0) / np.float32(7.0))) == \
        (int(np.float32(3.0 / 7.0).view(np.uint32) & 0x7FFFFF) | 0x800000) << (62 - 23 - 2)
    assert int(oracle.thresh_fixed_point(2.0 ** -70)) == 0


def _mass_rows(rng, nh, nb, peak):
    z = rng.standard_normal((nh, nb, nb)) * peak
    S = np.exp(z - z.max(axis=2, keepdims=True))
    return (S / S.sum(axis=2, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("tau", [0.25, 0.5, 0.9, 1e-12])
def test_threshold_prefix_is_minimal_and_sufficient(tau):
    rng = np.random.default_rng(7)
    S = _mass_rows(rng, 2, 9, 2.0)
    S[1, 2, :] = np.float32(1 / 9)          # all tied
    kv_idx, kv_cnt = oracle.select_thresh_global(S, tau, 0.0)   # budget 0: threshold sets only
    target = math.floor(tau * ONE)
    for h, rows in enumerate(_lists(kv_idx, kv_cnt)):
        for i, sel in enumerate(rows):
            row = [float(x) for x in S[h, i]]
            ranks = sorted(_rank(row, j) for j in sel)
            assert ranks == list(range(len(sel))), "the set is a prefix of the ranking"
            fx = [math.floor(row[j] * ONE) for j in sel]
            assert len(sel) >= 1
            assert sum(fx) >= target or len(sel) == 9
            if len(sel) > 1:
                last = max(sel, key=lambda j: _rank(row, j))
                assert sum(fx) - math.floor(row[last] * ONE) < target
    if tau == 1e-12:
        assert np.all(kv_cnt == 1)


@pytest.mark.parametrize("ratio", [0.0, 0.2, 0.45, 1.0])
def test_global_budget_fill(ratio):
    rng = np.random.default_rng(8)
    nb = 11
    S = _mass_rows(rng, 3, nb, 1.5)
    S[2, :, :] = np.float32(1 / nb)            # a head of exact ties
    base_idx, base_cnt = oracle.select_thresh_global(S, 0.3, 0.0)
    kv_idx, kv_cnt = oracle.select_thresh_global(S, 0.3, ratio)
    K = math.floor(ratio * nb * nb + 0.5)
    assert oracle.budget_pairs(ratio, nb) == K
    for h in range(3):
        T = {(i, j) for i, r in enumerate(_lists(base_idx, base_cnt)[h]) for j in r}
        F = {(i, j) for i, r in enumerate(_lists(kv_idx, kv_cnt)[h]) for j in r}
        assert T <= F
        assert len(F) == max(len(T), K)
        flat = [float(x) for x in S[h].ravel()]
        added = [i * nb + j for (i, j) in F - T]
        left = [p for p in range(nb * nb) if (p // nb, p % nb) not in F]
        if added and left:
            worst_added = max(_rank(flat, p) for p in added)
            best_left = min(_rank(flat, p) for p in left)
            assert worst_added < best_left


def test_budget_schedule_cfg5():
    # 929 blocks: 30% and 10% of 929**2 = 863041 pairs, rounded half up
    assert oracle.budget_pairs(0.30, 929) == 258912
    assert oracle.budget_pairs(0.10, 929) == 86304


def _golden_lvsa(golden_dir):
    out = []
    with open(os.path.join(golden_dir, "lvsa_T10_C5_P4.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                p = [int(v) for v in line.split()]
                out.append((p[0], p[1], p[2:]))
    return out


def test_lvsa_hand_derived(golden_dir):
    for s, t, frames in _golden_lvsa(golden_dir):
        sets = oracle.lvsa_frame_sets(10, 5, 4, s)
        assert sets[t].tolist() == frames


def test_lvsa_anchor_rotation_partitions_frames():
    """Each frame is a global anchor exactly once over T_per consecutive steps."""
    T, C, P = 61, 21, 8
    for s0 in range(0, 9):
        seen = []
        for s in range(s0, s0 + P):
            others = oracle.lvsa_frame_sets(T, T, P, s)   # C >= T: all frames
            assert all(len(a) == T for a in others)
            seen.extend(f for f in range(T) if (f - s) % P == 0)
        assert sorted(seen) == list(range(T))


@pytest.mark.parametrize("step", range(8))
def test_lvsa_constant_budget(step):
    T, C, P = 61, 21, 8
    sets = oracle.lvsa_frame_sets(T, C, P, step)
    anchors = {f for f in range(T) if f % P == step % P}
    for t, A in enumerate(sets):
        A = set(A.tolist())
        assert len(A) == C
        assert t in A
        assert anchors <= A
        W = A - anchors
        outside = [f for f in range(T) if f not in A]
        if W and outside:
            assert max(abs(f - t) for f in W) <= min(abs(f - t) for f in outside)


def test_lvsa_degenerate_cases_are_dense():
    for s in range(3):
        assert all(len(a) == 12 for a in oracle.lvsa_frame_sets(12, 3, 1, s))     # T_per = 1
        assert all(len(a) == 12 for a in oracle.lvsa_frame_sets(12, 12, 4, s))    # C >= T


def test_lvsa_tile_lists_and_cost():
    T, C, P, tiles = 61, 21, 8, 13
    kv_idx, kv_cnt = oracle.select_lvsa(T, tiles, C, P, 3)
    assert kv_idx.shape == (1, T * tiles, C * tiles)
    assert np.all(kv_cnt == C * tiles)
    sets = oracle.lvsa_frame_sets(T, C, P, 3)
    for I in range(T * tiles):
        frames = sorted({int(j) // tiles for j in kv_idx[0, I]})
        assert frames == sets[I // tiles].tolist()
        assert np.all(np.diff(kv_idx[0, I]) > 0)
    # LVSA, complexity: cost grows as T * C * P**2 * d (linear in T for fixed C)
    Pf, D, nh = 1560, 128, 12
    useful = sum(4 * D * nh * Pf * len(a) * Pf for a in sets)
    assert useful == 4 * D * nh * T * C * Pf * Pf


# ---------------------------------------------------------------- DynamicRad radial masks

def _golden_radial(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                head, ids = line.split(":")
                lam, t, j = head.split()
                rows.append((float(lam), int(t), int(j), [int(x) for x in ids.split()]))
    return rows


@pytest.mark.parametrize("name,T,P", [("radial_T5_P4.txt", 5, 4), ("radial_T3_P3.txt", 3, 3)])
def test_radial_hand_derived(golden_dir, name, T, P):
    for lam, t, j, ids in _golden_radial(golden_dir, name):
        kv_idx, kv_cnt = oracle.select_radial(T, P, lam)
        i = t * P + j
        assert list(kv_idx[0, i, :kv_cnt[0, i]]) == ids, (lam, t, j)


@pytest.mark.parametrize("T,P,lam", [(61, 13, 0.0), (61, 13, 0.1), (9, 5, 0.3), (4, 1, 0.0), (33, 24, 0.05)])
def test_radial_window_invariants(T, P, lam):
    """Own frame kept whole; own position kept in every frame; each frame's
    window is one contiguous run of tiles; widths never grow with distance
    and halve (rounded up) each time d + 1 doubles, down to the lam floor."""
    kv_idx, kv_cnt = oracle.select_radial(T, P, lam)
    widths = [oracle.radial_width(d, P, lam) for d in range(T)]
    assert widths[0] == P and all(a >= b for a, b in zip(widths, widths[1:]))
    floor = max(1, int(np.ceil(lam * P)))
    assert all(w >= floor for w in widths)
    k = 0
    while (1 << k) - 1 < T:                       # dyadic bands d + 1 in [2^k, 2^(k+1))
        band = widths[(1 << k) - 1:min((2 << k) - 1, T)]
        assert len(set(band)) == 1
        if k > 0:
            prev = widths[(1 << (k - 1)) - 1]
            assert band[0] == max(-(-prev // 2), floor) or band[0] == floor
        k += 1
    for t in range(T):
        for j in range(P):
            i = t * P + j
            ids = kv_idx[0, i, :kv_cnt[0, i]]
            assert kv_cnt[0, i] == sum(widths[abs(t - f)] for f in range(T))
            f_of, j_of = np.divmod(ids, P)
            for f in range(T):
                js = j_of[f_of == f]
                assert j in js
                assert np.array_equal(js, np.arange(js.min(), js.max() + 1))
                assert js.size == widths[abs(t - f)]


def test_radial_full_factor_is_dense():
    kv_idx, kv_cnt = oracle.select_radial(6, 3, 1.0)
    assert np.all(kv_cnt == 18)


def test_radial_dynamic_union_and_threshold():
    """The dynamic mode keeps the radial window plus every block whose logit
    is within delta of the row's best (float32); delta = 0 adds the row's
    best block(s), a huge delta keeps everything, and growing delta only adds."""
    rng = np.random.default_rng(7)
    T, P, nh = 6, 4, 2
    nb = T * P
    S = rng.standard_normal((nh, nb, nb)).astype(np.float32)
    S[0, 3, 5] = S[0, 3].max()            # a tie for the row's best
    base_idx, base_cnt = oracle.select_radial(T, P, 0.0)
    prev = None
    for delta in (0.0, 0.5, 1.5, 1e9):
        kv_idx, kv_cnt = oracle.select_radial_dynamic(S, T, P, 0.0, delta)
        sets = [[set(kv_idx[h, i, :kv_cnt[h, i]]) for i in range(nb)] for h in range(nh)]
        for h in range(nh):
            for i in range(nb):
                base = set(base_idx[0, i, :base_cnt[0, i]])
                strong = set(np.nonzero(S[h, i] >= np.float32(S[h, i].max()) - np.float32(delta))[0])
                assert sets[h][i] == base | strong
                assert int(np.argmax(S[h, i])) in sets[h][i]
                if prev is not None:
                    assert prev[h][i] <= sets[h][i]
                if delta == 1e9:
                    assert len(sets[h][i]) == nb
        prev = sets
    assert 5 in set(oracle.select_radial_dynamic(S, T, P, 0.0, 0.0)[0][0, 3])


def test_radial_dynamic_hand_derived(golden_dir):
    """The dynamic-threshold reading (best logit minus delta, at or above
    kept) on a hand-derived 2-frame case (tests/golden/radial_dyn_T2_P2.txt):
    a block exactly on the threshold is kept, one just below is dropped, and
    a block a mean-relative rule would keep is dropped."""
    S = np.zeros((1, 4, 4), dtype=np.float32)
    want = {}
    with open(os.path.join(golden_dir, "radial_dyn_T2_P2.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            head, vals = line.split(":")
            head = head.split()
            if head[0] == "S":
                S[0, int(head[1])] = [float(x) for x in vals.split()]
            else:
                want[(float(head[0]), int(head[1]))] = [int(x) for x in vals.split()]
    assert len(want) == 8
    for (delta, i), ids in want.items():
        kv_idx, kv_cnt = oracle.select_radial_dynamic(S, 2, 2, 0.0, delta)
        assert list(kv_idx[0, i, :kv_cnt[0, i]]) == ids, (delta, i)


def test_thresh_difference_explanations():
    """The helper that explains threshold-selection differences between
    float32 and float64 scores: lists from slightly perturbed scores are all
    explained; a planted low-score pair is not."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from _gpu_common import thresh_differences
    rng = np.random.default_rng(5)
    nh, nb = 2, 40
    S = rng.random((nh, nb, nb)) ** 6
    S /= S.sum(axis=2, keepdims=True)
    S32 = np.clip(S + rng.uniform(-1e-3, 1e-3, S.shape), 0, None)   # large enough to move pairs
    tau, ratio = 0.3, 0.12
    idx, cnt = oracle.select_thresh_global(S32, tau, ratio)
    diff, explained = thresh_differences(S, S32, idx, cnt, tau, ratio)
    assert diff > 0 and explained == diff
    # plant the lowest-scoring pair of a row into its list
    i = 3
    j = int(np.argmin(S[0, i]))
    assert j not in set(idx[0, i, :cnt[0, i]])
    row = np.sort(np.append(idx[0, i, :cnt[0, i]], j))
    idx2, cnt2 = idx.copy(), cnt.copy()
    cnt2[0, i] = row.size
    idx2[0, i, :row.size] = row
    diff2, explained2 = thresh_differences(S, S32, idx2, cnt2, tau, ratio)
    assert diff2 == diff + 1 and explained2 == explained
