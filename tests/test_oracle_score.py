"""Pins for the oracle's hierarchical block scoring (CPU only).

Pinned against: hand-computed values (tests/golden/mass_tiny.txt), the exact
block attention mass of dense attention (brute force with scipy's softmax),
piecewise-constant inputs where every sub-block size must agree with the
token-level mass, and closed-form uniform cases.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import softmax

import oracle


def _golden(golden_dir):
    out = []
    with open(os.path.join(golden_dir, "mass_tiny.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                case, s, I, J, expr = line.split(None, 4)
                out.append((case, int(s), int(I), int(J), eval(expr, {"math": math})))
    return out


def test_hand_computed_scores(golden_dir):
    ln2, ln3 = math.log(2), math.log(3)
    full_q = np.array([1, 0, 2, 0], float)[None, :, None]
    full_k = np.array([0, ln2, ln3, 0], float)[None, :, None]
    pad_q = np.array([1, 0, 2, 0], float)[None, :, None]
    pad_k = np.array([0, ln2, ln3, 0], float)[None, :, None]
    perm_full = np.arange(4)
    perm_pad = np.array([0, 1, 2, -1])
    pad_q[0, 3, 0] = pad_k[0, 3, 0] = 0.0
    cache = {}
    for case, s, I, J, val in _golden(golden_dir):
        if case == "full":
            S = cache.setdefault(("full", s), oracle.score_mass(full_q, full_k, perm_full, 2, s))
        elif case == "max":
            S = cache.setdefault(("max", s), oracle.score_max(full_q, full_k, perm_full, 2, s))
        else:
            S = cache.setdefault(("pad", s), oracle.score_mass(pad_q, pad_k, perm_pad, 2, s))
        assert S[0, I, J] == pytest.approx(val, rel=1e-14, abs=1e-15)


def _dense_block_mass(qp, kp, perm, B):
    """Exact block attention mass: token-level softmax over all real keys,
    summed over each key block, averaged over each query block's real rows."""
    nh, n_pad, D = qp.shape
    nb = n_pad // B
    real = perm >= 0
    out = np.zeros((nh, nb, nb))
    for h in range(nh):
        A = softmax(qp[h][real] @ kp[h][real].T / math.sqrt(D), axis=1)
        slots = np.nonzero(real)[0]
        for I in range(nb):
            rows = (slots // B) == I
            for J in range(nb):
                cols = (slots // B) == J
                out[h, I, J] = A[np.ix_(rows, cols)].sum(axis=1).mean()
    return out


@pytest.mark.parametrize("N,B,D", [(64, 16, 8), (52, 16, 8), (37, 8, 4)])
def test_subblock_size_one_is_exact_block_mass(N, B, D):
    rng = np.random.default_rng(1)
    perm, _ = oracle.plan(1, 1, N, "row", B)
    x = rng.standard_normal((2, 1, N, D))
    qp = oracle.gather(x[0].reshape(1, N, 1, D), perm)
    kp = oracle.gather(x[1].reshape(1, N, 1, D), perm)
    S = oracle.score_mass(qp, kp, perm, B, 1)
    np.testing.assert_allclose(S, _dense_block_mass(qp, kp, perm, B), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("s", [2, 4, 8, 16])
def test_piecewise_constant_inputs_match_token_level(s):
    """If every sub-block holds identical tokens, scoring on sub-block means
    with count weights must reproduce the token-level block attention mass."""
    rng = np.random.default_rng(2)
    B, D, N = 16, 6, 16 * 5 - 3       # ragged last block
    perm, _ = oracle.plan(1, 1, N, "row", B)
    n_pad = perm.size
    qs = rng.standard_normal((n_pad // s, D))
    ks = rng.standard_normal((n_pad // s, D))
    q = np.repeat(qs, s, axis=0)[:N].reshape(1, N, 1, D)
    k = np.repeat(ks, s, axis=0)[:N].reshape(1, N, 1, D)
    qp, kp = oracle.gather(q, perm), oracle.gather(k, perm)
    S = oracle.score_mass(qp, kp, perm, B, s)
    np.testing.assert_allclose(S, _dense_block_mass(qp, kp, perm, B), rtol=1e-12, atol=1e-14)


def test_rows_sum_to_one_and_uniform_case():
    rng = np.random.default_rng(3)
    perm, blk_len = oracle.plan(2, 5, 7, "hilbert", 16)
    N = 70
    x = rng.standard_normal((1, N, 3, 8))
    qp = kp = oracle.gather(x, perm)
    S = oracle.score_mass(qp, kp, perm, 16, 4)
    np.testing.assert_allclose(S.sum(axis=2), 1.0, atol=1e-13)
    const = oracle.gather(np.ones((1, N, 3, 8)), perm)
    U = oracle.score_mass(const, const, perm, 16, 4)
    # equal logits: each key block receives its share of real tokens
    np.testing.assert_allclose(U, np.broadcast_to(blk_len / N, U.shape), atol=1e-15)


def test_pool_is_mean_of_real_tokens():
    perm = np.array([0, 1, 2, -1, 3, -1, -1, -1])
    x = np.arange(4 * 2, dtype=float).reshape(1, 4, 1, 2)
    xp = oracle.gather(x, perm)
    means, counts = oracle.pool(xp, perm, 2)
    assert counts.tolist() == [2, 1, 1, 0]
    np.testing.assert_array_equal(means[0], [[1, 2], [4, 5], [6, 7], [0, 0]])


def test_max_aggregation_brute_force():
    rng = np.random.default_rng(4)
    N, B, s, D = 40, 8, 4, 5
    perm, _ = oracle.plan(1, 1, N, "row", B)
    q = rng.standard_normal((1, N, 1, D))
    k = rng.standard_normal((1, N, 1, D))
    qp, kp = oracle.gather(q, perm), oracle.gather(k, perm)
    S = oracle.score_max(qp, kp, perm, B, s)
    nb = perm.size // B
    for I in range(nb):
        for J in range(nb):
            best = -np.inf
            for u in range(I * B // s, (I + 1) * B // s):
                for v in range(J * B // s, (J + 1) * B // s):
                    qu = [perm[i] for i in range(u * s, u * s + s) if perm[i] >= 0]
                    kv = [perm[i] for i in range(v * s, v * s + s) if perm[i] >= 0]
                    if qu and kv:
                        z = float(np.mean(q[0, qu, 0], axis=0) @ np.mean(k[0, kv, 0], axis=0)) / math.sqrt(D)
                        best = max(best, z)
            assert S[0, I, J] == pytest.approx(best, rel=1e-12, abs=1e-12)
