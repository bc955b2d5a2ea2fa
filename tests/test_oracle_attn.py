"""Pins for the oracle's block-sparse attention (CPU only).

Pinned against: torch's float64 scaled_dot_product_attention when every
block is kept (a special case that must reduce to dense attention),
logsumexp, masking invariants (keys outside the list and pad slots cannot
matter), constant values, and row-subset consistency.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def _all_blocks(nh, nb):
    kv_idx = np.broadcast_to(np.arange(nb, dtype=np.int32), (nh, nb, nb)).copy()
    return kv_idx, np.full((nh, nb), nb, dtype=np.int32)


@pytest.mark.parametrize("idx", [1, 2])
def test_full_keep_equals_dense_sdpa(idx):
    w = wl.get(idx)
    q, k, v = wl.make_qkv(w, 0)
    perm, _ = oracle.plan(w.T, w.H, w.W, w.order, w.B)
    nb = perm.size // w.B
    qp, kp, vp = (oracle.gather(x, perm) for x in (q, k, v))
    op, lse = oracle.attn_blocks(qp, kp, vp, perm, w.B, *_all_blocks(w.heads, nb))
    o = oracle.scatter(op, perm, w.N)
    qt, kt, vt = (x.double().permute(0, 2, 1, 3) for x in (q, k, v))    # [1, heads, N, D]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt).permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)
    logits = torch.einsum("bhnd,bhmd->bhnm", qt, kt) / np.sqrt(w.D)
    ref_lse = torch.logsumexp(logits, dim=-1)[0].numpy()        # [heads, N]
    inv = oracle.inverse_perm(perm, w.N)
    np.testing.assert_allclose(lse[:, inv], ref_lse, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(o, oracle.attn_dense(*(x.double().numpy() for x in (q, k, v))),
                               rtol=1e-10, atol=1e-12)


def _random_case(seed=9, N=100, B=16, D=8, nh=2):
    rng = np.random.default_rng(seed)
    perm, _ = oracle.plan(1, 1, N, "row", B)
    xs = [oracle.gather(rng.standard_normal((1, N, nh, D)), perm) for _ in range(3)]
    nb = perm.size // B
    sel = np.stack([np.stack([np.sort(rng.choice(nb, 3, replace=False)) for _ in range(nb)])
                    for _ in range(nh)]).astype(np.int32)
    cnt = np.full((nh, nb), 3, dtype=np.int32)
    return perm, xs, sel, cnt, B


def test_keys_outside_the_list_do_not_matter():
    perm, (qp, kp, vp), sel, cnt, B = _random_case()
    op, lse = oracle.attn_blocks(qp, kp, vp, perm, B, sel, cnt)
    nb = sel.shape[1]
    rng = np.random.default_rng(10)
    kp2, vp2 = kp.copy(), vp.copy()
    for h in range(sel.shape[0]):
        I = 2
        out = [J for J in range(nb) if J not in sel[h, I]]
        for J in out:
            kp2[h, J * B:(J + 1) * B] += rng.standard_normal((B, kp.shape[2])) * 5
            vp2[h, J * B:(J + 1) * B] += rng.standard_normal((B, kp.shape[2])) * 5
        op2, _ = oracle.attn_blocks(qp, kp2, vp2, perm, B, sel, cnt)
        np.testing.assert_array_equal(op2[h, I * B:(I + 1) * B], op[h, I * B:(I + 1) * B])


def test_pad_slots_are_ignored():
    perm, (qp, kp, vp), sel, cnt, B = _random_case()
    op, lse = oracle.attn_blocks(qp, kp, vp, perm, B, sel, cnt)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[:, perm < 0] = 100.0
    vp2[:, perm < 0] = -7.0
    op2, lse2 = oracle.attn_blocks(qp, kp2, vp2, perm, B, sel, cnt)
    np.testing.assert_array_equal(op2, op)
    np.testing.assert_array_equal(lse2, lse)
    assert np.all(op[:, perm < 0] == 0)


def test_constant_values_pass_through():
    perm, (qp, kp, vp), sel, cnt, B = _random_case()
    vconst = np.zeros_like(vp)
    vconst[:, perm >= 0] = np.arange(vp.shape[2])[None, None, :] - 3.0
    op, _ = oracle.attn_blocks(qp, kp, vconst, perm, B, sel, cnt)
    np.testing.assert_allclose(op[:, perm >= 0], vconst[:, perm >= 0], rtol=1e-14, atol=1e-14)


def test_row_subset_matches_full_evaluation():
    perm, (qp, kp, vp), sel, cnt, B = _random_case()
    op, lse = oracle.attn_blocks(qp, kp, vp, perm, B, sel, cnt)
    rows = [np.array([0, 5, 17, 99]), np.array([3, 50])]
    op2, lse2 = oracle.attn_blocks(qp, kp, vp, perm, B, sel, cnt, rows=rows)
    for h, r in enumerate(rows):
        # same formula; only the BLAS blocking of the products differs
        np.testing.assert_allclose(op2[h, r], op[h, r], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(lse2[h, r], lse[h, r], rtol=1e-13, atol=1e-15)


def test_cached_mask_step_uses_step0_lists():
    """DFSAttn, Methodology, design 3: a cached mask is reused while attention
    is recomputed on the new step's inputs."""
    w = wl.get(2)
    q0, k0, v0 = wl.make_qkv(w, 0)
    q1, k1, v1 = wl.make_qkv(w, 1)
    r0 = oracle.run_layer(w.T, w.H, w.W, w.order, w.B, q0, k0, v0, select="topk", s=w.s, k_top=8)
    r1 = oracle.run_layer(w.T, w.H, w.W, w.order, w.B, q1, k1, v1, select="topk", s=w.s, k_top=8,
                          mask=(r0["kv_idx"], r0["kv_cnt"]))
    perm = r0["perm"]
    qp, kp, vp = (oracle.gather(x, perm) for x in (q1, k1, v1))
    op, _ = oracle.attn_blocks(qp, kp, vp, perm, w.B, r0["kv_idx"], r0["kv_cnt"])
    np.testing.assert_array_equal(r1["op"], op)
    assert r1["S"] is None


def test_block_mass_pins():
    """Exact per-block attention mass: every row sums to 1; averaged over the
    rows of a query block it equals MASS scoring at sub-block size 1 (itself
    pinned to brute-force softmax attention); full lists give recall 1 and a
    list of one block gives that block's mass."""
    rng = np.random.default_rng(11)
    T, H, W, nh, D, B = 2, 4, 5, 2, 8, 8           # 40 tokens, ragged last block
    perm, blk_len = oracle.plan(T, H, W, "row", B)
    x = [rng.standard_normal((1, T * H * W, nh, D)) for _ in range(2)]
    qp, kp = (oracle.gather(a, perm) for a in x)
    nb = perm.size // B
    real = np.nonzero(perm >= 0)[0]
    rows = [real, real]
    mass = oracle.block_mass(qp, kp, perm, B, rows)
    np.testing.assert_allclose(mass.sum(axis=2), 1.0, atol=1e-12)
    S1 = oracle.score_mass(qp, kp, perm, B, 1)
    blocks = real // B
    for h in range(nh):
        for I in range(nb):
            np.testing.assert_allclose(mass[h, blocks == I].mean(axis=0), S1[h, I], atol=1e-12)
    full = np.tile(np.arange(nb, dtype=np.int32), (nh, nb, 1))
    rec = oracle.recall(mass, rows, B, full, np.full((nh, nb), nb, dtype=np.int32))
    np.testing.assert_allclose(rec, 1.0, atol=1e-12)
    one = np.full((nh, nb, 1), 2, dtype=np.int32)
    rec1 = oracle.recall(mass, rows, B, one, np.ones((nh, nb), dtype=np.int32))
    np.testing.assert_allclose(rec1, mass[:, :, 2], atol=0)


def test_backward_full_keep_matches_autograd():
    """Keeping every block, the gradients equal torch autograd of dense fp64
    scaled-dot-product attention (an independent implementation)."""
    import torch
    rng = np.random.default_rng(21)
    T, H, W, nh, D, B = 2, 4, 5, 2, 8, 16           # 40 tokens, ragged last block
    perm, blk_len = oracle.plan(T, H, W, "hilbert", B)
    q, k, v, do = (rng.standard_normal((1, T * H * W, nh, D)) for _ in range(4))
    qp, kp, vp, dop = (oracle.gather(a, perm) for a in (q, k, v, do))
    nb = perm.size // B
    full = np.tile(np.arange(nb, dtype=np.int32), (nh, nb, 1))
    dq, dk, dv = oracle.attn_blocks_bwd(qp, kp, vp, dop, perm, B, full, np.full((nh, nb), nb, np.int32))
    tq, tk, tv = (torch.tensor(a[0].transpose(1, 0, 2), dtype=torch.float64, requires_grad=True)
                  for a in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(tq[None], tk[None], tv[None])[0]
    out.backward(torch.tensor(do[0].transpose(1, 0, 2)))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        back = oracle.scatter(mine, perm, T * H * W)[0].transpose(1, 0, 2)
        np.testing.assert_allclose(back, ref.numpy(), atol=1e-12)


def test_backward_finite_differences_sparse_lists():
    """With uneven sparse lists, the gradients match central finite
    differences of the oracle's own forward loss <dO, O>."""
    rng = np.random.default_rng(22)
    T, H, W, nh, D, B = 1, 4, 6, 1, 4, 8             # 24 tokens, 3 blocks
    perm, _ = oracle.plan(T, H, W, "row", B)
    qp, kp, vp, dop = (rng.standard_normal((nh, perm.size, D)) for _ in range(4))
    kv_idx = np.array([[[0, 2], [1, -1], [0, 1]]], dtype=np.int32)
    kv_cnt = np.array([[2, 1, 2]], dtype=np.int32)
    grads = oracle.attn_blocks_bwd(qp, kp, vp, dop, perm, B, kv_idx, kv_cnt)

    def loss(q, k, v):
        o, _ = oracle.attn_blocks(q, k, v, perm, B, kv_idx, kv_cnt)
        return float((o * dop).sum())
    eps = 1e-6
    for which, g in enumerate(grads):
        for (i, d) in [(0, 0), (5, 3), (9, 1), (17, 2), (23, 0)]:
            args = [qp.copy(), kp.copy(), vp.copy()]
            args[which][0, i, d] += eps
            up = loss(*args)
            args[which][0, i, d] -= 2 * eps
            down = loss(*args)
            assert abs((up - down) / (2 * eps) - g[0, i, d]) < 1e-7, (which, i, d)
