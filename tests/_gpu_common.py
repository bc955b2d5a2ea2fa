"""Shared helpers for the GPU parity tests (not collected by pytest)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as wl

TOL = {"f32": 1e-4, "bf16": 2e-2}       # max-abs attention tolerance vs the float64 oracle
SCORE_TOL = {"mass": 1e-5, "max": 1e-4}  # max-abs score tolerance (float32 scoring)


def dev():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return torch.device("cuda:0")


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu").to(torch.float64).numpy() if t.is_floating_point() else t.cpu().numpy()


def topk_k(w, nb):
    return w.k if w.k > 0 else max(1, int(np.floor(w.keep_ratio * nb + 0.5)))


def oracle_select(w, S, nb, step, max_kv=None):
    """The oracle's selection for a workload on a given score array."""
    if w.select == "topk":
        return oracle.select_topk(S, topk_k(w, nb), max_kv)
    if w.select == "thresh_global":
        return oracle.select_thresh_global(S, w.tau, wl.budget_ratio(w, step), max_kv)
    tiles = nb // w.T
    if w.select == "radial":
        return oracle.select_radial(w.T, tiles, w.lam, max_kv)
    if w.select == "radial_dyn":
        return oracle.select_radial_dynamic(S, w.T, tiles, w.lam, w.delta, max_kv)
    return oracle.select_lvsa(w.T, tiles, w.C, w.T_per, step, max_kv)


def lists_equal(a_idx, a_cnt, b_idx, b_cnt):
    """Same counts and the same first kv_cnt entries in every row (entries
    past a row's count are not part of the lists: the library leaves them
    unwritten, the oracle fills -1)."""
    a_idx, a_cnt, b_idx, b_cnt = (np.asarray(x) for x in (a_idx, a_cnt, b_idx, b_cnt))
    if not np.array_equal(a_cnt, b_cnt):
        return False
    w = min(a_idx.shape[-1], b_idx.shape[-1])
    if a_cnt.size and int(a_cnt.max()) > w:
        return False
    valid = np.arange(w)[None, None, :] < a_cnt[..., None]
    return bool(np.all((a_idx[..., :w] == b_idx[..., :w]) | ~valid))


def attn_rows(w, step, perm):
    """Per-head slot indices the oracle evaluates: every real slot for small
    workloads; otherwise all rows of sample_rows/B seeded query blocks per
    head (4096 rows at B = 128) plus the first and the ragged last block."""
    real = np.nonzero(perm >= 0)[0]
    if w.sample_rows == 0:
        return [real] * w.heads
    n_pad = perm.size
    nb = n_pad // w.B
    rows = []
    for h in range(w.heads):
        blocks = np.union1d(wl.sample_blocks(w, step, h, nb), [0, nb - 1])
        r = (blocks[:, None] * w.B + np.arange(w.B)[None, :]).ravel()
        rows.append(r[perm[r] >= 0])
    return rows


def max_err_rows(gpu_op, ref_op, rows):
    err = 0.0
    for h, r in enumerate(rows):
        err = max(err, float(np.abs(gpu_op[h, r] - ref_op[h, r]).max()))
    return err


def _row_prefix(S, tau):
    """Per-row shortest score-ranked prefix whose float64 sum reaches tau (at
    least one block), as a boolean mask [nb, nb] (the per-row part of the
    VMoBA threshold rule, recomputed here only to explain differences)."""
    nb = S.shape[0]
    order = np.argsort(-S, axis=1, kind="stable")
    srt = np.take_along_axis(S, order, axis=1)
    cs = np.cumsum(srt, axis=1)
    n = np.argmax(cs >= tau, axis=1) + 1
    n[~(cs[:, -1] >= tau)] = nb
    n = np.maximum(n, 1)
    mask = np.zeros((nb, nb), dtype=bool)
    for i in range(nb):
        mask[i, order[i, :n[i]]] = True
    return mask, order, cs


def thresh_differences(S64, S32, gpu_idx, gpu_cnt, tau, ratio):
    """Threshold selection on float32 GPU scores against the oracle's
    selection on its float64 scores (reading S26 iii). A pair chosen by one
    and not the other must be explained by the score error e = max|S32 - S64|:

    * row prefix: the pair's float64 prefix position sits near tau. With
      C = the float64 sum of the row's scores ranked strictly before it, the
      pair is in one prefix and not the other only if tau lies between C and
      the float32 sum before it, which differs from C by at most nb*e plus the
      scores of the m pairs whose float64 scores lie within 2e of it (they can
      swap places with it): |C - tau| <= nb*e + m*(s + 2e);
    * global fill: the pair's float64 score sits near the fill boundary. The
      float64 boundary (the score of the last pair added) can move by as many
      ranks as pairs that changed between the two row prefixes plus the pairs
      within 2e of the boundary; the pair's score must lie inside that rank
      window, widened by 2e.

    Returns (differing pairs, explained pairs) over all heads."""
    nh, nb, _ = S64.shape
    ref_idx, ref_cnt = oracle.select_thresh_global(S64, tau, ratio)
    K = oracle.budget_pairs(ratio, nb)
    e = float(np.abs(S32 - S64).max())
    diff = explained = 0
    for h in range(nh):
        m64 = np.zeros((nb, nb), dtype=bool)
        m32 = np.zeros((nb, nb), dtype=bool)
        for i in range(nb):
            m64[i, ref_idx[h, i, :ref_cnt[h, i]]] = True
            m32[i, gpu_idx[h, i, :gpu_cnt[h, i]]] = True
        bad = np.argwhere(m64 != m32)
        if bad.size == 0:
            continue
        T64, order, cs = _row_prefix(S64[h], tau)
        T32, _, _ = _row_prefix(S32[h].astype(np.float64), tau)
        dT = int((T64 != T32).sum())
        flat = S64[h].ravel()
        free = np.nonzero(~T64.ravel())[0]
        free = free[np.argsort(-flat[free], kind="stable")]
        need = max(K - int(T64.sum()), 0)
        pos_of = np.empty(nb, dtype=np.int64)
        for i, j in bad:
            diff += 1
            s = S64[h, i, j]
            pos_of[order[i]] = np.arange(nb)
            C = cs[i, pos_of[j]] - s
            m = int((np.abs(S64[h, i] - s) <= 2 * e).sum()) - 1
            row_ok = abs(C - tau) <= nb * e + m * (s + 2 * e) + 1e-12
            fill_ok = False
            if free.size:
                near = 0
                if need > 0:
                    g = flat[free[min(need - 1, free.size - 1)]]
                    near = int((np.abs(flat[free] - g) <= 2 * e).sum())
                w = dT + near + 1
                lo_r = min(max(need - 1 + w, 0), free.size - 1)
                hi_r = min(max(need - 1 - w, 0), free.size - 1)
                fill_ok = flat[free[lo_r]] - 2 * e <= s <= flat[free[hi_r]] + 2 * e
            explained += int(row_ok or fill_ok)
    return diff, explained
