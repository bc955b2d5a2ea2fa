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
    return np.array_equal(np.asarray(a_cnt), np.asarray(b_cnt)) and np.array_equal(
        np.asarray(a_idx), np.asarray(b_idx))


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
