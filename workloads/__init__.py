"""Seeded synthetic workloads for block-sparse video attention.

This module holds only shapes, parameters and seeded random draws. It contains
none of the method's arithmetic (no reordering, scoring, selection or
attention), so that both the CPU oracle and the HIP path can read identical
inputs from it without sharing any code with each other.

The five workloads follow the shapes of the video diffusion models the pages
discuss: a tiny case, a small structured case, a Wan-2.1-1.3B-like 480p
81-frame latent grid (DFSAttn page, "Experimental results": Wan2.1 and
HunyuanVideo), an LVSA-style long video at three times the Wan horizon (LVSA
page, section 2, frame budget C = 21), and a HunyuanVideo-like 720p 129-frame
grid with VMoBA-style threshold selection (VMoBA abstract). The models
themselves, their weights and prompts are not available, so seeded synthetic
Q/K/V tensors of those shapes stand in for the activations.

Input recipe (one generator per (workload, step, stream, head)):

* seed = idx * 10**6 + step * 10**4 + stream * 10**3 + head, fed to
  ``numpy.random.default_rng``; streams: 0 = smoothed field, 1 = Q noise,
  2 = K noise, 3 = i.i.d. Q, 4 = i.i.d. K, 5 = V, 8 = sampled query blocks,
  9 = sampled query rows.
* "iid": Q, K ~ N(0, 1) drawn in float64 as [N, D] per head.
* "smooth": one field F per (head, channel) on the T x H x W latent grid,
  white noise smoothed by a Gaussian of sigma 2 cells (scipy.ndimage,
  reflect boundary, truncate 4), then standardised per channel to zero mean
  and unit standard deviation; Q = F + 0.1 * noise_Q, K = F + 0.1 * noise_K.
  Sharing F between Q and K makes q.k largest for spatiotemporal neighbours,
  which is the locality the method exploits.
* V ~ N(0, 1) always.
* Token n of a head is grid cell (t, y, x) with n = (t * H + y) * W + x; heads
  are interleaved into [1, N, heads, D].
* Cast once: to float32 (tiny workload) or to bfloat16 with round-to-nearest-
  even (all others). Both sides read the same rounded values.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get", "seed_of", "make_qkv", "sample_rows", "sample_blocks",
           "budget_ratio", "n_tokens"]


@dataclass(frozen=True)
class Workload:
    idx: int
    name: str
    T: int
    H: int
    W: int
    heads: int
    D: int
    dtype: str             # "f32" or "bf16"
    qk: str                # "iid" or "smooth"
    order: str             # "row", "hilbert" or "frame"
    B: int                 # block (tile) size in tokens
    s: int                 # sub-block size used for scoring (0 = no scoring)
    select: str            # "topk", "thresh_global", "lvsa", "radial" or "radial_dyn"
    keep_ratio: float = 0.0      # top-k budget as a fraction of blocks
    k: int = 0                   # explicit top-k (0 = derive from keep_ratio)
    tau: float = 0.0             # cumulative-mass threshold per query block
    budget_start: float = 0.0    # global budget schedule (fraction of pairs)
    budget_end: float = 0.0
    C: int = 0                   # frame budget per query frame
    T_per: int = 0               # anchor period in frames
    steps: int = 1               # simulated denoising steps
    refresh: int = 1             # mask recomputed when step % refresh == 0
    sample_rows: int = 0         # 0 = compare every row
    agg: str = "mass"            # block score aggregation ("max": pre-softmax logits)
    lam: float = 0.0             # radial masks: long-range factor
    delta: float = 0.0           # dynamic radial mask: logit margin below the row's best
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def N(self) -> int:
        return self.T * self.H * self.W


WORKLOADS = {
    1: Workload(1, "tiny 4x8x8, 2 heads, d64, fp32, row-major, top-2 of 4",
                T=4, H=8, W=8, heads=2, D=64, dtype="f32", qk="iid", order="row",
                B=64, s=16, select="topk", k=2),
    2: Workload(2, "small 8x16x16, 4 heads, d64, bf16, Hilbert, top-25%",
                T=8, H=16, W=16, heads=4, D=64, dtype="bf16", qk="smooth",
                order="hilbert", B=64, s=16, select="topk", keep_ratio=0.25),
    3: Workload(3, "Wan-2.1-1.3B-like 480p 81 frames: 21x30x52, 12 heads, d128, bf16, "
                   "Hilbert, top-15%, mask cached over 5 steps",
                T=21, H=30, W=52, heads=12, D=128, dtype="bf16", qk="smooth",
                order="hilbert", B=128, s=32, select="topk", keep_ratio=0.15,
                steps=5, refresh=5, sample_rows=4096),
    4: Workload(4, "LVSA-style long video: 61x30x52, 12 heads, d128, bf16, "
                   "frame mask C=21, T_per=8",
                T=61, H=30, W=52, heads=12, D=128, dtype="bf16", qk="iid",
                order="frame", B=128, s=0, select="lvsa", C=21, T_per=8,
                steps=8, sample_rows=4096),
    5: Workload(5, "HunyuanVideo-like 720p 129 frames: 33x45x80, 24 heads, d128, bf16, "
                   "Hilbert, threshold 0.25 + global budget 30%->10%",
                T=33, H=45, W=80, heads=24, D=128, dtype="bf16", qk="smooth",
                order="hilbert", B=128, s=128, select="thresh_global", tau=0.25,
                budget_start=0.30, budget_end=0.10, steps=10, sample_rows=4096),
    6: Workload(6, "DynamicRad-style static radial mask: 61x30x52 frame tiles, 12 heads, d128, "
                   "bf16, long-range factor 1/8",
                T=61, H=30, W=52, heads=12, D=128, dtype="bf16", qk="smooth",
                order="frame", B=128, s=0, select="radial", lam=0.125, sample_rows=4096),
    7: Workload(7, "DynamicRad-style dynamic logit threshold: 61x30x52 frame tiles, 12 heads, "
                   "d128, bf16, radial window (factor 1/8) + blocks within 1.0 of the row's best "
                   "64-token sub-block logit",
                T=61, H=30, W=52, heads=12, D=128, dtype="bf16", qk="smooth",
                order="frame", B=128, s=64, select="radial_dyn", agg="max", lam=0.125,
                delta=1.0, sample_rows=4096),
}


def get(idx: int) -> Workload:
    return WORKLOADS[int(idx)]


def n_tokens(w: Workload) -> int:
    return w.N


def seed_of(idx: int, step: int, stream: int, head: int) -> int:
    return int(idx) * 10**6 + int(step) * 10**4 + int(stream) * 10**3 + int(head)


def budget_ratio(w: Workload, step: int) -> float:
    """Global keep budget for a step: linear from budget_start to budget_end over
    the workload's steps, endpoints included (the pages give a budget that
    decreases monotonically over the denoising steps)."""
    if w.steps <= 1:
        return float(w.budget_start)
    return float(w.budget_start) - (float(w.budget_start) - float(w.budget_end)) * step / (w.steps - 1)


def _smooth_field(w: Workload, step: int, head: int) -> np.ndarray:
    from scipy.ndimage import gaussian_filter
    rng = np.random.default_rng(seed_of(w.idx, step, 0, head))
    raw = rng.standard_normal((w.T, w.H, w.W, w.D))
    f = gaussian_filter(raw, sigma=(2.0, 2.0, 2.0, 0.0), mode="reflect", truncate=4.0)
    f = f.reshape(w.N, w.D)
    f -= f.mean(axis=0, keepdims=True)
    f /= f.std(axis=0, keepdims=True)
    return f


def _head_qkv(w: Workload, step: int, head: int):
    N, D = w.N, w.D
    if w.qk == "smooth":
        f = _smooth_field(w, step, head)
        q = f + 0.1 * np.random.default_rng(seed_of(w.idx, step, 1, head)).standard_normal((N, D))
        k = f + 0.1 * np.random.default_rng(seed_of(w.idx, step, 2, head)).standard_normal((N, D))
    elif w.qk == "iid":
        q = np.random.default_rng(seed_of(w.idx, step, 3, head)).standard_normal((N, D))
        k = np.random.default_rng(seed_of(w.idx, step, 4, head)).standard_normal((N, D))
    else:
        raise ValueError(w.qk)
    v = np.random.default_rng(seed_of(w.idx, step, 5, head)).standard_normal((N, D))
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


def make_qkv(w: Workload | int, step: int = 0, threads: int | None = None):
    """Return (q, k, v) as CPU torch tensors of shape [1, N, heads, D] in the
    workload's dtype (torch.float32 or torch.bfloat16, rounded to nearest even)."""
    import torch
    if not isinstance(w, Workload):
        w = get(w)
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    out = [torch.empty((1, w.N, w.heads, w.D), dtype=tdt) for _ in range(3)]
    if threads is None:
        threads = max(1, min(w.heads, len(os.sched_getaffinity(0)), 16))

    def fill(h):
        arrs = _head_qkv(w, step, h)
        for t, a in zip(out, arrs):
            t[0, :, h, :] = torch.from_numpy(a).to(tdt)
        return h

    if threads == 1:
        for h in range(w.heads):
            fill(h)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(w.heads)))
    return tuple(out)


def sample_rows(w: Workload | int, step: int, head: int, count: int | None = None) -> np.ndarray:
    """Seeded sorted draw without replacement of original token indices."""
    if not isinstance(w, Workload):
        w = get(w)
    count = w.sample_rows if count is None else count
    if count <= 0 or count >= w.N:
        return np.arange(w.N, dtype=np.int64)
    rng = np.random.default_rng(seed_of(w.idx, step, 9, head))
    return np.sort(rng.choice(w.N, size=count, replace=False)).astype(np.int64)


def sample_blocks(w: Workload | int, step: int, head: int, nb: int, count: int | None = None) -> np.ndarray:
    """Seeded sorted draw without replacement of query blocks whose rows are
    checked (count defaults to sample_rows / B, i.e. the same number of rows
    as sample_rows, grouped by block so the key sets are gathered once)."""
    if not isinstance(w, Workload):
        w = get(w)
    if count is None:
        count = max(1, -(-w.sample_rows // w.B)) if w.sample_rows > 0 else nb
    if count >= nb:
        return np.arange(nb, dtype=np.int64)
    rng = np.random.default_rng(seed_of(w.idx, step, 8, head))
    return np.sort(rng.choice(nb, size=count, replace=False)).astype(np.int64)


def topk_of(w: Workload, nb: int) -> int:
    """Blocks kept per query block for a top-k budget: the explicit k, else the
    keep ratio times the number of blocks, rounded half up, at least 1."""
    if w.k > 0:
        return int(w.k)
    return max(1, int(math.floor(w.keep_ratio * nb + 0.5)))
