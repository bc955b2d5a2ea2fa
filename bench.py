"""Benchmark: one block-sparse attention layer at the Wan-2.1-1.3B 480p shape.

A step is one pass of the whole path over one batch of synthetic Q/K/V that
is already resident in HBM: reorder (hsa_perm), score (hsa_score), select
(hsa_select), attention (hsa_attn) and restore (hsa_unperm). Two input sets
are rotated (each is 604 MB, above the 256 MB Infinity Cache).

Prints one JSON line: `value` is dense-equivalent TFLOP/s (dense attention
FLOP of the layer / layer time); `ms_per_step` is ms per layer. `roofline`
is for the dominant kernel (attention, bf16 matrix cores) with its time
taken from HIP events recorded on the stream the library launches on;
`stages` gives every step's time and its fraction of HBM or MFMA peak;
`cpu_baseline` times the CPU oracle on a bounded sample of the same layer.

Beside the headline workload the line carries `workloads`: the LVSA
long-video frame mask (61x30x52) and the HunyuanVideo-like 720p threshold
selection (33x45x80), each over every step of its schedule, with its own
per-stage times, roofline fractions and a smaller oracle sample.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload 3] [--no-cpu] [--no-extra]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 matrix-core peak
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 matrix-core peak
METRIC = "ms/layer + dense-equiv TFLOP/s of block-sparse attn at Wan-1.3B 480p shape"
COUNTERS = os.path.join(ROOT, "profiles", "attn_wan480p_counters.json")
ATTN_SRC = os.path.join(ROOT, "block_sparse_attention_hilbert3d_amd", "csrc", "attn.hip")


def _src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(w_idx):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current attention source; else None."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("attn_src_sha256_16") != _src_hash(ATTN_SRC) or c.get("workload") != w_idx:
        return None
    return c.get("hbm_bytes_per_launch")


def _oracle_select(w, S, nb, step):
    """The oracle's lists for a workload's selection rule at a step."""
    import oracle
    import workloads as wl
    if w.select == "topk":
        return oracle.select_topk(S, wl.topk_of(w, nb))
    if w.select == "thresh_global":
        return oracle.select_thresh_global(S, w.tau, wl.budget_ratio(w, step))
    tiles = nb // w.T
    if w.select == "lvsa":
        return oracle.select_lvsa(w.T, tiles, w.C, w.T_per, step)
    if w.select == "radial":
        return oracle.select_radial(w.T, tiles, w.lam)
    return oracle.select_radial_dynamic(S.astype("float32"), w.T, tiles, w.lam, w.delta)


def _cpu_baseline(w, q, k, v, step=0, blocks_per_head=32):
    """Time the CPU oracle on a bounded sample of the same layer: plan,
    gather, scoring and selection on the whole problem, attention on every
    row of `blocks_per_head` seeded query blocks per head, extrapolated
    linearly to all query blocks."""
    import numpy as np
    import oracle
    import workloads as wl

    t0 = time.perf_counter()
    perm, blk_len = oracle.plan(w.T, w.H, w.W, w.order, w.B)
    qp, kp, vp = (oracle.gather(x, perm) for x in (q, k, v))
    t1 = time.perf_counter()
    nb = perm.size // w.B
    S = oracle.score(qp, kp, perm, w.B, w.s, agg=w.agg) if w.s > 0 else None
    kv_idx, kv_cnt = _oracle_select(w, S, nb, step)
    t2 = time.perf_counter()
    nblk = min(blocks_per_head, nb)
    rows = []
    for h in range(w.heads):
        blocks = wl.sample_blocks(w, 0, h, nb, nblk)
        rows.append((blocks[:, None] * w.B + np.arange(w.B)[None, :]).ravel())
    oracle.attn_blocks(qp, kp, vp, perm, w.B, kv_idx, kv_cnt, rows=rows)
    t3 = time.perf_counter()
    full_attn = (t3 - t2) * nb / nblk
    layer_s = (t1 - t0) + (t2 - t1) + full_attn
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        blas = 1
    return dict(layer_s=layer_s, plan_gather_s=t1 - t0, score_select_s=t2 - t1,
                attn_sample_s=t3 - t2, attn_extrapolated_s=full_attn, wall_s=t3 - t0,
                cores=max(1, min(len(os.sched_getaffinity(0)), blas)), blocks_per_head=nblk,
                nb=nb)


def _cpu_record(cb, flop_dense):
    return {
        "value": flop_dense / cb["layer_s"] / 1e12, "unit": "TFLOP/s (dense-equivalent)",
        "cores": cb["cores"], "kind": "oracle",
        "sample": (f"float64 numpy oracle on this host: plan+gather {cb['plan_gather_s']:.2f}s and "
                   f"score+select {cb['score_select_s']:.2f}s on the whole layer, attention on "
                   f"{cb['blocks_per_head']} seeded query blocks/head ({cb['attn_sample_s']:.2f}s) "
                   f"extrapolated linearly to all {cb['nb']} blocks; layer {cb['layer_s']:.1f}s; "
                   f"cores = BLAS threads"),
        "ms_per_layer": cb["layer_s"] * 1e3,
    }


def _time_backward(hsa, L, qkv, K, stream, flop_fwd):
    """Attention backward on the layer's current lists: dQ, dK, dV for a seeded
    output gradient. FLOP: the algorithmic 2.5x the forward (five products per
    tile pair); the kernels compute seven (S and dP in both passes)."""
    import torch
    L.want_lse = True
    L.io = "reordered"   # the backward reads Qp, Kp, Vp and Op in the reordered layout
    if L.lse is None:
        L.lse = torch.empty((L.heads, L.n_pad), dtype=torch.float32, device=L.op.device)
    L.reorder(*qkv, pool=False)
    L.attend()
    g = torch.Generator(device=L.op.device).manual_seed(7)
    dop = torch.randn(L.op.shape, generator=g, device=L.op.device).to(L.op.dtype)
    outs = tuple(torch.empty_like(L.op) for _ in range(3))
    ws = torch.empty(max(hsa.lib().hsa_attn_bwd_ws_size(L.heads, L.nb, L.B, int(L.kv_idx.shape[0] == 1)), 16),
                     dtype=torch.uint8, device=L.op.device)
    args = (*L.xp, L.op, dop, L.lse, L.blk_len, L.kv_idx, L.kv_cnt, L.B)
    # warm-up: at least two passes and 50 ms of GPU time (clock settle)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    n, t = 0, 0.0
    while n < 2 or (t < 50.0 and n < 1000):
        hsa.hsa_attn_bwd(*args, outs=outs, ws=ws)
        n += 1
        e1.record(stream)
        e1.synchronize()
        t = e0.elapsed_time(e1)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(K):
        hsa.hsa_attn_bwd(*args, outs=outs, ws=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    return {"ms": ms, "tflops_algorithmic": 2.5 * flop_fwd / (ms * 1e-3) / 1e12,
            "tflops_computed": 3.5 * flop_fwd / (ms * 1e-3) / 1e12,
            "frac_mfma_peak_algorithmic": 2.5 * flop_fwd / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


def _keep_text(w, L, nb, tiles_steps, nh):
    mean_per_row = float(sum(tiles_steps)) / len(tiles_steps) / (nh * nb)
    if w.select == "topk":
        return f"top-{L.k} of {nb} key blocks per query block"
    if w.select == "lvsa":
        return (f"LVSA C={w.C} frames, T_per={w.T_per}: {mean_per_row:.1f} of {nb} tiles per "
                f"query tile (mean over {len(tiles_steps)} steps)")
    if w.select == "radial":
        return f"radial window, long-range factor {w.lam}: {mean_per_row:.1f} of {nb} tiles per query tile"
    if w.select == "radial_dyn":
        return (f"radial window (factor {w.lam}) + logits within {w.delta} of the row's best: "
                f"{mean_per_row:.1f} of {nb} tiles per query tile")
    return (f"cumulative threshold tau={w.tau} + global budget: {mean_per_row:.1f} of {nb} blocks per "
            f"query block (mean over {len(tiles_steps)} steps)")


def _copy_rate(torch, dev, stream):
    """Measured device-to-device copy bandwidth (context for the HBM
    fractions: the practical ceiling of plain streaming on this part)."""
    ca = torch.empty(256 << 20, dtype=torch.float32, device=dev).fill_(1.0)
    cb = torch.empty_like(ca)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    copy_us = []
    for r in range(4):
        flush.fill_(r)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        cb.copy_(ca)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_us.append(e0.elapsed_time(e1) * 1e3)
    return 2 * ca.numel() * 4 / min(copy_us[1:]) / 1e3


def _measure(hsa, wl, w, io, K, W, n_sets, detailed):
    """Time K layer steps of workload w (after W warm-up steps) on input sets
    rotated step by step; per-stage times from HIP events on the launch
    stream. Returns (record, layer, host input sets)."""
    import numpy as np
    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    sets_cpu = [wl.make_qkv(w, s) for s in range(n_sets)]
    sets = [tuple(x.to(dev) for x in st) for st in sets_cpu]
    L = hsa.layer_for_workload(w, device=dev, want_lse=False, io=io)
    nb, B, D, nh, N = L.nb, w.B, w.D, w.heads, w.N
    esz = 2 if w.dtype == "bf16" else 4
    scored = L.S is not None

    # the diffusion step a timed step stands for: its budget (threshold mode)
    # or its anchor rotation (LVSA); top-k steps refresh the same way each time
    def step_of(i):
        return i % max(w.steps, 1)

    def one_step(i, ev=None):
        q, k, v = sets[i % n_sets]
        st = step_of(i)
        if ev is not None:
            ev[0].record(stream)
        L.reorder(q, k, v, pool=scored)
        if ev is not None:
            ev[1].record(stream)
        if scored:
            qp, kp, _ = L.xp
            hsa.hsa_score(qp, kp, L.blk_len, B, w.s, L.agg, L.scale, out=L.S, pooled=L.pooled)
        if ev is not None:
            ev[2].record(stream)
        hsa.hsa_select(L.S, nh, nb, L.params(st, wl.budget_ratio(w, st)), L.max_kv,
                       outs=(L.kv_idx, L.kv_cnt), ws=L.select_ws, device=dev)
        if L.order is not None:  # longest lists first (threshold mode)
            hsa.hsa_attn_order(L.kv_cnt, L.max_kv, out=L.order)
        if ev is not None:
            ev[3].record(stream)
        L.attend()
        if ev is not None:
            ev[4].record(stream)
        L.restore()
        if ev is not None:
            ev[5].record(stream)

    # Bring the GPU to its working clock first. The host-side setup above
    # (input generation) leaves it idle for seconds, and after such a pause
    # its first ~15 layer steps run 10-20 % slower (clock and power ramp);
    # layers of a model run back to back, so the steps are repeated for at
    # least 50 ms of GPU time before the W warm-up steps (reported as
    # `settle`).
    def settle(min_ms=50.0):
        n, t = 0, 0.0
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record(stream)
        while t < min_ms and n < 1000:
            one_step(n)
            n += 1
            s1.record(stream)
            s1.synchronize()
            t = s0.elapsed_time(s1)
        return n, t

    settle_steps, settle_ms = settle()
    for i in range(W):
        one_step(i)
    torch.cuda.synchronize()
    # the timed steps: one event per step boundary, no markers between stages
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    bounds[0].record(stream)
    c0 = time.perf_counter()
    for i in range(K):
        one_step(i)
        bounds[i + 1].record(stream)
    enqueue_ms = (time.perf_counter() - c0) * 1e3 / K  # host time to issue one step
    torch.cuda.synchronize()
    ms_step = bounds[0].elapsed_time(bounds[K]) / K
    per_step = np.array([bounds[i].elapsed_time(bounds[i + 1]) for i in range(K)])
    # per-stage times from a second pass of the same steps with an event
    # between consecutive stages
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(K)]
    for i in range(K):
        one_step(i, evs[i])
    torch.cuda.synchronize()
    names = ["perm", "score", "select", "attn", "unperm"]
    stage_ms = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    ms_step_staged = float(np.mean([e[0].elapsed_time(e[5]) for e in evs]))

    # the lists of every timed step (they change with the step in threshold
    # and LVSA modes): computed tile pairs, useful (query, key) pairs over
    # real tokens, and list entries written
    G = L.kv_idx.shape[0]
    blk_len = L.blk_len.to(torch.int64)
    # A launch whose lists are shared by all heads, or whose plan has many
    # short blocks (bf16, 128-token blocks, no log-sum-exp, K/V not
    # gathered), walks the 64-key stages and leaves out a block's empty
    # second stage when it has at most 64 real keys: such a pair is half a
    # computed tile.
    walks = ((G == 1 and nh > 1) or L.short_blocks) and esz == 2 and B == 128 and L.io != "tokens"
    tiles_steps, useful_steps, entries_steps = [], [], []
    for i in range(K):
        one_step(i)
        cnt = L.kv_cnt.to(torch.int64)
        valid = torch.arange(L.max_kv, device=dev)[None, None, :] < cnt[..., None]
        ent_len = blk_len[L.kv_idx.clamp(0, nb - 1).to(torch.int64)]
        keys = torch.where(valid, ent_len, 0).sum(-1)
        halves = int((valid & (ent_len <= B // 2)).sum().item()) if walks else 0
        tiles_steps.append((int(cnt.sum().item()) - 0.5 * halves) * (nh // G))
        useful_steps.append(int((keys * blk_len[None, :]).sum().item()) * (nh // G))
        entries_steps.append(int(cnt.sum().item()))
    torch.cuda.synchronize()

    flop_tiles = 4.0 * B * B * D * float(np.mean(tiles_steps))
    flop_useful = 4.0 * D * float(np.mean(useful_steps))
    flop_dense = 4.0 * N * N * D * nh
    t_attn = stage_ms["attn"] * 1e-3
    achieved = flop_tiles / t_attn / 1e12
    row = N * nh * D * esz
    U = L.n_pad // w.s if scored else 0
    pooled_bytes = 2 * nh * U * D * 4
    stage_bytes = {
        # reordered: Q, K, V read and written once, plus the Q/K sub-block
        # means. tokens_qo: only K and V are reordered (Q is read for its
        # means on refresh steps). tokens: nothing is reordered; Q and K are
        # read for their means on refresh steps only.
        "perm": {"reordered": 3 * 2 * row + pooled_bytes,
                 "tokens_qo": 4 * row + ((row + pooled_bytes) if scored else 0),
                 "tokens": (2 * row + pooled_bytes) if scored else 0}[L.io],
        "score": pooled_bytes + nh * nb * nb * 4,
        # S read once (scored modes), the list entries and counts written
        "select": (nh * nb * nb * 4 if scored else 0) + (float(np.mean(entries_steps)) + G * nb) * 4,
        "unperm": 2 * row,
    }
    score_flop = 2.0 * U * U * D * nh
    stages = {}
    for n in names:
        t = stage_ms[n] * 1e-3
        if ((n == "score" and not scored) or (n == "unperm" and L.io != "reordered")
                or (n == "perm" and stage_bytes["perm"] == 0)):
            continue
        if n == "attn":
            stages[n] = {"ms": stage_ms[n], "tflops_computed_tiles": achieved,
                         "tflops_useful": flop_useful / t / 1e12,
                         "frac_mfma_peak": achieved / BF16_PEAK_TFLOPS,
                         "frac_mfma_peak_useful": flop_useful / t / 1e12 / BF16_PEAK_TFLOPS}
        elif n == "score":
            # pooling happens inside perm; what remains is the fp32 contraction
            stages[n] = {"ms": stage_ms[n], "bytes": stage_bytes[n], "flop": score_flop,
                         "tflops": score_flop / t / 1e12,
                         "frac_fp32_mfma_peak": score_flop / t / 1e12 / FP32_PEAK_TFLOPS,
                         "GB/s": stage_bytes[n] / t / 1e9,
                         "frac_hbm_peak": stage_bytes[n] / t / 1e9 / HBM_PEAK_GBS}
        else:
            gbs = stage_bytes[n] / t / 1e9
            stages[n] = {"ms": stage_ms[n], "bytes": stage_bytes[n], "GB/s": gbs,
                         "frac_hbm_peak": gbs / HBM_PEAK_GBS}
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
    rec = {
        "workload": w.name, "tokens": N, "heads": nh, "head_dim": D, "block": B,
        "sub_block": w.s, "order": w.order, "dtype": w.dtype,
        "keep": _keep_text(w, L, nb, tiles_steps, nh),
        "steps": K, "warmup": W,
        "ms_per_layer": ms_step,
        "ms_per_layer_p10_p50_p90": [float(np.percentile(per_step, p)) for p in (10, 50, 90)],
        "ms_per_layer_with_stage_events": ms_step_staged,
        "host_enqueue_ms_per_step": enqueue_ms,
        "settle": {"steps": settle_steps, "ms": settle_ms},
        "tflops_dense_equivalent": flop_dense / (ms_step * 1e-3) / 1e12,
        "stages": stages,
        "flop": {"dense": flop_dense, "computed_tiles": flop_tiles, "useful": flop_useful},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "frac_useful": flop_useful / t_attn / 1e12 / peak,
                     "kernel": "attn_bf16_pipe_kernel" if w.dtype == "bf16" else "attn_f32_kernel"},
    }
    if detailed:
        # cached-mask steps (mask reused: reorder, attention, restore), after
        # the clock is settled again (the list bookkeeping above syncs every
        # step and leaves the GPU idle in between)
        settle()
        cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for i in range(K):
            q, k, v = sets[(i + 1) % n_sets]
            cevs[i][0].record(stream)
            L.step(q, k, v, reuse_mask=True)
            cevs[i][1].record(stream)
        torch.cuda.synchronize()
        ms_cached = float(np.mean([a.elapsed_time(b) for a, b in cevs]))
        # the same refresh step captured once in a HIP graph and replayed (no
        # per-kernel launch cost); one graph per input set
        graphs = []
        for i in range(n_sets):
            L.step(*sets[i], step=0, budget_ratio=wl.budget_ratio(w, 0))
            torch.cuda.synchronize()
            gph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gph):
                L.step(*sets[i], step=0, budget_ratio=wl.budget_ratio(w, 0))
            graphs.append(gph)
        torch.cuda.synchronize()
        settle()
        for gph in graphs:
            gph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for i in range(K):
            graphs[i % n_sets].replay()
        g1.record(stream)
        torch.cuda.synchronize()
        rec["ms_per_layer_cached_mask"] = ms_cached
        rec["ms_per_step_hip_graph"] = g0.elapsed_time(g1) / K
        rec["ms_per_layer_refresh_cycle"] = ((ms_step + (w.refresh - 1) * ms_cached) / w.refresh
                                             if w.refresh > 1 else ms_step)
        rec["refresh_interval"] = w.refresh
        del graphs
    return rec, L, sets_cpu


# extra workloads reported beside the headline one: the LVSA long-video frame
# mask and the HunyuanVideo-like 720p threshold selection (one input set each,
# every step of their schedules, a smaller oracle sample)
EXTRA = {4: "lvsa_61x30x52", 5: "hunyuan720p_33x45x80"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--order", choices=["row", "hilbert", "frame", "tile2d", "cube3d"], default=None,
                    help="token order instead of the workload's own (e.g. the VMoBA 2D/3D partitions)")
    ap.add_argument("--backward", action="store_true",
                    help="also time the attention backward (hsa_attn_bwd) on the layer's lists")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the LVSA and 720p threshold workloads reported beside the default one")
    ap.add_argument("--io", choices=["auto", "reordered", "tokens_qo", "tokens"], default="tokens_qo",
                    help="where the reorders happen: five separate passes (reordered), the "
                         "attention kernel reading Q / writing O in token order (tokens_qo), "
                         "or also gathering K/V rows itself (tokens); auto picks tokens for "
                         "short top-k lists and tokens_qo otherwise")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run one device-to-device copy of this many MiB (a kernel of known "
                         "traffic, to scale hardware byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the attention path here runs on a single MI355X "
              "(multi-GPU sharding is designed, not built); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import block_sparse_attention_hilbert3d_amd as hsa
    import workloads as wl

    w = wl.get(args.workload)
    if args.order is not None:
        from dataclasses import replace
        w = replace(w, order=args.order)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    copy_gbs = _copy_rate(torch, dev, stream)
    if args.copy_calibration > 0:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).fill_(1.0)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    rec, L, sets_cpu = _measure(hsa, wl, w, args.io, args.steps, args.warmup, 2, detailed=True)
    K = args.steps
    out = {
        "metric": METRIC,
        "value": rec["tflops_dense_equivalent"],
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_layer"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded smoothed-field Q/K, i.i.d. V; no model weights)",
        "config": {"workload": f"Wan-2.1-1.3B-like 480p 81-frame latent {w.T}x{w.H}x{w.W}"
                               if w.idx == 3 else w.name,
                   "tokens": rec["tokens"], "heads": rec["heads"], "head_dim": rec["head_dim"],
                   "block": rec["block"], "sub_block": w.s, "order": w.order, "keep": rec["keep"],
                   "io": {"reordered": "five passes (reorder Q/K/V, attention, unperm)",
                          "tokens_qo": "K/V reordered; attention reads Q and writes O in token order",
                          "tokens": "attention gathers Q/K/V rows and writes O in token order; "
                                    "the reorder pass only pools Q/K on refresh steps"}[L.io],
                   "batch": 1},
        "ms_per_step_p10_p50_p90": rec["ms_per_layer_p10_p50_p90"],
        "ms_per_step_with_stage_events": rec["ms_per_layer_with_stage_events"],
        "host_enqueue_ms_per_step": rec["host_enqueue_ms_per_step"],
        "settle": rec["settle"],
        "ms_per_layer_cached_mask": rec["ms_per_layer_cached_mask"],
        "ms_per_step_hip_graph": rec["ms_per_step_hip_graph"],
        "ms_per_layer_refresh_cycle": rec["ms_per_layer_refresh_cycle"],
        "refresh_interval": rec["refresh_interval"],
        "stages": rec["stages"],
        "measured_copy_GB/s": copy_gbs,
        "flop": rec["flop"],
        "roofline": dict(rec["roofline"], traffic=_traffic(w.idx)),
    }
    if args.backward:
        out["backward"] = _time_backward(hsa, L, tuple(x.to(dev) for x in sets_cpu[0]), K, stream,
                                         rec["flop"]["computed_tiles"])
    del L
    torch.cuda.empty_cache()
    if not args.no_cpu:
        out["cpu_baseline"] = _cpu_record(_cpu_baseline(w, *sets_cpu[0]), rec["flop"]["dense"])
    del sets_cpu
    if args.workload == 3 and args.order is None and not args.no_extra:
        extra = {}
        for idx, key in EXTRA.items():
            we = wl.get(idx)
            r, Le, sc = _measure(hsa, wl, we, "tokens_qo", we.steps, 2, 1, detailed=False)
            del Le
            torch.cuda.empty_cache()
            if not args.no_cpu:
                r["cpu_baseline"] = _cpu_record(_cpu_baseline(we, *sc[0], step=0, blocks_per_head=8),
                                                r["flop"]["dense"])
            del sc
            extra[key] = r
        out["workloads"] = extra
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
