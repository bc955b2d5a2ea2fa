"""Attention recall of block selection across token orders and sub-block sizes.

DFSAttn (Problem, Methodology designs 1-2) argues that a global 3D Hilbert
order keeps semantically related tokens in the same block and that sub-block
scoring estimates block importance better than coarse pooling. This script
measures both claims on the synthetic smoothed-field inputs: for each token
order and sub-block size it builds the layer, selects the top-k key blocks
(the workload's keep ratio), and reports the share of the exact attention
mass that the selected blocks keep for seeded sampled query rows
(hsa_block_mass). Everything runs through the C ABI on the GPU.

    python -m block_sparse_attention_hilbert3d_amd.recall_study --workload 3
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys

import numpy as np
import torch


def study(widx: int = 3, orders=("row", "hilbert2d", "hilbert", "tile2d", "cube3d"),
          subs=(16, 32, 64, 128), rows_per_head: int = 4096, step: int = 0):
    from dataclasses import replace

    from . import binding as B_
    from .layer import layer_for_workload
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import workloads as wl

    base = wl.get(widx)
    dev = torch.device("cuda:0")
    q, k, v = (x.to(dev) for x in wl.make_qkv(base, step))
    results = []
    for order in orders:
        for s in subs:
            if base.B % s:
                continue
            w = replace(base, order=order, s=s, select="topk", k=0,
                        keep_ratio=base.keep_ratio if base.keep_ratio else 0.15)
            L = layer_for_workload(w, device=dev, want_lse=False)
            L.reorder(q, k, v)
            L.make_mask(step)
            perm = L.perm.cpu().numpy()
            real = np.nonzero(perm >= 0)[0]
            rows = []
            for h in range(w.heads):
                rng = np.random.default_rng(wl.seed_of(widx, step, 9, h))
                rows.append(np.sort(rng.choice(real, min(rows_per_head, real.size), replace=False)))
            rows_t = torch.from_numpy(np.stack(rows).astype(np.int32)).to(dev)
            rec = L.recall(rows_t).cpu().numpy()
            results.append({"order": order, "sub_block": s, "blocks": L.nb, "k": L.k,
                            "kept_fraction": L.k / L.nb, "mean_recall": float(rec.mean()),
                            "p10_recall": float(np.percentile(rec, 10))})
            print(json.dumps(results[-1]), flush=True)
            del L
    return results


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--rows", type=int, default=4096)
    ap.add_argument("--step", type=int, default=0)
    ap.add_argument("--orders", default="row,hilbert2d,hilbert,tile2d,cube3d")
    ap.add_argument("--subs", default="16,32,64,128")
    args = ap.parse_args()
    res = study(args.workload, orders=tuple(args.orders.split(",")),
                subs=tuple(int(x) for x in args.subs.split(",")), rows_per_head=args.rows, step=args.step)
    print("| order | s | blocks | k (kept) | mean recall | p10 recall |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in res:
        print(f"| {r['order']} | {r['sub_block']} | {r['blocks']} | {r['k']} ({100 * r['kept_fraction']:.1f} %) "
              f"| {r['mean_recall']:.4f} | {r['p10_recall']:.4f} |")


if __name__ == "__main__":
    main()
