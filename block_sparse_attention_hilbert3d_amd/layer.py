"""One block-sparse attention layer: the five C entry points in sequence.

reorder (hsa_perm) -> score (hsa_score) -> select (hsa_select) -> attend
(hsa_attn) -> restore order (hsa_unperm), with the plan computed once per
grid shape (hsa_plan). Buffers and workspaces are allocated once per layer
so a step enqueues kernels only.

``io`` chooses where the reorders happen; the output is bit-identical in
all three forms ("auto" picks "tokens" for top-k lists of at most 6144 keys
per query block and "tokens_qo" otherwise):
  "reordered"  the five passes above;
  "tokens_qo"  (default) the attention kernel reads Q and writes the output
               in token order (hsa_attn_tokens); hsa_perm reorders K and V
               and only pools Q; no hsa_unperm pass;
  "tokens"     the attention kernel also gathers K and V rows from the
               token-major tensors; hsa_perm runs on refresh steps only, to
               pool the Q/K sub-blocks that scoring needs. The per-stage row
               lookups cost the attention kernel ~4-5 %, so this pays only
               when lists are short (the reorder pass is then a larger
               share): at the Wan 480p shape with top-38 lists it equals
               "tokens_qo" on refresh steps and is ~2.5 % faster on cached
               ones; on the long LVSA / threshold lists it loses ~2 %.

``want_lse`` (off by default) also keeps the log-sum-exp of every row, which
the backward (hsa_attn_bwd) needs; inference does not, and the kernel that
produces it carries more registers (~7 % slower at the Wan 480p shape; with
gathered K/V it spills and runs ~25 % slower, so prefer "tokens_qo" when
the log-sum-exp is wanted).

Mask caching (DFSAttn, Methodology, design 3): ``step(..., reuse_mask=True)``
skips scoring and selection and attends with the lists kept from the last
refresh, on the new step's Q/K/V.
"""
from __future__ import annotations

import math

import torch

from . import binding as B_

IO_FORMS = ("reordered", "tokens_qo", "tokens")
AUTO_TOKENS_MAX_KEYS = 6144   # top-k lists up to this many keys per query block gather K/V


class SparseAttentionLayer:
    def __init__(self, T: int, H: int, W: int, heads: int, D: int, *, order: str, B: int,
                 select: str, s: int = 0, agg: str = "mass", k: int = 0, tau: float = 0.0,
                 C: int = 0, T_per: int = 1, lam: float = 0.0, delta: float = 0.0,
                 dtype=torch.bfloat16, device="cuda", want_lse: bool = False,
                 io: str = "tokens_qo"):
        self.T, self.H, self.W, self.heads, self.D = T, H, W, heads, D
        self.N = T * H * W
        self.order, self.B, self.select, self.s, self.agg = order, B, select, s, agg
        self.k, self.tau, self.C, self.T_per, self.lam, self.delta = k, tau, C, T_per, lam, delta
        if select == "radial_dyn":
            self.agg = "max"   # the dynamic threshold reads pre-softmax logits
        self.dtype, self.device = dtype, device
        if io == "auto":
            io = "tokens" if (select == "topk" and k * B <= AUTO_TOKENS_MAX_KEYS) else "tokens_qo"
        if io not in IO_FORMS:
            raise ValueError(f"io must be 'auto' or one of {IO_FORMS}")
        self.io = io
        self._qkv = None
        self.scale = 1.0 / math.sqrt(D)
        self.perm, self.blk_len = B_.hsa_plan(T, H, W, order, B, device=device)
        self.n_pad = self.perm.numel()
        self.nb = self.n_pad // B
        # Plans whose blocks often hold at most half a block of real tokens
        # (frame tiles, clipped 2D/3D partition tiles; not the Hilbert order,
        # whose only ragged block is the last) ask the attention kernel to
        # skip those blocks' empty second 64-key stage. The walk that does it
        # costs every stage a few scalar instructions, so it pays only when
        # short blocks are common: from 7 % of the plan's blocks on (frame
        # tiles 7.7 %, the 480p cubes 22 %; the 720p cubes, 5.9 % and rarely
        # selected, ran 1.6 % slower with it).
        n_short = int((self.blk_len <= B // 2).sum().item())
        self.short_blocks = n_short >= 0.07 * self.nb
        self.tiles_per_frame = self.nb // T if order == "frame" else 0
        shape = (heads, self.n_pad, D)
        self.xp = [torch.empty(shape, dtype=dtype, device=device) for _ in range(3)]
        self.op = torch.empty(shape, dtype=dtype, device=device)
        self.lse = torch.empty((heads, self.n_pad), dtype=torch.float32, device=device) if want_lse else None
        self.want_lse = want_lse
        self.o = torch.empty((1, self.N, heads, D), dtype=dtype, device=device)
        if select in ("lvsa", "radial"):   # geometry-only masks shared by all heads
            self.max_kv = self._lvsa_width() if select == "lvsa" else \
                B_.hsa_select_list_width(heads, self.nb, self.params(0, 0.0))
            G = 1
            self.S = None
            self.score_ws = None
        else:
            self.max_kv = k if select == "topk" else self.nb
            G = heads
            self.S = torch.empty((heads, self.nb, self.nb), dtype=torch.float32, device=device)
            self.score_ws = None
            # sub-block means written by the reorder pass (fused pooling)
            self.pooled = torch.empty((2, heads, self.n_pad // s, D), dtype=torch.float32,
                                      device=device)
        self.kv_idx = torch.empty((G, self.nb, self.max_kv), dtype=torch.int32, device=device)
        self.kv_cnt = torch.empty((G, self.nb), dtype=torch.int32, device=device)
        # threshold lists differ in length from row to row: attend longest first
        self.order = (torch.arange(G * self.nb, dtype=torch.int32, device=device)
                      if select in ("thresh_global", "radial_dyn") else None)
        p = self.params(0, 0.0)
        n = B_.lib().hsa_select_ws_size(heads, self.nb, p)
        self.select_ws = torch.empty(max(n, 16), dtype=torch.uint8, device=device)

    def _lvsa_width(self) -> int:
        """List capacity that holds the LVSA lists of every step: the widest
        of the T_per anchor rotations, as the library reports them."""
        return max(B_.hsa_select_list_width(self.heads, self.nb, self.params(step, 0.0))
                   for step in range(self.T_per))

    def params(self, step: int, budget_ratio: float) -> B_.SelectParams:
        return B_.make_params(self.select, k=self.k, tau=self.tau, budget_ratio=budget_ratio,
                              frames=self.T, tiles_per_frame=self.tiles_per_frame, C=self.C,
                              lam=self.lam, delta=self.delta,
                              T_per=self.T_per, step=step)

    def reorder(self, q, k, v, pool: bool = True):
        """Gather what the io form keeps reordered; on steps that refresh the
        mask also pool Q/K sub-blocks."""
        self._qkv = (q, k, v)
        pool = pool and self.S is not None
        if self.io == "tokens":
            if pool:
                B_.hsa_perm([q, k], self.perm, self.n_pad, outs=[None, None], pool_s=self.s,
                            pooled=self.pooled)
        elif self.io == "tokens_qo":
            if pool:
                B_.hsa_perm([q, k, v], self.perm, self.n_pad, outs=[None, self.xp[1], self.xp[2]],
                            pool_s=self.s, pooled=self.pooled)
            else:
                B_.hsa_perm([k, v], self.perm, self.n_pad, outs=self.xp[1:])
        elif pool:
            B_.hsa_perm([q, k, v], self.perm, self.n_pad, outs=self.xp, pool_s=self.s,
                        pooled=self.pooled)
        else:
            B_.hsa_perm([q, k, v], self.perm, self.n_pad, outs=self.xp)

    def make_mask(self, step: int = 0, budget_ratio: float = 0.0):
        qp, kp, _ = self.xp
        if self.S is not None:
            B_.hsa_score(qp, kp, self.blk_len, self.B, self.s, self.agg, self.scale, out=self.S,
                         pooled=self.pooled)
        B_.hsa_select(self.S, self.heads, self.nb, self.params(step, budget_ratio), self.max_kv,
                      device=self.device, outs=(self.kv_idx, self.kv_cnt), ws=self.select_ws)
        if self.order is not None:
            B_.hsa_attn_order(self.kv_cnt, self.max_kv, out=self.order)

    def attend(self):
        qp, kp, vp = self.xp
        if self.io != "reordered":
            q, k, v = self._qkv
            if self.io == "tokens_qo":
                k, v = kp, vp
            B_.hsa_attn_tokens(q, k, v, self.perm, self.blk_len, self.kv_idx, self.kv_cnt,
                               self.B, self.scale, want_lse=self.want_lse, out=self.o,
                               lse=self.lse, order=self.order, short_blocks=self.short_blocks)
        else:
            B_.hsa_attn(qp, kp, vp, self.blk_len, self.kv_idx, self.kv_cnt, self.B, self.scale,
                        want_lse=self.want_lse, out=self.op, lse=self.lse, order=self.order,
                        short_blocks=self.short_blocks)

    def restore(self):
        if self.io != "reordered":
            return self.o   # written by the attention kernel
        return B_.hsa_unperm(self.op, self.perm, self.N, out=self.o)

    def recall(self, rows):
        """Attention recall of the current lists for sampled query slots
        (rows int32 [heads, n] on the device): the share of each row's exact
        attention mass that its query block's list keeps (hsa_block_mass)."""
        qp, kp, _ = self.xp
        if self.io == "tokens_qo":   # Q is not kept reordered: gather it for the diagnostic
            B_.hsa_perm([self._qkv[0]], self.perm, self.n_pad, outs=[qp])
        elif self.io == "tokens":
            B_.hsa_perm(list(self._qkv[:2]), self.perm, self.n_pad, outs=[qp, kp])
        _, rec = B_.hsa_block_mass(qp, kp, self.blk_len, rows, self.B, self.scale, self.kv_idx,
                                   self.kv_cnt, want_mass=False)
        return rec

    def step(self, q, k, v, step: int = 0, budget_ratio: float = 0.0, reuse_mask: bool = False):
        """One layer: returns the output [1, N, heads, D] (a buffer owned by the layer)."""
        self.reorder(q, k, v, pool=not reuse_mask)
        if not reuse_mask:
            self.make_mask(step, budget_ratio)
        self.attend()
        return self.restore()


VMOBA_CYCLE = ("row", "tile2d", "cube3d")


def vmoba_order(layer_index: int) -> str:
    """Token order of transformer layer `layer_index` under VMoBA's layer-wise
    recurrent 1D-2D-3D block partitions (VMoBA abstract): 1D chunks of the
    row-major sequence, then per-frame 2D tiles, then 3D cubes, repeating."""
    return VMOBA_CYCLE[layer_index % 3]


def layer_for_workload(w, device="cuda", want_lse=False, io="tokens_qo") -> SparseAttentionLayer:
    """Layer configured for one of the synthetic workloads (workloads.Workload)."""
    dtype = torch.float32 if w.dtype == "f32" else torch.bfloat16
    nb = B_.hsa_plan_size(w.T, w.H, w.W, w.order, w.B)[1]
    k = 0
    if w.select == "topk":
        k = w.k if w.k > 0 else max(1, int(math.floor(w.keep_ratio * nb + 0.5)))
    return SparseAttentionLayer(w.T, w.H, w.W, w.heads, w.D, order=w.order, B=w.B,
                                select=w.select, s=w.s, agg=w.agg, k=k, tau=w.tau, C=w.C,
                                T_per=w.T_per, lam=w.lam, delta=w.delta, dtype=dtype,
                                device=device, want_lse=want_lse, io=io)
