"""CPU oracle for dynamic block-sparse video attention — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct numpy implementation of the
five-step path (reorder, score, select, attend, restore order) that the HIP
library computes. It exists to check the library, never to stand in for it:
only the tests, the smoke check and the benchmark's CPU-baseline leg may
import it. The product path has no CPU fallback and never calls into here.

It shares no code, headers, tables or constants with the HIP sources; the
only thing both sides read is the seeded input generator in ``workloads``.

Floating-point work is done in float64 from the exact float32/bfloat16 input
values. Each function cites the page and section it follows:

* DFSAttn (Dynamic Fine-grained Sparse Attention for Efficient Video
  Generation), Methodology, designs 1-3: 3D Hilbert reordering, hierarchical
  sub-block scoring, budgeted selection with mask caching.
* LVSA (Training-Free Sparse Attention for Long Video Diffusion), section 2:
  the frame set A(t) = G u W(t), rotating anchors, expanded windows; the
  complexity paragraph.
* VMoBA (Mixture of Block Attention for video diffusion), abstract: global
  block selection per head and threshold selection by cumulative similarity.
* DynamicRad (Content-Adaptive Sparse Attention), section 2: a shared
  candidate set aggregated block-wise for a block attention kernel; the
  static-ratio and dynamic-threshold modes over a logarithmic radial window
  with a long-range factor.

Readings of points the pages leave open are stated at each function that
takes them. Parity-unpinned items: the MASS
aggregation choice, the way threshold and global budget combine, the window
tie order and the synthetic-field recipe are readings that only invariants
pin, not values printed on the pages.
"""
from .hilbert import hilbert_index, hilbert_index_2d, hilbert_order_bits
from .plan import plan, inverse_perm
from .gather import gather, scatter
from .score import pool, score_mass, score_max, score
from .select import (select_topk, select_thresh_global, lvsa_frame_sets,
                     select_lvsa, thresh_fixed_point, budget_pairs, radial_width,
                     radial_window, select_radial, select_radial_dynamic)
from .attn import attn_blocks, attn_blocks_bwd, attn_dense, block_mass, recall
from .layer import run_layer

__all__ = [
    "hilbert_index", "hilbert_index_2d", "hilbert_order_bits", "plan", "inverse_perm", "gather", "scatter",
    "pool", "score_mass", "score_max", "score", "select_topk", "select_thresh_global",
    "lvsa_frame_sets", "select_lvsa", "thresh_fixed_point", "budget_pairs",
    "radial_width", "radial_window", "select_radial", "select_radial_dynamic",
    "attn_blocks", "attn_blocks_bwd", "attn_dense", "block_mass", "recall", "run_layer",
]
