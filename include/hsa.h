/*
 * hsa.h -- dynamic block-sparse self-attention over spatiotemporal video
 * tokens, MI355X (gfx950) HIP library, plain C ABI.
 *
 * The path has five steps, each one entry point (plus a once-per-shape plan):
 *   hsa_plan    token order for a latent grid (3D Hilbert, row-major, frame
 *               tiles, per-frame 2D Hilbert, VMoBA 2D tiles / 3D cubes)
 *   hsa_perm    gather Q, K, V into the reordered, padded, head-major layout
 *   hsa_score   sub-block pooled block-to-block importance scores
 *   hsa_select  per-query-block lists of key blocks (top-k, threshold +
 *               global budget, the LVSA frame mask, DynamicRad radial masks)
 *   hsa_attn    block-sparse flash attention over the listed key blocks
 *   hsa_unperm  scatter the output back to the original token order
 *   (hsa_attn_tokens fuses the gathers and this scatter into attention)
 *
 * Conventions shared by every entry point
 *  - The caller owns every buffer. Device buffers are device pointers (for
 *    example from torch), 16-byte aligned. The library never allocates or
 *    frees memory, never synchronises, and keeps no pointer after it returns.
 *    Host structs are read only during the call.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = null stream) and
 *    runs asynchronously; outputs are valid once the stream reaches the work.
 *  - Arguments are validated before any launch. On failure nothing is
 *    enqueued, no output is touched, a nonzero hsa_status_t is returned and
 *    hsa_last_error() (per thread) describes the problem.
 *  - Element types: HSA_F32 (float) or HSA_BF16 (bfloat16 bits). Head dim
 *    D in {64, 128}; block size B in {64, 128}; sub-block s in {16,32,64,128}
 *    dividing B.
 *  - Layouts (batch 1; a batch is a loop in the caller):
 *      token-major   x [N tokens][nh heads][D], consecutive tokens
 *                    `tok_stride` elements apart (>= nh*D, so fused QKV
 *                    buffers can be read in place);
 *      reordered     xp [nh][n_pad][D], slot i of head h at (h*n_pad+i)*D;
 *      perm          int32 [n_pad]: token held by slot i, -1 for a pad slot;
 *      blk_len       int32 [nb]: real tokens in block I (they are the first
 *                    blk_len[I] slots of the block; pads follow);
 *      scores        float [nh][nb][nb];
 *      lists         kv_idx int32 [G][nb][max_kv]: the first kv_cnt entries of
 *                    each row, ascending, are the list (hsa_select writes
 *                    only those; the rest of a row is not written and never
 *                    read); kv_cnt int32 [G][nb]; G = nh, or 1 when shared.
 *                    Kernels that read caller lists clamp each length to
 *                    [0, max_kv] and each entry to [0, nb), so a malformed
 *                    list gives wrong rows, never an access outside the
 *                    buffers; the backward pass and the block-mass
 *                    diagnostic search the lists and need them ascending.
 *  - Token n is grid cell (t, y, x) with n = (t*H + y)*W + x.
 */
#ifndef HSA_H
#define HSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSA_ABI_VERSION 4

typedef enum hsa_status {
  HSA_OK = 0,
  HSA_ERR_NULL_PTR = 1,     /* a required pointer is NULL */
  HSA_ERR_BAD_SHAPE = 2,    /* sizes inconsistent or out of range */
  HSA_ERR_BAD_DTYPE = 3,    /* element type not HSA_F32 / HSA_BF16 */
  HSA_ERR_UNSUPPORTED = 4,  /* valid but not implemented (e.g. D = 96) */
  HSA_ERR_WORKSPACE = 5,    /* workspace missing or too small */
  HSA_ERR_BAD_ARG = 6,      /* other invalid argument (mode, alignment, ...) */
  HSA_ERR_HIP = 7           /* the HIP runtime rejected a launch */
} hsa_status_t;

typedef enum { HSA_F32 = 0, HSA_BF16 = 1 } hsa_dtype_t;
typedef enum {
  HSA_ORDER_ROW = 0,
  HSA_ORDER_HILBERT3D = 1,
  HSA_ORDER_FRAME = 2,
  HSA_ORDER_TILE2D = 3, /* per-frame spatial tiles of 8 x (B/8) tokens */
  HSA_ORDER_CUBE3D = 4, /* spatiotemporal cubes of (B/64) x 8 x 8 tokens */
  HSA_ORDER_HILBERT2D = 5 /* frame-major, 2D Hilbert curve inside each frame */
} hsa_order_t;
typedef enum { HSA_AGG_MASS = 0, HSA_AGG_MAX = 1 } hsa_agg_t;
typedef enum {
  HSA_SELECT_TOPK = 0,
  HSA_SELECT_THRESH_GLOBAL = 1,
  HSA_SELECT_LVSA = 2,
  HSA_SELECT_RADIAL = 3,     /* DynamicRad static-ratio radial mask */
  HSA_SELECT_RADIAL_DYN = 4  /* DynamicRad dynamic logit threshold */
} hsa_select_mode_t;

typedef void *hsa_stream_t; /* a hipStream_t */

/* Selection parameters; which fields are read depends on `mode`. */
typedef struct hsa_select_params {
  int32_t mode;            /* hsa_select_mode_t */
  int32_t k;               /* TOPK: key blocks kept per query block, 1..nb */
  double tau;              /* THRESH_GLOBAL: cumulative score per query block, 0 <= tau < 4 */
  double budget_ratio;     /* THRESH_GLOBAL: head budget floor(ratio*nb*nb + 0.5) pairs */
  int32_t frames;          /* LVSA, RADIAL*: number of frames T (nb = frames*tiles_per_frame) */
  int32_t tiles_per_frame; /* LVSA, RADIAL*: tiles (blocks) per frame */
  int32_t C;               /* LVSA: frame budget per query frame, >= 1 */
  int32_t T_per;           /* LVSA: anchor period in frames, >= 1 */
  int32_t step;            /* LVSA: denoising step index, >= 0 */
  double lam;              /* RADIAL*: long-range factor in [0, 1] */
  double delta;            /* RADIAL_DYN: logit margin below the row's best, >= 0 */
} hsa_select_params_t;

/* Library version (HSA_ABI_VERSION) and status strings. */
int hsa_abi_version(void);
const char *hsa_status_str(hsa_status_t status);
/* Detail of the last failure on the calling thread ("" if none). */
const char *hsa_last_error(void);

/*
 * hsa_plan_size -- host-only: padded length and block count of a plan (the
 * blocks DFSAttn, Methodology, design 1, cuts the reordered sequence into;
 * LVSA section 2's per-frame tiles; VMoBA abstract's 2D and 3D partitions).
 * Closed forms, no device work; n_pad and nb are host outputs.
 * ROW / HILBERT3D / HILBERT2D: n_pad = ceil(N/B)*B. FRAME: n_pad = T*ceil(H*W/B)*B.
 * TILE2D / CUBE3D with tiles tT x tH x tW: one block per tile,
 * nb = ceil(T/tT)*ceil(H/tH)*ceil(W/tW). Grid sides 1..1024, n_pad < 2^31.
 * TILE2D needs B a multiple of 8, CUBE3D a multiple of 64.
 */
hsa_status_t hsa_plan_size(int32_t T, int32_t H, int32_t W, int32_t order, int32_t B,
                           int32_t *n_pad, int32_t *nb);

/* Workspace bytes hsa_plan needs (0 for every order but HILBERT3D and HILBERT2D). */
size_t hsa_plan_ws_size(int32_t T, int32_t H, int32_t W, int32_t order);

/*
 * hsa_plan -- token order for a T x H x W latent grid.
 * DFSAttn (Methodology, design 1): tokens are reordered along one global 3D
 * Hilbert curve so consecutive runs (blocks) are compact spatiotemporal
 * neighbourhoods. HILBERT3D walks the enclosing 2^b cube (b = ceil(log2 of
 * the longest side)) in curve order (Skilling's transpose construction, axes
 * (t, y, x), t most significant), keeps in-grid cells and pads the tail.
 * HILBERT2D is frame-major with each frame's cells along the 2D curve of the
 * enclosing square (b from max(H, W)), tail pads: the per-frame curve the
 * global 3D curve is measured against.
 * ROW is row-major with tail pads; FRAME is frame-major with each frame's
 * tokens padded to whole blocks (LVSA section 2 attends frame by frame).
 * TILE2D and CUBE3D are the 2D and 3D block partitions that VMoBA (abstract:
 * layer-wise recurrent 1D-2D-3D partitions; ROW is the 1D one) cycles
 * through: the grid is cut into tiles of 1 x 8 x B/8 (TILE2D) or
 * B/64 x 8 x 8 (CUBE3D) cells (t, y, x), edge tiles clipped to the grid;
 * each tile is one block (its cells in row-major order, then pads), blocks
 * in row-major order of their (t, y, x) tile coordinates.
 * Outputs: perm int32[n_pad] and blk_len int32[nb] (device).
 * ws: device workspace of hsa_plan_ws_size bytes (may be NULL if 0).
 */
hsa_status_t hsa_plan(int32_t T, int32_t H, int32_t W, int32_t order, int32_t B,
                      int32_t *perm, int32_t *blk_len, void *ws, size_t ws_bytes,
                      hsa_stream_t stream);

/*
 * hsa_perm -- gather into the reordered layout: xp[h][i][:] = x[perm[i]][h][:]
 * and zero rows for pad slots (DFSAttn, Methodology, design 1: reorder
 * before attention). Copies 1..3 tensors (Q, K, V) in one launch.
 * xs[j]: token-major input j; xps[j]: reordered output j (nh*n_pad*D
 * elements). xs and xps are host arrays of n_tensors device pointers.
 * tok_stride: elements between consecutive tokens of x; (tok_stride *
 * element size) must be a multiple of 16 bytes; nh*D*element size <= 16 KB.
 * pooled (optional, NULL to skip): also writes the sub-block means that
 * hierarchical scoring pools (DFSAttn, Methodology, design 2) for tensors 0
 * and 1 while they stream through: pooled[(j*nh + h)*(n_pad/pool_s) + u][d]
 * (float) = mean over the real slots of sub-block u (slots u*pool_s ..
 * u*pool_s + pool_s - 1) of x_j[perm[slot]][h][d], 0 for an empty sub-block.
 * pool_s in {16, 32, 64, 128} must divide n_pad; needs n_tensors >= 2.
 * With pooled given, xps[0] or xps[1] may be NULL: that tensor is pooled but
 * not stored (hsa_attn_tokens reads token-major tensors itself).
 */
hsa_status_t hsa_perm(int32_t n_tensors, const void *const *xs, void *const *xps,
                      const int32_t *perm, int32_t N, int32_t n_pad, int32_t nh, int32_t D,
                      int64_t tok_stride, int32_t dtype, int32_t pool_s, float *pooled,
                      hsa_stream_t stream);

/* Workspace bytes for hsa_score when it pools itself: pooled Q and K
 * sub-block means (float). */
size_t hsa_score_ws_size(int32_t nh, int32_t n_pad, int32_t s, int32_t D);

/*
 * hsa_score -- block importance from sub-block summaries.
 * DFSAttn (Methodology, design 2: hierarchical block scoring): blocks are
 * split into sub-blocks of s slots; sub-block means qbar_u, kbar_v (float,
 * over real tokens only) give logits z[u][v] = scale * qbar_u . kbar_v.
 * agg = MASS: p[u][v] = c_v exp(z[u][v] - max) / sum_v' c_v' exp(...) with
 *   c the real-token count of a sub-block; S[I][J] = sum_{u in I} c_u
 *   sum_{v in J} p[u][v] / sum_{u in I} c_u  (rows sum to 1).
 * agg = MAX: S[I][J] = max over u in I, v in J of z[u][v].
 * qp, kp: reordered [nh][nb*B][D]; blk_len: [nb]; S out: float [nh][nb][nb].
 * pooled (optional): the means hsa_perm wrote with pool_s = s; when given,
 * qp, kp and ws are not used (may be NULL) and no pooling pass runs.
 * Otherwise ws must hold hsa_score_ws_size bytes.
 * Limits: nb*B/s <= 2^20 sub-blocks per head. Computed in float32 (matrix
 * cores); beyond 2048 sub-blocks the key sub-blocks are streamed twice.
 */
hsa_status_t hsa_score(const void *qp, const void *kp, const float *pooled,
                       const int32_t *blk_len, int32_t nh, int32_t nb, int32_t B, int32_t s,
                       int32_t D, int32_t dtype, int32_t agg, float scale, float *S, void *ws,
                       size_t ws_bytes, hsa_stream_t stream);

/* Workspace bytes for hsa_select (0 for every mode but THRESH_GLOBAL). */
size_t hsa_select_ws_size(int32_t nh, int32_t nb, const hsa_select_params_t *p);

/*
 * hsa_select_list_width -- host-only: the smallest max_kv hsa_select accepts
 * for these parameters (k for TOPK; nb for THRESH_GLOBAL and RADIAL_DYN; the
 * longest list for LVSA and RADIAL). Returns 0 for invalid parameters.
 */
int32_t hsa_select_list_width(int32_t nh, int32_t nb, const hsa_select_params_t *p);

/*
 * hsa_select -- per-query-block ascending lists of key blocks.
 * Ranking is by score, ties to the lower index (lower I*nb + J globally).
 * TOPK (DFSAttn, Methodology, design 3: a sparsity budget): the k highest
 *   scores of each row. Lists [nh][nb][max_kv], max_kv >= k.
 * THRESH_GLOBAL (VMoBA abstract: threshold selection by cumulative similarity
 *   and global selection over the head; DFSAttn design 3: a budget that
 *   shrinks over steps): per row, the shortest score-ranked prefix whose sum
 *   reaches tau (sums exact in 2^-62 fixed point; at least one block); then
 *   per head the best-ranked remaining pairs are added until the head holds
 *   floor(budget_ratio*nb*nb + 0.5) pairs. Scores must be finite and >= 0
 *   (MASS). Lists [nh][nb][max_kv]; max_kv must be nb; nb <= 1024.
 * LVSA (LVSA section 2, A(t) = G_s u W(t)): frame t attends to the anchor
 *   frames f = step (mod T_per) and to the C - |G_s| nearest non-anchor
 *   frames (ties to the earlier frame; at least one); every tile of frame t
 *   lists every tile of those frames. S is not read (may be NULL). One list
 *   set shared by all heads: kv_idx [nb][max_kv], kv_cnt [nb].
 * RADIAL (DynamicRad section 2: static-ratio mode over a logarithmic radial
 *   window with long-range factor lam): blocks are frame tiles (block
 *   t*P + j is tile j of frame t, P = tiles_per_frame). Query tile (t, j)
 *   keeps, in every frame f at distance d = |t - f|, the
 *   w(d) = min(P, max(ceil(P / 2^floor(log2(d+1))), ceil(lam*P), 1)) tiles
 *   nearest to position j (ties to the lower tile): the run starting at
 *   clamp(j - floor(w/2), 0, P - w). S is not read (may be NULL). Shared by
 *   all heads: kv_idx [nb][max_kv], kv_cnt [nb]; max_kv >= the width that
 *   hsa_select_list_width reports.
 * RADIAL_DYN (DynamicRad section 2: dynamic-threshold mode, pre-softmax
 *   logits as importance): per head, the RADIAL window of each row plus
 *   every block J with S[h][I][J] >= max_J S[h][I][J] - (float)delta,
 *   formed and compared in float. S holds block logits (hsa_score with
 *   HSA_AGG_MAX), finite. Lists [nh][nb][max_kv]; max_kv must be nb.
 * ws: device workspace of hsa_select_ws_size bytes.
 */
hsa_status_t hsa_select(const float *S, int32_t nh, int32_t nb, const hsa_select_params_t *p,
                        int32_t *kv_idx, int32_t *kv_cnt, int32_t max_kv, void *ws,
                        size_t ws_bytes, hsa_stream_t stream);

/*
 * hsa_select_noalloc -- hsa_select without a caller workspace, for callers
 *   that cannot allocate device memory (code under HIP graph capture, tight
 *   serving loops, harnesses that forbid allocation). Same arguments, lists,
 *   results and errors as hsa_select minus ws/ws_bytes; the workspace is a
 *   static array of HSA_SELECT_NOALLOC_MAX_WS bytes that the library holds on
 *   every GPU it runs on until the process ends. Parameters whose workspace
 *   (hsa_select_ws_size) exceeds that size fail with HSA_ERR_UNSUPPORTED
 *   before anything is enqueued (THRESH_GLOBAL fits up to nh = 64 heads at
 *   nb = 1024; the other modes need no workspace). The call allocates nothing
 *   and clears what it needs itself; its first call on a device looks up
 *   that device's copy of the array (the device current at the call).
 *   Calls that overlap on one GPU (several streams or threads at once) share
 *   that GPU's array and race: serialise them.
 */
#define HSA_SELECT_NOALLOC_MAX_WS ((size_t)4 << 20)
hsa_status_t hsa_select_noalloc(const float *S, int32_t nh, int32_t nb, const hsa_select_params_t *p,
                                int32_t *kv_idx, int32_t *kv_cnt, int32_t max_kv, hsa_stream_t stream);

/*
 * hsa_attn -- block-sparse attention: for every query slot i of block I,
 *   o_i = sum_j softmax_j(scale * q_i . k_j) v_j over the real key slots j of
 *   the blocks listed for I (DFSAttn Significance: block-wise execution over
 *   reordered tokens; DynamicRad section 2.2: a shared candidate set
 *   aggregated block-wise). Non-causal. Unlisted blocks are never read.
 * qp, kp, vp, op: reordered [nh][nb*B][D]; op rows of pad slots are zero.
 * lse: optional float [nh][nb*B] natural-log log-sum-exp (NULL to skip).
 * kv_shared: bit 0 set if the lists are [nb][max_kv] shared by all heads;
 *   bit 1 set to say that the listed blocks often hold at most 64 real keys
 *   (frame tiles, clipped 2D/3D partition tiles): bf16 launches without lse
 *   and with 128-slot blocks then walk each list by 64-key stages and leave
 *   out such a block's empty second stage (same output bits; lists shared
 *   by all heads are walked that way whether or not the bit is set).
 *   Other bits must be zero.
 * order: optional int32 [G*nb] processing order from hsa_attn_order (G = nh,
 *   or 1 when shared): the b-th workgroup launched handles list row order[b]
 *   (when shared, the b-th group of nh workgroups handles block order[b] for
 *   every head). NULL: natural order, neighbouring blocks on one XCD. Entries
 *   are clamped to the valid range; a non-permutation computes some rows
 *   twice and leaves others unwritten.
 * BF16 runs on bf16 matrix cores with float accumulation and softmax; the
 * probabilities are rounded to bf16 for the value product and the output is
 * rounded to bf16 (nearest even); the output bits do not depend on whether
 * lse is requested. F32 computes in float throughout.
 * Results are deterministic, and the same lists give the same bits in
 * buffers of any capacity max_kv.
 */
hsa_status_t hsa_attn(const void *qp, const void *kp, const void *vp, void *op, float *lse,
                      const int32_t *blk_len, const int32_t *kv_idx, const int32_t *kv_cnt,
                      const int32_t *order, int32_t max_kv, int32_t kv_shared, int32_t nh,
                      int32_t nb, int32_t B, int32_t D, int32_t dtype, float scale,
                      hsa_stream_t stream);

/*
 * hsa_attn_tokens -- hsa_attn on token-major tensors: the reorder (DFSAttn,
 *   Methodology, design 1) of Q, optionally of K and V, and the inverse
 *   reorder of the output happen in the attention kernel's own loads and
 *   stores (rows are looked up in perm), so no reordered copy of those
 *   tensors is made and no hsa_unperm pass runs. Results are bit-identical
 *   to hsa_perm -> hsa_attn -> hsa_unperm on the same lists.
 * q: token-major [N][nh][D], q_stride elements between tokens (for example
 *   the Q slice of a fused QKV buffer). o: token-major output, o_stride
 *   elements between tokens; every real token's row is written once and
 *   nothing else in o is touched.
 * k, v: kv_stride > 0: token-major like q with that token stride (the byte
 *   span N*kv_stride*element size must stay below 4 GiB, N <= 2^24 and a
 *   token row below 16 MiB; otherwise HSA_ERR_UNSUPPORTED); kv_stride = 0:
 *   reordered [nh][nb*B][D] from hsa_perm.
 * Strides are >= nh*D elements and multiples of 16 bytes.
 * perm: the plan's int32 [nb*B] slot -> token map; entries are -1 or < N,
 *   and a slot is real exactly when it lies in the first blk_len[I] slots of
 *   its block (as hsa_plan writes them). Pad slots get zero query rows; pad
 *   key rows read token 0 and are masked.
 * lse, lists, order, scale, dtype: as for hsa_attn (lse stays in the
 *   reordered layout [nh][nb*B]).
 */
hsa_status_t hsa_attn_tokens(const void *q, const void *k, const void *v, void *o, int64_t q_stride,
                             int64_t kv_stride, int64_t o_stride, float *lse, const int32_t *perm,
                             int32_t N, const int32_t *blk_len, const int32_t *kv_idx,
                             const int32_t *kv_cnt, const int32_t *order, int32_t max_kv,
                             int32_t kv_shared, int32_t nh, int32_t nb, int32_t B, int32_t D,
                             int32_t dtype, float scale, hsa_stream_t stream);

/*
 * hsa_attn_order -- a processing order for hsa_attn that dispatches each
 *   head's longest lists first, so that rows with many key blocks (the
 *   cumulative threshold with a global budget gives rows very different list
 *   lengths, VMoBA abstract) do not trail at the end of the launch, while a
 *   head's rows stay together (they share key/value blocks in cache).
 * kv_cnt: int32 [G][nb] list lengths (G = nh, or 1 for shared lists), each in
 *   [0, max_kv] (values outside are clamped for sorting); max_kv <= 4095.
 * order: int32 [G*nb] output, a permutation of the list rows g*nb + I: head
 *   g's rows occupy positions g*nb .. g*nb + nb - 1 with non-increasing
 *   kv_cnt. Rows of equal length may appear in any order; hsa_attn's results
 *   do not depend on the order. One workgroup per head.
 */
hsa_status_t hsa_attn_order(const int32_t *kv_cnt, int32_t G, int32_t nb, int32_t max_kv,
                            int32_t *order, hsa_stream_t stream);

/*
 * hsa_attn_bwd -- gradients of hsa_attn (same lists, same attended keys) with
 *   respect to the reordered Q, K and V, for block-sparse training (VMoBA
 *   abstract: native training with block-sparse attention):
 *     P = softmax(scale q K^T) over the row's attended keys,
 *     dV = P^T dO,  dS = P * (dO V^T - rowsum(dO * O)),
 *     dQ = scale dS K,  dK = scale dS^T Q.
 * op: the forward output; lse: the forward's log-sum-exp (required); dop:
 *   dO, reordered like op. dqp, dkp, dvp: outputs [nh][nb*B][D] in the input
 *   dtype; rows of pad slots are zero, and pad rows of dop are ignored.
 * BF16 computes in float on matrix cores with P and dS rounded to bf16 for
 *   the products; F32 in float. Results are bit-reproducible (fixed sum
 *   order, no atomics).
 * ws: device workspace of hsa_attn_bwd_ws_size bytes (row deltas, the
 *   log-sum-exp in log2 units with pad rows at +inf, the transposed lists --
 *   for each key block, the query blocks that list it -- and longest-first
 *   processing orders for both list directions).
 */
size_t hsa_attn_bwd_ws_size(int32_t nh, int32_t nb, int32_t B, int32_t kv_shared);
hsa_status_t hsa_attn_bwd(const void *qp, const void *kp, const void *vp, const void *op,
                          const void *dop, const float *lse, const int32_t *blk_len,
                          const int32_t *kv_idx, const int32_t *kv_cnt, int32_t max_kv,
                          int32_t kv_shared, int32_t nh, int32_t nb, int32_t B, int32_t D,
                          int32_t dtype, float scale, void *dqp, void *dkp, void *dvp, void *ws,
                          size_t ws_bytes, hsa_stream_t stream);

/*
 * hsa_unperm -- scatter back to token order: o[perm[i]][h][:] = op[h][i][:]
 * for every real slot i (pad slots are dropped). DFSAttn (Methodology,
 * design 1): attention runs on the reordered sequence and its outputs go
 * back to the original token order (the inverse of hsa_perm's gather).
 * op: reordered [nh][n_pad][D]; o: token-major [N][nh][D] with tok_stride
 * elements between tokens (>= nh*D, a multiple of 16 bytes); perm: the
 * plan's slot -> token map. Rows of o that no real slot maps to are not
 * touched. Errors as hsa_perm (checked before any launch).
 */
hsa_status_t hsa_unperm(const void *op, void *o, const int32_t *perm, int32_t N, int32_t n_pad,
                        int32_t nh, int32_t D, int64_t tok_stride, int32_t dtype,
                        hsa_stream_t stream);

/*
 * hsa_block_mass -- selection diagnostic (off the hot path): for sampled
 *   query slots, the exact attention mass on every key block and the recall
 *   of the selected lists. Block selection (DFSAttn, Methodology, designs 2-3;
 *   VMoBA abstract; DynamicRad section 2) keeps the key blocks it estimates
 *   to carry a query block's attention; this measures what they really carry.
 * rows: int32 [nh][n_rows], slots of each head (values outside [0, nb*B) are
 *   clamped; pad slots give a zero query, i.e. uniform attention).
 * mass: optional float [nh][n_rows][nb]: the dense softmax of scale*q.k over
 *   every real key, summed over the real keys of block J (rows sum to 1).
 * recall: optional float [nh][n_rows]: the mass on the blocks listed for the
 *   row's own query block (kv_idx/kv_cnt as hsa_attn, required with recall).
 * At least one of mass and recall. Float arithmetic throughout.
 */
hsa_status_t hsa_block_mass(const void *qp, const void *kp, const int32_t *blk_len,
                            const int32_t *rows, int32_t n_rows, int32_t nh, int32_t nb,
                            int32_t B, int32_t D, int32_t dtype, float scale,
                            const int32_t *kv_idx, const int32_t *kv_cnt, int32_t max_kv,
                            int32_t kv_shared, float *mass, float *recall, hsa_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HSA_H */
