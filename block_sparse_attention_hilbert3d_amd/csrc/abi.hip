// C ABI: argument validation (before any launch) and dispatch to the kernels.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>
#include <string>

#include "common.h"

namespace hsa_host {

static thread_local std::string g_last_error;

hsa_status_t fail(hsa_status_t code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

hsa_status_t check_launch(const char *what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(HSA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return HSA_OK;
}

// Defined next to their kernels.
size_t plan_hilbert_groups(int T, int H, int W, int &bits, uint32_t &cube, int dims);
hsa_status_t launch_plan(int T, int H, int W, int order, int B, int n_pad, int nb, int32_t *perm,
                         int32_t *blk_len, void *ws, hipStream_t stream);
hsa_status_t launch_perm(int n, const void *const *xs, void *const *xps, const int32_t *perm,
                         int n_pad, int nh, int D, int64_t tok_stride, int esize, int pool_s,
                         float *pooled, hipStream_t stream);
hsa_status_t launch_unperm(const void *op, void *o, const int32_t *perm, int n_pad, int nh, int D,
                           int64_t tok_stride, int esize, hipStream_t stream);
size_t score_ws_bytes(int nh, int n_pad, int s, int D);
hsa_status_t launch_score(const void *qp, const void *kp, const float *pooled,
                          const int32_t *blk_len, int nh, int nb, int B, int s, int D, int dtype,
                          int agg, float scale, float *S, void *ws, hipStream_t stream);
size_t select_ws_bytes(int nh, int nb, int mode);
hsa_status_t launch_select(const float *S, int nh, int nb, const hsa_select_params_t *p,
                           int32_t *kv_idx, int32_t *kv_cnt, int max_kv, void *ws,
                           hipStream_t stream);
hsa_status_t launch_attn(const void *qp, const void *kp, const void *vp, void *op, float *lse,
                         const int32_t *blk_len, const int32_t *kv_idx, const int32_t *kv_cnt,
                         const int32_t *order, int max_kv, int kv_shared, int nh, int nb, int B,
                         int D, int dtype, float scale, const int32_t *perm, int64_t q_stride,
                         int64_t kv_stride, int64_t o_stride, hipStream_t stream);
size_t attn_bwd_ws_bytes(int nh, int nb, int B, int G);
hsa_status_t launch_attn_bwd(const void *qp, const void *kp, const void *vp, const void *op, const void *dop,
                             const float *lse, const int32_t *blk_len, const int32_t *kv_idx,
                             const int32_t *kv_cnt, int max_kv, int kv_shared, int nh, int nb, int B, int D,
                             int dtype, float scale, void *dqp, void *dkp, void *dvp, void *ws,
                             hipStream_t stream);
hsa_status_t launch_block_mass(const void *qp, const void *kp, const int32_t *blk_len, const int32_t *rows,
                               int n_rows, int nh, int nb, int B, int D, int dtype, float scale,
                               const int32_t *kv_idx, const int32_t *kv_cnt, int max_kv, int kv_shared,
                               float *mass, float *recall, hipStream_t stream);
hsa_status_t launch_attn_order(const int32_t *kv_cnt, int G, int nb, int max_kv, int32_t *order,
                               hipStream_t stream);

static int esize_of(int dtype) { return dtype == HSA_BF16 ? 2 : 4; }

static hsa_status_t check_dtype(int dtype) {
  if (dtype != HSA_F32 && dtype != HSA_BF16) return fail(HSA_ERR_BAD_DTYPE, "dtype %d is not HSA_F32 or HSA_BF16", dtype);
  return HSA_OK;
}

static hsa_status_t check_D(int D) {
  if (D != 64 && D != 128) return fail(HSA_ERR_UNSUPPORTED, "head dim %d not in {64, 128}", D);
  return HSA_OK;
}

static hsa_status_t check_B(int B) {
  if (B != 64 && B != 128) return fail(HSA_ERR_UNSUPPORTED, "block size %d not in {64, 128}", B);
  return HSA_OK;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

static hsa_status_t plan_size(int T, int H, int W, int order, int B, int32_t *n_pad, int32_t *nb) {
  if (T < 1 || H < 1 || W < 1 || T > 1024 || H > 1024 || W > 1024)
    return fail(HSA_ERR_BAD_SHAPE, "grid %dx%dx%d: each side must be in 1..1024", T, H, W);
  if (B < 1 || B > 4096) return fail(HSA_ERR_BAD_SHAPE, "block size %d out of range", B);
  const int64_t N = static_cast<int64_t>(T) * H * W;
  int64_t np;
  if (order == HSA_ORDER_ROW || order == HSA_ORDER_HILBERT3D || order == HSA_ORDER_HILBERT2D) {
    np = (N + B - 1) / B * B;
  } else if (order == HSA_ORDER_TILE2D || order == HSA_ORDER_CUBE3D) {
    const bool two = order == HSA_ORDER_TILE2D;
    const int unit = two ? 8 : 64;
    if (B % unit != 0) return fail(HSA_ERR_UNSUPPORTED, "%s needs B a multiple of %d (B=%d)", two ? "TILE2D" : "CUBE3D", unit, B);
    const int tT = two ? 1 : B / 64, tH = 8, tW = two ? B / 8 : 8;
    np = static_cast<int64_t>((T + tT - 1) / tT) * ((H + tH - 1) / tH) * ((W + tW - 1) / tW) * B;
  } else if (order == HSA_ORDER_FRAME) {
    np = static_cast<int64_t>(T) * ((static_cast<int64_t>(H) * W + B - 1) / B) * B;
  } else {
    return fail(HSA_ERR_BAD_ARG, "unknown order %d", order);
  }
  if (np >= (1ll << 31) - 1) return fail(HSA_ERR_BAD_SHAPE, "padded length %lld too large", static_cast<long long>(np));
  *n_pad = static_cast<int32_t>(np);
  *nb = static_cast<int32_t>(np / B);
  return HSA_OK;
}

}  // namespace hsa_host

using namespace hsa_host;

extern "C" {

int hsa_abi_version(void) { return HSA_ABI_VERSION; }

const char *hsa_status_str(hsa_status_t s) {
  switch (s) {
    case HSA_OK: return "ok";
    case HSA_ERR_NULL_PTR: return "null pointer";
    case HSA_ERR_BAD_SHAPE: return "bad shape";
    case HSA_ERR_BAD_DTYPE: return "bad dtype";
    case HSA_ERR_UNSUPPORTED: return "unsupported";
    case HSA_ERR_WORKSPACE: return "workspace too small";
    case HSA_ERR_BAD_ARG: return "bad argument";
    case HSA_ERR_HIP: return "hip error";
  }
  return "unknown status";
}

const char *hsa_last_error(void) { return g_last_error.c_str(); }

hsa_status_t hsa_plan_size(int32_t T, int32_t H, int32_t W, int32_t order, int32_t B,
                           int32_t *n_pad, int32_t *nb) {
  if (!n_pad || !nb) return fail(HSA_ERR_NULL_PTR, "hsa_plan_size: null output");
  g_last_error.clear();
  return plan_size(T, H, W, order, B, n_pad, nb);
}

size_t hsa_plan_ws_size(int32_t T, int32_t H, int32_t W, int32_t order) {
  if ((order != HSA_ORDER_HILBERT3D && order != HSA_ORDER_HILBERT2D) || T < 1 || H < 1 || W < 1 ||
      T > 1024 || H > 1024 || W > 1024)
    return 0;
  int bits;
  uint32_t cube;
  return plan_hilbert_groups(T, H, W, bits, cube, order == HSA_ORDER_HILBERT3D ? 3 : 2) * sizeof(int32_t);
}

hsa_status_t hsa_plan(int32_t T, int32_t H, int32_t W, int32_t order, int32_t B, int32_t *perm,
                      int32_t *blk_len, void *ws, size_t ws_bytes, hsa_stream_t stream) {
  g_last_error.clear();
  if (!perm || !blk_len) return fail(HSA_ERR_NULL_PTR, "hsa_plan: perm and blk_len are required");
  int32_t n_pad, nb;
  hsa_status_t st = plan_size(T, H, W, order, B, &n_pad, &nb);
  if (st != HSA_OK) return st;
  const size_t need = hsa_plan_ws_size(T, H, W, order);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(HSA_ERR_WORKSPACE, "hsa_plan: workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
  return launch_plan(T, H, W, order, B, n_pad, nb, perm, blk_len, ws, static_cast<hipStream_t>(stream));
}

hsa_status_t hsa_perm(int32_t n_tensors, const void *const *xs, void *const *xps,
                      const int32_t *perm, int32_t N, int32_t n_pad, int32_t nh, int32_t D,
                      int64_t tok_stride, int32_t dtype, int32_t pool_s, float *pooled,
                      hsa_stream_t stream) {
  g_last_error.clear();
  if (n_tensors < 1 || n_tensors > 3) return fail(HSA_ERR_BAD_ARG, "hsa_perm: n_tensors %d not in 1..3", n_tensors);
  if (!xs || !xps || !perm) return fail(HSA_ERR_NULL_PTR, "hsa_perm: null pointer array or perm");
  for (int i = 0; i < n_tensors; ++i) {
    if (!xs[i]) return fail(HSA_ERR_NULL_PTR, "hsa_perm: input %d is null", i);
    // a null output is allowed for a pooled tensor (0 or 1): pooled, not stored
    if (!xps[i] && !(pooled && i < 2)) return fail(HSA_ERR_NULL_PTR, "hsa_perm: output %d is null", i);
  }
  hsa_status_t st;
  if ((st = check_dtype(dtype)) != HSA_OK || (st = check_D(D)) != HSA_OK) return st;
  if (N < 1 || n_pad < N || nh < 1) return fail(HSA_ERR_BAD_SHAPE, "hsa_perm: N=%d n_pad=%d nh=%d", N, n_pad, nh);
  if (tok_stride < static_cast<int64_t>(nh) * D) return fail(HSA_ERR_BAD_SHAPE, "hsa_perm: tok_stride %lld < nh*D", static_cast<long long>(tok_stride));
  const int es = esize_of(dtype);
  if ((tok_stride * es) % 16 != 0) return fail(HSA_ERR_BAD_ARG, "hsa_perm: token stride must be a multiple of 16 bytes");
  if (static_cast<int64_t>(nh) * n_pad * D >= (1ll << 40)) return fail(HSA_ERR_BAD_SHAPE, "hsa_perm: tensor too large");
  if (static_cast<int64_t>(nh) * D * es / 16 > 1024) return fail(HSA_ERR_UNSUPPORTED, "hsa_perm: nh*D*elem_size must be <= 16 KB");
  for (int i = 0; i < n_tensors; ++i)
    if (!aligned16(xs[i]) || (xps[i] && !aligned16(xps[i]))) return fail(HSA_ERR_BAD_ARG, "hsa_perm: tensor %d not 16-byte aligned", i);
  if (pooled) {
    if (pool_s != 16 && pool_s != 32 && pool_s != 64 && pool_s != 128) return fail(HSA_ERR_UNSUPPORTED, "hsa_perm: pool_s %d not in {16,32,64,128}", pool_s);
    if (n_pad % pool_s) return fail(HSA_ERR_BAD_SHAPE, "hsa_perm: pool_s %d does not divide n_pad %d", pool_s, n_pad);
    if (n_tensors < 2) return fail(HSA_ERR_BAD_ARG, "hsa_perm: pooling needs Q and K (n_tensors >= 2)");
    if (!aligned16(pooled)) return fail(HSA_ERR_BAD_ARG, "hsa_perm: pooled must be 16-byte aligned");
  }
  return launch_perm(n_tensors, xs, xps, perm, n_pad, nh, D, tok_stride, es, pool_s, pooled,
                     static_cast<hipStream_t>(stream));
}

size_t hsa_score_ws_size(int32_t nh, int32_t n_pad, int32_t s, int32_t D) {
  if (nh < 1 || n_pad < 1 || s < 1 || D < 1 || n_pad % s) return 0;
  return score_ws_bytes(nh, n_pad, s, D);
}

hsa_status_t hsa_score(const void *qp, const void *kp, const float *pooled,
                       const int32_t *blk_len, int32_t nh, int32_t nb, int32_t B, int32_t s,
                       int32_t D, int32_t dtype, int32_t agg, float scale, float *S, void *ws,
                       size_t ws_bytes, hsa_stream_t stream) {
  g_last_error.clear();
  if ((!pooled && (!qp || !kp)) || !blk_len || !S) return fail(HSA_ERR_NULL_PTR, "hsa_score: null input or output");
  hsa_status_t st;
  if ((st = check_dtype(dtype)) != HSA_OK || (st = check_D(D)) != HSA_OK || (st = check_B(B)) != HSA_OK) return st;
  if (s != 16 && s != 32 && s != 64 && s != 128) return fail(HSA_ERR_UNSUPPORTED, "hsa_score: sub-block %d not in {16,32,64,128}", s);
  if (B % s) return fail(HSA_ERR_BAD_SHAPE, "hsa_score: sub-block %d does not divide block %d", s, B);
  if (nh < 1 || nb < 1) return fail(HSA_ERR_BAD_SHAPE, "hsa_score: nh=%d nb=%d", nh, nb);
  if (static_cast<int64_t>(nb) * (B / s) > (1 << 20)) return fail(HSA_ERR_UNSUPPORTED, "hsa_score: %lld sub-blocks > 2^20", static_cast<long long>(nb) * (B / s));
  if (agg != HSA_AGG_MASS && agg != HSA_AGG_MAX) return fail(HSA_ERR_BAD_ARG, "hsa_score: unknown aggregation %d", agg);
  if (!(scale > 0.f) || !isfinite(scale)) return fail(HSA_ERR_BAD_ARG, "hsa_score: scale must be finite and positive");
  if (!aligned16(S)) return fail(HSA_ERR_BAD_ARG, "hsa_score: S must be 16-byte aligned");
  if (pooled) {
    if (!aligned16(pooled)) return fail(HSA_ERR_BAD_ARG, "hsa_score: pooled must be 16-byte aligned");
  } else {
    if (!aligned16(qp) || !aligned16(kp)) return fail(HSA_ERR_BAD_ARG, "hsa_score: buffers must be 16-byte aligned");
    const size_t need = score_ws_bytes(nh, nb * B, s, D);
    if (!ws || ws_bytes < need) return fail(HSA_ERR_WORKSPACE, "hsa_score: workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
    if (!aligned16(ws)) return fail(HSA_ERR_BAD_ARG, "hsa_score: workspace must be 16-byte aligned");
  }
  return launch_score(qp, kp, pooled, blk_len, nh, nb, B, s, D, dtype, agg, scale, S, ws,
                      static_cast<hipStream_t>(stream));
}

// Radial window width at temporal distance d (DynamicRad static ratio): the
// frame's P tiles halved (rounded up) each time d + 1 doubles, floored at
// ceil(lam * P) and 1.
static int radial_w(int d, int P, int lam_tiles) {
  int k = 0;
  while ((2 << k) <= d + 1) ++k;
  const int w = (P + (1 << k) - 1) >> k;
  const int m = w > lam_tiles ? w : lam_tiles;
  return m < 1 ? 1 : (m > P ? P : m);
}

static int radial_lam_tiles(double lam, int P) { return static_cast<int>(ceil(lam * P)); }

static int radial_list_width(int T, int P, double lam) {
  const int lt = radial_lam_tiles(lam, P);
  int best = 0;
  for (int t = 0; t < T; ++t) {
    int n = 0;
    for (int f = 0; f < T; ++f) n += radial_w(t > f ? t - f : f - t, P, lt);
    best = n > best ? n : best;
  }
  return best;
}

static int lvsa_list_width(const hsa_select_params_t *p) {
  const int rot = p->step % p->T_per;
  const int anchors = rot < p->frames ? (p->frames - 1 - rot) / p->T_per + 1 : 0;
  const int others = p->frames - anchors;
  const int want = p->C - anchors > 1 ? p->C - anchors : 1;
  const int nw = others < want ? others : want;
  return (anchors + nw) * p->tiles_per_frame;
}

int32_t hsa_select_list_width(int32_t nh, int32_t nb, const hsa_select_params_t *p) {
  if (!p || nh < 1 || nb < 1) return 0;
  switch (p->mode) {
    case HSA_SELECT_TOPK: return p->k;
    case HSA_SELECT_THRESH_GLOBAL: return nb;
    case HSA_SELECT_RADIAL_DYN: return nb;
    case HSA_SELECT_LVSA:
      if (p->frames < 1 || p->tiles_per_frame < 1 || p->T_per < 1 || p->step < 0 || p->C < 1) return 0;
      return lvsa_list_width(p);
    case HSA_SELECT_RADIAL:
      if (p->frames < 1 || p->frames > 1024 || p->tiles_per_frame < 1 || !(p->lam >= 0.0) || !(p->lam <= 1.0)) return 0;
      return radial_list_width(p->frames, p->tiles_per_frame, p->lam);
    default: return 0;
  }
}

size_t hsa_select_ws_size(int32_t nh, int32_t nb, const hsa_select_params_t *p) {
  if (!p || nh < 1 || nb < 1) return 0;
  return select_ws_bytes(nh, nb, p->mode);
}

}  // extern "C"

namespace hsa_host {

// Argument checks shared by hsa_select and hsa_select_noalloc (everything
// but the workspace); `who` names the entry point in the message.
static hsa_status_t check_select_args(const char *who, const float *S, int32_t nh, int32_t nb,
                                      const hsa_select_params_t *p, const int32_t *kv_idx,
                                      const int32_t *kv_cnt, int32_t max_kv) {
  if (!p || !kv_idx || !kv_cnt) return fail(HSA_ERR_NULL_PTR, "%s: params and lists are required", who);
  if (nh < 1 || nb < 1) return fail(HSA_ERR_BAD_SHAPE, "%s: nh=%d nb=%d", who, nh, nb);
  if (max_kv < 1) return fail(HSA_ERR_BAD_SHAPE, "%s: max_kv=%d", who, max_kv);
  switch (p->mode) {
    case HSA_SELECT_TOPK:
      if (!S) return fail(HSA_ERR_NULL_PTR, "%s: scores required", who);
      if (nb > 1024) return fail(HSA_ERR_UNSUPPORTED, "%s: nb %d > 1024", who, nb);
      if (p->k < 1 || p->k > nb) return fail(HSA_ERR_BAD_ARG, "%s: k=%d not in 1..%d", who, p->k, nb);
      if (max_kv < p->k) return fail(HSA_ERR_BAD_SHAPE, "%s: max_kv %d < k %d", who, max_kv, p->k);
      break;
    case HSA_SELECT_THRESH_GLOBAL: {
      if (!S) return fail(HSA_ERR_NULL_PTR, "%s: scores required", who);
      if (nb > 1024) return fail(HSA_ERR_UNSUPPORTED, "%s: nb %d > 1024", who, nb);
      // tau * 2^62 must fit the unsigned 64-bit fixed-point target
      if (!(p->tau >= 0.0) || !(p->tau < 4.0)) return fail(HSA_ERR_BAD_ARG, "%s: tau %g not in [0, 4)", who, p->tau);
      if (!(p->budget_ratio >= 0.0) || !(p->budget_ratio <= 1.0)) return fail(HSA_ERR_BAD_ARG, "%s: budget_ratio %g not in [0, 1]", who, p->budget_ratio);
      if (max_kv != nb) return fail(HSA_ERR_BAD_SHAPE, "%s: THRESH_GLOBAL needs max_kv == nb", who);
      break;
    }
    case HSA_SELECT_LVSA: {
      if (p->frames < 1 || p->frames > 1024 || p->tiles_per_frame < 1) return fail(HSA_ERR_BAD_SHAPE, "%s: frames=%d tiles_per_frame=%d", who, p->frames, p->tiles_per_frame);
      if (static_cast<int64_t>(p->frames) * p->tiles_per_frame != nb) return fail(HSA_ERR_BAD_SHAPE, "%s: frames*tiles_per_frame != nb", who);
      if (p->C < 1 || p->T_per < 1 || p->step < 0) return fail(HSA_ERR_BAD_ARG, "%s: C=%d T_per=%d step=%d", who, p->C, p->T_per, p->step);
      // largest |A(t)|: all anchors plus max(C - anchors, 1) window frames
      const int64_t need = lvsa_list_width(p);
      if (max_kv < need) return fail(HSA_ERR_BAD_SHAPE, "%s: max_kv %d < %lld tiles per list", who, max_kv, static_cast<long long>(need));
      break;
    }
    case HSA_SELECT_RADIAL:
    case HSA_SELECT_RADIAL_DYN: {
      if (p->frames < 1 || p->frames > 1024 || p->tiles_per_frame < 1) return fail(HSA_ERR_BAD_SHAPE, "%s: frames=%d tiles_per_frame=%d", who, p->frames, p->tiles_per_frame);
      if (static_cast<int64_t>(p->frames) * p->tiles_per_frame != nb) return fail(HSA_ERR_BAD_SHAPE, "%s: frames*tiles_per_frame != nb", who);
      if (!(p->lam >= 0.0) || !(p->lam <= 1.0)) return fail(HSA_ERR_BAD_ARG, "%s: lam %g not in [0, 1]", who, p->lam);
      if (p->mode == HSA_SELECT_RADIAL) {
        const int need = radial_list_width(p->frames, p->tiles_per_frame, p->lam);
        if (max_kv < need) return fail(HSA_ERR_BAD_SHAPE, "%s: max_kv %d < %d tiles per list", who, max_kv, need);
      } else {
        if (!S) return fail(HSA_ERR_NULL_PTR, "%s: scores required", who);
        if (!(p->delta >= 0.0) || !isfinite(p->delta)) return fail(HSA_ERR_BAD_ARG, "%s: delta %g must be finite and >= 0", who, p->delta);
        if (max_kv != nb) return fail(HSA_ERR_BAD_SHAPE, "%s: RADIAL_DYN needs max_kv == nb", who);
        if (nb > 4096) return fail(HSA_ERR_UNSUPPORTED, "%s: nb %d > 4096", who, nb);
      }
      break;
    }
    default:
      return fail(HSA_ERR_BAD_ARG, "%s: unknown mode %d", who, p->mode);
  }
  return HSA_OK;
}

}  // namespace hsa_host

extern "C" {

hsa_status_t hsa_select(const float *S, int32_t nh, int32_t nb, const hsa_select_params_t *p,
                        int32_t *kv_idx, int32_t *kv_cnt, int32_t max_kv, void *ws,
                        size_t ws_bytes, hsa_stream_t stream) {
  g_last_error.clear();
  hsa_status_t st = check_select_args("hsa_select", S, nh, nb, p, kv_idx, kv_cnt, max_kv);
  if (st != HSA_OK) return st;
  const size_t need = select_ws_bytes(nh, nb, p->mode);
  if (need > 0) {
    if (!ws || ws_bytes < need) return fail(HSA_ERR_WORKSPACE, "hsa_select: workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
    if (!aligned16(ws)) return fail(HSA_ERR_BAD_ARG, "hsa_select: workspace must be 16-byte aligned");
  }
  return launch_select(S, nh, nb, p, kv_idx, kv_cnt, max_kv, ws, static_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace hsa_host {

// Workspace of hsa_select_noalloc: one array per GPU, part of the loaded
// code object (nothing is allocated at run time). In host code the name is a
// host-side stand-in, never a device address: kernels get the address that
// hipGetSymbolAddress reports for the current device.
constexpr size_t kSelectScratchBytes = HSA_SELECT_NOALLOC_MAX_WS;
static __device__ __align__(256) unsigned char scratch[kSelectScratchBytes];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void *g_scratch_dev[kMaxDevices];

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
static hsa_status_t scratch_on_current_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(HSA_ERR_HIP, "hsa_select_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(HSA_ERR_UNSUPPORTED, "hsa_select_noalloc: device %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(HSA_ERR_HIP, "hsa_select_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(e));
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return HSA_OK;
}

}  // namespace hsa_host

extern "C" {

hsa_status_t hsa_select_noalloc(const float *S, int32_t nh, int32_t nb, const hsa_select_params_t *p,
                                int32_t *kv_idx, int32_t *kv_cnt, int32_t max_kv, hsa_stream_t stream) {
  g_last_error.clear();
  hsa_status_t st = check_select_args("hsa_select_noalloc", S, nh, nb, p, kv_idx, kv_cnt, max_kv);
  if (st != HSA_OK) return st;
  const size_t need = select_ws_bytes(nh, nb, p->mode);
  if (need > kSelectScratchBytes)
    return fail(HSA_ERR_UNSUPPORTED, "hsa_select_noalloc: nh=%d nb=%d need %zu bytes of workspace, more than the "
                "%zu-byte static scratch; use hsa_select with a caller workspace", nh, nb, need, kSelectScratchBytes);
  void *ws = nullptr;
  if (need > 0 && (st = scratch_on_current_device(&ws)) != HSA_OK) return st;
  return launch_select(S, nh, nb, p, kv_idx, kv_cnt, max_kv, ws, static_cast<hipStream_t>(stream));
}

hsa_status_t hsa_attn(const void *qp, const void *kp, const void *vp, void *op, float *lse,
                      const int32_t *blk_len, const int32_t *kv_idx, const int32_t *kv_cnt,
                      const int32_t *order, int32_t max_kv, int32_t kv_shared, int32_t nh,
                      int32_t nb, int32_t B, int32_t D, int32_t dtype, float scale,
                      hsa_stream_t stream) {
  g_last_error.clear();
  if (!qp || !kp || !vp || !op || !blk_len || !kv_idx || !kv_cnt) return fail(HSA_ERR_NULL_PTR, "hsa_attn: null input or output");
  hsa_status_t st;
  if ((st = check_dtype(dtype)) != HSA_OK || (st = check_D(D)) != HSA_OK || (st = check_B(B)) != HSA_OK) return st;
  if (nh < 1 || nb < 1 || max_kv < 1) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn: nh=%d nb=%d max_kv=%d", nh, nb, max_kv);
  if (static_cast<int64_t>(nh) * nb >= (1ll << 31)) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn: too many blocks");
  if (kv_shared < 0 || kv_shared > 3) return fail(HSA_ERR_BAD_ARG, "hsa_attn: kv_shared must be 0..3");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(HSA_ERR_BAD_ARG, "hsa_attn: scale must be finite and positive");
  if (!aligned16(qp) || !aligned16(kp) || !aligned16(vp) || !aligned16(op)) return fail(HSA_ERR_BAD_ARG, "hsa_attn: tensors must be 16-byte aligned");
  if (order && !aligned4(order)) return fail(HSA_ERR_BAD_ARG, "hsa_attn: order must be 4-byte aligned");
  return launch_attn(qp, kp, vp, op, lse, blk_len, kv_idx, kv_cnt, order, max_kv, kv_shared, nh, nb, B, D, dtype, scale,
                     nullptr, 0, 0, 0, static_cast<hipStream_t>(stream));
}

hsa_status_t hsa_attn_tokens(const void *q, const void *k, const void *v, void *o, int64_t q_stride,
                             int64_t kv_stride, int64_t o_stride, float *lse, const int32_t *perm,
                             int32_t N, const int32_t *blk_len, const int32_t *kv_idx,
                             const int32_t *kv_cnt, const int32_t *order, int32_t max_kv,
                             int32_t kv_shared, int32_t nh, int32_t nb, int32_t B, int32_t D,
                             int32_t dtype, float scale, hsa_stream_t stream) {
  g_last_error.clear();
  if (!q || !k || !v || !o || !perm || !blk_len || !kv_idx || !kv_cnt) return fail(HSA_ERR_NULL_PTR, "hsa_attn_tokens: null input or output");
  hsa_status_t st;
  if ((st = check_dtype(dtype)) != HSA_OK || (st = check_D(D)) != HSA_OK || (st = check_B(B)) != HSA_OK) return st;
  if (nh < 1 || nb < 1 || max_kv < 1) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn_tokens: nh=%d nb=%d max_kv=%d", nh, nb, max_kv);
  if (static_cast<int64_t>(nh) * nb >= (1ll << 31)) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn_tokens: too many blocks");
  if (N < 1 || static_cast<int64_t>(N) > static_cast<int64_t>(nb) * B) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn_tokens: N=%d outside 1..nb*B", N);
  const int es = esize_of(dtype);
  const int64_t strides[3] = {q_stride, o_stride, kv_stride > 0 ? kv_stride : static_cast<int64_t>(nh) * D};
  for (const int64_t ts : strides) {
    if (ts < static_cast<int64_t>(nh) * D) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn_tokens: token stride %lld < nh*D", static_cast<long long>(ts));
    if ((ts * es) % 16 != 0) return fail(HSA_ERR_BAD_ARG, "hsa_attn_tokens: token strides must be multiples of 16 bytes");
    if (ts >= (1ll << 40) / N) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn_tokens: tensor too large");
  }
  if (kv_stride < 0) return fail(HSA_ERR_BAD_ARG, "hsa_attn_tokens: kv_stride must be 0 (reordered K/V) or a token stride");
  // gathered rows are addressed with 32-bit byte offsets from the tensor start
  if (kv_stride > 0 && static_cast<int64_t>(N) * kv_stride * es > (1ll << 32) - 1)
    return fail(HSA_ERR_UNSUPPORTED, "hsa_attn_tokens: token-major K/V span more than 4 GiB; reorder them with hsa_perm");
  // ... formed as token index x row bytes with 24-bit multiplies
  if (kv_stride > 0 && (N > (1 << 24) || kv_stride * es >= (1ll << 24)))
    return fail(HSA_ERR_UNSUPPORTED, "hsa_attn_tokens: gathered K/V need N <= 2^24 tokens and rows under 16 MiB; reorder them with hsa_perm");
  if (kv_shared < 0 || kv_shared > 3) return fail(HSA_ERR_BAD_ARG, "hsa_attn_tokens: kv_shared must be 0..3");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(HSA_ERR_BAD_ARG, "hsa_attn_tokens: scale must be finite and positive");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return fail(HSA_ERR_BAD_ARG, "hsa_attn_tokens: tensors must be 16-byte aligned");
  if (!aligned4(perm) || (order && !aligned4(order))) return fail(HSA_ERR_BAD_ARG, "hsa_attn_tokens: perm and order must be 4-byte aligned");
  return launch_attn(q, k, v, o, lse, blk_len, kv_idx, kv_cnt, order, max_kv, kv_shared, nh, nb, B, D, dtype, scale,
                     perm, q_stride, kv_stride, o_stride, static_cast<hipStream_t>(stream));
}

hsa_status_t hsa_attn_order(const int32_t *kv_cnt, int32_t G, int32_t nb, int32_t max_kv,
                            int32_t *order, hsa_stream_t stream) {
  g_last_error.clear();
  if (!kv_cnt || !order) return fail(HSA_ERR_NULL_PTR, "hsa_attn_order: null input or output");
  if (G < 1 || nb < 1 || max_kv < 1) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn_order: G=%d nb=%d max_kv=%d", G, nb, max_kv);
  if (static_cast<int64_t>(G) * nb >= (1ll << 31)) return fail(HSA_ERR_UNSUPPORTED, "hsa_attn_order: G*nb >= 2^31");
  if (max_kv > 4095) return fail(HSA_ERR_UNSUPPORTED, "hsa_attn_order: max_kv > 4095");
  if (!aligned4(kv_cnt) || !aligned4(order)) return fail(HSA_ERR_BAD_ARG, "hsa_attn_order: arrays must be 4-byte aligned");
  return launch_attn_order(kv_cnt, G, nb, max_kv, order, static_cast<hipStream_t>(stream));
}

size_t hsa_attn_bwd_ws_size(int32_t nh, int32_t nb, int32_t B, int32_t kv_shared) {
  if (nh < 1 || nb < 1 || B < 1 || (kv_shared != 0 && kv_shared != 1)) return 0;
  return attn_bwd_ws_bytes(nh, nb, B, kv_shared ? 1 : nh);
}

hsa_status_t hsa_attn_bwd(const void *qp, const void *kp, const void *vp, const void *op,
                          const void *dop, const float *lse, const int32_t *blk_len,
                          const int32_t *kv_idx, const int32_t *kv_cnt, int32_t max_kv,
                          int32_t kv_shared, int32_t nh, int32_t nb, int32_t B, int32_t D,
                          int32_t dtype, float scale, void *dqp, void *dkp, void *dvp, void *ws,
                          size_t ws_bytes, hsa_stream_t stream) {
  g_last_error.clear();
  if (!qp || !kp || !vp || !op || !dop || !lse || !blk_len || !kv_idx || !kv_cnt)
    return fail(HSA_ERR_NULL_PTR, "hsa_attn_bwd: null input (the forward's lse is required)");
  if (!dqp || !dkp || !dvp) return fail(HSA_ERR_NULL_PTR, "hsa_attn_bwd: null output");
  hsa_status_t st;
  if ((st = check_dtype(dtype)) != HSA_OK || (st = check_D(D)) != HSA_OK || (st = check_B(B)) != HSA_OK) return st;
  if (nh < 1 || nb < 1 || max_kv < 1) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn_bwd: nh=%d nb=%d max_kv=%d", nh, nb, max_kv);
  if (static_cast<int64_t>(nh) * nb * B >= (1ll << 31)) return fail(HSA_ERR_BAD_SHAPE, "hsa_attn_bwd: too many slots");
  if (kv_shared != 0 && kv_shared != 1) return fail(HSA_ERR_BAD_ARG, "hsa_attn_bwd: kv_shared must be 0 or 1");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(HSA_ERR_BAD_ARG, "hsa_attn_bwd: scale must be finite and positive");
  const void *ten[8] = {qp, kp, vp, op, dop, dqp, dkp, dvp};
  for (const void *t : ten)
    if (!aligned16(t)) return fail(HSA_ERR_BAD_ARG, "hsa_attn_bwd: tensors must be 16-byte aligned");
  const size_t need = attn_bwd_ws_bytes(nh, nb, B, kv_shared ? 1 : nh);
  if (!ws || ws_bytes < need) return fail(HSA_ERR_WORKSPACE, "hsa_attn_bwd: workspace needs %zu bytes, got %zu", need, ws ? ws_bytes : 0);
  if (!aligned16(ws)) return fail(HSA_ERR_BAD_ARG, "hsa_attn_bwd: workspace must be 16-byte aligned");
  return launch_attn_bwd(qp, kp, vp, op, dop, lse, blk_len, kv_idx, kv_cnt, max_kv, kv_shared, nh, nb, B, D,
                         dtype, scale, dqp, dkp, dvp, ws, static_cast<hipStream_t>(stream));
}

hsa_status_t hsa_block_mass(const void *qp, const void *kp, const int32_t *blk_len,
                            const int32_t *rows, int32_t n_rows, int32_t nh, int32_t nb,
                            int32_t B, int32_t D, int32_t dtype, float scale,
                            const int32_t *kv_idx, const int32_t *kv_cnt, int32_t max_kv,
                            int32_t kv_shared, float *mass, float *recall, hsa_stream_t stream) {
  g_last_error.clear();
  if (!qp || !kp || !blk_len || !rows) return fail(HSA_ERR_NULL_PTR, "hsa_block_mass: null input");
  if (!mass && !recall) return fail(HSA_ERR_NULL_PTR, "hsa_block_mass: no output requested");
  if (recall && (!kv_idx || !kv_cnt)) return fail(HSA_ERR_NULL_PTR, "hsa_block_mass: recall needs the lists");
  hsa_status_t st;
  if ((st = check_dtype(dtype)) != HSA_OK || (st = check_D(D)) != HSA_OK || (st = check_B(B)) != HSA_OK) return st;
  if (n_rows < 1 || nh < 1 || nb < 1) return fail(HSA_ERR_BAD_SHAPE, "hsa_block_mass: n_rows=%d nh=%d nb=%d", n_rows, nh, nb);
  if (recall && max_kv < 1) return fail(HSA_ERR_BAD_SHAPE, "hsa_block_mass: max_kv=%d", max_kv);
  if (kv_shared != 0 && kv_shared != 1) return fail(HSA_ERR_BAD_ARG, "hsa_block_mass: kv_shared must be 0 or 1");
  if (!(scale > 0.f) || !isfinite(scale)) return fail(HSA_ERR_BAD_ARG, "hsa_block_mass: scale must be finite and positive");
  if (!aligned16(qp) || !aligned16(kp)) return fail(HSA_ERR_BAD_ARG, "hsa_block_mass: tensors must be 16-byte aligned");
  return launch_block_mass(qp, kp, blk_len, rows, n_rows, nh, nb, B, D, dtype, scale, kv_idx, kv_cnt, max_kv,
                           kv_shared, mass, recall, static_cast<hipStream_t>(stream));
}

hsa_status_t hsa_unperm(const void *op, void *o, const int32_t *perm, int32_t N, int32_t n_pad,
                        int32_t nh, int32_t D, int64_t tok_stride, int32_t dtype,
                        hsa_stream_t stream) {
  g_last_error.clear();
  if (!op || !o || !perm) return fail(HSA_ERR_NULL_PTR, "hsa_unperm: null input or output");
  hsa_status_t st;
  if ((st = check_dtype(dtype)) != HSA_OK || (st = check_D(D)) != HSA_OK) return st;
  if (N < 1 || n_pad < N || nh < 1) return fail(HSA_ERR_BAD_SHAPE, "hsa_unperm: N=%d n_pad=%d nh=%d", N, n_pad, nh);
  if (tok_stride < static_cast<int64_t>(nh) * D) return fail(HSA_ERR_BAD_SHAPE, "hsa_unperm: tok_stride < nh*D");
  const int es = esize_of(dtype);
  if ((tok_stride * es) % 16 != 0) return fail(HSA_ERR_BAD_ARG, "hsa_unperm: token stride must be a multiple of 16 bytes");
  if (static_cast<int64_t>(nh) * D * es / 16 > 1024) return fail(HSA_ERR_UNSUPPORTED, "hsa_unperm: nh*D*elem_size must be <= 16 KB");
  if (!aligned16(op) || !aligned16(o)) return fail(HSA_ERR_BAD_ARG, "hsa_unperm: tensors must be 16-byte aligned");
  return launch_unperm(op, o, perm, n_pad, nh, D, tok_stride, es, static_cast<hipStream_t>(stream));
}

}  // extern "C"
