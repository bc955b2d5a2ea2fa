"""ctypes binding of libhsa.so: argument marshalling only.

Each function has the name of the C entry point it wraps, takes torch device
tensors, allocates outputs and workspaces with torch (device memory and the
current stream are all torch provides here), and calls the library on the
current HIP stream. Every step of the computation runs in the HIP kernels;
there is no CPU path. A missing library or a failing call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhsa.so")

HSA_F32, HSA_BF16 = 0, 1
ORDERS = {"row": 0, "hilbert": 1, "frame": 2, "tile2d": 3, "cube3d": 4, "hilbert2d": 5}
AGGS = {"mass": 0, "max": 1}
MODES = {"topk": 0, "thresh_global": 1, "lvsa": 2, "radial": 3, "radial_dyn": 4}

_c_i32, _c_i64, _c_f32, _c_sz, _p = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p


class SelectParams(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("k", ctypes.c_int32), ("tau", ctypes.c_double),
                ("budget_ratio", ctypes.c_double), ("frames", ctypes.c_int32),
                ("tiles_per_frame", ctypes.c_int32), ("C", ctypes.c_int32),
                ("T_per", ctypes.c_int32), ("step", ctypes.c_int32), ("lam", ctypes.c_double),
                ("delta", ctypes.c_double)]


_SIGS = {
    "hsa_abi_version": (ctypes.c_int, []),
    "hsa_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "hsa_last_error": (ctypes.c_char_p, []),
    "hsa_plan_size": (ctypes.c_int, [_c_i32] * 5 + [ctypes.POINTER(_c_i32)] * 2),
    "hsa_plan_ws_size": (_c_sz, [_c_i32] * 4),
    "hsa_plan": (ctypes.c_int, [_c_i32] * 5 + [_p, _p, _p, _c_sz, _p]),
    "hsa_perm": (ctypes.c_int, [_c_i32, _p, _p, _p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32,
                                _c_i32, _p, _p]),
    "hsa_score_ws_size": (_c_sz, [_c_i32] * 4),
    "hsa_score": (ctypes.c_int, [_p, _p, _p, _p] + [_c_i32] * 7 + [_c_f32, _p, _p, _c_sz, _p]),
    "hsa_select_ws_size": (_c_sz, [_c_i32, _c_i32, ctypes.POINTER(SelectParams)]),
    "hsa_select_list_width": (_c_i32, [_c_i32, _c_i32, ctypes.POINTER(SelectParams)]),
    "hsa_select": (ctypes.c_int, [_p, _c_i32, _c_i32, ctypes.POINTER(SelectParams), _p, _p, _c_i32, _p, _c_sz, _p]),
    "hsa_select_noalloc": (ctypes.c_int, [_p, _c_i32, _c_i32, ctypes.POINTER(SelectParams), _p, _p, _c_i32, _p]),
    "hsa_attn": (ctypes.c_int, [_p] * 9 + [_c_i32] * 7 + [_c_f32, _p]),
    "hsa_attn_tokens": (ctypes.c_int, [_p] * 4 + [_c_i64] * 3 + [_p, _p, _c_i32, _p, _p, _p, _p]
                        + [_c_i32] * 7 + [_c_f32, _p]),
    "hsa_attn_order": (ctypes.c_int, [_p, _c_i32, _c_i32, _c_i32, _p, _p]),
    "hsa_unperm": (ctypes.c_int, [_p, _p, _p, _c_i32, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _p]),
    "hsa_attn_bwd_ws_size": (_c_sz, [_c_i32] * 4),
    "hsa_attn_bwd": (ctypes.c_int, [_p] * 9 + [_c_i32] * 7 + [_c_f32, _p, _p, _p, _p, _c_sz, _p]),
    "hsa_block_mass": (ctypes.c_int, [_p, _p, _p, _p] + [_c_i32] * 6 + [_c_f32, _p, _p, _c_i32, _c_i32,
                                                                     _p, _p, _p]),
}

_lib = None


def lib():
    """Load libhsa.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_hilbert3d_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


class HsaError(RuntimeError):
    pass


def _check(status: int, name: str):
    if status != 0:
        L = lib()
        raise HsaError(f"{name}: {L.hsa_status_str(status).decode()} "
                       f"({L.hsa_last_error().decode()})")


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HSA_BF16
    if t.dtype == torch.float32:
        return HSA_F32
    raise HsaError(f"unsupported dtype {t.dtype}")


def _need_device(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise HsaError("tensors must be contiguous device tensors")


def hsa_plan_size(T: int, H: int, W: int, order: str, B: int):
    n_pad, nb = _c_i32(), _c_i32()
    _check(lib().hsa_plan_size(T, H, W, ORDERS[order], B, ctypes.byref(n_pad), ctypes.byref(nb)),
           "hsa_plan_size")
    return n_pad.value, nb.value


def hsa_plan(T: int, H: int, W: int, order: str, B: int, device="cuda"):
    """-> (perm int32[n_pad], blk_len int32[nb]) on the device."""
    n_pad, nb = hsa_plan_size(T, H, W, order, B)
    perm = torch.empty(n_pad, dtype=torch.int32, device=device)
    blk_len = torch.empty(nb, dtype=torch.int32, device=device)
    ws_n = lib().hsa_plan_ws_size(T, H, W, ORDERS[order])
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=device)
    _check(lib().hsa_plan(T, H, W, ORDERS[order], B, _ptr(perm), _ptr(blk_len), _ptr(ws), ws_n,
                          _stream()), "hsa_plan")
    return perm, blk_len


def hsa_perm(xs, perm: torch.Tensor, n_pad: int, outs=None, pool_s: int = 0, pooled=None):
    """xs: list of [1, N, nh, D] (token stride may exceed nh*D) -> list of [nh, n_pad, D].
    With pool_s > 0 also fills `pooled` (float32 [2, nh, n_pad // pool_s, D], allocated if
    None) with the sub-block means of xs[0] and xs[1]; returns (outs, pooled) then. When
    pooling, outs[0] or outs[1] may be None: that tensor is pooled but not stored."""
    xs = list(xs)
    x0 = xs[0]
    _, N, nh, D = x0.shape
    for x in xs:
        if x.shape != x0.shape or x.dtype != x0.dtype or not x.is_cuda:
            raise HsaError("hsa_perm: tensors must share shape, dtype and device")
        if x.stride(3) != 1 or x.stride(2) != D:
            raise HsaError("hsa_perm: heads and head dim must be contiguous")
        if x.stride(1) != x0.stride(1):
            raise HsaError("hsa_perm: tensors must share the token stride")
    _need_device(perm)
    if outs is None:
        outs = [torch.empty((nh, n_pad, D), dtype=x0.dtype, device=x0.device) for _ in xs]
    if pool_s and pooled is None:
        pooled = torch.empty((2, nh, n_pad // pool_s, D), dtype=torch.float32, device=x0.device)
    src = (ctypes.c_void_p * len(xs))(*[x.data_ptr() for x in xs])
    dst = (ctypes.c_void_p * len(xs))(*[None if y is None else y.data_ptr() for y in outs])
    _check(lib().hsa_perm(len(xs), src, dst, _ptr(perm), N, n_pad, nh, D, x0.stride(1),
                          _dtype_code(x0), int(pool_s), _ptr(pooled if pool_s else None),
                          _stream()), "hsa_perm")
    return (outs, pooled) if pool_s else outs


def hsa_score(qp, kp, blk_len, B: int, s: int, agg: str = "mass", scale: float | None = None,
              out=None, ws=None, pooled=None):
    """qp, kp [nh, n_pad, D] -> S float32 [nh, nb, nb]. With `pooled` (the means
    hsa_perm wrote for the same s) the pooling pass is skipped."""
    _need_device(qp, kp, blk_len, pooled)
    nh, n_pad, D = qp.shape
    nb = n_pad // B
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty((nh, nb, nb), dtype=torch.float32, device=qp.device)
    ws_n = 0
    if pooled is None:
        ws_n = lib().hsa_score_ws_size(nh, n_pad, s, D)
        if ws is None:
            ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=qp.device)
    _check(lib().hsa_score(_ptr(qp), _ptr(kp), _ptr(pooled), _ptr(blk_len), nh, nb, B, s, D,
                           _dtype_code(qp), AGGS[agg], scale, _ptr(out),
                           _ptr(ws if pooled is None else None),
                           ws.numel() if (pooled is None and ws is not None) else 0, _stream()),
           "hsa_score")
    return out


def make_params(mode: str, k=0, tau=0.0, budget_ratio=0.0, frames=0, tiles_per_frame=0, C=0,
                T_per=1, step=0, lam=0.0, delta=0.0) -> SelectParams:
    return SelectParams(MODES[mode], int(k), float(tau), float(budget_ratio), int(frames),
                        int(tiles_per_frame), int(C), int(T_per), int(step), float(lam), float(delta))


def hsa_select_list_width(nh: int, nb: int, params: SelectParams) -> int:
    """Smallest max_kv hsa_select accepts for these parameters."""
    n = lib().hsa_select_list_width(nh, nb, ctypes.byref(params))
    if n < 1:
        raise HsaError("hsa_select_list_width: invalid parameters")
    return n


def hsa_select(S, nh: int, nb: int, params: SelectParams, max_kv: int, device="cuda",
               outs=None, ws=None):
    """-> (kv_idx int32 [G, nb, max_kv], kv_cnt int32 [G, nb]); G = 1 for the head-shared
    modes (LVSA, RADIAL)."""
    if S is not None:
        _need_device(S)
        device = S.device
    G = 1 if params.mode in (MODES["lvsa"], MODES["radial"]) else nh
    if outs is None:
        outs = (torch.empty((G, nb, max_kv), dtype=torch.int32, device=device),
                torch.empty((G, nb), dtype=torch.int32, device=device))
    kv_idx, kv_cnt = outs
    ws_n = lib().hsa_select_ws_size(nh, nb, ctypes.byref(params))
    if ws is None:
        ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=device)
    _check(lib().hsa_select(_ptr(S), nh, nb, ctypes.byref(params), _ptr(kv_idx), _ptr(kv_cnt),
                            max_kv, _ptr(ws), ws.numel(), _stream()), "hsa_select")
    return kv_idx, kv_cnt


def hsa_select_noalloc(S, nh: int, nb: int, params: SelectParams, max_kv: int, outs):
    """hsa_select with the library's static workspace (no workspace argument;
    the caller passes the output lists `outs` = (kv_idx, kv_cnt))."""
    kv_idx, kv_cnt = outs
    _need_device(S, kv_idx, kv_cnt)
    _check(lib().hsa_select_noalloc(_ptr(S), nh, nb, ctypes.byref(params), _ptr(kv_idx), _ptr(kv_cnt),
                                    max_kv, _stream()), "hsa_select_noalloc")
    return kv_idx, kv_cnt


def hsa_attn_order(kv_cnt, max_kv: int, out=None):
    """kv_cnt int32 [G, nb] -> int32 [G*nb] row order, longest lists first."""
    _need_device(kv_cnt)
    G, nb = kv_cnt.shape
    if out is None:
        out = torch.empty(G * nb, dtype=torch.int32, device=kv_cnt.device)
    _check(lib().hsa_attn_order(_ptr(kv_cnt), G, nb, max_kv, _ptr(out), _stream()), "hsa_attn_order")
    return out


def hsa_attn(qp, kp, vp, blk_len, kv_idx, kv_cnt, B: int, scale: float | None = None,
             want_lse: bool = True, out=None, lse=None, order=None, short_blocks: bool = False):
    """-> (op [nh, n_pad, D] in the input dtype, lse float32 [nh, n_pad] or None).
    `order` (from hsa_attn_order) sets the processing order; results do not depend on it."""
    _need_device(qp, kp, vp, blk_len, kv_idx, kv_cnt, order)
    nh, n_pad, D = qp.shape
    nb = n_pad // B
    shared = (1 if kv_idx.shape[0] == 1 and nh > 1 else 0) | (2 if short_blocks else 0)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(qp)
    if want_lse and lse is None:
        lse = torch.empty((nh, n_pad), dtype=torch.float32, device=qp.device)
    _check(lib().hsa_attn(_ptr(qp), _ptr(kp), _ptr(vp), _ptr(out), _ptr(lse if want_lse else None),
                          _ptr(blk_len), _ptr(kv_idx), _ptr(kv_cnt), _ptr(order), kv_idx.shape[-1], shared,
                          nh, nb, B, D, _dtype_code(qp), scale, _stream()), "hsa_attn")
    return out, (lse if want_lse else None)


def hsa_attn_tokens(q, k, v, perm, blk_len, kv_idx, kv_cnt, B: int, scale: float | None = None,
                    want_lse: bool = True, out=None, lse=None, order=None, short_blocks: bool = False):
    """q [1, N, nh, D] token-major (token stride may exceed nh*D, e.g. a slice of a fused QKV
    buffer); k, v either token-major like q (same token stride) or reordered [nh, n_pad, D]
    (hsa_perm outputs) -> (o [1, N, nh, D], lse float32 [nh, n_pad] or None). Equals
    hsa_unperm(hsa_attn(Qp, Kp, Vp, ...)) with the reorders done inside the attention kernel."""
    _need_device(perm, blk_len, kv_idx, kv_cnt, order)
    _, N, nh, D = q.shape
    for x in (q, k, v):
        if not x.is_cuda or x.stride(-1) != 1 or (x.dim() == 4 and x.stride(2) != D):
            raise HsaError("hsa_attn_tokens: device tensors with contiguous heads and head dim")
    n_pad = perm.numel()
    nb = n_pad // B
    if k.dim() == 4:
        if k.stride(1) != v.stride(1) or k.shape != q.shape or v.shape != q.shape:
            raise HsaError("hsa_attn_tokens: token-major k and v must match q and share a stride")
        kv_stride = k.stride(1)
    else:
        _need_device(k, v)
        kv_stride = 0
    shared = (1 if kv_idx.shape[0] == 1 and nh > 1 else 0) | (2 if short_blocks else 0)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if out is None:
        out = torch.empty((1, N, nh, D), dtype=q.dtype, device=q.device)
    if out.stride(3) != 1 or out.stride(2) != D:
        raise HsaError("hsa_attn_tokens: heads and head dim of the output must be contiguous")
    if want_lse and lse is None:
        lse = torch.empty((nh, n_pad), dtype=torch.float32, device=q.device)
    _check(lib().hsa_attn_tokens(_ptr(q), _ptr(k), _ptr(v), _ptr(out), q.stride(1), kv_stride,
                                 out.stride(1), _ptr(lse if want_lse else None), _ptr(perm), N,
                                 _ptr(blk_len), _ptr(kv_idx), _ptr(kv_cnt), _ptr(order),
                                 kv_idx.shape[-1], shared, nh, nb, B, D, _dtype_code(q), scale,
                                 _stream()), "hsa_attn_tokens")
    return out, (lse if want_lse else None)


def hsa_unperm(op, perm, N: int, out=None):
    """op [nh, n_pad, D] -> o [1, N, nh, D]."""
    _need_device(op, perm)
    nh, n_pad, D = op.shape
    if out is None:
        out = torch.empty((1, N, nh, D), dtype=op.dtype, device=op.device)
    if out.stride(3) != 1 or out.stride(2) != D:
        raise HsaError("hsa_unperm: heads and head dim of the output must be contiguous")
    _check(lib().hsa_unperm(_ptr(op), _ptr(out), _ptr(perm), N, n_pad, nh, D, out.stride(1),
                            _dtype_code(op), _stream()), "hsa_unperm")
    return out


def hsa_block_mass(qp, kp, blk_len, rows, B: int, scale: float | None = None, kv_idx=None,
                   kv_cnt=None, want_mass: bool = True):
    """Selection diagnostic. rows int32 [nh, n_rows] (slots) -> (mass float32 [nh, n_rows, nb]
    or None, recall float32 [nh, n_rows] or None; recall needs kv_idx/kv_cnt)."""
    _need_device(qp, kp, blk_len, rows, kv_idx, kv_cnt)
    nh, n_pad, D = qp.shape
    nb = n_pad // B
    n_rows = rows.shape[1]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    mass = torch.empty((nh, n_rows, nb), dtype=torch.float32, device=qp.device) if want_mass else None
    rec = None
    shared, max_kv = 0, 0
    if kv_idx is not None:
        rec = torch.empty((nh, n_rows), dtype=torch.float32, device=qp.device)
        shared = 1 if kv_idx.shape[0] == 1 and nh > 1 else 0
        max_kv = kv_idx.shape[-1]
    _check(lib().hsa_block_mass(_ptr(qp), _ptr(kp), _ptr(blk_len), _ptr(rows), n_rows, nh, nb, B, D,
                                _dtype_code(qp), scale, _ptr(kv_idx), _ptr(kv_cnt), max_kv, shared,
                                _ptr(mass), _ptr(rec), _stream()), "hsa_block_mass")
    return mass, rec


def hsa_attn_bwd(qp, kp, vp, op, dop, lse, blk_len, kv_idx, kv_cnt, B: int, scale: float | None = None,
                 outs=None, ws=None):
    """Gradients of hsa_attn -> (dqp, dkp, dvp), each [nh, n_pad, D] in the input dtype.
    lse is the forward's log-sum-exp [nh, n_pad]."""
    _need_device(qp, kp, vp, op, dop, lse, blk_len, kv_idx, kv_cnt)
    nh, n_pad, D = qp.shape
    nb = n_pad // B
    shared = 1 if kv_idx.shape[0] == 1 and nh > 1 else 0
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if outs is None:
        outs = tuple(torch.empty_like(qp) for _ in range(3))
    dq, dk, dv = outs
    n = lib().hsa_attn_bwd_ws_size(nh, nb, B, shared)
    if ws is None:
        ws = torch.empty(max(n, 16), dtype=torch.uint8, device=qp.device)
    _check(lib().hsa_attn_bwd(_ptr(qp), _ptr(kp), _ptr(vp), _ptr(op), _ptr(dop), _ptr(lse), _ptr(blk_len),
                              _ptr(kv_idx), _ptr(kv_cnt), kv_idx.shape[-1], shared, nh, nb, B, D,
                              _dtype_code(qp), scale, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws), ws.numel(),
                              _stream()), "hsa_attn_bwd")
    return dq, dk, dv
