"""Thin Python binding of libhstu.so (include/hstu.h).

Argument marshalling only: tensors are torch device tensors (PyTorch supplies
device memory and the HIP stream); every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library is not built, or
no GPU is present, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# HSTU_LIB_PATH selects another build of the same library (the host-sanitizer
# build of the CPU tests); the default is the in-tree libhstu.so.
LIB_PATH = os.environ.get("HSTU_LIB_PATH") or os.path.join(_HERE, "libhstu.so")

HSTU_OK, HSTU_ERR_ARG, HSTU_ERR_UNSUPPORTED, HSTU_ERR_WORKSPACE, HSTU_ERR_DEVICE = range(5)
HSTU_F32, HSTU_BF16 = 0, 1
HSTU_ACT_SILU, HSTU_ACT_RELU = 0, 1
OP_ATTN_FWD, OP_ATTN_BWD, OP_LAYER_FWD, OP_MFALCON, OP_LAYER_BWD, OP_LAYER_APPEND = range(6)

EXPORTED = ["hstu_attn_fwd", "hstu_attn_bwd", "hstu_layer_fwd", "hstu_layer_bwd", "mfalcon_score",
            "hstu_workspace_size", "hstu_attn_fwd_noalloc", "hstu_layer_append", "hstu_softmax_attn_fwd",
            "hstu_sl_sample",
            "hstu_profile_enable", "hstu_profile_collect", "hstu_last_error", "hstu_abi_version"]


class HstuError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("libhstu status %d: %s" % (status, msg))
        self.status = status


class Jagged(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("total", ctypes.c_int32), ("n_max", ctypes.c_int32),
                ("offsets", ctypes.c_void_p), ("ts", ctypes.c_void_p)]


class Dims(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("heads", ctypes.c_int32), ("d_qk", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("ln_eps", ctypes.c_float)]


class Bias(ctypes.Structure):
    _fields_ = [("rab_p", ctypes.c_void_p), ("rab_p_hstride", ctypes.c_int64),
                ("rab_t", ctypes.c_void_p), ("rab_t_hstride", ctypes.c_int64)]


class CMat(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("ld", ctypes.c_int64)]


class Mat(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("ld", ctypes.c_int64)]


class Layer(ctypes.Structure):
    _fields_ = [("w1", ctypes.c_void_p), ("b1", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("b2", ctypes.c_void_p),
                ("rab", Bias), ("phi1", ctypes.c_int)]


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libhstu.so (needs no GPU: the HIP runtime initialises lazily)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libhstu.so is not built (%s); run __graft_entry__.build()" % path)
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.hstu_last_error.restype = ctypes.c_char_p
    lib.hstu_abi_version.restype = ctypes.c_int32
    lib.hstu_workspace_size.restype = ctypes.c_size_t
    lib.hstu_workspace_size.argtypes = [ctypes.c_int, P(Jagged), P(Dims), ctypes.c_int32, ctypes.c_int32]
    lib.hstu_attn_fwd.restype = ctypes.c_int
    lib.hstu_attn_fwd.argtypes = [P(Jagged), P(Dims), P(Bias), CMat, CMat, CMat, CMat, Mat, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hstu_attn_fwd_noalloc.restype = ctypes.c_int
    lib.hstu_attn_fwd_noalloc.argtypes = [P(Jagged), P(Dims), P(Bias), CMat, CMat, CMat, CMat, Mat, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_void_p]
    lib.hstu_attn_bwd.restype = ctypes.c_int
    lib.hstu_attn_bwd.argtypes = [P(Jagged), P(Dims), P(Bias), CMat, CMat, CMat, CMat, ctypes.c_void_p,
                                  ctypes.c_void_p, CMat, Mat, Mat, Mat, Mat, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hstu_layer_fwd.restype = ctypes.c_int
    lib.hstu_layer_fwd.argtypes = [P(Jagged), P(Dims), ctypes.c_int32, P(Layer), CMat, Mat, Mat, Mat,
                                   ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hstu_layer_bwd.restype = ctypes.c_int
    lib.hstu_layer_bwd.argtypes = [P(Jagged), P(Dims), ctypes.c_int32, P(Layer), CMat, CMat, Mat] + \
        [ctypes.c_void_p] * 6 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hstu_softmax_attn_fwd.restype = ctypes.c_int
    lib.hstu_softmax_attn_fwd.argtypes = [P(Jagged), P(Dims), CMat, CMat, CMat, Mat, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_size_t, ctypes.c_void_p]
    lib.hstu_sl_sample.restype = ctypes.c_int
    lib.hstu_sl_sample.argtypes = [P(Jagged), ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hstu_layer_append.restype = ctypes.c_int
    lib.hstu_layer_append.argtypes = [P(Jagged), P(Jagged), P(Dims), ctypes.c_int32, P(Layer), CMat, CMat, CMat, Mat,
                                      Mat, Mat, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mfalcon_score.restype = ctypes.c_int
    lib.mfalcon_score.argtypes = [P(Jagged), P(Dims), ctypes.c_int32, ctypes.c_int32, P(Layer), P(CMat), P(CMat),
                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, CMat, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.hstu_profile_enable.restype = None
    lib.hstu_profile_enable.argtypes = [ctypes.c_int32]
    lib.hstu_profile_collect.restype = ctypes.c_int32
    lib.hstu_profile_collect.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int32]
    _lib = lib
    return lib


def profile_enable(on: bool = True):
    load_library().hstu_profile_enable(1 if on else 0)


def profile_collect():
    """{kernel name: (launches, total ms)} since the previous collect."""
    arr = (KernelTime * 64)()
    n = load_library().hstu_profile_collect(arr, 64)
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n)}


def abi_version() -> int:
    return load_library().hstu_abi_version()


def last_error() -> str:
    return load_library().hstu_last_error().decode()


def _check(status: int):
    if status != HSTU_OK:
        raise HstuError(status, last_error())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return HSTU_BF16
    if t.dtype == torch.float32:
        return HSTU_F32
    raise TypeError("unsupported dtype %s" % t.dtype)


def _rowmat(t: Optional[torch.Tensor], width: int, cls=CMat):
    """A [T][...] tensor whose rows are contiguous blocks of `width` elements
    with token stride t.stride(0)."""
    if t is None:
        return cls(None, 0)
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if t.dim() == 3:
        T, a, b = t.shape
        if t.stride(2) != 1 or t.stride(1) != b:
            raise ValueError("per-head tensor must have contiguous heads")
    elif t.dim() == 2:
        if t.stride(1) != 1:
            raise ValueError("rows must be contiguous")
    else:
        raise ValueError("expected a 2-D or 3-D tensor")
    return cls(t.data_ptr(), t.stride(0) if t.shape[0] > 1 else max(width, t.stride(0)))


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


_ws_cache = {}


def _workspace(nbytes: int, device) -> torch.Tensor:
    key = (str(device),)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def _jagged(offsets: torch.Tensor, ts: Optional[torch.Tensor], n_max: int, total: Optional[int] = None) -> Jagged:
    if offsets.dtype != torch.int32 or not offsets.is_cuda:
        raise ValueError("offsets must be an int32 GPU tensor")
    if ts is not None and (ts.dtype != torch.int64 or not ts.is_cuda):
        raise ValueError("ts must be an int64 GPU tensor")
    B = offsets.numel() - 1
    if total is None:
        raise ValueError("total token count is required")
    return Jagged(B, int(total), int(n_max), offsets.data_ptr(), _ptr(ts))


def _bias(rab_p: Optional[torch.Tensor], rab_t: Optional[torch.Tensor]) -> Bias:
    for t in (rab_p, rab_t):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous()):
            raise ValueError("rab tables must be contiguous fp32")
    return Bias(_ptr(rab_p), rab_p.shape[-1] if rab_p is not None and rab_p.dim() == 2 else 0,
                _ptr(rab_t), rab_t.shape[-1] if rab_t is not None and rab_t.dim() == 2 else 0)


def workspace_size(op: int, jag: Jagged, dims: Dims, d_model: int = 0, total_cand: int = 0) -> int:
    lib = load_library()
    n = lib.hstu_workspace_size(op, ctypes.byref(jag), ctypes.byref(dims), d_model, total_cand)
    if n == 0:
        raise HstuError(HSTU_ERR_ARG, last_error())
    return n


def attn_fwd(offsets: torch.Tensor, total: int, ts: Optional[torch.Tensor], q: torch.Tensor, k: torch.Tensor,
             v: torch.Tensor, rab_p: Optional[torch.Tensor], rab_t: Optional[torch.Tensor], n_max: int,
             u: Optional[torch.Tensor] = None, eps: float = 1e-5, out: Optional[torch.Tensor] = None,
             o_save: Optional[torch.Tensor] = None, ln_stats: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_attn_fwd.  q, k, v: [T][H][d]; u: [T][H*d] or None.  Returns out
    ([T][H*d], dtype of q): O, or G = LayerNorm(O) (.) U when u is given."""
    lib = load_library()
    T, H, d = q.shape
    jag = _jagged(offsets, ts, n_max, total)
    dims = Dims(_dtype_code(q), H, d, v.shape[2], eps)
    if out is None:
        out = torch.empty((T, H * d), dtype=q.dtype, device=q.device)
    nws = workspace_size(OP_ATTN_FWD, jag, dims)
    ws = workspace if workspace is not None else _workspace(nws, q.device)
    bias = _bias(rab_p, rab_t)
    st = lib.hstu_attn_fwd(ctypes.byref(jag), ctypes.byref(dims), ctypes.byref(bias), _rowmat(q, H * d),
                           _rowmat(k, H * d), _rowmat(v, H * d), _rowmat(u, H * d), _rowmat(out, H * d, Mat),
                           _ptr(o_save), _ptr(ln_stats), ws.data_ptr(), ws.numel(), _stream(q.device))
    _check(st)
    return out


def sl_sample(offsets: torch.Tensor, total: int, ts: Optional[torch.Tensor], alpha: float, u: torch.Tensor,
              keys: torch.Tensor, x: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """hstu_sl_sample.  u: fp64 [B]; keys: int32 [T] read as uint32.
    Returns (out_offsets [B+1], out_index [T] (first out_offsets[B] valid),
    x_out [T][...] or None, ts_out [T] or None)."""
    lib = load_library()
    jag = _jagged(offsets, ts, 1, total)
    if u.dtype != torch.float64 or keys.dtype != torch.int32:
        raise ValueError("u must be float64 and keys int32 (bits read as uint32)")
    dev_ = offsets.device
    T = int(total)
    B = offsets.numel() - 1
    out_off = torch.empty(B + 1, dtype=torch.int32, device=dev_)
    out_idx = torch.empty(max(T, 1), dtype=torch.int32, device=dev_)
    x_out = torch.empty_like(x) if x is not None else None
    ts_out = torch.empty(max(T, 1), dtype=torch.int64, device=dev_) if ts is not None else None
    es = x.element_size() if x is not None else 0
    ws = workspace if workspace is not None else _workspace(256, dev_)
    st = lib.hstu_sl_sample(ctypes.byref(jag), float(alpha), u.data_ptr(), keys.data_ptr(), _ptr(x),
                            x.stride(0) * es if x is not None else 0, x.shape[1] * es if x is not None else 0,
                            out_off.data_ptr(), out_idx.data_ptr(), _ptr(x_out),
                            x_out.stride(0) * es if x_out is not None else 0, _ptr(ts_out), ws.data_ptr(), ws.numel(),
                            _stream(dev_))
    _check(st)
    return out_off, out_idx, x_out, ts_out


def softmax_attn_fwd(offsets: torch.Tensor, total: int, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, n_max: int,
                     out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_softmax_attn_fwd: causal softmax(Q K^T / sqrt(d)) V (the
    comparator).  Returns out [T][H*d]."""
    lib = load_library()
    T, H, d = q.shape
    jag = _jagged(offsets, None, n_max, total)
    dims = Dims(_dtype_code(q), H, d, v.shape[2], 1e-5)
    if out is None:
        out = torch.empty((T, H * d), dtype=q.dtype, device=q.device)
    nws = workspace_size(OP_ATTN_FWD, jag, dims)
    ws = workspace if workspace is not None else _workspace(nws, q.device)
    st = lib.hstu_softmax_attn_fwd(ctypes.byref(jag), ctypes.byref(dims), _rowmat(q, H * d), _rowmat(k, H * d),
                                   _rowmat(v, H * d), _rowmat(out, H * d, Mat), _ptr(lse), ws.data_ptr(), ws.numel(),
                                   _stream(q.device))
    _check(st)
    return out


def attn_fwd_noalloc(offsets: torch.Tensor, total: int, ts: Optional[torch.Tensor], q: torch.Tensor, k: torch.Tensor,
                     v: torch.Tensor, rab_p: Optional[torch.Tensor], rab_t: Optional[torch.Tensor], n_max: int,
                     u: Optional[torch.Tensor] = None, eps: float = 1e-5, out: Optional[torch.Tensor] = None,
                     o_save: Optional[torch.Tensor] = None, ln_stats: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_attn_fwd_noalloc: hstu_attn_fwd with the library's static scratch
    array instead of a workspace.  `out` should be given by callers that must
    not allocate (otherwise it is allocated here, by torch)."""
    lib = load_library()
    T, H, d = q.shape
    jag = _jagged(offsets, ts, n_max, total)
    dims = Dims(_dtype_code(q), H, d, v.shape[2], eps)
    if out is None:
        out = torch.empty((T, H * d), dtype=q.dtype, device=q.device)
    bias = _bias(rab_p, rab_t)
    st = lib.hstu_attn_fwd_noalloc(ctypes.byref(jag), ctypes.byref(dims), ctypes.byref(bias), _rowmat(q, H * d),
                                   _rowmat(k, H * d), _rowmat(v, H * d), _rowmat(u, H * d), _rowmat(out, H * d, Mat),
                                   _ptr(o_save), _ptr(ln_stats), _stream(q.device))
    _check(st)
    return out


def attn_bwd(offsets: torch.Tensor, total: int, ts: Optional[torch.Tensor], q, k, v, rab_p, rab_t, n_max: int,
             dout: torch.Tensor, u: Optional[torch.Tensor] = None, o_save: Optional[torch.Tensor] = None,
             ln_stats: Optional[torch.Tensor] = None, eps: float = 1e-5, want_drab: bool = True,
             workspace: Optional[torch.Tensor] = None):
    """hstu_attn_bwd.  Returns dict dq, dk, dv, du, drab_p, drab_t."""
    lib = load_library()
    T, H, d = q.shape
    jag = _jagged(offsets, ts, n_max, total)
    dims = Dims(_dtype_code(q), H, d, v.shape[2], eps)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dvv = torch.empty_like(v)
    du = torch.empty((T, H * d), dtype=q.dtype, device=q.device) if u is not None else None
    drp = torch.empty_like(rab_p) if (want_drab and rab_p is not None) else None
    drt = torch.empty_like(rab_t) if (want_drab and rab_t is not None and ts is not None) else None
    nws = workspace_size(OP_ATTN_BWD, jag, dims)
    ws = workspace if workspace is not None else _workspace(nws, q.device)
    bias = _bias(rab_p, rab_t)
    st = lib.hstu_attn_bwd(ctypes.byref(jag), ctypes.byref(dims), ctypes.byref(bias), _rowmat(q, H * d),
                           _rowmat(k, H * d), _rowmat(v, H * d), _rowmat(u, H * d), _ptr(o_save), _ptr(ln_stats),
                           _rowmat(dout, H * d), _rowmat(dq, H * d, Mat), _rowmat(dk, H * d, Mat),
                           _rowmat(dvv, H * d, Mat), _rowmat(du, H * d, Mat), _ptr(drp), _ptr(drt), ws.data_ptr(),
                           ws.numel(), _stream(q.device))
    _check(st)
    return dict(dq=dq, dk=dk, dv=dvv, du=du, drab_p=drp, drab_t=drt)


def _layer_struct(lay) -> Layer:
    return Layer(_ptr(lay["w1"]), _ptr(lay.get("b1")), _ptr(lay["w2"]), _ptr(lay.get("b2")),
                 _bias(lay.get("rab_p"), lay.get("rab_t")), int(lay.get("phi1", HSTU_ACT_SILU)))


def layer_fwd(offsets: torch.Tensor, total: int, ts: Optional[torch.Tensor], x: torch.Tensor, layer: dict,
              heads: int, d: int, n_max: int, eps: float = 1e-5, k_cache: Optional[torch.Tensor] = None,
              v_cache: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """hstu_layer_fwd.  layer: dict of device tensors w1 [4Hd][D], b1, w2 [D][Hd],
    b2, rab_p, rab_t, and phi1.  Returns y [T][D]."""
    lib = load_library()
    T, D = x.shape
    jag = _jagged(offsets, ts, n_max, total)
    dims = Dims(_dtype_code(x), heads, d, d, eps)
    y = out if out is not None else torch.empty_like(x)
    nws = workspace_size(OP_LAYER_FWD, jag, dims, D, 0)
    ws = workspace if workspace is not None else _workspace(nws, x.device)
    L = _layer_struct(layer)
    st = lib.hstu_layer_fwd(ctypes.byref(jag), ctypes.byref(dims), D, ctypes.byref(L), _rowmat(x, D),
                            _rowmat(y, D, Mat), _rowmat(k_cache, heads * d, Mat), _rowmat(v_cache, heads * d, Mat),
                            ws.data_ptr(), ws.numel(), _stream(x.device))
    _check(st)
    return y


def layer_bwd(offsets: torch.Tensor, total: int, ts: Optional[torch.Tensor], x: torch.Tensor, layer: dict,
              dy: torch.Tensor, heads: int, d: int, n_max: int, eps: float = 1e-5, want_bias_grads: bool = True,
              want_drab: bool = True, workspace: Optional[torch.Tensor] = None,
              out: Optional[dict] = None) -> dict:
    """hstu_layer_bwd (the forward recomputed from x).  Returns dict dx
    [T][D] (x's dtype), dw1 [4Hd][D], db1, dw2 [D][Hd], db2, drab_p, drab_t
    (fp32; the optional ones None when not requested).  `out`, if given, is
    a dict of that form from an earlier call whose tensors are reused."""
    lib = load_library()
    T, D = x.shape
    HD = heads * d
    jag = _jagged(offsets, ts, n_max, total)
    dims = Dims(_dtype_code(x), heads, d, d, eps)
    rp, rt = layer.get("rab_p"), layer.get("rab_t")
    if out is not None:
        dx, dw1, dw2, db1, db2, drp, drt = (out[k] for k in ("dx", "dw1", "dw2", "db1", "db2", "drab_p", "drab_t"))
    else:
        f32 = dict(dtype=torch.float32, device=x.device)
        dx = torch.empty_like(x)
        dw1 = torch.empty((4 * HD, D), **f32)
        dw2 = torch.empty((D, HD), **f32)
        db1 = torch.empty(4 * HD, **f32) if want_bias_grads else None
        db2 = torch.empty(D, **f32) if want_bias_grads else None
        drp = torch.empty_like(rp) if (want_drab and rp is not None) else None
        drt = torch.empty_like(rt) if (want_drab and rt is not None and ts is not None) else None
    nws = workspace_size(OP_LAYER_BWD, jag, dims, D, 0)
    ws = workspace if workspace is not None else _workspace(nws, x.device)
    L = _layer_struct(layer)
    st = lib.hstu_layer_bwd(ctypes.byref(jag), ctypes.byref(dims), D, ctypes.byref(L), _rowmat(x, D), _rowmat(dy, D),
                            _rowmat(dx, D, Mat), _ptr(dw1), _ptr(db1), _ptr(dw2), _ptr(db2), _ptr(drp), _ptr(drt),
                            ws.data_ptr(), ws.numel(), _stream(x.device))
    _check(st)
    return dict(dx=dx, dw1=dw1, db1=db1, dw2=dw2, db2=db2, drab_p=drp, drab_t=drt)


def layer_append(hist_offsets: torch.Tensor, hist_total: int, hist_ts: Optional[torch.Tensor],
                 add_offsets: torch.Tensor, add_total: int, add_ts: Optional[torch.Tensor], x_new: torch.Tensor,
                 layer: dict, k_cache: Optional[torch.Tensor], v_cache: Optional[torch.Tensor], heads: int, d: int,
                 n_max: int, eps: float = 1e-5, out: Optional[torch.Tensor] = None,
                 k_out: Optional[torch.Tensor] = None, v_out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None):
    """hstu_layer_append.  Returns (y_new [T_new][D], k_out, v_out
    [T_hist + T_new][H*d]): the new actions' layer output and the merged
    caches (user u's rows from hist_offsets[u] + add_offsets[u])."""
    lib = load_library()
    Tn, D = x_new.shape
    HD = heads * d
    hj = _jagged(hist_offsets, hist_ts, n_max, hist_total)
    aj = _jagged(add_offsets, add_ts, n_max, add_total)
    dims = Dims(_dtype_code(x_new), heads, d, d, eps)
    y = out if out is not None else torch.empty((Tn, D), dtype=x_new.dtype, device=x_new.device)
    Tm = int(hist_total) + int(add_total)
    ko = k_out if k_out is not None else torch.empty((Tm, HD), dtype=x_new.dtype, device=x_new.device)
    vo = v_out if v_out is not None else torch.empty((Tm, HD), dtype=x_new.dtype, device=x_new.device)
    nws = workspace_size(OP_LAYER_APPEND, hj, dims, D, int(add_total))
    ws = workspace if workspace is not None else _workspace(nws, x_new.device)
    L = _layer_struct(layer)
    st = lib.hstu_layer_append(ctypes.byref(hj), ctypes.byref(aj), ctypes.byref(dims), D, ctypes.byref(L),
                               _rowmat(k_cache, HD), _rowmat(v_cache, HD), _rowmat(x_new, D), _rowmat(y, D, Mat),
                               _rowmat(ko, HD, Mat), _rowmat(vo, HD, Mat), ws.data_ptr(), ws.numel(),
                               _stream(x_new.device))
    _check(st)
    return y, ko, vo


def mfalcon_score(hist_offsets: torch.Tensor, hist_total: int, hist_ts: Optional[torch.Tensor], layers: Sequence[dict],
                  k_caches: Sequence[torch.Tensor], v_caches: Sequence[torch.Tensor], cand_offsets: torch.Tensor,
                  total_cand: int, cand_ts: Optional[torch.Tensor], x_cand: torch.Tensor, b_m: int, heads: int,
                  d: int, n_max: int, eps: float = 1e-5, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mfalcon_score.  Returns the candidates' final hidden states, fp32 [M][D]."""
    lib = load_library()
    M, D = x_cand.shape
    jag = _jagged(hist_offsets, hist_ts, n_max, hist_total)
    dims = Dims(_dtype_code(x_cand), heads, d, d, eps)
    nl = len(layers)
    Ls = (Layer * nl)(*[_layer_struct(l) for l in layers])
    kc = (CMat * nl)(*[_rowmat(t, heads * d) for t in k_caches])
    vc = (CMat * nl)(*[_rowmat(t, heads * d) for t in v_caches])
    y = torch.empty((M, D), dtype=torch.float32, device=x_cand.device)
    nws = workspace_size(OP_MFALCON, jag, dims, D, total_cand)
    ws = workspace if workspace is not None else _workspace(nws, x_cand.device)
    st = lib.mfalcon_score(ctypes.byref(jag), ctypes.byref(dims), D, nl, Ls, kc, vc, cand_offsets.data_ptr(),
                           int(total_cand), _ptr(cand_ts), _rowmat(x_cand, D), int(b_m), y.data_ptr(), ws.data_ptr(),
                           ws.numel(), _stream(x_cand.device))
    _check(st)
    return y
