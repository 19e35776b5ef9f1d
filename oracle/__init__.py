"""CPU oracle for the HSTU attention path -- TEST INFRASTRUCTURE ONLY.

A plain fp64 implementation (``hstu_oracle.c``, nested loops, OpenMP over
independent rows) of what the GPU library computes, written from the paper
review page "Actions Speak Louder than Words" (arXiv 2402.17152), section 3:
Eq. 1-3 and M-FALCON.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg use it; the GPU library never imports or links
it, and it shares no code with the library.

Every function takes numpy arrays (any float dtype; converted to fp64) and
returns fp64 arrays.  Pins that tie it to the pages and to mathematics rather
than to itself live in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hstu_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _open(path):
    lib = ctypes.CDLL(path)
    lib.oracle_time_bucket.restype = ctypes.c_int
    lib.oracle_time_bucket.argtypes = [ctypes.c_int64]
    return lib


def _load():
    global _lib
    if _lib is None:
        build()
        _lib = _open(_LIB)
    return _lib


def swap_library(path: Optional[str]):
    """Point this module at another build of the oracle source (the mutation
    tests load deliberately broken copies); None restores the real one.
    Returns the previously loaded handle."""
    global _lib
    old = _lib
    _lib = _open(path) if path else None
    return old


def _d(a: Optional[np.ndarray]):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _i64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int64)


def time_bucket(dt: int) -> int:
    return _load().oracle_time_bucket(ctypes.c_int64(int(dt)))


def threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS, else all usable cores)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env:
        return int(env)
    return len(os.sched_getaffinity(0))


def attn_fwd(offsets, ts, q, k, v, rab_p, rab_t, n_max: int, rows: Optional[Sequence[int]] = None):
    """O = phi2(Q K^T + rab) V per Eq. 2; q, k [T][H][dqk], v [T][H][dv].
    Returns [T][H*dv] (or [len(rows)][H*dv] for the listed token rows)."""
    lib = _load()
    off = _i32(offsets)
    B = len(off) - 1
    q, k, v = _d(q), _d(k), _d(v)
    T, H, dqk = q.shape
    dv = v.shape[2]
    rp, rt = _d(rab_p), _d(rab_t)
    tsa = _i64(ts)
    if rows is not None:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.zeros((len(rows_a), H * dv), np.float64)
        nrows, rptr = len(rows_a), _p(rows_a)
    else:
        out = np.zeros((T, H * dv), np.float64)
        nrows, rptr = 0, None
    lib.oracle_attn_fwd(ctypes.c_int(B), _p(off), _p(tsa), ctypes.c_int(H), ctypes.c_int(dqk), ctypes.c_int(dv),
                        ctypes.c_int64(n_max), _p(rp), _p(rt), _p(q), _p(k), _p(v), _p(out),
                        ctypes.c_int64(nrows), rptr)
    return out


def ln_gate(O, U, eps: float):
    """G = LayerNorm(O) (.) U over each row's features (Eq. 3); returns
    (G, stats[T][2] = (mean, rstd))."""
    lib = _load()
    O = _d(O)
    T, F = O.shape
    Ud = _d(U)
    G = np.zeros_like(O)
    st = np.zeros((T, 2), np.float64)
    lib.oracle_ln_gate(ctypes.c_int64(T), ctypes.c_int(F), _p(O), _p(Ud), ctypes.c_double(eps), _p(G), _p(st))
    return G, st


def attn_bwd(offsets, ts, q, k, v, rab_p, rab_t, n_max: int, U, eps: float, dout):
    """Gradients of Eq. 2 (+ Norm (.) U when U is given) for the upstream
    gradient dout at G (or at O).  Returns dict dq, dk, dv, du, drab_p, drab_t."""
    lib = _load()
    off = _i32(offsets)
    B = len(off) - 1
    q, k, v = _d(q), _d(k), _d(v)
    T, H, dqk = q.shape
    dv = v.shape[2]
    rp, rt, Ud, do = _d(rab_p), _d(rab_t), _d(U), _d(dout)
    tsa = _i64(ts)
    res = dict(dq=np.zeros_like(q), dk=np.zeros_like(k), dv=np.zeros_like(v),
               du=np.zeros((T, H * dv)) if U is not None else None,
               drab_p=np.zeros_like(rp) if rp is not None else None,
               drab_t=np.zeros_like(rt) if rt is not None else None)
    lib.oracle_attn_bwd(ctypes.c_int(B), _p(off), _p(tsa), ctypes.c_int(H), ctypes.c_int(dqk), ctypes.c_int(dv),
                        ctypes.c_int64(n_max), _p(rp), _p(rt), _p(q), _p(k), _p(v), _p(Ud), ctypes.c_double(eps),
                        _p(do), _p(res["dq"]), _p(res["dk"]), _p(res["dv"]), _p(res["du"]), _p(res["drab_p"]),
                        _p(res["drab_t"]))
    return res


def attn_bwd_dq_rows(offsets, ts, q, k, v, rab_p, rab_t, n_max: int, U, eps: float, dout, rows):
    """dq of the listed token rows only (same chain as attn_bwd).  Returns
    [len(rows)][H][dqk]."""
    lib = _load()
    off = _i32(offsets)
    B = len(off) - 1
    q, k, v = _d(q), _d(k), _d(v)
    T, H, dqk = q.shape
    rows_a = np.ascontiguousarray(rows, dtype=np.int64)
    out = np.zeros((len(rows_a), H, dqk))
    lib.oracle_attn_bwd_dq_rows(ctypes.c_int(B), _p(off), _p(_i64(ts)), ctypes.c_int(H), ctypes.c_int(dqk),
                                ctypes.c_int(v.shape[2]), ctypes.c_int64(n_max), _p(_d(rab_p)), _p(_d(rab_t)), _p(q),
                                _p(k), _p(v), _p(_d(U)), ctypes.c_double(eps), _p(_d(dout)),
                                ctypes.c_int64(len(rows_a)), _p(rows_a), _p(out))
    return out


def layer_fwd(offsets, ts, x, layer, heads: int, d: int, n_max: int, phi1: int = 0, eps: float = 1e-5,
              return_kv: bool = False):
    """One HSTU layer (Eq. 1-3 + residual).  ``layer`` has w1 [4Hd][D], b1,
    w2 [D][Hd], b2, rab_p, rab_t.  Returns Y (and K, V [T][H][d] if asked)."""
    lib = _load()
    off = _i32(offsets)
    B = len(off) - 1
    X = _d(x)
    T, D = X.shape
    Y = np.zeros_like(X)
    kv = np.zeros((2, T, heads, d)) if return_kv else None
    lib.oracle_layer_fwd(ctypes.c_int(B), _p(off), _p(_i64(ts)), ctypes.c_int(heads), ctypes.c_int(d),
                         ctypes.c_int64(n_max), ctypes.c_int(D), _p(_d(layer.w1)), _p(_d(layer.b1)),
                         _p(_d(layer.w2)), _p(_d(layer.b2)), _p(_d(layer.rab_p)), _p(_d(layer.rab_t)),
                         ctypes.c_int(phi1), ctypes.c_double(eps), _p(X), _p(Y), _p(kv))
    return (Y, kv[0], kv[1]) if return_kv else Y


def layer_bwd(offsets, ts, x, layer, dy, heads: int, d: int, n_max: int, phi1: int = 0, eps: float = 1e-5):
    """Gradients of one HSTU layer (Eq. 1-3 + residual) for the upstream
    gradient ``dy`` at Y, the forward recomputed from ``x``.  Returns dict dx,
    dw1, db1, dw2, db2, drab_p, drab_t (the table gradients None when the
    table is None)."""
    lib = _load()
    off = _i32(offsets)
    B = len(off) - 1
    X, dY = _d(x), _d(dy)
    T, D = X.shape
    HD = heads * d
    rp, rt = _d(layer.rab_p), _d(layer.rab_t)
    res = dict(dx=np.zeros_like(X), dw1=np.zeros((4 * HD, D)), db1=np.zeros(4 * HD), dw2=np.zeros((D, HD)),
               db2=np.zeros(D), drab_p=np.zeros_like(rp) if rp is not None else None,
               drab_t=np.zeros_like(rt) if rt is not None else None)
    lib.oracle_layer_bwd(ctypes.c_int(B), _p(off), _p(_i64(ts)), ctypes.c_int(heads), ctypes.c_int(d),
                         ctypes.c_int64(n_max), ctypes.c_int(D), _p(_d(layer.w1)), _p(_d(layer.b1)),
                         _p(_d(layer.w2)), _p(rp), _p(rt), ctypes.c_int(phi1), ctypes.c_double(eps), _p(X), _p(dY),
                         _p(res["dx"]), _p(res["dw1"]), _p(res["db1"]), _p(res["dw2"]), _p(res["db2"]),
                         _p(res["drab_p"]), _p(res["drab_t"]))
    return res


def layer_kv(x, layer, heads: int, d: int, phi1: int = 0):
    """K and V of one layer for the tokens x [T][D] (the K and V column blocks
    of phi1(x W1^T + b1)).  Returns kv [2][T][H][d]."""
    lib = _load()
    X = _d(x)
    T, D = X.shape
    kv = np.zeros((2, T, heads, d))
    lib.oracle_layer_kv(ctypes.c_int64(T), ctypes.c_int(heads), ctypes.c_int(d), ctypes.c_int(D),
                        _p(_d(layer.w1)), _p(_d(layer.b1)), ctypes.c_int(phi1), _p(X), _p(kv))
    return kv


def history_cache(offsets, ts, x, layers, heads: int, d: int, n_max: int, phi1: int = 0, eps: float = 1e-5):
    """Run the layer stack over the user histories and keep every layer's K, V
    (the cacheable computations of M-FALCON).  The last layer's output is not
    part of the cache, so that layer only computes its K and V.  Returns kv
    [L][2][T][H][d]."""
    kvs = []
    h = x
    for i, layer in enumerate(layers):
        if i == len(layers) - 1:
            kvs.append(layer_kv(h, layer, heads, d, phi1))
        else:
            h, K, V = layer_fwd(offsets, ts, h, layer, heads, d, n_max, phi1, eps, return_kv=True)
            kvs.append(np.stack([K, V]))
    return np.stack(kvs)


def mfalcon(hist_offsets, hist_ts, cand_offsets, cand_ts, layers, kv, x_cand, heads: int, d: int, n_max: int,
            phi1: int = 0, eps: float = 1e-5):
    """Per-candidate, non-batched M-FALCON scoring against the cache ``kv``
    ([L][2][T_hist][H][d]).  Returns the candidates' final hidden states."""
    lib = _load()
    hoff, coff = _i32(hist_offsets), _i32(cand_offsets)
    U = len(hoff) - 1
    Xc = _d(x_cand)
    M, D = Xc.shape
    L = len(layers)
    W1 = _d(np.stack([l.w1 for l in layers]))
    b1 = _d(np.stack([l.b1 for l in layers]))
    W2 = _d(np.stack([l.w2 for l in layers]))
    b2 = _d(np.stack([l.b2 for l in layers]))
    rp = _d(np.stack([l.rab_p for l in layers]))
    rt = _d(np.stack([l.rab_t for l in layers]))
    kvd = _d(kv)
    y = np.zeros_like(Xc)
    lib.oracle_mfalcon(ctypes.c_int(U), _p(hoff), _p(_i64(hist_ts)), _p(coff), _p(_i64(cand_ts)), ctypes.c_int(L),
                       ctypes.c_int(heads), ctypes.c_int(d), ctypes.c_int64(n_max), ctypes.c_int(D), _p(W1), _p(b1),
                       _p(W2), _p(b2), _p(rp), _p(rt), ctypes.c_int(phi1), ctypes.c_double(eps), _p(kvd), _p(Xc),
                       _p(y))
    return y


def layer_append(hist_offsets, hist_ts, add_offsets, add_ts, layer, kv_cache, x_new, heads: int, d: int, n_max: int,
                 phi1: int = 0, eps: float = 1e-5):
    """One layer over newly appended actions against a cached history
    (kv_cache [2][T_hist][H][d], this layer's K, V of the history): new
    token i of user u sits at position n_u + i and attends to the history
    and to the new tokens up to itself.  Returns (y_new [T_new][D], the merged
    cache [2][T_hist + T_new][H][d], user u's rows starting at
    hist_offsets[u] + add_offsets[u])."""
    lib = _load()
    hoff, aoff = _i32(hist_offsets), _i32(add_offsets)
    U = len(hoff) - 1
    X = _d(x_new)
    Tn, D = X.shape
    Th = int(hoff[-1])
    y = np.zeros_like(X)
    kv_out = np.zeros((2, Th + Tn, heads, d))
    lib.oracle_layer_append(ctypes.c_int(U), _p(hoff), _p(_i64(hist_ts)), _p(aoff), _p(_i64(add_ts)),
                            ctypes.c_int(heads), ctypes.c_int(d), ctypes.c_int64(n_max), ctypes.c_int(D),
                            _p(_d(layer.w1)), _p(_d(layer.b1)), _p(_d(layer.w2)), _p(_d(layer.b2)),
                            _p(_d(layer.rab_p)), _p(_d(layer.rab_t)), ctypes.c_int(phi1), ctypes.c_double(eps),
                            _p(_d(kv_cache)), _p(X), _p(y), _p(kv_out))
    return y, kv_out


def softmax_attn_fwd(offsets, q, k, v, want_lse: bool = False):
    """The comparator: causal softmax(Q K^T / sqrt(d)) V per sequence and
    head (no bias).  Returns O [T][H*dv] (and lse [T][H] if asked)."""
    lib = _load()
    off = _i32(offsets)
    B = len(off) - 1
    q, k, v = _d(q), _d(k), _d(v)
    T, H, dqk = q.shape
    dv = v.shape[2]
    out = np.zeros((T, H * dv))
    lse = np.zeros((T, H)) if want_lse else None
    lib.oracle_softmax_attn_fwd(ctypes.c_int(B), _p(off), ctypes.c_int(H), ctypes.c_int(dqk), ctypes.c_int(dv), _p(q),
                                _p(k), _p(v), _p(out), _p(lse))
    return (out, lse) if want_lse else out


def sl_sample(offsets, alpha: float, u, keys):
    """Stochastic Length sampling: per sequence a length from the SL law and
    the actions with the L smallest keys, in order.  Returns (out_offsets
    [B+1] int32, out_index [out_offsets[B]] int32 rows of the input)."""
    lib = _load()
    off = _i32(offsets)
    B = len(off) - 1
    ua = np.ascontiguousarray(u, dtype=np.float64)
    ka = np.ascontiguousarray(keys, dtype=np.uint32)
    out_off = np.zeros(B + 1, np.int32)
    out_idx = np.zeros(max(1, int(off[-1])), np.int32)
    lib.oracle_sl_sample(ctypes.c_int(B), _p(off), ctypes.c_double(alpha), _p(ua), _p(ka), _p(out_off), _p(out_idx))
    return out_off, out_idx[:int(out_off[-1])]
