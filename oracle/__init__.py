"""fp64 CPU oracle for the Dynamic Mask Attention forward (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package; the HIP path never does.  The numerics
live in ``dma_oracle.cpp`` (plain C++17 + OpenMP, double precision), which
states each definition it follows.  This wrapper only marshals numpy arrays.

Functions (all inputs are copied to contiguous numpy arrays first):
  weights(V, Delta, A)                      -> delta [B, Hkv, Sk] float64
  vproj(X, Wv)                              -> V = X Wv [..., N] float64 (X [..., Cin])
  keep_row(delta_row, p, w)                 -> ascending int32 key list
  mask(delta, q0, Sq, w, Bq, Bk)            -> dict(evict, row_cnt, u_cnt, u_idx, kt_cnt, kt_idx)
  attn_rows(Q, K, V, delta, q0, w, rows, scale=None) -> (O [n, D], lse [n])
  attn(Q, K, V, delta, q0, w, scale=None)   -> (O [B, Sq, Hq, D], lse [B, Hq, Sq])
  attn_bwd(Q, K, V, delta, dO, q0, w, scale=None) -> (dQ, dK, dV, ddelta) float64
  weights_bwd(V, Delta, A, ddelta)          -> (dV [B, Sk, Hkv, D], dDelta, dA) float64
  attn_bwd_rows(Q, K, V, delta, dO, q0, w, rows)  -> dQ of (b, hq, i) rows [n, D]
  attn_bwd_keys(Q, K, V, delta, dO, q0, w, keys)  -> (dK, dV [m, D], ddelta [m]) of (b, h, j) keys
"""
import ctypes
import os

import numpy as np

from .build import build as _build, LIB_PATH

_lib = None
_I64 = ctypes.c_int64
_P = ctypes.c_void_p


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        _build()
    lib = ctypes.CDLL(LIB_PATH)
    lib.orc_num_threads.restype = ctypes.c_int
    lib.orc_weights.argtypes = [_P, _P, _P, _I64, _I64, _I64, _I64, _P]
    lib.orc_weights.restype = None
    lib.orc_vproj.argtypes = [_P, _P, _I64, _I64, _I64, _P]
    lib.orc_vproj.restype = None
    lib.orc_keep_row.argtypes = [_P, _I64, _I64, _P]
    lib.orc_keep_row.restype = _I64
    lib.orc_mask.argtypes = [_P, _I64, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P,
                             _I64, _P, _P, _I64]
    lib.orc_mask.restype = ctypes.c_int
    lib.orc_attn_rows.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                  _I64, ctypes.c_double, _P, _I64, _P, _P]
    lib.orc_attn_rows.restype = None
    lib.orc_attn_bwd.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _I64,
                                 _I64, ctypes.c_double, _P, _P, _P, _P]
    lib.orc_attn_bwd.restype = None
    lib.orc_attn_bwd_rows.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64,
                                      _I64, ctypes.c_double, _P, _I64, _P]
    lib.orc_attn_bwd_rows.restype = None
    lib.orc_attn_bwd_keys.argtypes = [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I64,
                                      _I64, ctypes.c_double, _P, _I64, _P, _P, _P]
    lib.orc_attn_bwd_keys.restype = None
    lib.orc_weights_bwd.argtypes = [_P, _P, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P]
    lib.orc_weights_bwd.restype = None
    _lib = lib
    return lib


def _np(x, dtype):
    """numpy copy (contiguous, given dtype) of a numpy array or torch tensor."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        import torch
        x = x.to(torch.float64 if dtype == np.float64 else
                 torch.float32 if dtype == np.float32 else torch.int64).numpy()
    return np.ascontiguousarray(x, dtype=dtype)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_load().orc_num_threads())


def weights(V, Delta, A):
    """delta[b,h,j] = exp(softplus(sum_c V[b,j,c] Delta[c,h]) * A[h]) in fp64."""
    lib = _load()
    V = _np(V, np.float32)
    B, Sk, Hkv, D = V.shape
    Dl = _np(Delta, np.float32)
    Av = _np(A, np.float32)
    assert Dl.shape == (Hkv * D, Hkv) and Av.shape == (Hkv,)
    out = np.empty((B, Hkv, Sk), np.float64)
    lib.orc_weights(_ptr(V), _ptr(Dl), _ptr(Av), B, Sk, Hkv, D, _ptr(out))
    return out


def vproj(X, Wv):
    """V[..., n] = sum_k X[..., k] Wv[k, n] in fp64 (the value projection)."""
    lib = _load()
    X = _np(X, np.float32)
    W = _np(Wv, np.float32)
    lead, Cin = X.shape[:-1], X.shape[-1]
    assert W.ndim == 2 and W.shape[0] == Cin
    N = W.shape[1]
    M = int(np.prod(lead)) if lead else 1
    out = np.empty((M, N), np.float64)
    lib.orc_vproj(_ptr(X), _ptr(W), M, Cin, N, _ptr(out))
    return out.reshape(*lead, N)


def keep_row(d, p, w):
    """Keys kept by query position p of one delta row (ascending)."""
    lib = _load()
    d = _np(d, np.float64)
    out = np.empty(max(p + 1, 1), np.int32)
    n = lib.orc_keep_row(_ptr(d), p, w, _ptr(out))
    return out[:n].copy()


def union_cap(q_lo, q_hi, w):
    """Largest possible number of keys kept by some row of [q_lo, q_hi]."""
    return min(q_hi + 1, w + q_hi - q_lo)


def mask(delta, q0, Sq, w, Bq, Bk):
    """Literal keep sets of rows q0..q0+Sq-1 for every leading (b, h) delta row."""
    lib = _load()
    d = _np(delta, np.float64)
    Sk = d.shape[-1]
    lead = d.shape[:-1]
    BH = int(np.prod(lead)) if lead else 1
    nQT = (Sq + Bq - 1) // Bq
    nKT = (Sk + Bk - 1) // Bk
    u_stride = max(1, min(Sk, w + Bq - 1))
    kt_stride = max(1, nKT)
    evict = np.empty((BH, Sk), np.int32)
    row_cnt = np.empty((BH, Sq), np.int64)
    u_cnt = np.empty((BH, nQT), np.int64)
    u_idx = np.full((BH, nQT, u_stride), -1, np.int32)
    kt_cnt = np.empty((BH, nQT), np.int64)
    kt_idx = np.full((BH, nQT, kt_stride), -1, np.int32)
    rc = lib.orc_mask(_ptr(d), BH, Sk, q0, Sq, w, Bq, Bk, _ptr(evict), _ptr(row_cnt),
                      _ptr(u_cnt), _ptr(u_idx), u_stride, _ptr(kt_cnt), _ptr(kt_idx), kt_stride)
    if rc == -2:
        raise RuntimeError("oracle mask: a tile list exceeded its stride")
    if rc == -1:
        raise RuntimeError("oracle mask: rows keeping a key are not one contiguous run")
    return dict(evict=evict.reshape(*lead, Sk), row_cnt=row_cnt.reshape(*lead, Sq),
                u_cnt=u_cnt.reshape(*lead, nQT), u_idx=u_idx.reshape(*lead, nQT, u_stride),
                kt_cnt=kt_cnt.reshape(*lead, nQT), kt_idx=kt_idx.reshape(*lead, nQT, kt_stride))


def attn_rows(Q, K, V, delta, q0, w, rows, scale=None):
    """Attention output and log-sum-exp of the listed (b, hq, i) query rows."""
    lib = _load()
    Qn = _np(Q, np.float32)
    Kn = _np(K, np.float32)
    Vn = _np(V, np.float32)
    d = _np(delta, np.float64)
    B, Sq, Hq, D = Qn.shape
    _, Sk, Hkv, _ = Kn.shape
    assert d.shape == (B, Hkv, Sk)
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
    n = rows.shape[0]
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    O = np.empty((n, D), np.float64)
    lse = np.empty((n,), np.float64)
    if n:
        lib.orc_attn_rows(_ptr(Qn), _ptr(Kn), _ptr(Vn), _ptr(d), B, Sq, Sk, Hq, Hkv, D, q0, w,
                          float(scale), _ptr(rows), n, _ptr(O), _ptr(lse))
    return O, lse


def attn(Q, K, V, delta, q0, w, scale=None):
    """Attention over every query row: O [B, Sq, Hq, D], lse [B, Hq, Sq]."""
    B, Sq, Hq, D = Q.shape
    b, h, i = np.meshgrid(np.arange(B), np.arange(Hq), np.arange(Sq), indexing="ij")
    rows = np.stack([b.ravel(), h.ravel(), i.ravel()], 1)
    O, lse = attn_rows(Q, K, V, delta, q0, w, rows, scale)
    return (O.reshape(B, Hq, Sq, D).transpose(0, 2, 1, 3).copy(), lse.reshape(B, Hq, Sq))


def attn_bwd(Q, K, V, delta, dO, q0, w, scale=None):
    """Gradients of sum(dO * O) with the keep sets held fixed:
    dQ [B,Sq,Hq,D], dK and dV [B,Sk,Hkv,D], ddelta [B,Hkv,Sk] (float64)."""
    lib = _load()
    Qn, Kn, Vn, gn = (_np(x, np.float32) for x in (Q, K, V, dO))
    d = _np(delta, np.float64)
    B, Sq, Hq, D = Qn.shape
    _, Sk, Hkv, _ = Kn.shape
    assert d.shape == (B, Hkv, Sk) and gn.shape == Qn.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    dQ = np.empty((B, Sq, Hq, D), np.float64)
    dK = np.empty((B, Sk, Hkv, D), np.float64)
    dV = np.empty((B, Sk, Hkv, D), np.float64)
    dd = np.empty((B, Hkv, Sk), np.float64)
    lib.orc_attn_bwd(_ptr(Qn), _ptr(Kn), _ptr(Vn), _ptr(d), _ptr(gn), B, Sq, Sk, Hq, Hkv, D, q0,
                     w, float(scale), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dd))
    return dQ, dK, dV, dd


def weights_bwd(V, Delta, A, ddelta):
    """Gradients through delta = exp(softplus(V . Delta) * A) given ddelta:
    dV [B,Sk,Hkv,D], dDelta [Hkv*D, Hkv], dA [Hkv] (float64)."""
    lib = _load()
    Vn = _np(V, np.float32)
    Dn = _np(Delta, np.float32)
    An = _np(A, np.float32)
    gd = _np(ddelta, np.float64)
    B, Sk, Hkv, D = Vn.shape
    assert gd.shape == (B, Hkv, Sk)
    dV = np.empty((B, Sk, Hkv, D), np.float64)
    dDelta = np.empty((Hkv * D, Hkv), np.float64)
    dA = np.empty((Hkv,), np.float64)
    lib.orc_weights_bwd(_ptr(Vn), _ptr(Dn), _ptr(An), _ptr(gd), B, Sk, Hkv, D, _ptr(dV),
                        _ptr(dDelta), _ptr(dA))
    return dV, dDelta, dA


def _bwd_inputs(Q, K, V, delta, dO):
    Qn, Kn, Vn, gn = (_np(x, np.float32) for x in (Q, K, V, dO))
    return Qn, Kn, Vn, _np(delta, np.float64), gn


def attn_bwd_rows(Q, K, V, delta, dO, q0, w, rows, scale=None):
    """dQ of the listed (b, hq, i) rows, float64 [n, D]."""
    lib = _load()
    Qn, Kn, Vn, d, gn = _bwd_inputs(Q, K, V, delta, dO)
    B, Sq, Hq, D = Qn.shape
    _, Sk, Hkv, _ = Kn.shape
    rows = np.ascontiguousarray(np.asarray(rows, np.int64).reshape(-1, 3))
    out = np.empty((rows.shape[0], D), np.float64)
    lib.orc_attn_bwd_rows(_ptr(Qn), _ptr(Kn), _ptr(Vn), _ptr(d), _ptr(gn), Sq, Sk, Hq, Hkv, D, q0,
                          w, float(scale or 1.0 / np.sqrt(D)), _ptr(rows), rows.shape[0],
                          _ptr(out))
    return out


def attn_bwd_keys(Q, K, V, delta, dO, q0, w, keys, scale=None):
    """dK, dV [m, D] and ddelta [m] of the listed (b, h, j) keys (float64)."""
    lib = _load()
    Qn, Kn, Vn, d, gn = _bwd_inputs(Q, K, V, delta, dO)
    B, Sq, Hq, D = Qn.shape
    _, Sk, Hkv, _ = Kn.shape
    keys = np.ascontiguousarray(np.asarray(keys, np.int64).reshape(-1, 3))
    m = keys.shape[0]
    dK = np.empty((m, D), np.float64)
    dV = np.empty((m, D), np.float64)
    dd = np.empty((m,), np.float64)
    lib.orc_attn_bwd_keys(_ptr(Qn), _ptr(Kn), _ptr(Vn), _ptr(d), _ptr(gn), Sq, Sk, Hq, Hkv, D,
                          q0, w, float(scale or 1.0 / np.sqrt(D)), _ptr(keys), m, _ptr(dK),
                          _ptr(dV), _ptr(dd))
    return dK, dV, dd
