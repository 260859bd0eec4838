"""Dynamic Mask Attention (DMA) forward for MI355X (gfx950).

The method is the one of the Hugging Face blog "Trainable Dynamic Mask
Sparse Attention": per-key dynamic weights delta = exp(softplus(v Delta) A)
from the value states, a causal top-w keep mask per query, and attention
softmax(q k^T / sqrt(d) + delta) v over only the kept keys.  Every step runs
in hand-written HIP kernels behind a C ABI (include/dma.h); this module only
marshals torch tensors (device memory and the current stream) into it.

    delta = weights(V, Delta, A)
    mask  = topk_mask(delta, Sq, q_offset, w)
    O     = attn_fwd(Q, K, V, delta, mask, q_offset, w)
or  O = forward(Q, K, V, Delta, A, w)
"""
import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import DmaMask, DmaMaskDims, check, load

__all__ = ["weights", "topk_mask", "attn_fwd", "forward", "mask_dims", "Mask", "tile_sizes",
           "load"]


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return _lib.DMA_BF16
    if t == torch.float32:
        return _lib.DMA_F32
    raise TypeError(f"unsupported dtype {t}")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr() if t is not None and t.numel() else 0)


def _need_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("DMA tensors must live on the GPU")


def _check_delta(delta: torch.Tensor, B: int, Hkv: int, Sk: int):
    if delta.dtype != torch.float32 or tuple(delta.shape) != (B, Hkv, Sk):
        raise ValueError(f"delta must be float32 [B, Hkv, Sk] = {[B, Hkv, Sk]}, got "
                         f"{delta.dtype} {list(delta.shape)}")


def _check_mask(mask: "Mask", B: int, Hkv: int, Sq: int, Sk: int):
    """The kernels index the mask arrays by these sizes, so a mask built for
    other sizes would be read out of bounds."""
    if (mask.B, mask.Hkv, mask.Sq, mask.Sk) != (B, Hkv, Sq, Sk):
        raise ValueError(f"mask was built for (B, Hkv, Sq, Sk) = "
                         f"{(mask.B, mask.Hkv, mask.Sq, mask.Sk)}, the call has {(B, Hkv, Sq, Sk)}")
    d = mask_dims(B, Hkv, Sq, Sk, mask.q_offset, mask.w)
    n = d["n_tiles_total"]
    for name, t, need in (("u_idx", mask.u_idx, d["u_elems"]), ("u_cnt", mask.u_cnt, n),
                          ("u_nfull", mask.u_nfull, n), ("u_dmax", mask.u_dmax, n),
                          ("evict", mask.evict, d["evict_elems"]),
                          ("u_dlo", mask.u_dlo, n if Sq > 1 else 0)):
        if need and (t is None or t.numel() < need):
            raise ValueError(f"mask array {name} holds fewer than {need} entries")
    if Sq == 1 and mask.u_dval is not None and mask.u_dval.numel() < d["u_elems"]:
        raise ValueError(f"mask array u_dval holds fewer than {d['u_elems']} entries")


def _check_qkv(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor):
    if Q.dim() != 4 or K.dim() != 4 or V.shape != K.shape:
        raise ValueError("Q must be [B,Sq,Hq,D], K and V [B,Sk,Hkv,D]")
    if Q.dtype != K.dtype or Q.dtype != V.dtype:
        raise ValueError("Q, K and V must share one dtype")
    if Q.shape[0] != K.shape[0] or Q.shape[3] != K.shape[3]:
        raise ValueError("Q and K/V disagree on batch or head size")
    if K.stride() != V.stride() or Q.stride(3) != 1 or K.stride(3) != 1:
        raise ValueError("K and V must share strides; the D values must be contiguous")


def tile_sizes():
    bq, bk = ctypes.c_int32(), ctypes.c_int32()
    load().dma_tile_sizes(ctypes.byref(bq), ctypes.byref(bk))
    return bq.value, bk.value


def mask_dims(B, Hkv, Sq, Sk, q_offset, w):
    d = DmaMaskDims()
    check("dma_mask_dims_for", load().dma_mask_dims_for(B, Hkv, Sq, Sk, q_offset, w,
                                                          ctypes.byref(d)))
    return {f: getattr(d, f) for f, _ in DmaMaskDims._fields_}


@dataclass
class Mask:
    """Device arrays of one mask (layouts in include/dma.h)."""
    B: int
    Hkv: int
    Sq: int
    Sk: int
    q_offset: int
    w: int
    dims: dict
    evict: Optional[torch.Tensor]
    u_idx: torch.Tensor
    u_cnt: torch.Tensor
    u_nfull: torch.Tensor
    u_dmax: torch.Tensor
    kt_idx: Optional[torch.Tensor]
    kt_cnt: Optional[torch.Tensor]
    u_dlo: Optional[torch.Tensor] = None
    u_dval: Optional[torch.Tensor] = None

    def cstruct(self):
        return DmaMask(_ptr(self.evict), _ptr(self.u_idx), _ptr(self.u_cnt), _ptr(self.u_nfull),
                       _ptr(self.u_dmax), _ptr(self.kt_idx), _ptr(self.kt_cnt), _ptr(self.u_dlo),
                       _ptr(self.u_dval))


def alloc_mask(B, Hkv, Sq, Sk, q_offset, w, device, kt_lists=True) -> Mask:
    d = mask_dims(B, Hkv, Sq, Sk, q_offset, w)
    i32 = dict(dtype=torch.int32, device=device)
    n = d["n_tiles_total"]
    return Mask(B, Hkv, Sq, Sk, q_offset, w, d,
                evict=torch.empty(d["evict_elems"], **i32) if d["evict_elems"] else None,
                u_idx=torch.empty(max(1, d["u_elems"]), **i32),
                u_cnt=torch.empty(max(1, n), **i32),
                u_nfull=torch.empty(max(1, n), **i32),
                u_dmax=torch.empty(max(1, n), dtype=torch.float32, device=device),
                kt_idx=torch.empty(max(1, d["kt_elems"]), **i32) if kt_lists else None,
                kt_cnt=torch.empty(max(1, n), **i32) if kt_lists else None,
                u_dlo=torch.empty(max(1, n), dtype=torch.float32, device=device)
                if Sq > 1 else None,
                u_dval=torch.empty(max(1, d["u_elems"]), dtype=torch.float32, device=device)
                if Sq == 1 else None)


def weights(V: torch.Tensor, Delta: torch.Tensor, A: torch.Tensor,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """delta[b,h,j] = exp(softplus(V[b,j,:] . Delta[:,h]) * A[h]);  V [B,Sk,Hkv,D]."""
    _need_cuda(V, Delta, A)
    B, Sk, Hkv, D = V.shape
    if V.stride(3) != 1 or V.stride(2) != D:
        raise ValueError("V rows must be contiguous over (kv head, channel)")
    Delta = Delta.contiguous().float()
    A = A.contiguous().float()
    if out is None:
        out = torch.empty(B, Hkv, Sk, dtype=torch.float32, device=V.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (B, Hkv, Sk) or not out.is_contiguous():
        raise ValueError("out must be contiguous float32 [B, Hkv, Sk]")
    check("dma_weights", load().dma_weights(_ptr(V), _dtype_code(V.dtype), B, Sk, Hkv, D,
                                            V.stride(0), V.stride(1), _ptr(Delta), _ptr(A),
                                            _ptr(out), _stream(V.device)))
    return out


def vproj_weights(X: torch.Tensor, Wv: torch.Tensor, Hkv: int, Delta: Optional[torch.Tensor] = None,
                  A: Optional[torch.Tensor] = None, V: Optional[torch.Tensor] = None,
                  delta: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Value projection V = X Wv (X [B,Sk,Cin] bf16, Wv [Cin, Hkv*D] bf16) with the
    dynamic weights formed in its epilogue when Delta and A are given:
    returns (V [B,Sk,Hkv,D] bf16, delta [B,Hkv,Sk] float32), or V alone."""
    _need_cuda(X, Wv)
    if X.dim() != 3 or X.dtype != torch.bfloat16 or X.stride(2) != 1:
        raise ValueError("X must be bf16 [B, Sk, Cin] with contiguous rows")
    B, Sk, Cin = X.shape
    if Wv.dim() != 2 or Wv.dtype != torch.bfloat16 or Wv.shape[0] != Cin or Wv.shape[1] % Hkv:
        raise ValueError("Wv must be bf16 [Cin, Hkv*D]")
    Wv = Wv.contiguous()
    D = Wv.shape[1] // Hkv
    if V is None:
        V = torch.empty(B, Sk, Hkv, D, dtype=torch.bfloat16, device=X.device)
    elif V.dtype != torch.bfloat16 or tuple(V.shape) != (B, Sk, Hkv, D) or V.stride(3) != 1 \
            or V.stride(2) != D:
        raise ValueError("V must be bf16 [B, Sk, Hkv, D] with contiguous rows")
    lib = load()
    fused = Delta is not None
    if fused:
        _need_cuda(Delta, A)
        Delta = Delta.contiguous().float()
        A = A.contiguous().float()
        if delta is None:
            delta = torch.empty(B, Hkv, Sk, dtype=torch.float32, device=X.device)
        elif delta.dtype != torch.float32 or tuple(delta.shape) != (B, Hkv, Sk) \
                or not delta.is_contiguous():
            raise ValueError("delta must be contiguous float32 [B, Hkv, Sk]")
    nbytes = lib.dma_vproj_workspace_bytes(B, Sk, Hkv, D) if fused else 0
    if nbytes and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=X.device)
    check("dma_vproj_weights", lib.dma_vproj_weights(
        _ptr(X), B, Sk, Cin, X.stride(0), X.stride(1), _ptr(Wv), Hkv, D, _ptr(V), V.stride(0),
        V.stride(1), _ptr(Delta), _ptr(A), _ptr(delta) if fused else ctypes.c_void_p(0),
        _ptr(workspace) if nbytes else ctypes.c_void_p(0), nbytes, _stream(X.device)))
    return (V, delta) if fused else V


def topk_mask(delta: torch.Tensor, Sq: int, q_offset: int, w: int, kt_lists: bool = True,
              mask: Optional[Mask] = None, workspace: Optional[torch.Tensor] = None,
              noalloc: bool = False) -> Mask:
    """Causal top-w keep mask of query positions q_offset..q_offset+Sq-1.
    noalloc: use the library's static scratch (dma_topk_mask_noalloc) instead
    of a workspace; `mask` must then be given for the call to allocate nothing."""
    _need_cuda(delta)
    delta = delta.contiguous()
    B, Hkv, Sk = delta.shape
    _check_delta(delta, B, Hkv, Sk)
    lib = load()
    if mask is None:
        mask = alloc_mask(B, Hkv, Sq, Sk, q_offset, w, delta.device, kt_lists)
    if noalloc:
        ms = mask.cstruct()
        check("dma_topk_mask_noalloc", lib.dma_topk_mask_noalloc(
            _ptr(delta), B, Hkv, Sq, Sk, q_offset, w, ctypes.byref(ms), _stream(delta.device)))
        return mask
    nbytes = lib.dma_topk_workspace_bytes(B, Hkv, Sq, Sk, w)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(16, nbytes), dtype=torch.uint8, device=delta.device)
    ms = mask.cstruct()
    check("dma_topk_mask", lib.dma_topk_mask(_ptr(delta), B, Hkv, Sq, Sk, q_offset, w,
                                             ctypes.byref(ms), _ptr(workspace), nbytes,
                                             _stream(delta.device)))
    return mask


def decode_keep_append(delta: torch.Tensor, mask: Mask) -> Mask:
    """One decode step of a one-row keep set: `mask` holds keep(Sk-2) over keys
    0..Sk-2 (built with kt_lists=False); delta [B,Hkv,Sk] adds key Sk-1.  The
    lists are updated in place to keep(Sk-1) and `mask` describes that row."""
    _need_cuda(delta)
    delta = delta.contiguous()
    B, Hkv, Sk = delta.shape
    if mask.Sq != 1 or mask.kt_idx is not None or (B, Hkv) != (mask.B, mask.Hkv) \
            or Sk != mask.Sk + 1:
        raise ValueError("decode_keep_append needs a one-row mask without key-tile lists "
                         "over one key fewer than delta")
    ms = mask.cstruct()
    check("dma_decode_keep_append", load().dma_decode_keep_append(
        _ptr(delta), B, Hkv, Sk, mask.w, ctypes.byref(ms), _stream(delta.device)))
    mask.Sk, mask.q_offset = Sk, Sk - 1
    mask.dims = mask_dims(B, Hkv, 1, Sk, Sk - 1, mask.w)
    return mask


def attn_fwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, delta: torch.Tensor, mask: Mask,
             scale: Optional[float] = None, return_lse: bool = False,
             out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
             lib=None):
    """Masked attention; Q [B,Sq,Hq,D], K/V [B,Sk,Hkv,D] (any b/s/h strides).
    lib: the loaded library to call (default load(); the tests pass load_safe())."""
    _check_qkv(Q, K, V)
    B, Sq, Hq, D = Q.shape
    _, Sk, Hkv, _ = K.shape
    _check_delta(delta, B, Hkv, Sk)
    _check_mask(mask, B, Hkv, Sq, Sk)
    _need_cuda(Q, K, V, delta)
    delta_c = delta.contiguous()  # bound to a name: it must outlive the enqueued kernels
    lib = lib or load()
    if out is None:
        out = torch.empty(B, Sq, Hq, D, dtype=Q.dtype, device=Q.device)
    lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=Q.device) if return_lse else None
    nbytes = lib.dma_attn_workspace_bytes(B, Hq, Sq, D, mask.w)
    if nbytes and (workspace is None or workspace.numel() < nbytes):
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=Q.device)
    qs = (ctypes.c_int64 * 3)(Q.stride(0), Q.stride(1), Q.stride(2))
    ks = (ctypes.c_int64 * 3)(K.stride(0), K.stride(1), K.stride(2))
    ms = mask.cstruct()
    check("dma_attn_fwd", lib.dma_attn_fwd(
        _ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q.dtype), B, Sq, Sk, Hq, Hkv, D, qs, ks,
        mask.q_offset, mask.w, _ptr(delta_c), ctypes.byref(ms),
        float(scale) if scale is not None else 0.0, _ptr(out), _ptr(lse),
        _ptr(workspace) if nbytes else ctypes.c_void_p(0), nbytes, _stream(Q.device)))
    return (out, lse) if return_lse else out


def forward(Q, K, V, Delta, A, w, q_offset=0, scale=None, return_all=False):
    """The whole DMA forward: weights, keep mask, attention."""
    delta = weights(V, Delta, A)
    mask = topk_mask(delta, Q.shape[1], q_offset, w)
    O = attn_fwd(Q, K, V, delta, mask, scale=scale)
    if return_all:
        return O, delta, mask
    return O


def attn_fwd_train(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, delta: torch.Tensor,
                   mask: Mask, scale: Optional[float] = None):
    """attn_fwd for training (bf16 prefill): returns O, lse and O_res, the
    rounding residual of O that attn_bwd uses for dO . O."""
    _check_qkv(Q, K, V)
    B, Sq, Hq, D = Q.shape
    _, Sk, Hkv, _ = K.shape
    _check_delta(delta, B, Hkv, Sk)
    _check_mask(mask, B, Hkv, Sq, Sk)
    _need_cuda(Q, K, V, delta)
    delta_c = delta.contiguous()
    O = torch.empty(B, Sq, Hq, D, dtype=Q.dtype, device=Q.device)
    Ores = torch.empty_like(O)
    lse = torch.empty(B, Hq, Sq, dtype=torch.float32, device=Q.device)
    qs = (ctypes.c_int64 * 3)(Q.stride(0), Q.stride(1), Q.stride(2))
    ks = (ctypes.c_int64 * 3)(K.stride(0), K.stride(1), K.stride(2))
    ms = mask.cstruct()
    check("dma_attn_fwd_train", load().dma_attn_fwd_train(
        _ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q.dtype), B, Sq, Sk, Hq, Hkv, D, qs, ks,
        mask.q_offset, mask.w, _ptr(delta_c), ctypes.byref(ms),
        0.0 if scale is None else float(scale), _ptr(O), _ptr(lse), _ptr(Ores), _stream(Q.device)))
    return O, lse, Ores


def attn_bwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, delta: torch.Tensor, mask: Mask,
             O: torch.Tensor, lse: torch.Tensor, dO: torch.Tensor,
             O_res: Optional[torch.Tensor] = None,
             scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
             lib=None):
    """Gradients of sum(dO * O) of attn_fwd (keep sets fixed): float32 dQ
    [B,Sq,Hq,D], dK and dV [B,Sk,Hkv,D], ddelta [B,Hkv,Sk].  O and lse are
    the forward's outputs; O_res (from attn_fwd_train) makes dO . O exact.
    lib: the loaded library to call (default load(); the tests pass load_safe())."""
    _check_qkv(Q, K, V)
    B, Sq, Hq, D = Q.shape
    _, Sk, Hkv, _ = K.shape
    _check_delta(delta, B, Hkv, Sk)
    _check_mask(mask, B, Hkv, Sq, Sk)
    if O.shape != Q.shape or dO.shape != Q.shape or O.dtype != Q.dtype or dO.dtype != Q.dtype:
        raise ValueError("O and dO must have Q's shape and dtype")
    if O_res is not None and (O_res.shape != Q.shape or O_res.dtype != Q.dtype):
        raise ValueError("O_res must have Q's shape and dtype")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("lse must be float32 [B, Hq, Sq]")
    _need_cuda(Q, K, V, delta, O, lse, dO)
    # contiguous copies bound to names: each must outlive the enqueued kernels
    # (a temporary freed at once could hand its memory to the next copy)
    delta_c, O_c, lse_c, dO_c = (t.contiguous() for t in (delta, O, lse, dO))
    Ores_c = O_res.contiguous() if O_res is not None else None
    lib = lib or load()
    dev = Q.device
    dQ = torch.empty(B, Sq, Hq, D, dtype=torch.float32, device=dev)
    dK = torch.empty(B, Sk, Hkv, D, dtype=torch.float32, device=dev)
    dV = torch.empty(B, Sk, Hkv, D, dtype=torch.float32, device=dev)
    dd = torch.empty(B, Hkv, Sk, dtype=torch.float32, device=dev)
    nbytes = lib.dma_attn_bwd_workspace_bytes(B, Hq, Hkv, Sq, Sk, mask.w)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(256, nbytes), dtype=torch.uint8, device=dev)
    qs = (ctypes.c_int64 * 3)(Q.stride(0), Q.stride(1), Q.stride(2))
    ks = (ctypes.c_int64 * 3)(K.stride(0), K.stride(1), K.stride(2))
    ms = mask.cstruct()
    check("dma_attn_bwd", lib.dma_attn_bwd(
        _ptr(Q), _ptr(K), _ptr(V), _dtype_code(Q.dtype), B, Sq, Sk, Hq, Hkv, D, qs, ks,
        mask.q_offset, mask.w, _ptr(delta_c), ctypes.byref(ms),
        0.0 if scale is None else float(scale), _ptr(O_c),
        _ptr(Ores_c) if Ores_c is not None else None, _ptr(lse_c),
        _ptr(dO_c), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dd), _ptr(workspace), nbytes,
        _stream(dev)))
    return dQ, dK, dV, dd


def weights_bwd(V: torch.Tensor, Delta: torch.Tensor, A: torch.Tensor, ddelta: torch.Tensor,
                dV: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Backward of weights() given ddelta [B,Hkv,Sk]: returns (dV, dDelta, dA), float32.
    dV [B,Sk,Hkv,D] is accumulated into when given (the attention's dV)."""
    _need_cuda(V, Delta, A, ddelta)
    B, Sk, Hkv, D = V.shape
    if V.stride(3) != 1 or V.stride(2) != D:
        raise ValueError("V rows must be contiguous over (kv head, channel)")
    _check_delta(ddelta, B, Hkv, Sk)
    if dV is not None and (dV.dtype != torch.float32 or tuple(dV.shape) != (B, Sk, Hkv, D)
                           or not dV.is_contiguous()):
        raise ValueError("dV must be contiguous float32 [B, Sk, Hkv, D]")
    # converted copies bound to names: each must outlive the enqueued kernels
    Delta_c = Delta.contiguous().float()
    A_c = A.contiguous().float()
    dd_c = ddelta.contiguous()
    dev = V.device
    if dV is None:
        dV = torch.zeros(B, Sk, Hkv, D, dtype=torch.float32, device=dev)
    dDelta = torch.empty(Hkv * D, Hkv, dtype=torch.float32, device=dev)
    dA = torch.empty(Hkv, dtype=torch.float32, device=dev)
    lib = load()
    nbytes = lib.dma_weights_bwd_workspace_bytes(B, Sk, Hkv)
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(16, nbytes), dtype=torch.uint8, device=dev)
    check("dma_weights_bwd", lib.dma_weights_bwd(
        _ptr(V), _dtype_code(V.dtype), B, Sk, Hkv, D, V.stride(0), V.stride(1),
        _ptr(Delta_c), _ptr(A_c), _ptr(dd_c), _ptr(dV), _ptr(dDelta), _ptr(dA), _ptr(workspace),
        nbytes,
        _stream(dev)))
    return dV, dDelta, dA
