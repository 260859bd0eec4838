"""Seeded synthetic inputs for the DMA forward.

This module only draws random numbers; it holds none of the method's
arithmetic.  Both the HIP path and the fp64 oracle are fed the tensors it
returns (the oracle receives exact fp32 widenings of the stored values).

Recipe (one torch.Generator on the target device, seeded with the workload
seed; draws in this order):
  Q, K, V  ~ N(0, 1) drawn in fp32, then rounded to the storage dtype (bf16
             round-to-nearest-even; fp32 kept as drawn).  Layout BSHD:
             Q [B, Sq, Hq, D], K and V [B, Sk, Hkv, D], contiguous.
  Delta    ~ N(0, delta_std^2), fp32, shape [Hkv*D, Hkv] (row c = flattened
             (kv head, channel) index h*D + d of a value row, column = head).
  A        ~ U(0.5, 1.5), fp32, shape [Hkv].
K and V are drawn one batch slab at a time so that peak fp32 scratch stays
at one slab even for the 32K-token cache of the decode workload.
The backward's upstream gradient (make_grad) comes from a second generator
seeded with seed + 7919: dO ~ N(0, 1) in fp32, rounded to the storage dtype,
shape [B, Sq, Hq, D].
"""
import torch

from .configs import Workload

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _randn_slabs(g, shape, dtype, device):
    out = torch.empty(shape, dtype=dtype, device=device)
    for b in range(shape[0]):
        out[b].copy_(torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32))
    return out


def make_inputs(wl: Workload, device="cpu", seed=None):
    """Return dict(Q, K, V, Delta, A) for workload ``wl`` on ``device``."""
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed if seed is None else seed)
    dt = _DT[wl.dtype]
    Q = _randn_slabs(g, (wl.B, wl.Sq, wl.Hq, wl.D), dt, device)
    K = _randn_slabs(g, (wl.B, wl.Sk, wl.Hkv, wl.D), dt, device)
    V = _randn_slabs(g, (wl.B, wl.Sk, wl.Hkv, wl.D), dt, device)
    Delta = torch.randn(wl.Hkv * wl.D, wl.Hkv, generator=g, device=device,
                        dtype=torch.float32) * wl.delta_std
    A = torch.rand(wl.Hkv, generator=g, device=device, dtype=torch.float32) + 0.5
    return dict(Q=Q, K=K, V=V, Delta=Delta, A=A)


def make_small(B, Hq, Hkv, Sq, Sk, D, w, dtype="bf16", q_offset=0, delta_std=0.02,
               seed=0, device="cpu"):
    """Inputs for an ad-hoc shape (tests of ragged tiles and edge cases)."""
    wl = Workload("adhoc", dtype, B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, q_offset=q_offset,
                  D=D, w=w, delta_std=delta_std, seed=seed)
    return wl, make_inputs(wl, device=device)


def make_grad(wl: Workload, device="cpu", seed=None):
    """Upstream gradient dO [B, Sq, Hq, D] for workload ``wl``."""
    g = torch.Generator(device=device)
    g.manual_seed((wl.seed if seed is None else seed) + 7919)
    return _randn_slabs(g, (wl.B, wl.Sq, wl.Hq, wl.D), _DT[wl.dtype], device)
