"""GPU value projection with the dynamic weights in its epilogue (Hugging
Face blog "Trainable Dynamic Mask Sparse Attention", section "Dynamic Sparse
Mask Generation": delta computed from the value matrix) against the fp64
oracle, through the C ABI.

V = X Wv is checked against the oracle's fp64 product within the bound of
fp32 sums and one bf16 rounding; delta against the oracle's weights of the V
the kernel stored (the fused call's definition); and the fused call against
the projection alone followed by the separate weights call."""
import numpy as np
import pytest
import torch

import oracle
import trainable_dynamic_mask_amd as dma
from tests.dma_check import delta_tol, to64

pytestmark = pytest.mark.gpu


def _inputs(B, Sk, Cin, Hkv, D, seed, x_pad=0):
    g = torch.Generator().manual_seed(seed)
    X = torch.randn(B, Sk, Cin + x_pad, generator=g).to(torch.bfloat16)
    Wv = (torch.randn(Cin, Hkv * D, generator=g) / Cin ** 0.5).to(torch.bfloat16)
    Delta = torch.randn(Hkv * D, Hkv, generator=g) * 0.02
    A = torch.rand(Hkv, generator=g) + 0.5
    X = X.cuda()[:, :, :Cin]  # x_pad > 0: rows further apart than Cin
    return X, Wv.cuda(), Delta.cuda(), A.cuda()


def _check_v(V, X, Wv, rows=None):
    """|V - X Wv| within one bf16 rounding of the fp32 sum plus the fp32 sum's error."""
    Xr = X.reshape(-1, X.shape[-1])
    Vr = V.reshape(Xr.shape[0], -1)
    if rows is not None:
        Xr, Vr = Xr[rows], Vr[rows]
    want = oracle.vproj(Xr, Wv)
    Cin = Xr.shape[1]
    s = np.abs(to64(Xr)) @ np.abs(to64(Wv))   # sum of |products| per output
    e32 = Cin * 2.0 ** -24 * s
    bound = 2.0 ** -8 * (np.abs(want) + e32) + e32
    err = np.abs(to64(Vr) - want)
    assert (err <= bound).all(), f"V off by {float((err - bound).max()):.3e} over its bound"
    return float((err / (np.abs(want) + 1e-3)).max())


@pytest.mark.parametrize("B,Sk,Cin,Hkv,D,x_pad", [
    (1, 300, 128, 2, 128, 0),      # one column tile, a ragged row tile
    (2, 1000, 512, 8, 128, 0),     # four column tiles, rows across batches
    (3, 77, 64, 4, 64, 0),         # one K step
    (2, 513, 256, 8, 64, 64),      # rows of X further apart than Cin
    (1, 257, 192, 1, 256, 0)])     # a single head
def test_vproj_weights_small(gpu_lib, B, Sk, Cin, Hkv, D, x_pad):
    X, Wv, Delta, A = _inputs(B, Sk, Cin, Hkv, D, seed=Sk + Cin, x_pad=x_pad)
    print(f"vproj B={B} Sk={Sk} Cin={Cin} Hkv={Hkv} D={D}", flush=True)
    V, d = dma.vproj_weights(X, Wv, Hkv, Delta, A)
    torch.cuda.synchronize()
    rel = _check_v(V, X, Wv)
    want = oracle.weights(V, Delta, A)  # the weights of the stored values
    err = float(np.max(np.abs(to64(d) - want) / np.abs(want)))
    print(f"  V max rel {rel:.2e}  delta max rel {err:.2e}")
    assert err <= delta_tol("bf16")
    # the projection alone writes the same V; the separate weights call agrees
    V2 = dma.vproj_weights(X, Wv, Hkv)
    assert torch.equal(V, V2)
    if D in (64, 128):  # the head sizes dma_weights takes
        d2 = dma.weights(V, Delta, A)
        assert float(((d - d2).abs() / d2.abs()).max()) <= 1e-5


def test_vproj_weights_prefill_shape(gpu_lib):
    # the 16K prefill's value projection: hidden 4096 (32 heads x 128) to 8 kv
    # heads x 128; V on sampled rows (every row tile's first and last, and
    # random ones), delta on every key
    B, Sk, Cin, Hkv, D = 1, 16384, 4096, 8, 128
    X, Wv, Delta, A = _inputs(B, Sk, Cin, Hkv, D, seed=16)
    V, d = dma.vproj_weights(X, Wv, Hkv, Delta, A)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    rows = sorted(set(range(0, Sk, 256)) | set(range(255, Sk, 256)) |
                  set(rng.integers(0, Sk, 256).tolist()))
    _check_v(V, X, Wv, rows=np.array(rows))
    want = oracle.weights(V, Delta, A)
    err = float(np.max(np.abs(to64(d) - want) / np.abs(want)))
    print(f"prefill shape: delta max rel {err:.2e}")
    assert err <= delta_tol("bf16")
    V2 = dma.vproj_weights(X, Wv, Hkv)
    assert torch.equal(V, V2)
