"""GPU backward of the dynamic weights (Hugging Face blog "Trainable Dynamic
Mask Sparse Attention", section "Dynamic Sparse Mask Generation", delta
equation with softplus) against the fp64 oracle, through the C ABI.

The pre-activation is recomputed with exact products (three-way bf16 split
of Delta) and fp32 sums, and the reductions over keys run in fp32, so the
gradients match the oracle to fp32 accumulation error: max abs error <= 1e-4
of the largest reference entry."""
import numpy as np
import pytest
import torch

import oracle
import trainable_dynamic_mask_amd as dma
from trainable_dynamic_mask_amd.inputs import make_small
from tests.dma_check import to64

pytestmark = pytest.mark.gpu


def _close(got, want, name, tol=1e-4):
    got = to64(got)
    scale = max(np.abs(want).max(), 1e-30)
    err = np.abs(got - want).max() / scale
    print(f"{name}: max err / max ref {err:.2e}")
    assert err <= tol, name


@pytest.mark.parametrize("B,Sk,Hkv,D,std", [(2, 300, 8, 128, 0.02), (1, 77, 3, 64, 0.05),
                                            (1, 1000, 16, 128, 0.02), (1, 513, 8, 128, 0.05)])
def test_weights_bwd_matches_oracle(gpu_lib, B, Sk, Hkv, D, std):
    wl, x = make_small(B, Hkv, Hkv, Sk, Sk, D, 5, dtype="bf16", delta_std=std, seed=Sk + D,
                       device="cuda")
    g = torch.Generator(device="cuda").manual_seed(Sk)
    gd = torch.randn(B, Hkv, Sk, generator=g, device="cuda")
    dV0 = torch.randn(B, Sk, Hkv, D, generator=g, device="cuda")
    print(f"weights bwd B={B} Sk={Sk} Hkv={Hkv} D={D}", flush=True)
    dV, dDelta, dA = dma.weights_bwd(x["V"], x["Delta"], x["A"], gd, dV=dV0.clone())
    torch.cuda.synchronize()
    wV, wD, wA = oracle.weights_bwd(x["V"], x["Delta"], x["A"], to64(gd))
    _close(dV - dV0, wV, "dV")
    _close(dDelta, wD, "dDelta")
    _close(dA, wA, "dA")


def test_weights_bwd_chain_from_attention(gpu_lib):
    # ddelta of the attention backward feeds the weights backward; the total dV is
    # the attention's plus the weights' (the value matrix feeds both)
    from trainable_dynamic_mask_amd.inputs import make_grad
    wl, x = make_small(1, 4, 2, 400, 400, 128, 50, dtype="bf16", seed=21, device="cuda")
    dO = make_grad(wl, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    m = dma.topk_mask(d, 400, 0, 50)
    O, lse, Ores = dma.attn_fwd_train(x["Q"], x["K"], x["V"], d, m)
    dQ, dK, dVa, dd = dma.attn_bwd(x["Q"], x["K"], x["V"], d, m, O, lse, dO, O_res=Ores)
    dV, dDelta, dA = dma.weights_bwd(x["V"], x["Delta"], x["A"], dd, dV=dVa.clone())
    torch.cuda.synchronize()
    _, _, wVa, wdd = oracle.attn_bwd(x["Q"], x["K"], x["V"], to64(d), dO, 0, 50)
    wVw, wD, wA = oracle.weights_bwd(x["V"], x["Delta"], x["A"], wdd)
    _close(dV, wVa + wVw, "dV total", tol=3e-2)
    _close(dDelta, wD, "dDelta", tol=3e-2)
    # dA[h] = sum_j ddelta_j * delta_j * softplus(pre_j), and ddelta sums to zero per
    # head, so dA is a small sum of cancelling terms: its error is bounded against
    # the sum of the terms' magnitudes, not against dA itself
    dl = oracle.weights(x["V"], x["Delta"], x["A"])                  # [1, Hkv, Sk]
    sp = np.log(dl) / to64(x["A"])[None, :, None]
    mag = np.abs(wdd * dl * sp).sum(axis=(0, 2))
    err = np.abs(to64(dA) - wA)
    print(f"dA: max err / sum |terms| {np.max(err / mag):.2e}")
    assert np.all(err <= 1e-2 * mag)
