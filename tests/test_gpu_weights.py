"""GPU parity of the dynamic weights (Hugging Face blog "Trainable Dynamic
Mask Sparse Attention", section "Dynamic Sparse Mask Generation") against
the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import trainable_dynamic_mask_amd as dma
from trainable_dynamic_mask_amd.configs import WORKLOADS
from trainable_dynamic_mask_amd.inputs import make_inputs, make_small
from tests.dma_check import delta_tol, to64

pytestmark = pytest.mark.gpu


def _rel_err(got, want):
    return float(np.max(np.abs(got - want) / np.abs(want)))


@pytest.mark.parametrize("name", ["tiny_f32", "prefill_4k", "prefill_16k", "prefill_64k"])
def test_weights_workloads(gpu_lib, name):
    wl = WORKLOADS[name]
    x = make_inputs(wl, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    torch.cuda.synchronize()
    want = oracle.weights(x["V"], x["Delta"], x["A"])
    err = _rel_err(to64(d), want)
    print(f"{name}: delta max rel err {err:.2e}")
    assert err <= delta_tol(wl.dtype)


def test_weights_decode_cache_sampled(gpu_lib):
    wl = WORKLOADS["decode_32k"]
    x = make_inputs(wl, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    torch.cuda.synchronize()
    for b in (0, 31, 63):
        want = oracle.weights(x["V"][b:b + 1], x["Delta"], x["A"])
        assert _rel_err(to64(d[b:b + 1]), want) <= delta_tol(wl.dtype)


@pytest.mark.parametrize("Hkv,D,dtype", [(1, 64, "f32"), (3, 64, "bf16"), (5, 128, "bf16"),
                                         (16, 128, "bf16"), (8, 64, "f32")])
def test_weights_shapes_and_ragged_rows(gpu_lib, Hkv, D, dtype):
    wl, x = make_small(B=2, Hq=Hkv, Hkv=Hkv, Sq=77, Sk=77, D=D, w=5, dtype=dtype,
                       delta_std=0.05, seed=Hkv * D, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    want = oracle.weights(x["V"], x["Delta"], x["A"])
    assert _rel_err(to64(d), want) <= delta_tol(dtype)


def test_weights_zero_projection_is_two_to_the_a(gpu_lib):
    wl, x = make_small(B=1, Hq=8, Hkv=8, Sq=100, Sk=100, D=128, w=5, device="cuda")
    d = dma.weights(x["V"], torch.zeros_like(x["Delta"]), x["A"])
    want = torch.pow(2.0, x["A"].double()).cpu().numpy()
    np.testing.assert_allclose(to64(d), np.broadcast_to(want[None, :, None], d.shape), rtol=1e-6)


def test_weights_strided_value_rows(gpu_lib):
    # V as a slice of a wider per-token buffer (row stride > Hkv*D)
    wl, x = make_small(B=2, Hq=4, Hkv=4, Sq=64, Sk=64, D=64, w=5, device="cuda")
    big = torch.zeros(2, 64, 6, 64, dtype=torch.bfloat16, device="cuda")
    big[:, :, 1:5] = x["V"]
    Vs = big[:, :, 1:5]
    d = dma.weights(Vs, x["Delta"], x["A"])
    want = oracle.weights(x["V"], x["Delta"], x["A"])
    assert _rel_err(to64(d), want) <= 3e-5


def test_weights_empty(gpu_lib):
    V = torch.empty(0, 10, 2, 64, dtype=torch.bfloat16, device="cuda")
    d = dma.weights(V, torch.zeros(128, 2, device="cuda"), torch.ones(2, device="cuda"))
    assert d.shape == (0, 2, 10)
