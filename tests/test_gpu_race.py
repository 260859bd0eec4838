"""Cross-check of the hand-synchronised prefill attention (through the C ABI).

The bf16 prefill kernel gathers K/V rows and key metadata straight into LDS
with direct loads the compiler does not track, and waits for each batch with
a hand-counted vmcnt at a later phase barrier.  libdma_hip_safe.so is the
same source built with DMA_SAFE_SYNC, where every barrier waits for all
loads in flight.  Any read of LDS before its data landed would make the two
differ, so their outputs must be bit-identical (O and the log-sum-exp, both
forwards).  The backward's dq kernel (four query heads per workgroup) runs
the same ping-pong with loads in flight across a barrier; its gradients are
compared the same way.
"""
import pytest
import torch

import trainable_dynamic_mask_amd as dma
from trainable_dynamic_mask_amd import _lib
from trainable_dynamic_mask_amd.configs import WORKLOADS
from trainable_dynamic_mask_amd.inputs import make_inputs, make_small

pytestmark = pytest.mark.gpu


def _both(x, d, gm, return_lse):
    safe = _lib.load_safe()
    fast = dma.attn_fwd(x["Q"], x["K"], x["V"], d, gm, return_lse=return_lse)
    slow = dma.attn_fwd(x["Q"], x["K"], x["V"], d, gm, return_lse=return_lse, lib=safe)
    torch.cuda.synchronize()
    return fast, slow


def _equal(a, b, what):
    if isinstance(a, tuple):
        for u, v, n in zip(a, b, ("O", "lse")):
            _equal(u, v, f"{what} {n}")
        return
    diff = (a.float() != b.float()).sum().item()
    assert diff == 0, f"{what}: {diff} elements differ between the fast and safe builds"


@pytest.mark.parametrize("name,q_rows", [("prefill_16k", None), ("prefill_64k", 4096)])
def test_fast_and_safe_sync_agree_bitwise(gpu_lib, name, q_rows):
    wl = WORKLOADS[name]
    print(f"race cross-check {name} rows {q_rows or wl.Sq}", flush=True)
    x = make_inputs(wl, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    if q_rows is None:
        gm = dma.topk_mask(d, wl.Sq, wl.q_offset, wl.w)
    else:
        # the last q_rows rows of the sequence: full-length lists (w keys)
        q0 = wl.Sk - q_rows
        x["Q"] = x["Q"][:, q0:].contiguous()
        gm = dma.topk_mask(d, q_rows, q0, wl.w)
    for lse in (False, True):
        fast, slow = _both(x, d, gm, lse)
        _equal(fast, slow, f"{name} (lse={lse})")


@pytest.mark.parametrize("B,Hq,Hkv,S,w", [(2, 8, 2, 1000, 100), (1, 16, 2, 777, 300),
                                          (1, 4, 4, 200, 1)])
def test_fast_and_safe_sync_agree_small(gpu_lib, B, Hq, Hkv, S, w):
    # ragged tiles, G = 4, 8 and 1 (head groups of 4, 2 and 1 per workgroup)
    wl, x = make_small(B, Hq, Hkv, S, S, 128, w, dtype="bf16", delta_std=0.05, seed=S,
                       device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, S, 0, w)
    for lse in (False, True):
        fast, slow = _both(x, d, gm, lse)
        _equal(fast, slow, f"{(B, Hq, Hkv, S, w)} (lse={lse})")


@pytest.mark.parametrize("name,shape", [("prefill_16k", None),
                                        ("adhoc", (1, 8, 2, 700, 300, 150))])
def test_backward_fast_and_safe_sync_agree_bitwise(gpu_lib, name, shape):
    from trainable_dynamic_mask_amd.inputs import make_grad
    if shape is None:
        wl = WORKLOADS[name]
        x = make_inputs(wl, device="cuda")
    else:
        B, Hq, Hkv, S, w, q0 = shape
        wl, x = make_small(B, Hq, Hkv, S - q0, S, 128, w, dtype="bf16", q_offset=q0,
                           seed=41, device="cuda")
    print(f"backward race cross-check {name} Sq {wl.Sq}", flush=True)
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, wl.Sq, wl.q_offset, wl.w)
    O, lse, Ores = dma.attn_fwd_train(x["Q"], x["K"], x["V"], d, gm)
    dO = make_grad(wl, device="cuda")
    fast = dma.attn_bwd(x["Q"], x["K"], x["V"], d, gm, O, lse, dO, O_res=Ores)
    slow = dma.attn_bwd(x["Q"], x["K"], x["V"], d, gm, O, lse, dO, O_res=Ores,
                        lib=_lib.load_safe())
    torch.cuda.synchronize()
    for u, v, n in zip(fast, slow, ("dQ", "dK", "dV", "ddelta")):
        _equal(u, v, f"{name} backward {n}")
