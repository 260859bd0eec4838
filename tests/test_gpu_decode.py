"""GPU one-row (decode) attention against the fp64 oracle, through the C ABI:
one query per sequence at position Sk-1 keeps the w best keys of the cache."""
import numpy as np
import pytest
import torch

import oracle
import trainable_dynamic_mask_amd as dma
from trainable_dynamic_mask_amd.configs import WORKLOADS
from trainable_dynamic_mask_amd.inputs import make_inputs, make_small
from tests.dma_check import compare_rows, to64

pytestmark = pytest.mark.gpu


def _decode(x, wl):
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, 1, wl.q_offset, wl.w)
    O, lse = dma.attn_fwd(x["Q"], x["K"], x["V"], d, gm, return_lse=True)
    torch.cuda.synchronize()
    return d, gm, O, lse


@pytest.mark.parametrize("B,Hq,Hkv,Sk,w,dtype,D", [
    (2, 8, 2, 300, 37, "bf16", 128), (3, 4, 4, 1000, 1000, "bf16", 128),
    (1, 16, 2, 5000, 700, "bf16", 128), (2, 4, 2, 600, 257, "f32", 64),
    (1, 8, 8, 100, 1, "bf16", 64), (1, 2, 1, 1, 5, "f32", 128),
    (1, 8, 2, 50000, 2048, "bf16", 128)])  # a cache past 32768 keys
def test_decode_small(gpu_lib, B, Hq, Hkv, Sk, w, dtype, D):
    wl, x = make_small(B, Hq, Hkv, 1, Sk, D, w, dtype=dtype, q_offset=Sk - 1, seed=Sk + w,
                       device="cuda")
    d, gm, O, lse = _decode(x, wl)
    rows = np.array([(b, hq, 0) for b in range(B) for hq in range(Hq)], np.int64)
    Or, Lr = oracle.attn_rows(x["Q"], x["K"], x["V"], to64(d), wl.q_offset, w, rows)
    compare_rows(O, lse, Or, Lr, rows, dtype, "decode small")


@pytest.mark.parametrize("Sk,w", [(5000, 700), (40000, 2048)])
def test_decode_kept_delta_copy(gpu_lib, Sk, w):
    # the attention reads the mask's copy of delta at the listed keys; without
    # the copy it gathers delta itself: the outputs must be bit-identical
    wl, x = make_small(2, 8, 2, 1, Sk, 128, w, dtype="bf16", q_offset=Sk - 1, seed=Sk,
                       device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, 1, wl.q_offset, w)
    O1, L1 = dma.attn_fwd(x["Q"], x["K"], x["V"], d, gm, return_lse=True)
    gm.u_dval = None
    O2, L2 = dma.attn_fwd(x["Q"], x["K"], x["V"], d, gm, return_lse=True)
    assert torch.equal(O1, O2) and torch.equal(L1, L2)


def test_decode_equals_last_prefill_row(gpu_lib):
    # the same sequence as a 4096-row prefill: its last row must match decode
    wl, x = make_small(1, 8, 2, 4096, 4096, 128, 512, dtype="bf16", seed=9, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    Op = dma.attn_fwd(x["Q"], x["K"], x["V"], d, dma.topk_mask(d, 4096, 0, 512))
    Od = dma.attn_fwd(x["Q"][:, -1:], x["K"], x["V"], d, dma.topk_mask(d, 1, 4095, 512))
    err = (Op[:, -1:].float() - Od.float()).abs().max().item()
    assert err <= 2e-2


def test_decode_workload_every_row(gpu_lib):
    # all 2048 (batch, query head) rows of the decode workload
    wl = WORKLOADS["decode_32k"]
    print("decode_32k: every row", flush=True)
    x = make_inputs(wl, device="cuda")
    d, gm, O, lse = _decode(x, wl)
    rows = np.array([(b, hq, 0) for b in range(wl.B) for hq in range(wl.Hq)], np.int64)
    # the oracle reads one batch slab at a time (the whole cache is 8 GiB in fp32)
    Or = np.empty((len(rows), wl.D))
    Lr = np.empty(len(rows))
    d64 = to64(d)
    for b in range(wl.B):
        sel = rows[:, 0] == b
        sub = rows[sel].copy()
        sub[:, 0] = 0
        o, l = oracle.attn_rows(x["Q"][b:b + 1], x["K"][b:b + 1], x["V"][b:b + 1],
                                d64[b:b + 1], wl.q_offset, wl.w, sub)
        Or[sel], Lr[sel] = o, l
    m, r = compare_rows(O, lse, Or, Lr, rows, "bf16", "decode_32k")
    print(f"decode_32k: {len(rows)} rows (all), max abs {m:.2e} rel L2 {r:.2e}")
