"""GPU decode steps of the one-row keep set (Hugging Face blog "Trainable
Dynamic Mask Sparse Attention", section "Mask Combination with Causal
Constraints"), through the C ABI: after every appended key the lists must be
bit-identical to a fresh one-row selection over the grown sequence, and
equal to the fp64 oracle's keep set of that row."""
import numpy as np
import pytest
import torch

import oracle
import trainable_dynamic_mask_amd as dma
from tests.dma_check import to64

pytestmark = pytest.mark.gpu


def _lists(m, w):
    BH = m.B * m.Hkv
    cnt = m.u_cnt[:BH].cpu().numpy()
    idx = m.u_idx[:BH * w].view(BH, w).cpu().numpy()
    dval = m.u_dval[:BH * w].view(BH, w).cpu().numpy().view(np.uint32)  # bits: -0 != +0 here
    return cnt, idx, m.u_nfull[:BH].cpu().numpy(), m.u_dmax[:BH].cpu().numpy(), dval


def _delta(kind, B, Hkv, S, seed):
    g = torch.Generator(device="cpu").manual_seed(seed)
    if kind == "random":
        d = torch.rand(B, Hkv, S, generator=g) * 10 + 1
    elif kind == "ties":         # three values only: the lower index must win every tie
        d = torch.randint(1, 4, (B, Hkv, S), generator=g).float()
    elif kind == "signed_zeros":  # -0 and +0 tie: a new +0 never displaces a kept -0
        vals = torch.tensor([-0.0, 0.0, -0.0, 0.0, -1.0, 1.0])
        d = vals[torch.randint(0, 6, (B, Hkv, S), generator=g)]
    elif kind == "rising":       # every new key beats every kept key
        d = torch.arange(S, dtype=torch.float32).repeat(B, Hkv, 1) + 1
    else:                        # falling: no new key ever enters
        d = torch.arange(S, 0, -1, dtype=torch.float32).repeat(B, Hkv, 1)
    return d.cuda()


@pytest.mark.parametrize("kind,B,Hkv,w,steps", [
    ("random", 2, 4, 256, 150), ("random", 1, 3, 1, 60), ("random", 2, 2, 7, 80),
    ("ties", 2, 4, 33, 120), ("ties", 1, 2, 1, 40), ("signed_zeros", 2, 2, 1, 60),
    ("signed_zeros", 2, 2, 2, 60), ("rising", 1, 2, 16, 30),
    ("falling", 1, 2, 16, 30)])
def test_append_matches_selection(gpu_lib, kind, B, Hkv, w, steps):
    S0 = w + 1
    full = _delta(kind, B, Hkv, S0 + steps, seed=w + steps)
    print(f"append {kind} B={B} Hkv={Hkv} w={w} steps={steps}", flush=True)
    m = dma.topk_mask(full[:, :, :S0].contiguous(), 1, S0 - 1, w, kt_lists=False)
    for Sk in range(S0 + 1, S0 + steps + 1):
        d = full[:, :, :Sk].contiguous()
        dma.decode_keep_append(d, m)
        ref = dma.topk_mask(d, 1, Sk - 1, w, kt_lists=False)
        got, want = _lists(m, w), _lists(ref, w)
        for a, b, name in zip(got, want, ("u_cnt", "u_idx", "u_nfull", "u_dmax", "u_dval")):
            assert np.array_equal(a, b), f"{name} differs after key {Sk - 1}"
        if Sk in (S0 + 1, S0 + steps):
            dd = to64(d)
            for bh in range(B * Hkv):
                keep = oracle.keep_row(dd.reshape(B * Hkv, Sk)[bh], Sk - 1, w)
                assert np.array_equal(got[1][bh], keep)


def test_append_decode_size(gpu_lib):
    # 64 steps at the decode workload's size: w = 2048 over ~30K keys, 32 sequences
    B, Hkv, w, S0, steps = 4, 8, 2048, 30000, 64
    full = _delta("random", B, Hkv, S0 + steps, seed=5)
    print("append decode size", flush=True)
    m = dma.topk_mask(full[:, :, :S0].contiguous(), 1, S0 - 1, w, kt_lists=False)
    for Sk in range(S0 + 1, S0 + steps + 1):
        dma.decode_keep_append(full[:, :, :Sk].contiguous(), m)
    ref = dma.topk_mask(full.contiguous(), 1, S0 + steps - 1, w, kt_lists=False)
    for a, b in zip(_lists(m, w), _lists(ref, w)):
        assert np.array_equal(a, b)


def test_append_then_attention(gpu_lib):
    # the appended lists drive the one-row attention exactly like selected ones
    B, Hq, Hkv, D, w, S0, steps = 2, 8, 2, 128, 64, 200, 20
    g = torch.Generator(device="cpu").manual_seed(3)
    S = S0 + steps
    Q = torch.randn(B, 1, Hq, D, generator=g).bfloat16().cuda()
    K = torch.randn(B, S, Hkv, D, generator=g).bfloat16().cuda()
    V = torch.randn(B, S, Hkv, D, generator=g).bfloat16().cuda()
    full = _delta("random", B, Hkv, S, seed=4)
    m = dma.topk_mask(full[:, :, :S0].contiguous(), 1, S0 - 1, w, kt_lists=False)
    for Sk in range(S0 + 1, S + 1):
        dma.decode_keep_append(full[:, :, :Sk].contiguous(), m)
    ref = dma.topk_mask(full, 1, S - 1, w, kt_lists=False)
    O1 = dma.attn_fwd(Q, K, V, full, m)
    O2 = dma.attn_fwd(Q, K, V, full, ref)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2)
