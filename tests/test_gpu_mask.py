"""GPU keep masks and block-skip lists (Hugging Face blog "Trainable Dynamic
Mask Sparse Attention", section "Mask Combination with Causal Constraints")
against the oracle's literal per-row top-w sets, bit-exact on a shared delta,
through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import trainable_dynamic_mask_amd as dma
from trainable_dynamic_mask_amd.configs import WORKLOADS
from trainable_dynamic_mask_amd.inputs import make_inputs
from tests.dma_check import check_mask, to64

pytestmark = pytest.mark.gpu


def _delta(kind, B, H, S, seed):
    g = torch.Generator().manual_seed(seed)
    if kind == "ties":       # few distinct values: exact ties everywhere
        d = torch.randint(0, 5, (B, H, S), generator=g).float() + 1.0
    elif kind == "allequal":
        d = torch.full((B, H, S), 2.0)
    elif kind == "increasing":  # newest key always best: a sliding window
        d = torch.arange(S, dtype=torch.float32).expand(B, H, S).contiguous() + 1.0
    elif kind == "decreasing":  # oldest keys always best: the first w keys
        d = (S - torch.arange(S, dtype=torch.float32)).expand(B, H, S).contiguous()
    elif kind == "signed_zeros":  # -0 and +0 are equal: they tie, the lower index wins
        vals = torch.tensor([-0.0, 0.0, -0.0, 0.0, -1.0, 1.0])
        d = vals[torch.randint(0, 6, (B, H, S), generator=g)]
    elif kind == "periodic":  # depends on j mod 512 only: a spaced sample sees few values
        d = ((torch.arange(S) * 37) % 512 + 1).float().expand(B, H, S).contiguous()
    elif kind == "clusters":  # two far-apart groups with a spread inside each
        hi = torch.rand(B, H, S, generator=g) < 0.5
        d = torch.exp(torch.randn(B, H, S, generator=g)) * torch.where(hi, 1e3, 1e-3)
    elif kind == "narrow":  # every weight within a few hundred ulps of 1
        d = 1.0 + torch.randint(0, 300, (B, H, S), generator=g).float() * 2.0 ** -23
    elif kind == "negative":  # all below zero, some -inf
        d = -torch.exp(torch.randn(B, H, S, generator=g))
        d[torch.rand(B, H, S, generator=g) < 0.01] = float("-inf")
    else:
        d = torch.exp(torch.randn(B, H, S, generator=g))
    return d.cuda()


@pytest.mark.parametrize("kind", ["random", "ties", "allequal", "increasing", "decreasing"])
@pytest.mark.parametrize("S,w", [(1, 1), (2, 1), (63, 5), (64, 64), (65, 7), (200, 37),
                                 (300, 300), (333, 1000), (1000, 130)])
def test_mask_small(gpu_lib, kind, S, w):
    d = _delta(kind, 2, 3, S, seed=S * 7 + w)
    gm = dma.topk_mask(d, S, 0, w)
    torch.cuda.synchronize()
    check_mask(gm, d)


@pytest.mark.parametrize("S,w", [(2, 1), (9, 1), (9, 2), (300, 1), (300, 2), (5000, 1),
                                 (5000, 2), (20000, 2)])
def test_mask_signed_zeros(gpu_lib, S, w):
    # mixed -0 / +0 weights: the order code must treat them as one value
    d = _delta("signed_zeros", 2, 2, S, seed=S + w)
    assert torch.signbit(d[d == 0]).any() and (~torch.signbit(d[d == 0])).any()
    gm = dma.topk_mask(d, S, 0, w)
    check_mask(gm, d)


@pytest.mark.parametrize("p,w", [(1, 1), (7, 2), (100, 1), (100, 2), (32767, 1), (32767, 2)])
def test_decode_select_signed_zeros(gpu_lib, p, w):
    d = _delta("signed_zeros", 3, 2, p + 1, seed=p * 3 + w)
    gm = dma.topk_mask(d, 1, p, w)
    check_mask(gm, d)


@pytest.mark.parametrize("S,w", [(4097, 100), (8192, 3000), (12345, 2048), (9000, 6000),
                                 (12000, 9000), (20000, 9500), (16385, 700)])
def test_mask_multi_chunk_sort(gpu_lib, S, w):
    # up to 16384 keys: 1024-key sort chunks ranked by binary searches (ties
    # resolved by index); beyond: 4096-key chunks and merge passes (16385,
    # 20000); w = 9000 and 9500 give tile groups with more candidates than
    # the LDS of the one-kernel list path holds, so they take the two-kernel
    # path
    d = _delta("ties", 1, 2, S, seed=S)
    gm = dma.topk_mask(d, S, 0, w)
    check_mask(gm, d)


@pytest.mark.parametrize("q0,Sq,Sk,w", [(10, 50, 60, 7), (100, 130, 300, 40), (0, 70, 200, 9),
                                        (4000, 200, 4200, 512)])
def test_mask_query_offset(gpu_lib, q0, Sq, Sk, w):
    d = _delta("ties", 1, 2, Sk, seed=q0 + Sq)
    gm = dma.topk_mask(d, Sq, q0, w)
    check_mask(gm, d)


@pytest.mark.parametrize("name", ["tiny_f32", "prefill_4k", "prefill_16k", "prefill_64k",
                                  "chunk_16k"])
def test_mask_workloads(gpu_lib, name):
    wl = WORKLOADS[name]
    x = make_inputs(wl, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, wl.Sq, wl.q_offset, wl.w)
    torch.cuda.synchronize()
    check_mask(gm, d)


def test_mask_deterministic(gpu_lib):
    d = _delta("ties", 2, 4, 9000, seed=3)
    a = dma.topk_mask(d, 9000, 0, 700)
    b = dma.topk_mask(d, 9000, 0, 700)
    for f in ("evict", "u_cnt", "u_nfull", "u_dmax", "kt_cnt"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    # list entries past each tile's count are never written: compare the counted ones
    nt = a.dims["n_tiles_total"]
    for f, cnt, stride in (("u_idx", a.u_cnt, a.dims["u_stride"]),
                           ("kt_idx", a.kt_cnt, a.dims["kt_stride"])):
        ta = getattr(a, f)[: nt * stride].view(nt, stride).cpu()
        tb = getattr(b, f)[: nt * stride].view(nt, stride).cpu()
        for g, c in enumerate(cnt.cpu().tolist()):
            assert torch.equal(ta[g, :c], tb[g, :c]), (f, g)


@pytest.mark.parametrize("kind", ["random", "ties", "allequal"])
@pytest.mark.parametrize("p,w", [(0, 1), (5, 10), (4095, 2048), (32767, 2048), (20000, 1)])
def test_decode_select(gpu_lib, kind, p, w):
    Sk = p + 1 + 3  # cache longer than the row's prefix
    d = _delta(kind, 3, 2, Sk, seed=p + w)
    gm = dma.topk_mask(d, 1, p, w)
    torch.cuda.synchronize()
    check_mask(gm, d)


@pytest.mark.parametrize("kind", ["random", "increasing", "decreasing", "periodic", "clusters",
                                  "narrow", "negative", "ties"])
@pytest.mark.parametrize("p,w", [(300, 100), (1000, 999), (8191, 2048), (25000, 3000),
                                 (32767, 1), (32767, 2048), (32767, 16384), (32767, 31000)])
def test_decode_select_bracket(gpu_lib, kind, p, w):
    # rows of at most 32768 keys: the sampled bracket with radix passes, and
    # the full bit search when the bracket misses (structured rows, ties,
    # half the row kept)
    Sk = p + 1 + 2
    d = _delta(kind, 2, 2, Sk, seed=p * 5 + w)
    gm = dma.topk_mask(d, 1, p, w)
    torch.cuda.synchronize()
    check_mask(gm, d)


@pytest.mark.parametrize("kind", ["random", "ties", "allequal", "signed_zeros"])
@pytest.mark.parametrize("p,w", [(32768, 2048), (40000, 1), (40000, 5000), (70000, 2048),
                                 (131071, 40000)])
def test_decode_select_long_rows(gpu_lib, kind, p, w):
    # rows past 32768 keys take the radix-pass selection; ties and equal
    # weights exercise its equal-code handling, the last case a list larger
    # than one key tile per thread
    Sk = p + 1 + 5
    d = _delta(kind, 2, 2, Sk, seed=p + w)
    gm = dma.topk_mask(d, 1, p, w)
    torch.cuda.synchronize()
    check_mask(gm, d)


def test_decode_workload(gpu_lib):
    wl = WORKLOADS["decode_32k"]
    x = make_inputs(wl, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    gm = dma.topk_mask(d, 1, wl.q_offset, wl.w)
    torch.cuda.synchronize()
    u = gm.u_idx.cpu().numpy().reshape(wl.B, wl.Hkv, -1)
    cnt = gm.u_cnt.cpu().numpy().reshape(wl.B, wl.Hkv)
    d64 = to64(d)
    assert (cnt == wl.w).all()
    for b in range(wl.B):
        for h in range(wl.Hkv):
            np.testing.assert_array_equal(u[b, h, : cnt[b, h]],
                                          oracle.keep_row(d64[b, h], wl.q_offset, wl.w))


def test_mask_empty(gpu_lib):
    d = torch.ones(0, 2, 10, device="cuda")
    gm = dma.topk_mask(d, 10, 0, 3)
    assert gm.dims["n_tiles_total"] == 0
    d = torch.ones(1, 2, 10, device="cuda")
    gm = dma.topk_mask(d, 0, 10, 3)
    assert gm.dims["n_tiles_total"] == 0
