"""GPU backward of the masked attention against the fp64 oracle, through the
C ABI (Hugging Face blog "Trainable Dynamic Mask Sparse Attention", section
"Efficient Sparse Attention Computation": gradients of sum(dO * O) with the
keep sets fixed).

The forward runs through dma_attn_fwd_train, whose O rounding residual lets
the backward form dO . O to ~2^-18 (bf16 O alone is not enough where the
attention is nearly one-hot, e.g. the 64K workload's delta range).
Tolerances: the backward rounds P and dS to bf16 for the MFMA products
(relative 2^-9 per operand), so each gradient is compared as a whole against
its largest entry: rel-L2 <= 1e-2 and max abs error <= 3e-2 of max
|reference|.  ddelta, summed in fp32 from fp32 dS, gets the same bar."""
import numpy as np
import pytest
import torch

import oracle
import trainable_dynamic_mask_amd as dma
from trainable_dynamic_mask_amd.inputs import make_grad, make_small
from tests.dma_check import ddelta_term_sizes, to64

pytestmark = pytest.mark.gpu


def _close(got, want, name):
    got = to64(got) if hasattr(got, "detach") else got
    scale = max(np.abs(want).max(), 1e-30)
    err = np.abs(got - want)
    rel_l2 = np.sqrt((err ** 2).sum() / max((want ** 2).sum(), 1e-300))
    print(f"{name}: max err / max ref {err.max() / scale:.2e}  rel-L2 {rel_l2:.2e}")
    assert err.max() <= 3e-2 * scale, name
    assert rel_l2 <= 1e-2, name


def _run(B, Hq, Hkv, Sq, Sk, w, q0=0, seed=0, delta_std=0.02, residual=True):
    wl, x = make_small(B, Hq, Hkv, Sq, Sk, 128, w, dtype="bf16", q_offset=q0, seed=seed,
                       delta_std=delta_std, device="cuda")
    dO = make_grad(wl, device="cuda")
    print(f"bwd B={B} Hq={Hq} Hkv={Hkv} Sq={Sq} Sk={Sk} w={w} q0={q0}", flush=True)
    d = dma.weights(x["V"], x["Delta"], x["A"])
    m = dma.topk_mask(d, Sq, q0, w)
    if residual:
        O, lse, Ores = dma.attn_fwd_train(x["Q"], x["K"], x["V"], d, m)
        # the training forward writes the same O as the forward asked for the
        # log-sum-exp (both round the logits as the backward recomputes them)
        O2, _ = dma.attn_fwd(x["Q"], x["K"], x["V"], d, m, return_lse=True)
        assert torch.equal(O, O2)
    else:
        O, lse = dma.attn_fwd(x["Q"], x["K"], x["V"], d, m, return_lse=True)
        Ores = None
    dQ, dK, dV, dd = dma.attn_bwd(x["Q"], x["K"], x["V"], d, m, O, lse, dO, O_res=Ores)
    torch.cuda.synchronize()
    want = oracle.attn_bwd(x["Q"], x["K"], x["V"], to64(d), dO, q0, w)
    return (dQ, dK, dV, dd), want


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,w,q0", [
    (1, 4, 1, 300, 300, 37, 0),       # ragged tiles, G = 4
    (2, 8, 2, 1000, 1000, 200, 0),    # two groups of 512 rows, ragged
    (1, 4, 2, 600, 600, 600, 0),      # w >= S: every causal key
    (1, 6, 2, 200, 777, 150, 500),    # chunked prefill, G = 3
    (1, 2, 2, 1100, 1100, 700, 0),    # G = 1, keys kept across three groups
])
def test_bwd_matches_oracle(gpu_lib, B, Hq, Hkv, Sq, Sk, w, q0):
    got, want = _run(B, Hq, Hkv, Sq, Sk, w, q0, seed=Sq + w)
    for g, r, name in zip(got, want, ("dQ", "dK", "dV", "ddelta")):
        _close(g, r, name)


def test_bwd_heavy_tailed_delta(gpu_lib):
    # the 64K workload's delta range (pre-activation std ~1.6, delta up to ~2e4):
    # P is formed from delta - lse, never from their raw sum
    got, want = _run(1, 4, 2, 700, 700, 100, seed=3, delta_std=0.1)
    for g, r, name in zip(got, want, ("dQ", "dK", "dV", "ddelta")):
        _close(g, r, name)


def test_bwd_heavy_tail_chunked(gpu_lib):
    # delta std 0.05 (delta up to ~2e3) in a chunked prefill: fp32 logits of that
    # size carry absolute errors ~ulp(delta)*log2(e), i.e. weights with relative
    # errors ~1e-4, and rows that do not see the tile's largest delta are not
    # shifted exactly.  dQ, dK and dV stay within the usual bounds; the delta
    # gradient sums terms up to ~1e3 times larger than itself (nearly one-hot
    # rows), so each key's error is bounded relative to the size of its terms
    # (twice the bf16 rounding of the forward's weights, which reaches dL/ddelta
    # through D = dO . O).
    B, Hq, Hkv, Sq, Sk, q0, w = 2, 9, 3, 229, 773, 544, 344
    wl, x = make_small(B, Hq, Hkv, Sq, Sk, 128, w, dtype="bf16", q_offset=q0, seed=76114265,
                       delta_std=0.05, device="cuda")
    dO = make_grad(wl, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    m = dma.topk_mask(d, Sq, q0, w)
    O, lse, Ores = dma.attn_fwd_train(x["Q"], x["K"], x["V"], d, m)
    got = dma.attn_bwd(x["Q"], x["K"], x["V"], d, m, O, lse, dO, O_res=Ores)
    torch.cuda.synchronize()
    d64 = to64(d)
    want = oracle.attn_bwd(x["Q"], x["K"], x["V"], d64, dO, q0, w)
    for g, r, name in zip(got[:3], want[:3], ("dQ", "dK", "dV")):
        _close(g, r, name)
    T = ddelta_term_sizes(x["Q"], x["K"], x["V"], d64, dO, q0, w)
    err = np.abs(to64(got[3]) - want[3])
    ratio = err / np.maximum(T, 1e-30)
    print(f"ddelta: error / term size max {ratio.max():.2e}, median {np.median(ratio[T > 0]):.2e}")
    assert (err <= 4e-3 * T + 1e-6).all()


def test_bwd_w1_only_dv(gpu_lib):
    # w = 1: each row keeps one key with weight 1, so dQ, dK, ddelta vanish
    got, want = _run(1, 4, 1, 400, 400, 1, seed=5)
    dQ, dK, dV, dd = got
    assert float(dQ.abs().max()) < 1e-3 and float(dK.abs().max()) < 1e-3
    assert float(dd.abs().max()) < 1e-3
    _close(dV, want[2], "dV")


def test_bwd_delta_gradient_sums_to_zero(gpu_lib):
    got, _ = _run(1, 4, 2, 900, 900, 300, seed=8)
    dd = to64(got[3])
    assert np.abs(dd.sum(-1)).max() < 1e-3 * np.abs(dd).sum(-1).max()


def test_bwd_without_residual(gpu_lib):
    # dO . O from the bf16 O alone (no training forward): fine away from one-hot rows
    got, want = _run(1, 4, 2, 600, 600, 150, seed=12, residual=False)
    for g, r, name in zip(got, want, ("dQ", "dK", "dV", "ddelta")):
        _close(g, r, name)


def test_bwd_prefill_16k_sampled(gpu_lib):
    # the bench workload at full size: dQ of sampled rows and dK/dV/ddelta of sampled
    # keys against the oracle's one-at-a-time backward, ddelta summing to zero per
    # head, and exact zeros for keys no row keeps
    from trainable_dynamic_mask_amd.configs import WORKLOADS
    from trainable_dynamic_mask_amd.inputs import make_inputs
    wl = WORKLOADS["prefill_16k"]
    x = make_inputs(wl, device="cuda")
    dO = make_grad(wl, device="cuda")
    print("bwd prefill_16k sampled", flush=True)
    d = dma.weights(x["V"], x["Delta"], x["A"])
    m = dma.topk_mask(d, wl.Sq, 0, wl.w)
    O, lse, Ores = dma.attn_fwd_train(x["Q"], x["K"], x["V"], d, m)
    dQ, dK, dV, dd = dma.attn_bwd(x["Q"], x["K"], x["V"], d, m, O, lse, dO, O_res=Ores)
    torch.cuda.synchronize()
    d64 = to64(d)
    rows = [(0, hq, i) for hq, i in ((0, 0), (5, 2047), (9, 2048), (31, 16383), (17, 8191),
                                      (2, 64), (30, 12345), (12, 4095))]
    want = oracle.attn_bwd_rows(x["Q"], x["K"], x["V"], d64, dO, 0, wl.w, rows)
    got = np.stack([to64(dQ[b, i, hq]) for b, hq, i in rows])
    _close(got, want, "dQ rows")
    ev = m.evict.view(wl.B, wl.Hkv, wl.Sk).cpu().numpy()
    # two kept keys (a late one and one kept for thousands of rows) and two never kept
    late = [j for j in range(16300, 16384) if ev[0, 3, j] > j][0]
    mid = [j for j in range(12000, 12400) if ev[0, 6, j] - j > 2000][0]
    dead = [j for j in range(9000, 16384) if ev[0, 1, j] == j][:2]
    keys = [(0, 3, late), (0, 6, mid)]
    wk, wv, wd = oracle.attn_bwd_keys(x["Q"], x["K"], x["V"], d64, dO, 0, wl.w, keys)
    for t, (b, h, j) in enumerate(keys):
        _close(to64(dK[b, j, h]), wk[t], f"dK key {j}")
        _close(to64(dV[b, j, h]), wv[t], f"dV key {j}")
        scale = np.abs(to64(dd[b, h])).max()
        assert abs(float(dd[b, h, j]) - wd[t]) <= 3e-2 * scale, f"ddelta key {j}"
    for j in dead:
        assert float(dK[0, j, 1].abs().max()) == 0 and float(dV[0, j, 1].abs().max()) == 0
        assert float(dd[0, 1, j]) == 0
    ddn = to64(dd)
    assert np.abs(ddn.sum(-1)).max() < 1e-3 * np.abs(ddn).sum(-1).max()


def test_bwd_noncontiguous_views_match_contiguous(gpu_lib):
    # O, O_res and dO handed over as non-contiguous views of one buffer each, and
    # Delta/A in bf16: the binding makes contiguous float copies, which must all
    # stay alive until the kernels have read them (a copy freed early could be
    # overwritten by the next one).  Results must equal the contiguous call's.
    B, Hq, Hkv, S, w = 1, 8, 2, 300, 64
    wl, x = make_small(B, Hq, Hkv, S, S, 128, w, dtype="bf16", seed=31, device="cuda")
    dO = make_grad(wl, device="cuda")
    d = dma.weights(x["V"], x["Delta"], x["A"])
    m = dma.topk_mask(d, S, 0, w)
    O, lse, Ores = dma.attn_fwd_train(x["Q"], x["K"], x["V"], d, m)
    ref = dma.attn_bwd(x["Q"], x["K"], x["V"], d, m, O, lse, dO, O_res=Ores)
    # the same values behind transposed storage: [B, Hq, S, D] buffers viewed as [B, S, Hq, D]
    def strided(t):
        buf = t.transpose(1, 2).contiguous()
        v = buf.transpose(1, 2)
        assert not v.is_contiguous()
        return v
    lse_nc = lse.transpose(1, 2).contiguous().transpose(1, 2)
    assert not lse_nc.is_contiguous()
    got = dma.attn_bwd(x["Q"], x["K"], x["V"], d, m, strided(O), lse_nc, strided(dO),
                       O_res=strided(Ores))
    torch.cuda.synchronize()
    for a, b, name in zip(got, ref, ("dQ", "dK", "dV", "ddelta")):
        assert torch.equal(a, b), name
    # weights backward with bf16 Delta and A: the float copies must survive the call
    Dl, Al = x["Delta"].bfloat16(), x["A"].bfloat16()
    dV1, dD1, dA1 = dma.weights_bwd(x["V"], Dl, Al, ref[3], dV=ref[2].clone())
    dV2, dD2, dA2 = dma.weights_bwd(x["V"], Dl.float(), Al.float(), ref[3], dV=ref[2].clone())
    torch.cuda.synchronize()
    assert torch.equal(dV1, dV2)
    assert torch.allclose(dD1, dD2, rtol=1e-5, atol=1e-7) and torch.allclose(dA1, dA2, rtol=1e-5)
