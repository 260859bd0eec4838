"""Pins of the oracle's backward (CPU only).

The gradients are those of L = sum(dO * O) through the attention of the
Hugging Face blog "Trainable Dynamic Mask Sparse Attention" (section
"Efficient Sparse Attention Computation", with the mask of section "Mask
Combination with Causal Constraints" added to the scaled scores) and through
the dynamic weights of section "Dynamic Sparse Mask Generation" (delta
equation, softplus).  The keep sets are piecewise constant in delta, so
they are held fixed (masked positions get exactly zero gradient, the
section's "Backward Pass Safety" item).  The pins do not retype the
oracle's formulas: central finite differences of the oracle's own forward,
torch fp64 autograd through a plain masked softmax, the w = 1 closed form,
and the shift invariance of softmax.
"""
import numpy as np
import pytest
import torch

import oracle


def _inputs(B, S, Hq, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    # bf16-valued, so that x +/- 2^-10 is exact in float32
    Q = torch.randn(B, S, Hq, D, generator=g).bfloat16().float()
    K = torch.randn(B, S, Hkv, D, generator=g).bfloat16().float()
    V = torch.randn(B, S, Hkv, D, generator=g).bfloat16().float()
    dO = torch.randn(B, S, Hq, D, generator=g).bfloat16().float()
    delta = (torch.rand(B, Hkv, S, generator=g, dtype=torch.float64) * 3 + 1)
    return Q, K, V, dO, delta


def _loss(Q, K, V, delta, dO, w):
    O, _ = oracle.attn(Q, K, V, delta, 0, w)
    return float((O * dO.double().numpy()).sum())


@pytest.mark.parametrize("w", [1, 4, 12])
def test_attn_bwd_finite_differences(w):
    B, S, Hq, Hkv, D = 1, 12, 4, 2, 8
    Q, K, V, dO, delta = _inputs(B, S, Hq, Hkv, D, seed=w)
    dQ, dK, dV, dd = oracle.attn_bwd(Q, K, V, delta, dO, 0, w)
    rng = np.random.default_rng(w)
    h = 2.0 ** -10
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in X.shape)
            Xp, Xm = X.clone(), X.clone()
            Xp[idx] += h
            Xm[idx] -= h
            args = {"Q": Q, "K": K, "V": V}
            fp = _loss(*(Xp if k == name else args[k] for k in "QKV"), delta, dO, w)
            fm = _loss(*(Xm if k == name else args[k] for k in "QKV"), delta, dO, w)
            fd = (fp - fm) / (2 * h)
            assert abs(fd - G[idx]) <= 1e-6 + 1e-4 * abs(G[idx]), (name, idx, fd, G[idx])
    hd = 1e-6   # delta is fp64; the keep sets do not move at this step
    for _ in range(8):
        idx = tuple(int(rng.integers(0, n)) for n in delta.shape)
        dp, dm = delta.clone(), delta.clone()
        dp[idx] += hd
        dm[idx] -= hd
        fd = (_loss(Q, K, V, dp, dO, w) - _loss(Q, K, V, dm, dO, w)) / (2 * hd)
        assert abs(fd - dd[idx]) <= 1e-7 + 1e-6 * abs(dd[idx]), (idx, fd, dd[idx])


def _autograd_reference(Q, K, V, delta, dO, q0, w):
    """torch fp64: keep sets from the oracle's row selection, additive -inf mask,
    plain softmax attention, autograd for every input."""
    B, Sq, Hq, D = Q.shape
    _, Sk, Hkv, _ = K.shape
    G = Hq // Hkv
    keep = torch.zeros(B, Hkv, Sq, Sk, dtype=torch.bool)
    for b in range(B):
        for h in range(Hkv):
            for i in range(Sq):
                keep[b, h, i, oracle.keep_row(delta[b, h].numpy(), q0 + i, w)] = True
    q = Q.double().requires_grad_()
    k = K.double().requires_grad_()
    v = V.double().requires_grad_()
    d = delta.clone().requires_grad_()
    kk = k.repeat_interleave(G, dim=2)
    vv = v.repeat_interleave(G, dim=2)
    s = torch.einsum("bihd,bjhd->bhij", q, kk) / D ** 0.5
    s = s + d.repeat_interleave(G, dim=1)[:, :, None, :]
    s = s.masked_fill(~keep.repeat_interleave(G, dim=1), float("-inf"))
    O = torch.einsum("bhij,bjhd->bihd", torch.softmax(s, -1), vv)
    (O * dO.double()).sum().backward()
    return q.grad, k.grad, v.grad, d.grad


@pytest.mark.parametrize("B,S,Hq,Hkv,D,w,q0", [(2, 40, 4, 2, 16, 9, 0), (1, 30, 3, 1, 8, 30, 0),
                                               (1, 50, 2, 2, 8, 5, 20)])
def test_attn_bwd_matches_autograd(B, S, Hq, Hkv, D, w, q0):
    Q, K, V, dO, delta = _inputs(B, S, Hq, Hkv, D, seed=S + w)
    Q, dO = Q[:, q0:], dO[:, q0:]       # rows q0..S-1 against keys 0..S-1 (chunked prefill)
    want = _autograd_reference(Q, K, V, delta, dO, q0, w)
    got = oracle.attn_bwd(Q, K, V, delta, dO, q0, w)
    for g, r in zip(got, want):
        np.testing.assert_allclose(g, r.numpy(), rtol=1e-9, atol=1e-12)


def test_attn_bwd_w1_closed_form():
    # w = 1: each row keeps one key with weight exactly 1, so only dV is nonzero and
    # dV_j is the sum of dO over the rows (and query heads) that keep key j
    B, S, Hq, Hkv, D = 1, 25, 4, 2, 8
    Q, K, V, dO, delta = _inputs(B, S, Hq, Hkv, D, seed=7)
    dQ, dK, dV, dd = oracle.attn_bwd(Q, K, V, delta, dO, 0, 1)
    assert np.abs(dQ).max() == 0 and np.abs(dK).max() == 0 and np.abs(dd).max() == 0
    want = np.zeros_like(dV)
    G = Hq // Hkv
    for h in range(Hkv):
        best = -1
        for p in range(S):   # running argmax, lower index on ties
            if best < 0 or delta[0, h, p] > delta[0, h, best]:
                best = p
            want[0, best, h] += dO[0, p, h * G:(h + 1) * G].double().sum(0).numpy()
    np.testing.assert_allclose(dV, want, rtol=0, atol=1e-12)


def test_attn_bwd_delta_gradient_sums_to_zero():
    # softmax is invariant to adding one constant to every logit of a row, so the
    # delta gradient of each (batch, kv head) sums to zero over its keys
    Q, K, V, dO, delta = _inputs(2, 60, 4, 2, 16, seed=11)
    _, _, _, dd = oracle.attn_bwd(Q, K, V, delta, dO, 0, 17)
    assert np.abs(dd.sum(-1)).max() < 1e-12 * max(1.0, np.abs(dd).sum())


def test_weights_bwd_finite_differences_and_autograd():
    g = torch.Generator().manual_seed(5)
    B, S, Hkv, D = 2, 9, 3, 8
    V = torch.randn(B, S, Hkv, D, generator=g).bfloat16().float()
    Delta = (torch.randn(Hkv * D, Hkv, generator=g) * 0.25).bfloat16().float()
    A = (torch.rand(Hkv, generator=g) + 0.5).bfloat16().float()
    gd = torch.randn(B, Hkv, S, generator=g, dtype=torch.float64)
    dV, dDelta, dA = oracle.weights_bwd(V, Delta, A, gd)
    # autograd of the plain definition in fp64
    v = V.double().requires_grad_()
    dl = Delta.double().requires_grad_()
    a = A.double().requires_grad_()
    pre = v.reshape(B, S, Hkv * D) @ dl
    dlt = torch.exp(torch.nn.functional.softplus(pre) * a).permute(0, 2, 1)
    (dlt * gd).sum().backward()
    np.testing.assert_allclose(dV, v.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dDelta, dl.grad.numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(dA, a.grad.numpy(), rtol=1e-10, atol=1e-12)
    # central differences of the oracle's own forward
    h = 2.0 ** -10
    L = lambda V_, Dl_, A_: float((oracle.weights(V_, Dl_, A_) * gd.numpy()).sum())
    rng = np.random.default_rng(0)
    for name, X, Gr in (("V", V, dV), ("Delta", Delta, dDelta), ("A", A, dA)):
        for _ in range(5):
            idx = tuple(int(rng.integers(0, n)) for n in X.shape)
            Xp, Xm = X.clone(), X.clone()
            Xp[idx] += h
            Xm[idx] -= h
            args = {"V": V, "Delta": Delta, "A": A}
            fp = L(*(Xp if k == name else args[k] for k in ("V", "Delta", "A")))
            fm = L(*(Xm if k == name else args[k] for k in ("V", "Delta", "A")))
            fd = (fp - fm) / (2 * h)
            assert abs(fd - Gr[idx]) <= 1e-6 + 1e-4 * abs(Gr[idx]), (name, idx, fd, Gr[idx])


def test_sampled_backward_equals_full():
    # the per-row and per-key oracles agree with the full backward
    Q, K, V, dO, delta = _inputs(2, 70, 4, 2, 16, seed=31)
    dQ, dK, dV, dd = oracle.attn_bwd(Q, K, V, delta, dO, 0, 20)
    rows = [(0, 0, 0), (1, 3, 69), (0, 2, 33), (1, 1, 19)]
    got = oracle.attn_bwd_rows(Q, K, V, delta, dO, 0, 20, rows)
    for r, (b, hq, i) in enumerate(rows):
        np.testing.assert_allclose(got[r], dQ[b, i, hq], rtol=1e-12, atol=1e-14)
    keys = [(0, 0, 0), (1, 1, 69), (0, 1, 40), (1, 0, 5)]
    gk, gv, gd = oracle.attn_bwd_keys(Q, K, V, delta, dO, 0, 20, keys)
    for t, (b, h, j) in enumerate(keys):
        np.testing.assert_allclose(gk[t], dK[b, j, h], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(gv[t], dV[b, j, h], rtol=1e-12, atol=1e-14)
        assert abs(gd[t] - dd[b, h, j]) <= 1e-12 * max(1.0, abs(dd[b, h, j]))
