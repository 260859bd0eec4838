"""Pins of the oracle's dynamic weights (CPU only).

Definition under test: delta = exp(tau(v Delta) x A) from the Hugging Face
blog "Trainable Dynamic Mask Sparse Attention", section "Dynamic Sparse Mask
Generation", with tau = softplus, v the whole value row of key j
(Hkv*D entries, kv head major) and Delta a [Hkv*D, Hkv] matrix.
"""
import math

import numpy as np
import torch

import oracle


def _inputs(B=2, Sk=5, Hkv=3, D=4, seed=0):
    rng = np.random.default_rng(seed)
    V = rng.standard_normal((B, Sk, Hkv, D)).astype(np.float32)
    Dl = (rng.standard_normal((Hkv * D, Hkv)) * 0.3).astype(np.float32)
    A = (rng.random(Hkv) + 0.5).astype(np.float32)
    return V, Dl, A


def test_zero_projection_gives_two_to_the_a():
    # softplus(0) = ln 2, so delta = exp(A ln 2) = 2^A exactly up to rounding
    V, Dl, A = _inputs()
    d = oracle.weights(V, np.zeros_like(Dl), A)
    want = np.power(2.0, A.astype(np.float64))
    np.testing.assert_allclose(d, np.broadcast_to(want[None, :, None], d.shape), rtol=1e-15)
    d0 = oracle.weights(np.zeros_like(V), Dl, A)
    np.testing.assert_allclose(d0, np.broadcast_to(want[None, :, None], d.shape), rtol=1e-15)


def test_single_entry_pins_flattening_and_column():
    # Delta has one nonzero entry at row c = h_src*D + ch, column h_dst:
    # only head h_dst sees pre = V[b, j, h_src, ch] * s; all others get 2^A.
    V, Dl, A = _inputs(Hkv=3, D=4)
    h_src, ch, h_dst, s = 2, 1, 0, np.float32(0.75)
    Z = np.zeros_like(Dl)
    Z[h_src * 4 + ch, h_dst] = s
    d = oracle.weights(V, Z, A)
    pre = V[:, :, h_src, ch].astype(np.float64) * float(s)
    sp = np.logaddexp(0.0, pre)  # library softplus
    np.testing.assert_allclose(d[:, h_dst, :], np.exp(sp * float(A[h_dst])), rtol=1e-14)
    for h in (1, 2):
        np.testing.assert_allclose(d[:, h, :], 2.0 ** float(A[h]), rtol=1e-15)


def test_softplus_known_point():
    # softplus(ln(e - 1)) = 1, so delta = e^A (input rounded to fp32: ~1e-7)
    V = np.zeros((1, 1, 1, 2), np.float32)
    V[0, 0, 0, 1] = 1.0
    Dl = np.zeros((2, 1), np.float32)
    Dl[1, 0] = math.log(math.e - 1.0)
    A = np.array([1.3], np.float32)
    d = oracle.weights(V, Dl, A)
    assert abs(d[0, 0, 0] - math.exp(float(A[0]))) < 1e-6


def test_softplus_tails():
    # large positive pre: softplus(x) -> x; large negative: -> e^x -> 0
    V = np.array([[[[1.0]]], [[[-1.0]]]], np.float32).reshape(2, 1, 1, 1)
    Dl = np.array([[60.0]], np.float32)
    A = np.array([0.1], np.float32)
    d = oracle.weights(V, Dl, A)
    a = float(A[0])  # the fp32 value of 0.1
    assert abs(d[0, 0, 0] - math.exp(60.0 * a)) / math.exp(60.0 * a) < 1e-14
    assert abs(d[1, 0, 0] - math.exp(math.exp(-60.0) * a)) < 1e-15


def test_matches_library_composition():
    # torch fp64 matmul + softplus (threshold disabled) + exp as libraries
    V, Dl, A = _inputs(B=2, Sk=7, Hkv=4, D=8, seed=3)
    d = oracle.weights(V, Dl, A)
    Vt = torch.from_numpy(V).double().reshape(2, 7, 32)
    pre = Vt @ torch.from_numpy(Dl).double()              # [B, Sk, Hkv]
    ref = torch.exp(torch.nn.functional.softplus(pre, threshold=1e9) * torch.from_numpy(A).double())
    np.testing.assert_allclose(d, ref.permute(0, 2, 1).numpy(), rtol=1e-13)


def test_weights_at_least_one_for_positive_a():
    V, Dl, A = _inputs(B=1, Sk=50, Hkv=2, D=16, seed=4)
    assert (oracle.weights(V, Dl, A) >= 1.0).all()
