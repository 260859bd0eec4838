"""Pins of the oracle's attention (CPU only).

Definition under test: o_t = softmax(q_t k^T / sqrt(d_h) o m_t) v from the
Hugging Face blog "Trainable Dynamic Mask Sparse Attention", section
"Efficient Sparse Attention Computation", with "o" read as adding the mask
m_t (delta on kept keys, -inf elsewhere, section "Mask Combination with
Causal Constraints") to the scaled scores; query head hq reads kv head
hq // (Hq/Hkv).
"""
import math

import numpy as np
import torch
import torch.nn.functional as F

import oracle
from tests import brute
from tests.golden import load


def _qkv(B, Sq, Sk, Hq, Hkv, D, seed):
    g = torch.Generator().manual_seed(seed)
    Q = torch.randn(B, Sq, Hq, D, generator=g)
    K = torch.randn(B, Sk, Hkv, D, generator=g)
    V = torch.randn(B, Sk, Hkv, D, generator=g)
    return Q, K, V


def _dense_reference(Q, K, V, delta, q0, w, scale):
    """torch fp64: scores + additive mask from the stable-sort keep rule, softmax, matmul."""
    B, Sq, Hq, D = Q.shape
    _, Sk, Hkv, _ = K.shape
    G = Hq // Hkv
    O = torch.empty(B, Sq, Hq, D, dtype=torch.float64)
    L = torch.empty(B, Hq, Sq, dtype=torch.float64)
    for b in range(B):
        for hq in range(Hq):
            h = hq // G
            keep = torch.from_numpy(brute.dense_keep(delta[b, h], q0, Sq, w))
            bias = torch.where(keep, torch.from_numpy(delta[b, h])[None, :].expand(Sq, Sk),
                               torch.tensor(-math.inf, dtype=torch.float64))
            s = scale * (Q[b, :, hq].double() @ K[b, :, h].double().T) + bias
            O[b, :, hq] = torch.softmax(s, -1) @ V[b, :, h].double()
            L[b, hq] = torch.logsumexp(s, -1)
    return O.numpy(), L.numpy()


def test_hand_derived_fixture():
    g = load("attn_two_keys.txt")
    Q = np.zeros((1, 3, 1, 2), np.float32)
    Q[0, int(g["row"][0]), 0] = g["q"]
    K = np.array([g["k0"], g["k1"], g["k2"]], np.float32).reshape(1, 3, 1, 2)
    V = np.array([g["v0"], g["v1"], g["v2"]], np.float32).reshape(1, 3, 1, 2)
    delta = np.array(g["delta"]).reshape(1, 1, 3)
    O, lse = oracle.attn_rows(Q, K, V, delta, 0, int(g["w"][0]), [[0, 0, int(g["row"][0])]])
    np.testing.assert_allclose(O[0], g["o"], atol=2e-7)
    assert abs(lse[0] - g["lse"][0]) < 2e-7


def test_zero_delta_projection_full_window_is_causal_sdpa():
    # Delta = 0 makes delta = 2^A[h] on every key; with w >= S every causal key is
    # kept and the constant cancels in the softmax: plain causal attention.
    B, S, H, D = 2, 37, 3, 16
    Q, K, V = _qkv(B, S, S, H, H, D, 1)
    A = torch.rand(H) + 0.5
    delta = oracle.weights(V, torch.zeros(H * D, H), A)
    O, _ = oracle.attn(Q, K, V, delta, 0, S)
    ref = F.scaled_dot_product_attention(Q.double().transpose(1, 2), K.double().transpose(1, 2),
                                         V.double().transpose(1, 2), is_causal=True)
    np.testing.assert_allclose(O, ref.transpose(1, 2).numpy(), atol=1e-12)


def test_full_window_is_sdpa_with_float_bias():
    B, S, H, D = 1, 41, 2, 8
    Q, K, V = _qkv(B, S, S, H, H, D, 2)
    rng = np.random.default_rng(2)
    delta = rng.random((B, H, S)) * 3
    O, _ = oracle.attn(Q, K, V, delta, 0, S)
    causal = torch.ones(S, S, dtype=torch.bool).tril()
    bias = torch.where(causal[None], torch.from_numpy(delta)[:, :, None, :].expand(B, H, S, S),
                       torch.tensor(-math.inf, dtype=torch.float64))
    ref = F.scaled_dot_product_attention(Q.double().transpose(1, 2), K.double().transpose(1, 2),
                                         V.double().transpose(1, 2), attn_mask=bias)
    np.testing.assert_allclose(O, ref.transpose(1, 2).numpy(), atol=1e-12)


def test_window_one_copies_the_argmax_value_row():
    B, S, H, D = 1, 30, 2, 8
    Q, K, V = _qkv(B, S, S, H, H, D, 3)
    rng = np.random.default_rng(3)
    delta = rng.integers(0, 4, (B, H, S)).astype(np.float64)
    O, lse = oracle.attn(Q, K, V, delta, 0, 1)
    for h in range(H):
        for i in range(S):
            j = int(np.argmax(delta[0, h, : i + 1]))
            assert (O[0, i, h] == V[0, j, h].double().numpy()).all()


def test_gqa_general_window_against_dense_masked_softmax():
    B, S, Hq, Hkv, D = 2, 53, 4, 2, 16
    Q, K, V = _qkv(B, S, S, Hq, Hkv, D, 4)
    rng = np.random.default_rng(4)
    delta = rng.integers(0, 5, (B, Hkv, S)).astype(np.float64) * 0.7
    for w in (1, 5, 19):
        O, L = oracle.attn(Q, K, V, delta, 0, w)
        Or, Lr = _dense_reference(Q, K, V, delta, 0, w, 1 / math.sqrt(D))
        np.testing.assert_allclose(O, Or, atol=1e-12)
        np.testing.assert_allclose(L, Lr, atol=1e-12)


def test_query_offset_rows_and_custom_scale():
    B, Sq, Sk, Hq, Hkv, D = 1, 9, 40, 2, 1, 8
    Q, K, V = _qkv(B, Sq, Sk, Hq, Hkv, D, 5)
    rng = np.random.default_rng(5)
    delta = rng.random((B, Hkv, Sk)) * 2
    O, L = oracle.attn(Q, K, V, delta, 31, 12, scale=0.3)
    Or, Lr = _dense_reference(Q, K, V, delta, 31, 12, 0.3)
    np.testing.assert_allclose(O, Or, atol=1e-12)
    np.testing.assert_allclose(L, Lr, atol=1e-12)


def test_output_inside_value_hull():
    B, S, H, D = 1, 64, 2, 8
    Q, K, V = _qkv(B, S, S, H, H, D, 6)
    delta = np.random.default_rng(6).random((B, H, S)) * 4
    O, _ = oracle.attn(Q, K, V, delta, 0, 7)
    vmax = V.abs().amax(dim=1).double().numpy()  # [B, H, D]
    assert (np.abs(O) <= vmax[:, None, :, :] + 1e-12).all()
