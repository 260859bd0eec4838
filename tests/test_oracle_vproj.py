"""Pins of the oracle's value projection (CPU only).

Definition under test: V = X Wv, the linear map whose output is the value
matrix that the delta equation of the Hugging Face blog "Trainable Dynamic
Mask Sparse Attention" (section "Dynamic Sparse Mask Generation") starts
from: V[m, n] = sum_k X[m, k] Wv[k, n].
"""
import numpy as np

import oracle


def test_one_hot_rows_pick_weight_rows():
    # X row m = e_{k(m)}: V row m is row k(m) of Wv, exactly
    rng = np.random.default_rng(1)
    Cin, N = 12, 7
    W = rng.standard_normal((Cin, N)).astype(np.float32)
    ks = np.array([3, 0, 11, 3, 5])
    X = np.zeros((len(ks), Cin), np.float32)
    X[np.arange(len(ks)), ks] = 1.0
    np.testing.assert_array_equal(oracle.vproj(X, W), W[ks].astype(np.float64))


def test_identity_weight_returns_input():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((2, 3, 6)).astype(np.float32)
    np.testing.assert_array_equal(oracle.vproj(X, np.eye(6, dtype=np.float32)),
                                  X.astype(np.float64))


def test_small_integer_case_by_hand():
    # integers: every product and sum is exact in fp64
    X = np.array([[1, 2, 0, -1, 3], [0, 0, 4, 1, -2], [5, -1, 1, 0, 0]], np.float32)
    W = np.array([[1, 0, 2, -1], [3, 1, 0, 0], [0, 2, 1, 1], [-2, 0, 0, 4], [1, 1, -1, 0]],
                 np.float32)
    want = np.zeros((3, 4))
    for m in range(3):
        for n in range(4):
            want[m, n] = sum(float(X[m, k]) * float(W[k, n]) for k in range(5))
    np.testing.assert_array_equal(oracle.vproj(X, W), want)
    assert want[0, 0] == 1 + 6 + 0 + 2 + 3  # one entry spelled out


def test_linear_in_x_and_shape_kept():
    rng = np.random.default_rng(3)
    X1 = rng.standard_normal((4, 2, 9)).astype(np.float32)
    X2 = rng.standard_normal((4, 2, 9)).astype(np.float32)
    W = rng.standard_normal((9, 5)).astype(np.float32)
    V1, V2 = oracle.vproj(X1, W), oracle.vproj(X2, W)
    assert V1.shape == (4, 2, 5)
    V12 = oracle.vproj((X1 + 2 * X2).astype(np.float64).astype(np.float32), W)
    # X1 + 2*X2 is rounded to fp32 on the way in: compare against that input
    Xs = (X1 + 2 * X2).astype(np.float32).astype(np.float64)
    np.testing.assert_allclose(V12, np.einsum("abk,kn->abn", Xs, W.astype(np.float64)),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(V1 + 2 * V2, V12, rtol=1e-5, atol=1e-5)


def test_transposed_weight_swaps_roles():
    # (X W)^T = W^T X^T: the projection of W^T by X^T is the transpose
    rng = np.random.default_rng(4)
    X = rng.integers(-3, 4, (6, 5)).astype(np.float32)
    W = rng.integers(-3, 4, (5, 7)).astype(np.float32)
    np.testing.assert_array_equal(oracle.vproj(W.T.copy(), X.T.copy()), oracle.vproj(X, W).T)
