"""Pins of the oracle's keep mask, eviction rows and tile lists (CPU only).

Rule under test: the causal top-w combine of the Hugging Face blog
"Trainable Dynamic Mask Sparse Attention", section "Mask Combination with
Causal Constraints": row p keeps the w keys j <= p with the largest delta,
equal delta going to the lower index (all p+1 keys when p+1 <= w).
"""
import numpy as np
import pytest

import oracle
from tests import brute
from tests.golden import load


@pytest.mark.parametrize("name", ["keep_ties_w2.txt", "keep_ties_w3.txt",
                                  "keep_signed_zeros_w1.txt", "keep_signed_zeros_w2.txt"])
def test_hand_derived_fixture(name):
    g = load(name)
    d = np.array(g["delta"])
    if "signed_zeros" in name:
        assert np.signbit(d[d == 0]).any() and (~np.signbit(d[d == 0])).any()
    w, Bq, Bk = int(g["w"][0]), int(g["Bq"][0]), int(g["Bk"][0])
    S = len(d)
    for p, want in g["row"].items():
        assert oracle.keep_row(d, p, w).tolist() == [int(x) for x in want]
    m = oracle.mask(d[None], 0, S, w, Bq, Bk)
    assert m["evict"][0].tolist() == [int(x) for x in g["evict"]]
    for t, want in g["tile"].items():
        assert m["u_idx"][0, t, : m["u_cnt"][0, t]].tolist() == [int(x) for x in want]
    for t, want in g["ktile"].items():
        assert m["kt_idx"][0, t, : m["kt_cnt"][0, t]].tolist() == [int(x) for x in want]


def _rand_delta(rng, S, kind):
    if kind == "ties":
        return rng.integers(0, 4, S).astype(np.float64)
    if kind == "allequal":
        return np.full(S, 2.0)
    if kind == "signed_zeros":  # -0 and +0 tie (IEEE equality); also -1 and 1
        return rng.choice(np.array([-0.0, 0.0, -1.0, 1.0]), S)
    return rng.random(S) + 1.0


@pytest.mark.parametrize("kind", ["ties", "random", "allequal", "signed_zeros"])
def test_brute_force_enumeration(kind):
    rng = np.random.default_rng(7)
    for trial in range(40):
        S = int(rng.integers(1, 10))
        w = int(rng.integers(1, 11))
        d = _rand_delta(rng, S, kind)
        for p in range(S):
            assert oracle.keep_row(d, p, w).tolist() == brute.keep_by_enumeration(d, p, w)


@pytest.mark.parametrize("kind", ["ties", "random"])
def test_stable_sort_and_counts(kind):
    rng = np.random.default_rng(11)
    for trial in range(10):
        S = int(rng.integers(50, 300))
        w = int(rng.integers(1, 80))
        d = _rand_delta(rng, S, kind)
        m = oracle.mask(d[None], 0, S, w, 16, 16)
        K = brute.dense_keep(d, 0, S, w)
        rows = np.arange(S)
        # every row keeps exactly min(p+1, w) keys
        assert (m["row_cnt"][0] == np.minimum(rows + 1, w)).all()
        assert (K.sum(1) == np.minimum(rows + 1, w)).all()
        # eviction rows reproduce every row's keep set: keep(p,j) <=> j <= p < e_j
        e = m["evict"][0]
        P, J = rows[:, None], rows[None, :]
        assert ((J <= P) & (P < e[None, :]) == K).all()


def test_window_at_least_sequence_is_causal():
    rng = np.random.default_rng(3)
    d = rng.random(40)
    for w in (40, 41, 1000):
        for p in range(40):
            assert oracle.keep_row(d, p, w).tolist() == list(range(p + 1))


def test_window_one_is_running_argmax():
    rng = np.random.default_rng(5)
    d = rng.integers(0, 5, 60).astype(np.float64)
    for p in range(60):
        # np.argmax returns the first (lowest-index) maximum
        assert oracle.keep_row(d, p, 1).tolist() == [int(np.argmax(d[: p + 1]))]


def test_monotone_transform_invariance():
    rng = np.random.default_rng(9)
    d = rng.integers(0, 6, 120).astype(np.float64) + rng.integers(0, 2, 120) * 0.5
    base = oracle.mask(d[None], 0, 120, 17, 8, 8)
    for f in (np.exp, lambda x: x ** 3 + x, lambda x: 2.0 * x - 7.0):
        m = oracle.mask(f(d)[None], 0, 120, 17, 8, 8)
        for k in ("evict", "u_cnt", "u_idx", "kt_cnt", "kt_idx"):
            assert (m[k] == base[k]).all(), k


def test_nesting():
    """keep(p) is contained in keep(p-1) plus key p."""
    rng = np.random.default_rng(13)
    d = rng.integers(0, 3, 200).astype(np.float64)
    prev = set()
    for p in range(200):
        cur = set(oracle.keep_row(d, p, 23).tolist())
        assert cur <= prev | {p}
        prev = cur


def test_tile_lists_are_unions():
    rng = np.random.default_rng(17)
    for trial in range(6):
        S = int(rng.integers(20, 260))
        w = int(rng.integers(1, 70))
        Bq, Bk = [(4, 8), (16, 16), (64, 64), (7, 5)][trial % 4]
        d = rng.integers(0, 8, S).astype(np.float64)
        m = oracle.mask(d[None], 0, S, w, Bq, Bk)
        K = brute.dense_keep(d, 0, S, w)
        for t in range((S + Bq - 1) // Bq):
            r0, r1 = t * Bq, min(S, t * Bq + Bq)
            want = np.nonzero(K[r0:r1].any(0))[0].tolist()
            got = m["u_idx"][0, t, : m["u_cnt"][0, t]].tolist()
            assert got == want
            assert len(got) <= oracle.union_cap(r0, r1 - 1, w)
            kts = sorted({j // Bk for j in want})
            assert m["kt_idx"][0, t, : m["kt_cnt"][0, t]].tolist() == kts


def test_query_offset_window_matches_full_rows():
    rng = np.random.default_rng(19)
    S, w = 150, 20
    d = rng.integers(0, 5, S).astype(np.float64)
    full = oracle.mask(d[None], 0, S, w, 8, 8)
    q0, Sq = 61, 53
    part = oracle.mask(d[None], q0, Sq, w, 8, 8)
    assert (part["row_cnt"][0] == full["row_cnt"][0, q0:q0 + Sq]).all()
    K = brute.dense_keep(d, q0, Sq, w)
    e = part["evict"][0]
    P = (q0 + np.arange(Sq))[:, None]
    J = np.arange(S)[None, :]
    assert (((J <= P) & (P < e[None, :])) == K).all()
    # the windowed eviction row is the full one clamped to the observed rows
    ef = full["evict"][0]
    j = np.arange(S)
    start = np.maximum(j, q0)
    clamped = np.where(j >= q0 + Sq, j, np.minimum(np.maximum(ef, start), q0 + Sq))
    assert (e == clamped).all()


def test_multiple_heads_independent():
    rng = np.random.default_rng(23)
    d = rng.integers(0, 4, (2, 3, 90)).astype(np.float64)
    m = oracle.mask(d, 0, 90, 9, 16, 16)
    for b in range(2):
        for h in range(3):
            one = oracle.mask(d[b, h][None], 0, 90, 9, 16, 16)
            assert (m["evict"][b, h] == one["evict"][0]).all()
            assert (m["u_idx"][b, h] == one["u_idx"][0]).all()
