"""Brute-force and library cross-checks used to pin the oracle (tiny inputs).

Nothing here is shared with the HIP path.  The keep-set checks follow the
causal top-w rule of the Hugging Face blog "Trainable Dynamic Mask Sparse
Attention" (section "Mask Combination with Causal Constraints"), with ties
toward the lower key index, using methods unlike the oracle's selection:
exhaustive subset enumeration and a library stable sort.
"""
import itertools

import numpy as np


def beats(d, a, b):
    return d[a] > d[b] or (d[a] == d[b] and a < b)


def keep_by_enumeration(d, p, w):
    """The unique subset of {0..p} of size min(p+1, w) whose every member beats
    every non-member.  Raises if zero or several subsets qualify."""
    cand = list(range(p + 1))
    m = min(p + 1, w)
    found = []
    for sub in itertools.combinations(cand, m):
        s = set(sub)
        if all(beats(d, a, b) for a in s for b in cand if b not in s):
            found.append(sub)
    if len(found) != 1:
        raise AssertionError(f"{len(found)} dominating subsets for row {p}")
    return list(found[0])


def keep_by_stable_sort(d, p, w):
    """numpy's stable sort of -delta keeps equal keys in index order, so the
    first w entries are the keep set."""
    d = np.asarray(d, np.float64)[: p + 1]
    return sorted(np.argsort(-d, kind="stable")[:w].tolist())


def dense_keep(d, q0, Sq, w):
    """Boolean [Sq, Sk] keep matrix from the stable-sort rule."""
    d = np.asarray(d, np.float64)
    K = np.zeros((Sq, d.shape[0]), bool)
    for r in range(Sq):
        K[r, keep_by_stable_sort(d, q0 + r, w)] = True
    return K
