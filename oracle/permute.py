"""Semantic-aware permutation, fp64/int.  TEST INFRASTRUCTURE ONLY.

Source: Sparse VideoGen2 explainer, technical summary section 2.a: tokens are
reordered so that each cluster occupies one contiguous range; the permutations
pi_q and pi_k are applied so that the final output is mathematically equivalent
to the dense one.

Readings: clusters appear in ascending cluster id; inside a cluster tokens keep
ascending original index (a stable sort), which makes the permutation unique;
V follows K's permutation.  ``perm[i]`` is the original row of permuted row i and
``offsets[c]`` is the first permuted row of cluster c (``offsets[C] == n``).
"""
from __future__ import annotations

import numpy as np


def cluster_permutation(assign: np.ndarray, c: int):
    """Stable sort of token indices by cluster id.  Returns (perm int64 [n], offsets int64 [c+1])."""
    assign = np.asarray(assign)
    perm = np.argsort(assign, kind="stable").astype(np.int64)
    sizes = np.bincount(assign, minlength=c)
    offsets = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)
    return perm, offsets


def permute_rows(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """x_p[i] = x[perm[i]]."""
    return np.asarray(x)[perm]


def unpermute_rows(x_p: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """out[perm[i]] = x_p[i]  (the inverse of ``permute_rows``)."""
    out = np.empty_like(x_p)
    out[perm] = x_p
    return out
