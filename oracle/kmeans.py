"""Lloyd k-means, fp64.  TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Source: Sparse VideoGen2 explainer, technical summary section 2.a
("semantic-aware permutation"): the Q and K vectors of a head are clustered
independently with k-means into C_q and C_k clusters before attention.  The
centroid cache of section 2.c means the caller supplies the initial centroids.

Readings where the page is silent:
* metric: squared Euclidean distance (Lloyd's algorithm);
* exactly ``iters`` iterations, no tolerance, no early stop;
* an argmin tie goes to the lowest cluster index;
* an empty cluster keeps its previous centroid and has size 0;
* the result is the last iteration's assignment together with the means of
  that assignment (a consistent pair).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class KMeansResult:
    assign: np.ndarray      # int64 [n], cluster of each row (last iteration)
    sizes: np.ndarray       # int64 [c], rows per cluster
    centroids: np.ndarray   # float64 [c, d], means of the last assignment
    margin: np.ndarray      # float64 [n], second-best minus best squared distance (last iteration)


def sq_distances(x: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """Squared Euclidean distances ||x_n - mu_c||^2, float64 [n, c].

    Written as ||x||^2 - 2 x.mu + ||mu||^2 so that one matrix product (a library
    primitive) does the work; in float64 the cancellation error is ~1e-13 for
    activations of order 1, far below the 1e-5 tie margin used in comparisons.
    """
    x = np.asarray(x, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    xx = np.einsum("nd,nd->n", x, x)
    mm = np.einsum("cd,cd->c", mu, mu)
    return xx[:, None] - 2.0 * (x @ mu.T) + mm[None, :]


def assign_step(x: np.ndarray, mu: np.ndarray):
    """E-step: a_n = argmin_c ||x_n - mu_c||^2 (ties -> lowest c).

    Returns (assign int64 [n], margin float64 [n]) where margin is the gap between
    the second-smallest and the smallest distance (inf when c == 1).
    """
    dist = sq_distances(x, mu)
    assign = np.argmin(dist, axis=1)          # first minimum = lowest index
    if dist.shape[1] == 1:
        return assign.astype(np.int64), np.full(dist.shape[0], np.inf)
    part = np.partition(dist, 1, axis=1)
    return assign.astype(np.int64), part[:, 1] - part[:, 0]


def update_step(x: np.ndarray, assign: np.ndarray, mu_prev: np.ndarray):
    """M-step: mu_c = mean of the rows assigned to c; an empty cluster keeps mu_prev[c].

    Returns (centroids float64 [c, d], sizes int64 [c]).
    """
    x = np.asarray(x, dtype=np.float64)
    c, d = mu_prev.shape
    sizes = np.bincount(assign, minlength=c).astype(np.int64)
    sums = np.zeros((c, d), dtype=np.float64)
    np.add.at(sums, assign, x)
    mu = np.array(mu_prev, dtype=np.float64, copy=True)
    nz = sizes > 0
    mu[nz] = sums[nz] / sizes[nz, None]
    return mu, sizes


def kmeans(x: np.ndarray, mu0: np.ndarray, iters: int) -> KMeansResult:
    """``iters`` Lloyd iterations (assign, then update) from the initial centroids mu0."""
    if iters < 1:
        raise ValueError("iters must be >= 1")
    mu = np.asarray(mu0, dtype=np.float64)
    assign = margin = sizes = None
    for _ in range(iters):
        assign, margin = assign_step(x, mu)
        mu, sizes = update_step(x, assign, mu)
    return KMeansResult(assign, sizes, mu, margin)


def objective(x: np.ndarray, assign: np.ndarray, mu: np.ndarray) -> float:
    """Lloyd's objective sum_n ||x_n - mu_{a_n}||^2 (for the monotonicity pin)."""
    diff = np.asarray(x, np.float64) - np.asarray(mu, np.float64)[assign]
    return float(np.einsum("nd,nd->", diff, diff))
