"""Centroid-based top-p block selection, fp64.  TEST INFRASTRUCTURE ONLY.

Source: Sparse VideoGen2 explainer, technical summary section 2.b
("centroid-based top-p selection"): instead of full attention scores, scores
are computed between cluster centroids; clusters are sorted by their estimated
score and taken one after another until the cumulative sum reaches the
threshold p, so the kept density follows the content.  DynamicRad explainer,
technical summary section 2.a (dynamic-threshold mode) adds the safeguard that
a block never ends empty.

Readings where the pages are silent:
* centroid score S_ij = (mu_q_i . mu_k_j) * scale, scale = 1/sqrt(d);
* the quantity that is accumulated is the size-weighted softmax
  P_ij = n_k_j exp(S_ij - max) / sum_j' n_k_j' exp(S_ij' - max) over non-empty K
  clusters.  This is what full softmax attention of the Q centroid gives each K
  cluster if every key is replaced by its centroid, so the kept mass estimates
  the attention mass kept;
* selection is per Q cluster over K clusters; every row of a Q cluster shares
  one key set;
* order by descending P, ties by ascending K-cluster id;
* keep the shortest prefix whose cumulative sum is >= p (the element that
  crosses p is kept); p >= 1 keeps every non-empty K cluster.  Because p > 0 and
  at least one K cluster is non-empty, a non-empty Q cluster always keeps one;
* an empty Q cluster keeps nothing (it has no rows).

``threshold_select`` is DynamicRad's dynamic-threshold ("quality-first") mode
(DynamicRad explainer, technical summary section 2.a): pre-softmax logits serve
as cheap importance proxies, one global threshold keeps only the high-scoring
pairs, and a block left empty keeps its top-scoring pair so it never loses all
context.  Readings: the proxy of block pair (i, j) is the centroid score S_ij
above (block means on uniform blocks, cluster centroids after k-means); the
threshold is absolute, S_ij >= theta; only pairs inside the candidate set (all
pairs when none is given) whose key block is non-empty are eligible; a
non-empty query block with no eligible pair at or above theta keeps its
eligible argmax (ties by the lower key id); an empty query block keeps nothing.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass
class SelectResult:
    mask: np.ndarray        # bool [cq, ck]
    kept_count: np.ndarray  # int64 [cq]
    kept_idx: np.ndarray    # int64 [cq, ck]; ascending K ids, then -1
    weights: np.ndarray     # float64 [cq, ck]; P_ij (0 for empty K clusters)
    cut_margin: np.ndarray  # float64 [cq]; distance of the cut decision from a tie (inf if none)


def centroid_scores(mu_q: np.ndarray, mu_k: np.ndarray, scale: float) -> np.ndarray:
    """S = (mu_q mu_k^T) * scale, float64 [cq, ck]."""
    return (np.asarray(mu_q, np.float64) @ np.asarray(mu_k, np.float64).T) * float(scale)


def top_p_select(scores: np.ndarray, size_q: np.ndarray, size_k: np.ndarray,
                 top_p: float) -> SelectResult:
    scores = np.asarray(scores, np.float64)
    cq, ck = scores.shape
    size_q = np.asarray(size_q)
    size_k = np.asarray(size_k)
    valid = size_k > 0
    mask = np.zeros((cq, ck), dtype=bool)
    weights = np.zeros((cq, ck), dtype=np.float64)
    margin = np.full(cq, np.inf)
    n_valid = int(valid.sum())
    for i in range(cq):
        if size_q[i] == 0 or n_valid == 0:
            continue
        s = scores[i]
        smax = s[valid].max()
        w = np.where(valid, size_k * np.exp(np.where(valid, s - smax, 0.0)), 0.0)
        p_row = w / w.sum()
        weights[i] = p_row
        cand = np.flatnonzero(valid)                     # empty K clusters are never candidates
        order = cand[np.lexsort((cand, -p_row[cand]))]   # P descending, then id ascending
        if top_p >= 1.0:
            m = n_valid
        else:
            cum = np.cumsum(p_row[order])
            hit = np.flatnonzero(cum >= top_p)
            m = int(hit[0]) + 1 if hit.size else n_valid
            # how close the decision is to flipping
            gaps = [cum[m - 1] - top_p]
            if m >= 2:
                gaps.append(top_p - cum[m - 2])
            if m < n_valid:
                gaps.append(p_row[order[m - 1]] - p_row[order[m]])
            margin[i] = min(abs(g) for g in gaps)
        mask[i, order[:m]] = True
    kept_count = mask.sum(axis=1).astype(np.int64)
    kept_idx = np.full((cq, ck), -1, dtype=np.int64)
    for i in range(cq):
        ids = np.flatnonzero(mask[i])
        kept_idx[i, :ids.size] = ids
    return SelectResult(mask, kept_count, kept_idx, weights, margin)


@dataclass
class ThresholdResult:
    mask: np.ndarray        # bool [nq, nk]
    kept_count: np.ndarray  # int64 [nq]
    kept_idx: np.ndarray    # int64 [nq, nk]; ascending key ids, then -1
    margin: np.ndarray      # float64 [nq]; distance of the row's decisions from a tie


def threshold_select(scores: np.ndarray, size_q: np.ndarray, size_k: np.ndarray, theta: float,
                     cand: np.ndarray = None) -> ThresholdResult:
    scores = np.asarray(scores, np.float64)
    nq, nk = scores.shape
    size_q = np.asarray(size_q)
    size_k = np.asarray(size_k)
    elig = np.broadcast_to(size_k > 0, (nq, nk)).copy()
    if cand is not None:
        elig &= np.asarray(cand, dtype=bool)
    mask = np.zeros((nq, nk), dtype=bool)
    margin = np.full(nq, np.inf)
    for i in range(nq):
        if size_q[i] == 0:
            continue
        ids = np.flatnonzero(elig[i])
        if ids.size == 0:
            continue
        s = scores[i, ids]
        keep = s >= theta
        margin[i] = float(np.min(np.abs(s - theta)))
        if keep.any():
            mask[i, ids[keep]] = True
        else:   # the safeguard: the top-scoring eligible pair (lowest id on ties)
            top = int(np.argmax(s))
            mask[i, ids[top]] = True
            rest = np.delete(s, top)
            if rest.size:
                margin[i] = min(margin[i], float(s[top] - rest.max()))
    kept_count = mask.sum(axis=1).astype(np.int64)
    kept_idx = np.full((nq, nk), -1, dtype=np.int64)
    for i in range(nq):
        ids = np.flatnonzero(mask[i])
        kept_idx[i, :ids.size] = ids
    return ThresholdResult(mask, kept_count, kept_idx, margin)
