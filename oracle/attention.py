"""Masked softmax attention, fp64.  TEST INFRASTRUCTURE ONLY.

Sources:
* Long-video blog ("Why long video is hard", the VRAM wall): full bidirectional
  attention over all latent tokens, cost O(n^2) -- ``full_attention``.
* Sparse VideoGen2 explainer, technical summary section 2.a (the permuted
  computation is equivalent to the dense one) and 2.c (attention over only the
  selected blocks) -- ``cluster_sparse_attention``, evaluated in ORIGINAL
  token coordinates: the allowed keys of token n are those n' whose K cluster is
  kept for n's Q cluster.  No permutation is ever materialised here.
* DynamicRad explainer, technical summary section 2.a (static-ratio mode, a
  fixed mask over the radial candidate set) -- ``block_sparse_attention`` with
  allowed(n, n') = mask[n // block, n' // block].

For each query row: O_n = sum_{n' allowed} softmax(q_n.k_n' * scale) v_n' and
LSE_n = log sum_{n' allowed} exp(q_n.k_n' * scale).  A row with no allowed key
gets O = 0 and LSE = -inf.  The logit scale is 1/sqrt(d) unless given.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float):
    """Dense softmax attention of the rows of q over all rows of k / v.

    Returns (o float64 [nq, dv], lse float64 [nq])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    nq = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((nq, v.shape[1])), np.full(nq, -np.inf)
    s = (q @ k.T) * float(scale)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    den = e.sum(axis=1)
    return (e @ v) / den[:, None], m + np.log(den)


def full_attention(q, k, v, scale: Optional[float] = None, rows: Optional[np.ndarray] = None):
    """Every key allowed.  ``rows`` optionally restricts the query rows computed
    (rows are independent, so a sample is exact for the rows it covers)."""
    scale = 1.0 / np.sqrt(q.shape[-1]) if scale is None else scale
    qq = q if rows is None else np.asarray(q)[rows]
    return attend(qq, k, v, scale)


def cluster_sparse_attention(q, k, v, assign_q, assign_k, cluster_mask, scale=None,
                             rows: Optional[np.ndarray] = None):
    """Attention where token n sees key n' iff cluster_mask[assign_q[n], assign_k[n']].

    Returns (o, lse) for all rows, or for ``rows`` in the given order."""
    scale = 1.0 / np.sqrt(q.shape[-1]) if scale is None else scale
    q = np.asarray(q)
    assign_q = np.asarray(assign_q)
    assign_k = np.asarray(assign_k)
    cluster_mask = np.asarray(cluster_mask, dtype=bool)
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    o = np.zeros((rows.size, np.asarray(v).shape[1]))
    lse = np.full(rows.size, -np.inf)
    cl = assign_q[rows]
    for i in np.unique(cl):
        sel = np.flatnonzero(cl == i)
        keys = np.flatnonzero(cluster_mask[i][assign_k])
        o[sel], lse[sel] = attend(q[rows[sel]], np.asarray(k)[keys], np.asarray(v)[keys], scale)
    return o, lse


def block_sparse_attention(q, k, v, block_mask, block: int, scale=None,
                           rows: Optional[np.ndarray] = None):
    """Attention where token n sees key n' iff block_mask[n // block, n' // block]."""
    scale = 1.0 / np.sqrt(q.shape[-1]) if scale is None else scale
    q = np.asarray(q)
    nk = np.asarray(k).shape[0]
    rows = np.arange(q.shape[0]) if rows is None else np.asarray(rows)
    key_block = np.arange(nk) // block
    o = np.zeros((rows.size, np.asarray(v).shape[1]))
    lse = np.full(rows.size, -np.inf)
    qb = rows // block
    for i in np.unique(qb):
        sel = np.flatnonzero(qb == i)
        keys = np.flatnonzero(np.asarray(block_mask, bool)[i][key_block])
        o[sel], lse[sel] = attend(q[rows[sel]], np.asarray(k)[keys], np.asarray(v)[keys], scale)
    return o, lse
