"""One SVG2-form sparse attention layer, end to end, fp64.  TEST INFRASTRUCTURE ONLY.

Source: Sparse VideoGen2 explainer, technical summary section 2 (a: k-means
of Q and K and the permutation; b: centroid scores and top-p; c: attention over
the kept blocks).  The stages run in the page's order; attention is evaluated
in original coordinates, so the permutation itself is only reported (it is
what the GPU path materialises) and never used to compute the output.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .attention import cluster_sparse_attention
from .kmeans import kmeans
from .permute import cluster_permutation
from .select import centroid_scores, top_p_select


def svg2_layer(q, k, v, mu0_q, mu0_k, iters: int, top_p: float, scale: Optional[float] = None,
               rows: Optional[np.ndarray] = None) -> dict:
    """One (batch, head) slice: q, k, v are [n, d]; mu0_* are initial centroids [c, d]."""
    d = q.shape[-1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    km_q = kmeans(q, mu0_q, iters)
    km_k = kmeans(k, mu0_k, iters)
    perm_q, off_q = cluster_permutation(km_q.assign, mu0_q.shape[0])
    perm_k, off_k = cluster_permutation(km_k.assign, mu0_k.shape[0])
    sel = top_p_select(centroid_scores(km_q.centroids, km_k.centroids, scale),
                       km_q.sizes, km_k.sizes, top_p)
    o, lse = cluster_sparse_attention(q, k, v, km_q.assign, km_k.assign, sel.mask, scale, rows)
    kept_pairs = int((km_q.sizes[:, None] * km_k.sizes[None, :] * sel.mask).sum())
    return dict(km_q=km_q, km_k=km_k, perm_q=perm_q, off_q=off_q, perm_k=perm_k, off_k=off_k,
                select=sel, o=o, lse=lse, kept_pairs=kept_pairs,
                density=kept_pairs / float(q.shape[0] * k.shape[0]))
