"""DynamicRad's radial candidate set, static-ratio mask and block means, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: DynamicRad explainer, technical summary section 2.a ("unified
candidate set and dual-mode selection"): one hardware-friendly candidate set
comes from a radial locality prior -- the attention a block receives fades with
spatial and temporal distance -- and two exclusive modes select from it.  The
static-ratio ("throughput-first") mode keeps a fixed retention ratio that
depends on the temporal distance t and needs no content scoring: it takes a
fixed share of the candidates.  The dynamic-threshold mode is
``oracle.select.threshold_select``.

Readings where the pages are silent (the pages give no formula):

* tokens are cut into uniform blocks of ``block`` consecutive tokens (the last
  may be short); token index n = (t * H + y) * W + x, so a frame holds
  hw = H * W tokens;
* block b starts at token block * b; its frame is t_b = floor(block * b / hw)
  and its spatial window index s_b = floor((block * b mod hw) / block);
* candidate pair (a, b): dt = |t_a - t_b| <= dt_max and
  |s_a - s_b| <= window0 >> dt (the spatial window halves with every frame of
  temporal distance -- the radial decay);
* static ratio: for query block a and temporal distance dt, of the n candidates
  at that distance keep the first ceil(r[dt] * n) in the order
  (|s_a - s_b| ascending, b ascending) -- "a fixed percentage of the candidate
  set", taken nearest first as the radial prior ranks them.  ceil(r * n) is
  evaluated in float64 with r the float32 ratio widened exactly;
* block means (the proxies of the dynamic mode on uniform blocks) are the
  arithmetic mean of each block's rows, returned rounded to float32, the
  precision the library exchanges centroids in.
"""
from __future__ import annotations

import math

import numpy as np


def block_geometry(n: int, hw: int, block: int):
    """(frame t_b, window index s_b) of every uniform block, int64 [nb] each."""
    nb = -(-n // block)
    t = np.empty(nb, np.int64)
    s = np.empty(nb, np.int64)
    for b in range(nb):
        start = block * b
        t[b] = start // hw
        s[b] = (start % hw) // block
    return t, s


def radial_candidates(n: int, hw: int, block: int, dt_max: int, window0: int) -> np.ndarray:
    """bool [nb, nb]: the radial locality candidate set (loops, no vectorisation)."""
    t, s = block_geometry(n, hw, block)
    nb = t.size
    cand = np.zeros((nb, nb), dtype=bool)
    for a in range(nb):
        for b in range(nb):
            dt = abs(int(t[a]) - int(t[b]))
            if dt <= dt_max and abs(int(s[a]) - int(s[b])) <= (window0 >> dt):
                cand[a, b] = True
    return cand


def static_ratio_mask(n: int, hw: int, block: int, dt_max: int, window0: int,
                      ratios) -> np.ndarray:
    """bool [nb, nb]: per query block and temporal distance dt, the nearest
    ceil(ratios[dt] * n_candidates) candidates (ties by block id)."""
    r = np.asarray(ratios, dtype=np.float32).astype(np.float64)
    if r.size != dt_max + 1:
        raise ValueError("one ratio per temporal distance 0..dt_max")
    t, s = block_geometry(n, hw, block)
    cand = radial_candidates(n, hw, block, dt_max, window0)
    nb = t.size
    keep = np.zeros((nb, nb), dtype=bool)
    for a in range(nb):
        for dt in range(dt_max + 1):
            ids = [b for b in range(nb) if cand[a, b] and abs(int(t[a]) - int(t[b])) == dt]
            ids.sort(key=lambda b: (abs(int(s[a]) - int(s[b])), b))
            k = int(math.ceil(float(r[dt]) * len(ids)))
            for b in ids[:k]:
                keep[a, b] = True
    return keep


def block_means(x: np.ndarray, block: int):
    """Mean of each uniform block of rows of x [n, d]: (float32 [nb, d], int64 sizes [nb])."""
    x = np.asarray(x, np.float64)
    n = x.shape[0]
    nb = -(-n // block)
    means = np.empty((nb, x.shape[1]), np.float64)
    sizes = np.empty(nb, np.int64)
    for b in range(nb):
        rows = x[block * b: min(n, block * b + block)]
        sizes[b] = rows.shape[0]
        means[b] = rows.sum(axis=0) / rows.shape[0]
    return means.astype(np.float32), sizes
