"""Pins for DynamicRad's radial candidate set, static-ratio mask, block means and
dynamic-threshold selection in the oracle (CPU only).

* closed-form candidate counts for an interior block of a frame-aligned grid;
* the 5 s clip geometry's radial density 0.1296 and per-row counts 15 / 33.2 / 41
  (figures recorded for the full-size geometry, kept as a regression pin);
* symmetry, the diagonal, ratio 1 = the candidate set, ratio 0 = nothing,
  monotonicity in the ratios, ceil(r * n) kept per distance and nearest first;
* block means of an arithmetic ramp in closed form;
* the hand-derived threshold example in tests/golden/threshold_hand.json, and
  the threshold rule against a direct set construction on random scores.
"""
import json
import math
import os

import numpy as np

import oracle


def _interior_geometry():
    # 40 blocks per frame (frame-aligned), 9 frames; block 200 sits in frame 5 at window 0
    block, per = 16, 40
    hw = block * per
    n = hw * 9
    return n, hw, block


def test_candidate_counts_closed_form():
    n, hw, block = _interior_geometry()
    cand = oracle.radial_candidates(n, hw, block, 2, 8)
    t, s = oracle.block_geometry(n, hw, block)
    a = 4 * 40 + 20                       # frame 4, window 20: every neighbour exists
    assert t[a] == 4 and s[a] == 20
    dts = np.abs(t - t[a])
    row = cand[a]
    assert row[dts == 0].sum() == 2 * 8 + 1
    assert row[dts == 1].sum() == 2 * (2 * 4 + 1)
    assert row[dts == 2].sum() == 2 * (2 * 2 + 1)
    assert row[dts > 2].sum() == 0
    assert row.sum() == 17 + 18 + 10


def test_candidates_symmetric_with_diagonal():
    for n, hw, block in [(32760, 1560, 128), _interior_geometry(), (1000, 96, 32)]:
        cand = oracle.radial_candidates(n, hw, block, 2, 8)
        assert (cand == cand.T).all()
        assert cand.diagonal().all()


def test_five_second_clip_radial_statistics():
    cand = oracle.radial_candidates(32760, 30 * 52, 128, 2, 8)
    assert cand.shape == (256, 256)
    assert round(cand.mean(), 4) == 0.1296
    per_row = cand.sum(axis=1)
    assert per_row.min() == 15 and per_row.max() == 41
    assert round(per_row.mean(), 1) == 33.2


def test_static_ratio_limits_and_monotone():
    n, hw, block = 6000, 640, 32
    cand = oracle.radial_candidates(n, hw, block, 3, 8)
    assert (oracle.static_ratio_mask(n, hw, block, 3, 8, [1, 1, 1, 1]) == cand).all()
    assert not oracle.static_ratio_mask(n, hw, block, 3, 8, [0, 0, 0, 0]).any()
    lo = oracle.static_ratio_mask(n, hw, block, 3, 8, [0.5, 0.25, 0.1, 0.0])
    hi = oracle.static_ratio_mask(n, hw, block, 3, 8, [0.75, 0.5, 0.3, 0.2])
    assert (lo <= hi).all() and (lo <= cand).all() and lo.diagonal().all()


def test_static_ratio_counts_and_nearest_first():
    n, hw, block = _interior_geometry()
    t, s = oracle.block_geometry(n, hw, block)
    ratios = [0.5, 0.5, 0.25]
    keep = oracle.static_ratio_mask(n, hw, block, 2, 8, ratios)
    a = 4 * 40 + 20
    dts = np.abs(t - t[a])
    ds = np.abs(s - s[a])
    # ceil(0.5 * 17) = 9 at dt 0: windows 16..24 (|ds| <= 4)
    assert keep[a, dts == 0].sum() == math.ceil(0.5 * 17) == 9
    assert set(np.flatnonzero(keep[a] & (dts == 0))) == {a + k for k in range(-4, 5)}
    # ceil(0.5 * 18) = 9 at dt 1: |ds| <= 1 in both frames (6), then |ds| = 2 by id (3 of 4)
    sel1 = np.flatnonzero(keep[a] & (dts == 1))
    assert sel1.size == 9
    assert (ds[sel1] <= 2).all() and (ds[sel1] <= 1).sum() == 6
    two = np.flatnonzero((dts == 1) & (ds == 2))
    assert set(sel1[ds[sel1] == 2]) == set(sorted(two)[:3])
    # ceil(0.25 * 10) = 3 at dt 2: |ds| = 0 in both frames, then the lower-id |ds| = 1
    sel2 = np.flatnonzero(keep[a] & (dts == 2))
    assert sel2.size == 3 and (ds[sel2] == 0).sum() == 2
    one = np.flatnonzero((dts == 2) & (ds == 1))
    assert set(sel2[ds[sel2] == 1]) == {one.min()}
    # ratios are float32: ceil(float32(0.3) * 10) = 4, not 3
    keep3 = oracle.static_ratio_mask(n, hw, block, 2, 8, [0.5, 0.5, 0.3])
    assert (keep3[a] & (dts == 2)).sum() == 4


def test_block_means_of_a_ramp():
    n, d, block = 70, 3, 16
    x = np.arange(n, dtype=np.float64)[:, None] * np.array([1.0, -2.0, 0.5])
    means, sizes = oracle.block_means(x, block)
    assert sizes.tolist() == [16, 16, 16, 16, 6]
    for b in range(5):
        lo, hi = 16 * b, min(n, 16 * b + 16)
        mid = (lo + hi - 1) / 2.0                     # mean of lo .. hi-1
        np.testing.assert_array_equal(means[b], np.float32(mid * np.array([1.0, -2.0, 0.5])))


def test_threshold_golden(golden_dir):
    with open(os.path.join(golden_dir, "threshold_hand.json")) as f:
        fx = json.load(f)
    s = np.array(fx["scores"])
    for case in fx["cases"]:
        cand = np.ones(s.shape, dtype=bool)
        for i, j in case.get("cand_exclude", []):
            cand[i, j] = False
        r = oracle.threshold_select(s, np.array(fx["size_q"]), np.array(fx["size_k"]),
                                    case["theta"], cand)
        for i, kept in enumerate(case["kept"]):
            assert np.flatnonzero(r.mask[i]).tolist() == kept
            assert r.kept_count[i] == len(kept)
            assert r.kept_idx[i, :len(kept)].tolist() == kept
            assert (r.kept_idx[i, len(kept):] == -1).all()


def test_threshold_rule_on_random_scores():
    rng = np.random.default_rng(3)
    for trial in range(20):
        nq, nk = 9, 13
        s = rng.standard_normal((nq, nk))
        size_q = rng.integers(0, 3, nq)
        size_k = rng.integers(0, 3, nk)
        cand = rng.random((nq, nk)) < 0.7
        theta = rng.normal() * 1.5
        r = oracle.threshold_select(s, size_q, size_k, theta, cand)
        for i in range(nq):
            elig = [j for j in range(nk) if cand[i, j] and size_k[j] > 0]
            want = set()
            if size_q[i] > 0 and elig:
                want = {j for j in elig if s[i, j] >= theta}
                if not want:
                    want = {max(elig, key=lambda j: (s[i, j], -j))}
            assert set(np.flatnonzero(r.mask[i])) == want
