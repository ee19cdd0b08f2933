"""Pins for the k-means oracle (CPU only).

What pins it, independently of its own code:
* a hand-derived 1-D worked example (tests/golden/kmeans_1d.json);
* scikit-learn's Lloyd k-means from the same initial centroids;
* brute-force distances (explicit per-coordinate differences, math.fsum);
* Lloyd invariants: the objective never increases, a fixed point is stable,
  centroids are the means of their members, sizes add up to n.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth


def test_golden_1d(golden_dir):
    with open(os.path.join(golden_dir, "kmeans_1d.json")) as f:
        fx = json.load(f)
    for case in fx["cases"]:
        x = np.array(case["x"], float)
        mu0 = np.array(case["mu0"], float)
        for st in case["steps"]:
            r = oracle.kmeans(x, mu0, st["iters"])
            assert r.assign.tolist() == st["assign"], case["name"]
            assert r.sizes.tolist() == st["sizes"], case["name"]
            np.testing.assert_allclose(r.centroids, st["centroids"], rtol=0, atol=1e-12)
        if "margin_iter2" in case:
            r = oracle.kmeans(x, mu0, 2)
            np.testing.assert_allclose(r.margin, case["margin_iter2"], atol=1e-9)
        if "margin_iter1" in case:
            r = oracle.kmeans(x, mu0, 1)
            np.testing.assert_allclose(r.margin, case["margin_iter1"], atol=1e-12)


def _brute_assign(x, mu):
    assign, margin = [], []
    for row in x:
        dists = [math.fsum((a - b) ** 2 for a, b in zip(row, c)) for c in mu]
        best = 0
        for j in range(1, len(dists)):
            if dists[j] < dists[best]:
                best = j
        assign.append(best)
        rest = sorted(dists)
        margin.append(rest[1] - rest[0] if len(rest) > 1 else math.inf)
    return np.array(assign), np.array(margin)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_assign_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((40, 5))
    mu = rng.standard_normal((7, 5))
    a, m = oracle.assign_step(x, mu)
    ab, mb = _brute_assign(x, mu)
    assert (a == ab).all()
    np.testing.assert_allclose(m, mb, atol=1e-12)


def test_tiny_config_matches_brute_force_every_iteration():
    cfg = synth.CONFIGS["tiny"]
    x = synth.video_qkv(cfg)["k"][0, 1].astype(np.float64)
    idx = synth.kmeans_init_indices(cfg, "k", cfg.ck)[0, 1]
    mu = x[idx]
    for _ in range(cfg.iters):
        a, _ = oracle.assign_step(x, mu)
        ab, _ = _brute_assign(x, mu)
        assert (a == ab).all()
        new, sizes = oracle.update_step(x, a, mu)
        for c in range(mu.shape[0]):
            members = x[ab == c]
            if len(members):
                for j in range(x.shape[1]):
                    assert abs(new[c, j] - math.fsum(members[:, j]) / len(members)) < 1e-12
            else:
                assert (new[c] == mu[c]).all()
        mu = new


def _blobs(seed, n=400, d=8, k=5):
    rng = np.random.default_rng(seed)
    centres = 4.0 * rng.standard_normal((k, d))
    lab = rng.integers(0, k, n)
    return centres[lab] + rng.standard_normal((n, d))


@pytest.mark.parametrize("iters", [1, 2, 5])
@pytest.mark.parametrize("seed", [3, 4])
def test_matches_sklearn_lloyd(iters, seed):
    from sklearn.cluster import KMeans
    x = _blobs(seed)
    c = 6
    mu0 = x[np.sort(np.random.default_rng(seed + 10).choice(len(x), c, replace=False))]
    # the comparison needs every cluster non-empty at every iteration (scikit-learn
    # relocates empty clusters; this oracle keeps them)
    mu = mu0
    for _ in range(iters):
        a, _ = oracle.assign_step(x, mu)
        mu, sizes = oracle.update_step(x, a, mu)
        assert (sizes > 0).all()
    r = oracle.kmeans(x, mu0, iters)
    km = KMeans(n_clusters=c, init=mu0, n_init=1, max_iter=iters, tol=0.0,
                algorithm="lloyd").fit(x)
    np.testing.assert_allclose(r.centroids, km.cluster_centers_, rtol=0, atol=1e-10)
    # scikit-learn's labels come from one more assignment step on its final centres
    a_next, _ = oracle.assign_step(x, r.centroids)
    assert (a_next == km.labels_).all()


def test_objective_never_increases_and_fixed_point_is_stable():
    cfg = synth.CONFIGS["tiny"]
    x = synth.video_qkv(cfg)["q"][0, 0].astype(np.float64)
    mu = x[synth.kmeans_init_indices(cfg, "q", 6)[0, 0]]
    prev = math.inf
    for _ in range(50):
        a, _ = oracle.assign_step(x, mu)
        obj_before = oracle.objective(x, a, mu)
        mu, _ = oracle.update_step(x, a, mu)
        obj_after = oracle.objective(x, a, mu)
        assert obj_before <= prev + 1e-9
        assert obj_after <= obj_before + 1e-9
        prev = obj_after
    # converged: another iteration changes nothing
    a1, _ = oracle.assign_step(x, mu)
    mu2, _ = oracle.update_step(x, a1, mu)
    a2, _ = oracle.assign_step(x, mu2)
    assert (a1 == a2).all()
    np.testing.assert_allclose(mu2, mu, atol=1e-12)


def test_sizes_and_consistent_pair():
    cfg = synth.CONFIGS["tiny"]
    x = synth.video_qkv(cfg)["k"][0, 0].astype(np.float64)
    mu0 = x[synth.kmeans_init_indices(cfg, "k", 4)[0, 0]]
    r = oracle.kmeans(x, mu0, 10)
    assert r.sizes.sum() == x.shape[0]
    assert (np.bincount(r.assign, minlength=4) == r.sizes).all()
    for c in range(4):
        if r.sizes[c]:
            np.testing.assert_allclose(r.centroids[c], x[r.assign == c].mean(0), atol=1e-12)


def test_single_cluster_and_c_equals_n():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((9, 3))
    r = oracle.kmeans(x, x[:1], 3)
    assert (r.assign == 0).all() and np.isinf(r.margin).all()
    np.testing.assert_allclose(r.centroids[0], x.mean(0), atol=1e-12)
    r = oracle.kmeans(x, x.copy(), 2)          # every row its own cluster
    assert (r.assign == np.arange(9)).all()
    np.testing.assert_allclose(r.centroids, x, atol=0)


def test_duplicate_centroids_tie_to_lowest():
    x = np.array([[0.0, 0.0], [5.0, 5.0]])
    mu = np.array([[5.0, 5.0], [0.0, 0.0], [0.0, 0.0]])
    a, m = oracle.assign_step(x, mu)
    assert a.tolist() == [1, 0]
    assert m[0] == 0.0


def test_iters_must_be_positive():
    with pytest.raises(ValueError):
        oracle.kmeans(np.zeros((2, 2)), np.zeros((1, 2)), 0)
