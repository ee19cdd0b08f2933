"""Pins for the top-p selection oracle (CPU only).

* the hand-derived example in tests/golden/top_p_hand.json;
* the size-weighted softmax equals plain softmax attention of the Q centroid over
  the expanded key set in which every key is its cluster's centroid (torch, fp64);
* brute force over all subsets for C_k <= 8: the kept set has the minimum
  cardinality reaching mass p and the maximum mass among sets of that size;
* p = 1 keeps every non-empty cluster; a tiny p keeps only the top cluster;
  empty Q clusters keep nothing; empty K clusters are never kept.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle


def test_golden_hand_example(golden_dir):
    with open(os.path.join(golden_dir, "top_p_hand.json")) as f:
        fx = json.load(f)
    s = np.array(fx["scores"])
    for case in fx["cases"]:
        r = oracle.top_p_select(s, np.array(fx["size_q"]), np.array(fx["size_k"]), case["top_p"])
        np.testing.assert_allclose(r.weights, fx["weights"], atol=1e-15)
        assert np.flatnonzero(r.mask[0]).tolist() == case["kept"]
        assert r.kept_count[0] == len(case["kept"])
        assert r.kept_idx[0, :len(case["kept"])].tolist() == case["kept"]
        assert (r.kept_idx[0, len(case["kept"]):] == -1).all()


def _expanded_softmax_mass(mu_q_row, mu_k, size_k, scale):
    keys = torch.tensor(np.repeat(mu_k, size_k, axis=0), dtype=torch.float64)
    owner = np.repeat(np.arange(len(size_k)), size_k)
    w = torch.softmax(torch.tensor(mu_q_row, dtype=torch.float64) @ keys.T * scale, dim=0).numpy()
    return np.bincount(owner, weights=w, minlength=len(size_k))


@pytest.mark.parametrize("seed", range(4))
def test_weights_equal_expanded_key_softmax(seed):
    rng = np.random.default_rng(seed)
    d = 8
    mu_q = rng.standard_normal((3, d))
    mu_k = rng.standard_normal((6, d))
    size_k = rng.integers(0, 5, 6)
    size_k[0] = max(size_k[0], 1)
    scale = 1 / np.sqrt(d)
    r = oracle.top_p_select(oracle.centroid_scores(mu_q, mu_k, scale), np.ones(3, int), size_k,
                            0.7)
    for i in range(3):
        np.testing.assert_allclose(r.weights[i], _expanded_softmax_mass(mu_q[i], mu_k, size_k,
                                                                        scale), atol=1e-14)


@pytest.mark.parametrize("seed", range(30))
def test_brute_force_subsets(seed):
    rng = np.random.default_rng(100 + seed)
    ck = int(rng.integers(1, 9))
    s = rng.standard_normal((2, ck)) * rng.uniform(0.1, 4)
    size_k = rng.integers(0, 4, ck)
    if size_k.sum() == 0:
        size_k[rng.integers(0, ck)] = 1
    p = float(rng.uniform(0.05, 0.999))
    r = oracle.top_p_select(s, np.array([1, 1]), size_k, p)
    valid = np.flatnonzero(size_k > 0)
    for i in range(2):
        w = np.zeros(ck)
        w[valid] = size_k[valid] * np.exp(s[i, valid])
        P = w / w.sum()
        best_card, best_mass = None, -1.0
        for m in range(1, len(valid) + 1):
            masses = [sum(P[list(sub)]) for sub in itertools.combinations(valid, m)]
            if max(masses) >= p - 1e-12:
                best_card, best_mass = m, max(masses)
                break
        kept = np.flatnonzero(r.mask[i])
        assert len(kept) == best_card
        assert abs(P[kept].sum() - best_mass) < 1e-12
        assert all(size_k[j] > 0 for j in kept)


def test_p_one_keeps_all_nonempty_and_tiny_p_keeps_top():
    rng = np.random.default_rng(9)
    s = rng.standard_normal((4, 10))
    size_k = np.array([3, 0, 1, 1, 0, 2, 5, 1, 1, 1])
    size_q = np.array([1, 0, 2, 2])
    r = oracle.top_p_select(s, size_q, size_k, 1.0)
    for i in (0, 2, 3):
        assert (r.mask[i] == (size_k > 0)).all()
    assert not r.mask[1].any() and r.kept_count[1] == 0
    r = oracle.top_p_select(s, size_q, size_k, 1e-12)
    for i in (0, 2, 3):
        w = np.where(size_k > 0, size_k * np.exp(s[i]), 0)
        assert np.flatnonzero(r.mask[i]).tolist() == [int(np.argmax(w))]


def test_equal_weights_tie_to_lowest_id():
    s = np.zeros((1, 4))
    r = oracle.top_p_select(s, np.array([1]), np.array([1, 1, 1, 1]), 0.5)
    assert np.flatnonzero(r.mask[0]).tolist() == [0, 1]


def test_kept_mass_is_minimal():
    rng = np.random.default_rng(11)
    s = rng.standard_normal((20, 50)) * 2
    size_k = rng.integers(1, 20, 50)
    for p in (0.3, 0.8, 0.9, 0.99):
        r = oracle.top_p_select(s, np.ones(20, int), size_k, p)
        for i in range(20):
            kept = np.flatnonzero(r.mask[i])
            mass = r.weights[i, kept].sum()
            assert mass >= p - 1e-12
            assert mass - r.weights[i, kept].min() < p


def test_underflowed_weight_still_beats_empty_cluster():
    # cluster 1 is non-empty but its weight underflows to 0; cluster 0 is empty.
    # With p = 1 every non-empty cluster is kept and the empty one never is.
    s = np.array([[0.0, -2000.0, 5.0]])
    r = oracle.top_p_select(s, np.array([1]), np.array([0, 1, 1]), 1.0)
    assert np.flatnonzero(r.mask[0]).tolist() == [1, 2]
