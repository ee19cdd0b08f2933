"""Pins for the permutation oracle (CPU only): brute-force bucket construction,
bijection, contiguity, stability, prefix-sum offsets and unpermute(permute(x)) == x
bit for bit (Sparse VideoGen2 explainer, technical summary section 2.a)."""
import numpy as np
import pytest

import oracle


def _buckets(assign, c):
    lists = [[] for _ in range(c)]
    for i, a in enumerate(assign):
        lists[a].append(i)
    perm = [i for lst in lists for i in lst]
    offsets = [0]
    for lst in lists:
        offsets.append(offsets[-1] + len(lst))
    return np.array(perm), np.array(offsets)


@pytest.mark.parametrize("n,c,seed", [(1, 1, 0), (10, 3, 1), (257, 16, 2), (1000, 1000, 3),
                                      (500, 7, 4)])
def test_matches_bucket_brute_force(n, c, seed):
    rng = np.random.default_rng(seed)
    assign = rng.integers(0, c, n)
    perm, off = oracle.cluster_permutation(assign, c)
    pb, ob = _buckets(assign, c)
    assert (perm == pb).all() and (off == ob).all()
    assert sorted(perm.tolist()) == list(range(n))             # bijection
    for cl in range(c):                                        # contiguous, stable
        seg = perm[off[cl]:off[cl + 1]]
        assert (assign[seg] == cl).all()
        assert (np.diff(seg) > 0).all()


def test_round_trip_is_identity_bitwise():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((300, 16)).astype(np.float32)
    x[3, 2] = np.nan
    x[7, 1] = -0.0
    assign = rng.integers(0, 9, 300)
    perm, _ = oracle.cluster_permutation(assign, 9)
    back = oracle.unpermute_rows(oracle.permute_rows(x, perm), perm)
    assert back.tobytes() == x.tobytes()


def test_empty_clusters_have_empty_ranges():
    assign = np.array([2, 2, 0, 2])
    perm, off = oracle.cluster_permutation(assign, 4)
    assert off.tolist() == [0, 1, 1, 4, 4]
    assert perm.tolist() == [2, 0, 1, 3]
