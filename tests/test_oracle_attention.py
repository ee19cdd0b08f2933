"""Pins for the attention oracle (CPU only).

* a hand-derived worked example (tests/golden/attention_hand.json);
* torch's float64 scaled_dot_product_attention (a library routine) for the
  dense case, scipy's logsumexp for LSE;
* brute-force per-element loops with math.fsum on a tiny masked case;
* closed forms: identical keys give the mean of V; constant V gives V;
* invariants: every row's softmax weights sum to 1; an all-ones mask equals
  full attention; the permuted block formulation equals the original-coordinate
  one after unpermuting (Sparse VideoGen2 explainer, technical summary
  section 2.a: the permuted output is equivalent to the dense one).
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import logsumexp

import oracle


def test_golden_hand_example(golden_dir):
    with open(os.path.join(golden_dir, "attention_hand.json")) as f:
        fx = json.load(f)
    o, lse = oracle.full_attention(np.array(fx["q"]), np.array(fx["k"]), np.array(fx["v"]))
    np.testing.assert_allclose(o, fx["o"], atol=1e-12)
    np.testing.assert_allclose(lse, fx["lse"], atol=1e-12)


@pytest.mark.parametrize("n,m,d", [(1, 1, 4), (17, 33, 16), (64, 128, 64)])
def test_full_matches_torch_sdpa(n, m, d):
    rng = np.random.default_rng(n + m)
    q, k, v = rng.standard_normal((n, d)), rng.standard_normal((m, d)), rng.standard_normal((m, d))
    o, lse = oracle.full_attention(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None]).numpy()[0]
    np.testing.assert_allclose(o, ref, atol=1e-12)
    np.testing.assert_allclose(lse, logsumexp(q @ k.T / math.sqrt(d), axis=1), atol=1e-12)


def test_weights_sum_to_one():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal((20, 8)) * 3, rng.standard_normal((30, 8)) * 3
    _, lse = oracle.full_attention(q, k, np.zeros((30, 8)))
    for r in range(20):
        w = [math.exp(float(np.dot(q[r], k[j])) / math.sqrt(8) - lse[r]) for j in range(30)]
        assert abs(math.fsum(w) - 1.0) < 1e-12


def test_brute_force_masked_tiny():
    rng = np.random.default_rng(4)
    n, d = 7, 3
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    aq = np.array([0, 1, 1, 0, 2, 2, 1])
    ak = np.array([1, 0, 2, 2, 0, 1, 1])
    cm = np.array([[1, 0, 1], [0, 1, 0], [1, 1, 1]], bool)
    o, lse = oracle.cluster_sparse_attention(q, k, v, aq, ak, cm, scale=0.5)
    for r in range(n):
        allowed = [j for j in range(n) if cm[aq[r], ak[j]]]
        logits = [0.5 * math.fsum(q[r, t] * k[j, t] for t in range(d)) for j in allowed]
        mx = max(logits)
        ex = [math.exp(s - mx) for s in logits]
        den = math.fsum(ex)
        for t in range(d):
            assert abs(o[r, t] - math.fsum(e * v[j, t] for e, j in zip(ex, allowed)) / den) < 1e-12
        assert abs(lse[r] - (mx + math.log(den))) < 1e-12


def test_closed_forms():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((5, 8))
    k = np.tile(rng.standard_normal((1, 8)), (9, 1))     # identical keys: uniform weights
    v = rng.standard_normal((9, 8))
    o, lse = oracle.full_attention(q, k, v)
    np.testing.assert_allclose(o, np.tile(v.mean(0), (5, 1)), atol=1e-12)
    np.testing.assert_allclose(lse, q @ k[0] / math.sqrt(8) + math.log(9), atol=1e-12)
    vc = np.tile(rng.standard_normal((1, 8)), (9, 1))      # constant V
    o, _ = oracle.full_attention(q, rng.standard_normal((9, 8)), vc)
    np.testing.assert_allclose(o, np.tile(vc[0], (5, 1)), atol=1e-12)


def test_all_ones_masks_equal_full():
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((70, 16)) for _ in range(3))
    o_full, lse_full = oracle.full_attention(q, k, v)
    o_b, lse_b = oracle.block_sparse_attention(q, k, v, np.ones((3, 3), bool), block=32)
    aq, ak = rng.integers(0, 4, 70), rng.integers(0, 5, 70)
    o_c, lse_c = oracle.cluster_sparse_attention(q, k, v, aq, ak, np.ones((4, 5), bool))
    for o, lse in ((o_b, lse_b), (o_c, lse_c)):
        np.testing.assert_allclose(o, o_full, atol=1e-12)
        np.testing.assert_allclose(lse, lse_full, atol=1e-12)


def test_empty_key_set():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((4, 4)) for _ in range(3))
    o, lse = oracle.cluster_sparse_attention(q, k, v, np.zeros(4, int), np.zeros(4, int),
                                             np.zeros((1, 1), bool))
    assert (o == 0).all() and np.isneginf(lse).all()


def test_permuted_formulation_equals_original_coordinates():
    rng = np.random.default_rng(8)
    n, d, cq, ck = 90, 8, 5, 7
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    aq, ak = rng.integers(0, cq, n), rng.integers(0, ck, n)
    cm = rng.random((cq, ck)) < 0.5
    cm[:, 0] = True
    o, lse = oracle.cluster_sparse_attention(q, k, v, aq, ak, cm)
    pq, offq = oracle.cluster_permutation(aq, cq)
    pk, offk = oracle.cluster_permutation(ak, ck)
    qp, kp, vp = q[pq], k[pk], v[pk]
    op = np.zeros_like(qp)
    lp = np.zeros(n)
    for i in range(cq):
        rows = slice(offq[i], offq[i + 1])
        keys = np.concatenate([np.arange(offk[j], offk[j + 1]) for j in range(ck) if cm[i, j]])
        op[rows], lp[rows] = oracle.attend(qp[rows], kp[keys], vp[keys], 1 / math.sqrt(d))
    np.testing.assert_allclose(oracle.unpermute_rows(op, pq), o, atol=1e-12)
    np.testing.assert_allclose(oracle.unpermute_rows(lp, pq), lse, atol=1e-12)


def test_row_sample_is_exact():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((300, 16)) for _ in range(3))
    mask = rng.random((3, 3)) < 0.6
    mask[np.arange(3), np.arange(3)] = True
    o, lse = oracle.block_sparse_attention(q, k, v, mask, 128)
    rows = np.array([299, 0, 130, 5])
    o2, lse2 = oracle.block_sparse_attention(q, k, v, mask, 128, rows=rows)
    # equal up to BLAS blocking (one ulp)
    np.testing.assert_allclose(o2, o[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse[rows], rtol=0, atol=1e-13)


def _brute_block_sparse(q, k, v, mask, block, scale):
    """Per-element loops with math.fsum: query row r sees key j iff
    mask[r // block][j // block]; a row that sees no key gets O = 0, LSE = -inf."""
    nq, d = q.shape
    o = np.zeros((nq, v.shape[1]))
    lse = np.full(nq, -np.inf)
    for r in range(nq):
        allowed = [j for j in range(k.shape[0]) if mask[r // block][j // block]]
        if not allowed:
            continue
        logits = [scale * math.fsum(q[r, t] * k[j, t] for t in range(d)) for j in allowed]
        mx = max(logits)
        ex = [math.exp(s - mx) for s in logits]
        den = math.fsum(ex)
        for t in range(v.shape[1]):
            o[r, t] = math.fsum(e * v[j, t] for e, j in zip(ex, allowed)) / den
        lse[r] = mx + math.log(den)
    return o, lse


@pytest.mark.parametrize("nq,nk,block,seed", [(11, 11, 4, 0), (37, 45, 8, 1), (9, 30, 4, 2)])
def test_block_sparse_matches_brute_force(nq, nk, block, seed):
    """Uniform-block masked attention (DynamicRad explainer, technical summary
    section 2.a: a fixed block mask) on asymmetric masks with ragged last blocks,
    different query and key lengths and a query block that keeps nothing: a
    transposed mask, keys taken from the query's block, or a dropped ragged tail
    all fail here."""
    rng = np.random.default_rng(40 + seed)
    d = 5
    q, k, v = (rng.standard_normal((n, d)) for n in (nq, nk, nk))
    nqb, nkb = -(-nq // block), -(-nk // block)
    if (nq, nk) == (11, 11):
        mask = np.array([[1, 1, 0], [0, 0, 0], [1, 0, 1]], bool)
    else:
        mask = rng.random((nqb, nkb)) < 0.45
        mask[1] = False                              # an empty query block
        mask[0, nkb - 1] = True                      # the ragged key tail is reached
        mask[nqb - 1, 0] = True
    assert (mask != mask.T).any() if nqb == nkb else True
    o, lse = oracle.block_sparse_attention(q, k, v, mask, block, scale=0.7)
    ob, lb = _brute_block_sparse(q, k, v, mask, block, 0.7)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    assert (np.isneginf(lse) == np.isneginf(lb)).all()
    fin = ~np.isneginf(lb)
    np.testing.assert_allclose(lse[fin], lb[fin], rtol=0, atol=1e-12)
    assert np.isneginf(lse[block:2 * block]).all() and (o[block:2 * block] == 0).all()


def test_nan_reaches_exactly_the_rows_that_read_it():
    """The NaN rule: a NaN in query row n, or in a K row that row n keeps, makes
    all of O_n and LSE_n NaN (it enters every logit of that row, or one logit and
    then the row's normaliser); a NaN in element c of a kept V row makes O_n[c]
    NaN and leaves LSE_n alone; a row whose kept keys and query hold no NaN is
    bitwise the clean result.  This is IEEE arithmetic applied to the masked
    definition (Sparse VideoGen2 explainer, technical summary section 2.c:
    only the selected blocks are read), checked here on the oracle."""
    rng = np.random.default_rng(17)
    nq, nk, block, d = 40, 36, 8, 6
    q, k, v = (rng.standard_normal((n, d)) for n in (nq, nk, nk))
    mask = rng.random((5, 5)) < 0.45
    mask[np.arange(5), np.arange(5)] = True
    mask[:, 0] = False                    # a key block that nobody keeps
    mask[2] = False                       # a query block that keeps nothing
    o0, l0 = oracle.block_sparse_attention(q, k, v, mask, block)
    keeps = lambda j: np.repeat(mask[:, j // block], block)[:nq]   # noqa: E731
    # NaN in one K row (of key block 3)
    kn = k.copy()
    kn[27, 4] = np.nan
    o, lse = oracle.block_sparse_attention(q, kn, v, mask, block)
    hit = keeps(27)
    assert hit.any() and (~hit).any()
    assert np.isnan(o[hit]).all() and np.isnan(lse[hit]).all()
    assert np.array_equal(o[~hit], o0[~hit]) and np.array_equal(lse[~hit], l0[~hit])
    # NaN in one V element (key block 1, column 2)
    vn = v.copy()
    vn[11, 2] = np.nan
    o, lse = oracle.block_sparse_attention(q, k, vn, mask, block)
    hit = keeps(11)
    assert hit.any() and (~hit).any()
    assert np.isnan(o[hit, 2]).all() and not np.isnan(np.delete(o, 2, axis=1)).any()
    assert np.array_equal(o[~hit], o0[~hit]) and np.array_equal(lse, l0)
    # NaN in one query row: that row only, even within its block
    qn = q.copy()
    qn[5, 0] = np.nan
    o, lse = oracle.block_sparse_attention(qn, k, v, mask, block)
    assert np.isnan(o[5]).all() and np.isnan(lse[5])
    rest = np.arange(nq) != 5
    assert np.array_equal(o[rest], o0[rest]) and np.array_equal(lse[rest], l0[rest])
    # a NaN in a key block that no query block keeps changes nothing
    kn = k.copy()
    kn[0:8] = np.nan
    vn = v.copy()
    vn[0:8] = np.nan
    o, lse = oracle.block_sparse_attention(q, kn, vn, mask, block)
    assert np.array_equal(o, o0) and np.array_equal(lse, l0)
