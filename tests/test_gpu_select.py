"""GPU parity of sva_select_blocks against the oracle's top-p (both fp64).

Masks, kept counts and kept-id lists must be identical for every Q cluster
whose cut decision is further than 1e-9 from flipping (cumulative sum vs p, or
the P values on either side of the cut).  Both sides compute in fp64, so the
only admissible differences are rounding-level; the count of rows within the
contract's 1e-5 tie margin is reported as well.
"""
import numpy as np
import pytest
import torch

import oracle
from parity import device, host, to_dev
from sparse_attention_long_head_amd import sva_select_blocks

pytestmark = pytest.mark.gpu


def _centroids(rng, heads, c, d, spread):
    base = spread * rng.standard_normal((8, d))
    pick = rng.integers(0, 8, c)
    return (base[pick] + 0.3 * rng.standard_normal((c, d)))[None].repeat(heads, 0)[None]


def _compare(mu_q, size_q, mu_k, size_k, scale, p):
    mask, kc, ki = sva_select_blocks(to_dev(mu_q.astype(np.float32)), to_dev(size_q, torch.int32),
                                     to_dev(mu_k.astype(np.float32)), to_dev(size_k, torch.int32),
                                     scale, p)
    mask, kc, ki = host(mask), host(kc), host(ki)
    near = 0
    for h in range(mu_q.shape[1]):
        r = oracle.top_p_select(oracle.centroid_scores(mu_q[0, h].astype(np.float32),
                                                       mu_k[0, h].astype(np.float32), scale),
                                size_q[0, h], size_k[0, h], p)
        for i in range(mu_q.shape[2]):
            near += int(r.cut_margin[i] < 1e-5)
            if r.cut_margin[i] < 1e-9:
                continue
            assert np.array_equal(mask[0, h, i].astype(bool), r.mask[i]), (h, i)
            assert kc[0, h, i] == r.kept_count[i], (h, i)
            assert np.array_equal(ki[0, h, i], r.kept_idx[i]), (h, i)
    return near


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("ck", [1, 7, 100, 500, 1000, 2000, 4096])
@pytest.mark.parametrize("p", [0.5, 0.9, 1.0])
def test_select_matches_oracle(d, ck, p):
    rng = np.random.default_rng(ck + d)
    heads, cq = 2, 40
    mu_q = _centroids(rng, heads, cq, d, 1.75)
    mu_k = _centroids(rng, heads, ck, d, 1.75)
    size_q = rng.integers(0, 400, (1, heads, cq)).astype(np.int32)
    size_q[0, 0, :3] = 0                                  # empty Q clusters keep nothing
    size_k = rng.integers(0, 120, (1, heads, ck)).astype(np.int32)
    if ck > 1:
        size_k[0, :, ::5] = 0                             # empty K clusters are never kept
    size_k[0, :, 0] = 17
    _compare(mu_q, size_q, mu_k, size_k, float(np.float32(1 / np.sqrt(d))), p)
    if p == 1.0:
        mask, _, _ = sva_select_blocks(to_dev(mu_q.astype(np.float32)),
                                       to_dev(size_q, torch.int32),
                                       to_dev(mu_k.astype(np.float32)),
                                       to_dev(size_k, torch.int32), 0.1, 1.0)
        m = host(mask).astype(bool)
        for h in range(heads):
            for i in range(cq):
                want = (size_k[0, h] > 0) & (size_q[0, h, i] > 0)
                assert np.array_equal(m[0, h, i], want)


def test_deterministic():
    rng = np.random.default_rng(1)
    args = [to_dev(_centroids(rng, 4, 100, 128, 2.0).astype(np.float32)),
            to_dev(rng.integers(1, 50, (1, 4, 100)).astype(np.int32), torch.int32),
            to_dev(_centroids(rng, 4, 500, 128, 2.0).astype(np.float32)),
            to_dev(rng.integers(0, 50, (1, 4, 500)).astype(np.int32), torch.int32), 0.088, 0.9]
    a = sva_select_blocks(*args)
    b = sva_select_blocks(*args)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    device()
