"""GPU parity of sva_permute / sva_unpermute: permutation and offsets bit-exact
against the oracle's stable sort, gathered rows bitwise equal to x[perm], and
unpermute(permute(x)) == x bitwise (Sparse VideoGen2 explainer, section 2.a)."""
import numpy as np
import pytest
import torch

import oracle
from parity import device, host, rand_inputs, to_dev
from sparse_attention_long_head_amd import sva_permute, sva_unpermute

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,c", [(1, 1), (100, 7), (2048, 2048), (5000, 300), (4097, 1),
                                 (32760, 500), (32760, 100), (9000, 16384 // 4),
                                 (20000, 8192), (20000, 10000)])
def test_permutation_matches_oracle(n, c):
    heads = 3
    rng = np.random.default_rng(n + c)
    # spatially coherent runs (like clusters of video tokens), with some clusters empty
    assign = np.minimum(rng.integers(0, c, (1, heads, n)), c - 1)
    runs = rng.integers(0, c, (1, heads, max(1, n // 37) + 1))
    assign[..., : (n // 37) * 37] = np.repeat(runs[..., : n // 37], 37, axis=-1)[..., : (n // 37) * 37]
    if c > 3:
        assign[assign == 2] = 3
    assign = assign.astype(np.int32)
    perm, off, _ = sva_permute(to_dev(assign, torch.int32), c)
    perm, off = host(perm), host(off)
    for h in range(heads):
        p_ref, o_ref = oracle.cluster_permutation(assign[0, h], c)
        assert np.array_equal(perm[0, h], p_ref), h
        assert np.array_equal(off[0, h], o_ref), h


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.bfloat16, 64),
                                     (torch.float32, 128), (torch.float32, 64)])
def test_gather_and_round_trip_bitwise(dtype, d):
    heads, n, c = 2, 3001, 57
    rng = np.random.default_rng(d)
    assign = rng.integers(0, c, (1, heads, n)).astype(np.int32)
    xk = rand_inputs((1, heads, n, d), 1, "bf16" if dtype == torch.bfloat16 else "f32")
    xv = rand_inputs((1, heads, n, d), 2, "bf16" if dtype == torch.bfloat16 else "f32")
    tk, tv = to_dev(xk, dtype), to_dev(xv, dtype)
    perm, off, (pk, pv) = sva_permute(to_dev(assign, torch.int32), c, [tk, tv])
    p = host(perm)
    for h in range(heads):
        assert np.array_equal(host(pk)[0, h], xk[0, h][p[0, h]])
        assert np.array_equal(host(pv)[0, h], xv[0, h][p[0, h]])
    back = sva_unpermute(pk, perm)
    assert torch.equal(back, tk)
    assert torch.equal(sva_unpermute(pv, perm), tv)


def test_deterministic():
    rng = np.random.default_rng(3)
    a = to_dev(rng.integers(0, 200, (1, 4, 20000)).astype(np.int32), torch.int32)
    p1, o1, _ = sva_permute(a, 200)
    p2, o2, _ = sva_permute(a, 200)
    assert torch.equal(p1, p2) and torch.equal(o1, o2)
    device()
