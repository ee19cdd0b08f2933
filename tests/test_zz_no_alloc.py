"""sva_block_sparse_attn_noalloc (static schedule scratch, no allocation)
against sva_block_sparse_attn with a caller workspace, through the C ABI:
bit-identical outputs and LSE on two calls in a row, the second smaller than
the first (the static array keeps the first call's schedule, which the second
must fully rewrite), and the cluster-shaped and uniform-block layouts."""
import numpy as np
import pytest
import torch

import synth
from parity import device, host, rand_inputs, to_dev
from sparse_attention_long_head_amd import (sva_block_sparse_attn,
                                            sva_block_sparse_attn_noalloc)

pytestmark = pytest.mark.gpu


def _case(heads, n, block, seed, density):
    rng = np.random.default_rng(seed)
    nb = -(-n // block)
    q, k, v = (rand_inputs((1, heads, n, 128), seed + i) for i in range(3))
    mask = rng.random((1, heads, nb, nb)) < density
    mask[..., np.arange(nb), np.arange(nb)] = True
    kc, ki = synth.mask_to_ell(mask)
    off = np.broadcast_to(synth.uniform_offsets(n, block), (1, heads, nb + 1)).copy()
    dev = device()
    t = {n_: to_dev(a, torch.bfloat16) for n_, a in (("q", q), ("k", k), ("v", v))}
    return (t["q"], t["k"], t["v"], torch.from_numpy(off).to(dev), torch.from_numpy(kc).to(dev),
            torch.from_numpy(ki).to(dev))


def test_noalloc_equals_workspace_variant_on_two_calls():
    dev = device()
    scale = float(np.float32(1 / np.sqrt(128)))
    for heads, n, block, seed, dens in ((6, 9000, 128, 1, 0.3), (2, 1300, 100, 7, 0.5)):
        q, k, v, off, kc, ki = _case(heads, n, block, seed, dens)
        o_ref, lse_ref = sva_block_sparse_attn(q, k, v, off, off, kc, ki, scale, want_lse=True)
        o = torch.empty_like(q)
        lse = torch.empty((1, heads, n), dtype=torch.float32, device=dev)
        sva_block_sparse_attn_noalloc(q, k, v, off, off, kc, ki, scale, o, lse)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), (heads, n)
        assert torch.equal(lse, lse_ref), (heads, n)
    # the second call again, after an unrelated launch on the same stream
    sva_block_sparse_attn_noalloc(q, k, v, off, off, kc, ki, scale, o, lse)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
