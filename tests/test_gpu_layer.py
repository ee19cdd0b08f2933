"""End-to-end GPU parity of one SVG2-form layer (k-means -> permute -> select
-> block-sparse attention -> unpermute) against the fp64 oracle layer.

* tiny config (fp32): every stage equal to the chained oracle, output to 1e-4;
* top_p = 1: the sparse layer equals dense attention (density-1 invariant);
* full size (32,760 tokens x 40 heads, the benchmark's launch configuration):
  the last k-means iteration in lockstep for every head, selection in lockstep
  for every head, and the unpermuted output on sampled rows of several heads
  against the oracle's attention under the GPU's own clusters and mask.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (assign_parity, check_attention, device, host, to_dev)
from sparse_attention_long_head_amd import SparseVideoAttention, sva_full_attn, sva_kmeans

pytestmark = pytest.mark.gpu


def _layer_inputs(cfg, heads=None):
    x = synth.video_qkv(cfg, heads=heads)
    h = tuple(range(cfg.heads)) if heads is None else heads
    iq = synth.gather_init(x["q"], synth.kmeans_init_indices(cfg, "q", cfg.cq, heads=h))
    ik = synth.gather_init(x["k"], synth.kmeans_init_indices(cfg, "k", cfg.ck, heads=h))
    return x, iq, ik


@pytest.mark.parametrize("fused", [True, False])
def test_tiny_end_to_end_fp32(fused):
    cfg = synth.CONFIGS["tiny"]
    x, iq, ik = _layer_inputs(cfg)
    dev = device()
    layer = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters,
                                 cfg.top_p, dtype=torch.float32, device=dev, want_lse=True,
                                 fuse_permutation=fused)
    t = {k: to_dev(v) for k, v in x.items()}
    o = host(layer(t["q"], t["k"], t["v"], to_dev(iq), to_dev(ik)))
    for h in range(cfg.heads):
        r = oracle.svg2_layer(*(x[n][0, h].astype(np.float64) for n in "qkv"),
                              iq[0, h].astype(np.float64), ik[0, h].astype(np.float64),
                              cfg.iters, cfg.top_p, scale=np.float32(layer.scale))
        assert np.array_equal(host(layer.assign_q)[0, h], r["km_q"].assign)
        assert np.array_equal(host(layer.assign_k)[0, h], r["km_k"].assign)
        assert np.array_equal(host(layer.perm_q)[0, h], r["perm_q"])
        assert np.array_equal(host(layer.off_k)[0, h], r["off_k"])
        assert np.array_equal(host(layer.mask)[0, h].astype(bool), r["select"].mask)
        check_attention(o[0, h], r["o"], False, f"head {h}")
        if fused:                              # LSE in original token order
            lse = host(layer.lse)[0, h]
        else:                                  # LSE in permuted query order
            lse = np.empty(cfg.n)
            lse[host(layer.perm_q)[0, h]] = host(layer.lse)[0, h]
        assert np.abs(lse - r["lse"]).max() < 1e-5


def test_top_p_one_equals_dense():
    cfg = synth.CONFIGS["5s"].with_(T=2, heads=2)
    x, iq, ik = _layer_inputs(cfg)
    dev = device()
    layer = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters, 1.0,
                                 device=dev)
    t = {k: to_dev(v, torch.bfloat16) for k, v in x.items()}
    o = host(layer(t["q"], t["k"], t["v"], to_dev(iq), to_dev(ik)))
    od, _ = sva_full_attn(t["q"], t["k"], t["v"], layer.scale)
    for h in range(cfg.heads):
        ro, _ = oracle.full_attention(x["q"][0, h], x["k"][0, h], x["v"][0, h],
                                      np.float32(layer.scale))
        check_attention(o[0, h], ro, True, f"sparse p=1 head {h}")
        check_attention(host(od)[0, h], ro, True, f"dense head {h}")


@pytest.fixture(scope="module")
def full_layer():
    cfg = synth.CONFIGS["5s"]
    x, iq, ik = _layer_inputs(cfg)
    dev = device()
    t = {k: to_dev(v, torch.bfloat16) for k, v in x.items()}
    layer = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters,
                                 cfg.top_p, device=dev)
    layer(t["q"], t["k"], t["v"], to_dev(iq), to_dev(ik))
    torch.cuda.synchronize()
    return cfg, x, iq, ik, t, layer


def test_full_size_last_kmeans_iteration_lockstep(full_layer):
    cfg, x, iq, ik, t, layer = full_layer
    ties = 0
    for name, init, c, assign in (("q", iq, cfg.cq, layer.assign_q),
                                  ("k", ik, cfg.ck, layer.assign_k)):
        cent = to_dev(init)
        sva_kmeans(t[name], c, cfg.iters - 1, cent)          # centroids entering the last step
        before = host(cent).astype(np.float64)
        _, a_last, _ = sva_kmeans(t[name], c, 1, cent)      # one more step = the 10-step run
        assert torch.equal(a_last, assign)
        a = host(assign)
        for h in range(cfg.heads):
            ref, margin = oracle.assign_step(x[name][0, h].astype(np.float64), before[0, h])
            ties += assign_parity(a[0, h], ref, margin, f"{name} head {h}")
    print(f"\nfull size: k-means tie mismatches {ties}")
    assert ties <= 20


def test_full_size_select_lockstep(full_layer):
    cfg, x, iq, ik, t, layer = full_layer
    mq, mk = host(layer.cent_q), host(layer.cent_k)
    sq, sk = host(layer.sizes_q), host(layer.sizes_k)
    mask, kc, ki = host(layer.mask), host(layer.kept_count), host(layer.kept_idx)
    near = 0
    for h in range(cfg.heads):
        r = oracle.top_p_select(oracle.centroid_scores(mq[0, h], mk[0, h], layer.scale),
                                sq[0, h], sk[0, h], cfg.top_p)
        for i in range(cfg.cq):
            near += int(r.cut_margin[i] < 1e-5)
            if r.cut_margin[i] < 1e-9:
                continue
            assert np.array_equal(mask[0, h, i].astype(bool), r.mask[i]), (h, i)
            assert kc[0, h, i] == r.kept_count[i]
            assert np.array_equal(ki[0, h, i], r.kept_idx[i])
    density = layer.kept_pairs() / (cfg.heads * cfg.n * cfg.n)
    print(f"\nfull size: density {density:.4f}, Q clusters within 1e-5 of a cut tie {near}")
    assert 0.05 < density < 0.3


def test_full_size_output_sampled(full_layer):
    cfg, x, iq, ik, t, layer = full_layer
    o = host(layer.o)
    aq, ak, mask = host(layer.assign_q), host(layer.assign_k), host(layer.mask).astype(bool)
    rng = np.random.default_rng(2)
    for h in (0, 21, 39):
        rows = np.unique(np.concatenate([[0, 1, cfg.n - 1], rng.integers(0, cfg.n, 40)]))
        ro, _ = oracle.cluster_sparse_attention(x["q"][0, h], x["k"][0, h], x["v"][0, h],
                                                aq[0, h], ak[0, h], mask[0, h],
                                                np.float32(layer.scale), rows=rows)
        check_attention(o[0, h, rows], ro, True, f"layer head {h}")


@pytest.mark.parametrize("fused", [True, False])
def test_two_stream_forward_equals_sequential_stages(fused):
    # forward runs the Q clustering on a side stream, concurrently with K/V;
    # the result must be bit-identical to the stages run one after another
    cfg = synth.CONFIGS["5s"].with_(heads=4)
    x, iq, ik = _layer_inputs(cfg, heads=(0, 1, 2, 3))
    dev = device()
    layer = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters,
                                 cfg.top_p, device=dev, fuse_permutation=fused)
    t = {k: to_dev(v, torch.bfloat16) for k, v in x.items()}
    iq_d, ik_d = to_dev(iq), to_dev(ik)
    outs = []
    for _ in range(2):
        layer(t["q"], t["k"], t["v"], iq_d, ik_d)
        outs.append(layer.o.clone())
    layer.kmeans(t["q"], t["k"], iq_d, ik_d)
    layer.permute(t["q"], t["k"], t["v"])
    layer.select()
    layer.attend(t["q"], t["k"], t["v"])
    layer.unpermute()
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])
    assert torch.equal(outs[0], layer.o)


def test_fused_permutation_layer_equals_unfused():
    # reading Q, K, V through the permutation inside attention (and writing O
    # back in token order) gives the same bits as gather -> attend -> unpermute
    cfg = synth.CONFIGS["5s"].with_(heads=3)
    x, iq, ik = _layer_inputs(cfg, heads=(5, 6, 7))
    dev = device()
    t = {k: to_dev(v, torch.bfloat16) for k, v in x.items()}
    iq_d, ik_d = to_dev(iq), to_dev(ik)
    res = {}
    for fused in (True, False):
        layer = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters,
                                     cfg.top_p, device=dev, want_lse=True,
                                     fuse_permutation=fused)
        layer(t["q"], t["k"], t["v"], iq_d, ik_d)
        lse = layer.lse.clone()
        if not fused:
            lse = torch.empty_like(lse).scatter_(2, layer.perm_q.long(), lse)
        res[fused] = (layer.o.clone(), lse, layer.perm_q.clone(), layer.mask.clone())
    for a, b in zip(res[True], res[False]):
        assert torch.equal(a, b)
