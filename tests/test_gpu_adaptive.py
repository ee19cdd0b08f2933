"""Per-head cluster counts (the layer's adaptive-C mode) on the GPU.

* sva_cluster_spread against the same sums in fp64 NumPy (J: the k-means
  objective under the GPU's assignment and centroids; T: the scatter about the
  mean);
* a layer whose heads have different (C_q, C_k), two of them equal but not
  adjacent (a packed group), head by head against the fp64 oracle: the last
  k-means iteration in lockstep, the top-p selection in lockstep, and the
  output against the oracle's attention under the GPU's own clusters and mask;
  each head group equals a plain layer run on its heads; the slice gather and
  scatter against torch indexing;
* the rule (smallest C of a ladder within (1 + delta) of the objective at the
  largest C) on heads drawn with few and with many mixture regions.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assign_parity, check_attention, device, host, to_dev
from sparse_attention_long_head_amd import (AdaptiveSparseVideoAttention, SparseVideoAttention,
                                            choose_clusters, sva_cluster_spread,
                                            sva_gather_slices, sva_kmeans)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_cluster_spread_parity(dtype, d):
    cfg = synth.CONFIGS["5s"].with_(T=2, heads=3, d=d)        # 3,120 tokens
    x = synth.video_qkv(cfg)["k"]
    c = 70
    init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "k", c))
    xt = to_dev(x, dtype)
    cent = to_dev(init)
    _, a, _ = sva_kmeans(xt, c, 3, cent)
    sp = host(sva_cluster_spread(xt, c, cent, a))
    xs = host(xt).astype(np.float64)
    for h in range(cfg.heads):
        ah, ch = host(a)[0, h], host(cent)[0, h].astype(np.float64)
        j = float(((xs[0, h] - ch[ah]) ** 2).sum())
        t = float(((xs[0, h] - xs[0, h].mean(0)) ** 2).sum())
        assert abs(sp[0, h, 0] - j) <= 1e-9 * j, (h, sp[0, h, 0], j)
        assert abs(sp[0, h, 1] - t) <= 1e-8 * t, (h, sp[0, h, 1], t)
    # deterministic
    assert np.array_equal(sp, host(sva_cluster_spread(xt, c, cent, a)))


CQ = [30, 60, 30, 20]
CK = [150, 300, 150, 90]


@pytest.fixture(scope="module")
def adaptive():
    cfg = synth.CONFIGS["5s"].with_(T=3, heads=len(CQ))        # 4,680 tokens
    x = synth.video_qkv(cfg)
    dev = device()
    t = {n: to_dev(x[n], torch.bfloat16) for n in "qkv"}
    layer = AdaptiveSparseVideoAttention(cfg.heads, cfg.n, cfg.d, CQ, CK, cfg.iters, cfg.top_p,
                                         device=dev)
    # heads 0 and 2 share their counts (a packed group), heads 1 and 3 are alone
    assert [hs for hs, _ in layer.groups] == [[0, 2], [1], [3]]
    inits_q, inits_k = [], []
    for hs, g in layer.groups:
        inits_q.append(to_dev(synth.gather_init(
            x["q"][:, hs], synth.kmeans_init_indices(cfg, "q", g.cq, heads=tuple(hs)))))
        inits_k.append(to_dev(synth.gather_init(
            x["k"][:, hs], synth.kmeans_init_indices(cfg, "k", g.ck, heads=tuple(hs)))))
    o = layer(t["q"], t["k"], t["v"], inits_q, inits_k)
    torch.cuda.synchronize()
    return cfg, x, t, layer, inits_q, inits_k, host(o)


def test_heads_with_different_c_match_the_oracle(adaptive):
    cfg, x, t, layer, inits_q, inits_k, o = adaptive
    ties = 0
    for gi, (hs, g) in enumerate(layer.groups):
        for name, init, c, assign in (("q", inits_q[gi], g.cq, g.assign_q),
                                      ("k", inits_k[gi], g.ck, g.assign_k)):
            cent = init.clone()
            sva_kmeans(t[name][:, hs].contiguous(), c, cfg.iters - 1, cent)   # entering the last step
            before = host(cent).astype(np.float64)
            for j, h in enumerate(hs):
                ref, margin = oracle.assign_step(x[name][0, h].astype(np.float64), before[0, j])
                ties += assign_parity(host(assign)[0, j], ref, margin, f"{name} head {h}")
        for j, h in enumerate(hs):
            r = oracle.top_p_select(oracle.centroid_scores(host(g.cent_q)[0, j],
                                                           host(g.cent_k)[0, j], g.scale),
                                    host(g.sizes_q)[0, j], host(g.sizes_k)[0, j], cfg.top_p)
            firm = r.cut_margin >= 1e-9
            assert np.array_equal(host(g.mask)[0, j].astype(bool)[firm], r.mask[firm]), h
            ro, _ = oracle.cluster_sparse_attention(x["q"][0, h], x["k"][0, h], x["v"][0, h],
                                                    host(g.assign_q)[0, j],
                                                    host(g.assign_k)[0, j],
                                                    host(g.mask)[0, j].astype(bool),
                                                    np.float32(g.scale))
            check_attention(o[0, h], ro, True, f"head {h} (C_q {g.cq}, C_k {g.ck})")
    assert ties <= 2


def test_each_group_equals_a_plain_layer(adaptive):
    cfg, x, t, layer, inits_q, inits_k, o = adaptive
    for gi, (hs, g) in enumerate(layer.groups):
        plain = SparseVideoAttention(1, len(hs), cfg.n, cfg.d, g.cq, g.ck, cfg.iters, cfg.top_p,
                                     device=device())
        op = plain(t["q"][:, hs].contiguous(), t["k"][:, hs].contiguous(),
                   t["v"][:, hs].contiguous(), inits_q[gi], inits_k[gi])
        assert np.array_equal(host(op), o[:, hs])


def test_gather_slices_round_trip():
    dev = device()
    src = torch.randn(7, 33, 64, device=dev).to(torch.bfloat16)
    idx = torch.tensor([5, 0, 3], dtype=torch.int32, device=dev)
    packed = torch.empty(3, 33, 64, dtype=torch.bfloat16, device=dev)
    sva_gather_slices(src, idx, packed)
    assert torch.equal(packed, src[idx.long()])
    back = torch.zeros_like(src)
    sva_gather_slices(packed, idx, back, scatter=True)
    ref = torch.zeros_like(src)
    ref[idx.long()] = src[idx.long()]
    assert torch.equal(back, ref)


def test_rule_gives_fewer_clusters_to_simpler_content():
    """Head 0 drawn with 8 mixture regions, head 1 with 64: the objective at
    the largest ladder step is reached early for head 0 only."""
    base = synth.CONFIGS["5s"].with_(T=3, heads=1)
    ks = [synth.video_qkv(base.with_(centres=m))["k"] for m in (8, 64)]
    x = to_dev(np.concatenate(ks, axis=1), torch.bfloat16)
    ladder = (20, 60, 180)
    chosen, ratio = choose_clusters(x, ladder, iters=5, delta=0.1)
    assert chosen[0] < chosen[1], (chosen, ratio)
    # the choice is the rule applied to the reported objectives
    for j, c in enumerate(chosen):
        first = next(i for i in range(len(ladder)) if ratio[i, j] <= 1.1 * ratio[-1, j])
        assert c == ladder[first]
