"""GPU parity of the whole layer on the 10 s (63,960 tokens, C_q/C_k = 200/1000)
and 30 s (195,000 tokens, 400/2000) clips, two heads each so the fp64 oracle
stays bounded: the last k-means iteration in lockstep, and, for top-p 0.8, 0.9
and 0.95, the selection in lockstep and the output on sampled rows against the
oracle's attention under the GPU's own clusters and mask.  Kept lists here run past one LDS segment of
the attention kernel (more than 1,024 kept key clusters are possible with
C_k = 2,000), and the k-means tiles cover ragged tails.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import assign_parity, check_attention, device, host, to_dev
from sparse_attention_long_head_amd import SparseVideoAttention, sva_kmeans

pytestmark = pytest.mark.gpu

HEADS = {"10s": (0, 23), "30s": (0, 7)}
TOP_P = (0.8, 0.9, 0.95)


@pytest.fixture(scope="module", params=["10s", "30s"])
def long_layer(request):
    heads = HEADS[request.param]
    cfg = synth.CONFIGS[request.param].with_(heads=len(heads))
    full = synth.CONFIGS[request.param]
    x = synth.video_qkv(full, heads=heads)
    iq = synth.gather_init(x["q"], synth.kmeans_init_indices(full, "q", cfg.cq, heads=heads))
    ik = synth.gather_init(x["k"], synth.kmeans_init_indices(full, "k", cfg.ck, heads=heads))
    t = {k: to_dev(v, torch.bfloat16) for k, v in x.items()}
    layer = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters,
                                 cfg.top_p, device=device())
    layer(t["q"], t["k"], t["v"], to_dev(iq), to_dev(ik))
    torch.cuda.synchronize()
    return cfg, x, iq, ik, t, layer


def test_last_kmeans_iteration_lockstep(long_layer):
    cfg, x, iq, ik, t, layer = long_layer
    ties = 0
    for name, init, c, assign in (("q", iq, cfg.cq, layer.assign_q),
                                  ("k", ik, cfg.ck, layer.assign_k)):
        cent = to_dev(init)
        sva_kmeans(t[name], c, cfg.iters - 1, cent)
        before = host(cent).astype(np.float64)
        _, a_last, _ = sva_kmeans(t[name], c, 1, cent)
        assert torch.equal(a_last, assign)
        for j in range(cfg.heads):
            ref, margin = oracle.assign_step(x[name][0, j].astype(np.float64), before[0, j])
            ties += assign_parity(host(assign)[0, j], ref, margin, f"{cfg.name} {name} {j}")
    print(f"\n{cfg.name}: k-means tie mismatches {ties}")
    assert ties <= 10


def _with_top_p(layer, t, p):
    layer.top_p = p
    layer.select()
    layer.attend(t["q"], t["k"], t["v"])
    torch.cuda.synchronize()


@pytest.mark.parametrize("p", TOP_P)
def test_select_lockstep(long_layer, p):
    cfg, x, iq, ik, t, layer = long_layer
    _with_top_p(layer, t, p)
    mask, kc = host(layer.mask).astype(bool), host(layer.kept_count)
    for j in range(cfg.heads):
        r = oracle.top_p_select(oracle.centroid_scores(host(layer.cent_q)[0, j],
                                                       host(layer.cent_k)[0, j], layer.scale),
                                host(layer.sizes_q)[0, j], host(layer.sizes_k)[0, j], p)
        firm = r.cut_margin >= 1e-9
        assert firm.mean() > 0.98
        assert np.array_equal(mask[0, j][firm], r.mask[firm]), (p, j)
        assert np.array_equal(kc[0, j][firm], r.kept_count[firm]), (p, j)
    density = layer.kept_pairs() / float(cfg.heads * cfg.n * cfg.n)
    print(f"\n{cfg.name} p={p}: density {density:.4f}, max kept K clusters {kc.max()}")
    assert 0.005 < density < 0.6


@pytest.mark.parametrize("p", TOP_P)
def test_output_sampled(long_layer, p):
    cfg, x, iq, ik, t, layer = long_layer
    _with_top_p(layer, t, p)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([[0, 1, cfg.n - 1], rng.integers(0, cfg.n, 48)]))
    for j in range(cfg.heads):
        ro, _ = oracle.cluster_sparse_attention(x["q"][0, j], x["k"][0, j], x["v"][0, j],
                                                host(layer.assign_q)[0, j],
                                                host(layer.assign_k)[0, j],
                                                host(layer.mask)[0, j].astype(bool),
                                                np.float32(layer.scale), rows=rows)
        check_attention(host(layer.o)[0, j, rows], ro, True, f"{cfg.name} p={p} head {j}")


@pytest.fixture(scope="module", params=[1.5, 2.0])
def alpha_layer(request):
    # the sweep's other centre scales (less / more separable content), one head
    heads = (11,)
    full = synth.CONFIGS["10s"]
    cfg = full.with_(heads=len(heads), alpha=request.param)
    x = synth.video_qkv(full, heads=heads, alpha=request.param)
    iq = synth.gather_init(x["q"], synth.kmeans_init_indices(full, "q", cfg.cq, heads=heads))
    ik = synth.gather_init(x["k"], synth.kmeans_init_indices(full, "k", cfg.ck, heads=heads))
    t = {k: to_dev(v, torch.bfloat16) for k, v in x.items()}
    layer = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters, 0.9,
                                 device=device())
    layer(t["q"], t["k"], t["v"], to_dev(iq), to_dev(ik))
    torch.cuda.synchronize()
    return cfg, x, iq, ik, t, layer


def test_alpha_points_lockstep_and_output(alpha_layer):
    cfg, x, iq, ik, t, layer = alpha_layer
    # last k-means iteration in lockstep with the oracle
    ties = 0
    for name, init, c, assign in (("q", iq, cfg.cq, layer.assign_q),
                                  ("k", ik, cfg.ck, layer.assign_k)):
        cent = to_dev(init)
        sva_kmeans(t[name], c, cfg.iters - 1, cent)
        before = host(cent).astype(np.float64)
        _, a_last, _ = sva_kmeans(t[name], c, 1, cent)
        assert torch.equal(a_last, assign)
        ref, margin = oracle.assign_step(x[name][0, 0].astype(np.float64), before[0, 0])
        ties += assign_parity(host(assign)[0, 0], ref, margin, f"alpha {cfg.alpha} {name}")
    assert ties <= 5
    # the selection in lockstep
    _with_top_p(layer, t, 0.9)
    r = oracle.top_p_select(oracle.centroid_scores(host(layer.cent_q)[0, 0],
                                                   host(layer.cent_k)[0, 0], layer.scale),
                            host(layer.sizes_q)[0, 0], host(layer.sizes_k)[0, 0], 0.9)
    firm = r.cut_margin >= 1e-9
    assert firm.mean() > 0.98
    assert np.array_equal(host(layer.mask)[0, 0].astype(bool)[firm], r.mask[firm])
    # sampled output rows under the GPU's clusters and mask
    rows = np.unique(np.concatenate([[0, cfg.n - 1],
                                     np.random.default_rng(5).integers(0, cfg.n, 40)]))
    ro, _ = oracle.cluster_sparse_attention(x["q"][0, 0], x["k"][0, 0], x["v"][0, 0],
                                            host(layer.assign_q)[0, 0], host(layer.assign_k)[0, 0],
                                            host(layer.mask)[0, 0].astype(bool),
                                            np.float32(layer.scale), rows=rows)
    check_attention(host(layer.o)[0, 0, rows], ro, True, f"alpha {cfg.alpha}")
