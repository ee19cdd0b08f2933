"""Pins for the end-to-end oracle layer (CPU only).

* p = 1 keeps every non-empty K cluster, so the layer equals full attention
  (torch float64 SDPA) -- the density-1.0 invariant;
* the kept-pair count equals the number of (q, k) pairs the mask allows;
* the layer is deterministic.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _tiny_head(h=0):
    cfg = synth.CONFIGS["tiny"]
    x = synth.video_qkv(cfg)
    q, k, v = (x[n][0, h].astype(np.float64) for n in "qkv")
    mq = q[synth.kmeans_init_indices(cfg, "q", cfg.cq)[0, h]]
    mk = k[synth.kmeans_init_indices(cfg, "k", cfg.ck)[0, h]]
    return cfg, q, k, v, mq, mk


def test_density_one_equals_full_attention():
    cfg, q, k, v, mq, mk = _tiny_head()
    r = oracle.svg2_layer(q, k, v, mq, mk, cfg.iters, 1.0)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(q)[None], torch.tensor(k)[None], torch.tensor(v)[None]).numpy()[0]
    np.testing.assert_allclose(r["o"], ref, atol=1e-12)
    assert r["density"] == 1.0


def test_kept_pairs_count():
    cfg, q, k, v, mq, mk = _tiny_head(1)
    r = oracle.svg2_layer(q, k, v, mq, mk, cfg.iters, cfg.top_p)
    aq, ak = r["km_q"].assign, r["km_k"].assign
    allowed = r["select"].mask[aq][:, ak]
    assert allowed.sum() == r["kept_pairs"]
    assert 0 < r["density"] <= 1
    assert (allowed.sum(1) > 0).all()          # no row is left without keys


def test_deterministic():
    cfg, q, k, v, mq, mk = _tiny_head()
    a = oracle.svg2_layer(q, k, v, mq, mk, cfg.iters, cfg.top_p)
    b = oracle.svg2_layer(q, k, v, mq, mk, cfg.iters, cfg.top_p)
    assert a["o"].tobytes() == b["o"].tobytes()
    assert (a["select"].mask == b["select"].mask).all()


# --- p < 1: the layer against its stages composed independently here -------
# Sparse VideoGen2 explainer, technical summary section 2: k-means of Q and of
# K (2.a), centroid scores and the cumulative top-p over K clusters (2.b),
# attention of every token over the keys of its Q cluster's kept K clusters,
# in original coordinates (2.a: the permuted computation is equivalent).

def _lloyd_loops(x, mu0, iters):
    """Plain-loop Lloyd: fsum distances, argmin with ties to the lowest id,
    fsum means, an empty cluster keeps its centroid."""
    mu = [list(map(float, r)) for r in mu0]
    rows = [list(map(float, r)) for r in x]
    for _ in range(iters):
        assign = []
        for r in rows:
            dist = [math.fsum((a - b) ** 2 for a, b in zip(r, m)) for m in mu]
            best = min(range(len(mu)), key=lambda c: (dist[c], c))
            srt = sorted(dist)
            assert srt[1] - srt[0] > 1e-9            # no near tie in these inputs
            assign.append(best)
        for c in range(len(mu)):
            mem = [rows[i] for i in range(len(rows)) if assign[i] == c]
            if mem:
                mu[c] = [math.fsum(col) / len(mem) for col in zip(*mem)]
    sizes = [assign.count(c) for c in range(len(mu))]
    return assign, sizes, mu


def _top_p_subsets(mu_q, size_q, mu_k, size_k, scale, p):
    """Per Q cluster: P_j = n_j exp(S_j) / sum over non-empty K clusters; the
    kept set is, among all subsets of non-empty K clusters whose mass reaches
    p, one of the fewest clusters with the largest mass."""
    ck = len(mu_k)
    live = [j for j in range(ck) if size_k[j] > 0]
    keep = np.zeros((len(mu_q), ck), bool)
    for i, mq in enumerate(mu_q):
        if size_q[i] == 0:
            continue
        s = {j: scale * math.fsum(a * b for a, b in zip(mq, mu_k[j])) for j in live}
        top = max(s.values())
        w = {j: size_k[j] * math.exp(s[j] - top) for j in live}
        tot = math.fsum(w.values())
        pj = {j: w[j] / tot for j in live}
        best = None
        for m in range(1, len(live) + 1):
            for sub in itertools.combinations(live, m):
                mass = math.fsum(pj[j] for j in sub)
                if mass >= p and (best is None or mass > best[0]):
                    best = (mass, sub)
            if best is not None:
                break
        keep[i, list(best[1])] = True
    return keep


def _attention_loops(q, k, v, aq, ak, keep, scale):
    o = np.zeros_like(v, dtype=np.float64)
    lse = np.zeros(q.shape[0])
    for r in range(q.shape[0]):
        allowed = [j for j in range(k.shape[0]) if keep[aq[r], ak[j]]]
        logits = [scale * float(np.dot(q[r], k[j])) for j in allowed]
        mx = max(logits)
        ex = [math.exp(t - mx) for t in logits]
        den = math.fsum(ex)
        for t in range(v.shape[1]):
            o[r, t] = math.fsum(e * v[j, t] for e, j in zip(ex, allowed)) / den
        lse[r] = mx + math.log(den)
    return o, lse


@pytest.mark.parametrize("h,cq,ck,p", [(0, 3, 5, 0.6), (1, 5, 3, 0.85)])
def test_layer_below_p1_matches_composed_stages(h, cq, ck, p):
    """svg2_layer at p < 1 with C_q != C_k on the tiny clip: swapping the Q and
    K sides anywhere (sizes, centroids, assignments) or cutting after the wrong
    element changes the result."""
    cfg = synth.CONFIGS["tiny"]
    x = synth.video_qkv(cfg)
    q, k, v = (x[n][0, h].astype(np.float64) for n in "qkv")
    mq = q[synth.kmeans_init_indices(cfg, "q", cq)[0, h]]
    mk = k[synth.kmeans_init_indices(cfg, "k", ck)[0, h]]
    scale = 1.0 / math.sqrt(cfg.d)
    r = oracle.svg2_layer(q, k, v, mq, mk, cfg.iters, p, scale=scale)
    aq, sq, cen_q = _lloyd_loops(q, mq, cfg.iters)
    ak, sk, cen_k = _lloyd_loops(k, mk, cfg.iters)
    assert list(r["km_q"].assign) == aq and list(r["km_k"].assign) == ak
    np.testing.assert_allclose(r["km_q"].centroids, cen_q, rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["km_k"].centroids, cen_k, rtol=0, atol=1e-13)
    keep = _top_p_subsets(cen_q, sq, cen_k, sk, scale, p)
    assert (r["select"].mask == keep).all()
    assert not keep[np.array(sq) > 0].all()          # p < 1 really drops clusters here
    o, lse = _attention_loops(q, k, v, np.array(aq), np.array(ak), keep, scale)
    np.testing.assert_allclose(r["o"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], lse, rtol=0, atol=1e-12)
    assert r["kept_pairs"] == int(sum(sq[i] * sk[j] for i in range(cq) for j in range(ck)
                                      if keep[i, j]))
