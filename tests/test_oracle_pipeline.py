"""Pins for the end-to-end oracle layer (CPU only).

* p = 1 keeps every non-empty K cluster, so the layer equals full attention
  (torch float64 SDPA) -- the density-1.0 invariant;
* the kept-pair count equals the number of (q, k) pairs the mask allows;
* the layer is deterministic.
"""
import numpy as np
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
