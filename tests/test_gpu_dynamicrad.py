"""GPU parity of DynamicRad's selection modes (DynamicRad explainer, technical
summary section 2.a) against the fp64 oracle, through the C ABI.

* sva_radial_mask: the radial candidate set with a static ratio per temporal
  distance, bit-exact against ``oracle.static_ratio_mask`` on the 5 s, 10 s and
  30 s clip geometries and on ragged ones (frames that do not align with
  blocks, a short last block, blocks longer than a frame), same mask for every
  slice, ascending ELL lists;
* sva_block_means: bit-exact for bf16 inputs (an fp64 sum of at most `block`
  bf16 values is exact, so the order cannot matter), within one fp32 ulp for
  fp32 inputs, ragged last block;
* sva_select_threshold: bit-exact against ``oracle.threshold_select`` on the
  same fp32 proxies, with and without a candidate set, empty query and key
  blocks, thresholds from "keep everything" to "safeguard only"; rows whose
  oracle decision lies within 1e-9 of a tie are counted, not compared (none
  are expected for random inputs);
* both modes end to end on uniform blocks of the 5 s clip: mask -> block-sparse
  attention against ``oracle.block_sparse_attention`` on sampled rows;
* RadialSparseAttention equals the manual call sequence bit for bit, and the
  SVG2 layer with a threshold in place of top-p matches the oracle (tiny, fp32).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import check_attention, device, host, rand_inputs, to_dev
from sparse_attention_long_head_amd import (RadialSparseAttention, SparseVideoAttention,
                                            sva_block_means, sva_block_sparse_attn,
                                            sva_radial_mask, sva_select_threshold)

pytestmark = pytest.mark.gpu


def _check_ell(mask, count, idx):
    m = mask.astype(bool)
    assert (count == m.sum(axis=-1)).all()
    nk = m.shape[-1]
    for row in np.ndindex(m.shape[:-1]):
        ids = np.flatnonzero(m[row])
        assert (idx[row][:ids.size] == ids).all()
        assert (idx[row][ids.size:] == -1).all()


GEOMETRIES = [
    # (n, hw, block, dt_max, window0, ratios)
    (32760, 30 * 52, 128, 2, 8, [1.0, 1.0, 1.0]),          # 5 s clip, candidate set
    (32760, 30 * 52, 128, 2, 8, [0.5, 0.3, 0.1]),          # 5 s clip, static ratio
    (63960, 30 * 52, 128, 2, 8, [0.75, 0.5, 0.25]),        # 10 s clip
    (195000, 30 * 52, 128, 3, 8, [1.0, 0.5, 0.25, 0.1]),   # 30 s clip
    (5000, 96, 32, 4, 6, [0.6, 0.4, 0.4, 0.2, 1.0]),       # ragged frames, short last block
    (3000, 50, 128, 1, 3, [1.0, 0.5]),                     # blocks longer than a frame
    (777, 777, 64, 0, 2, [0.5]),                           # one frame
]


@pytest.mark.parametrize("geom", GEOMETRIES, ids=lambda g: f"n{g[0]}_hw{g[1]}_b{g[2]}_dt{g[3]}")
def test_radial_mask_matches_oracle(geom):
    n, hw, block, dt_max, w0, ratios = geom
    want = oracle.static_ratio_mask(n, hw, block, dt_max, w0, ratios)
    mask, count, idx = sva_radial_mask(n, hw, block, dt_max, w0, ratios, 1, 3, device())
    mask, count, idx = host(mask), host(count), host(idx)
    for h in range(3):
        assert np.array_equal(mask[0, h].astype(bool), want), f"head {h}"
    _check_ell(mask, count, idx)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("bf16", [True, False])
def test_block_means(bf16, d):
    n, block = 1000, 128                       # 8 blocks, the last one 104 rows
    x = rand_inputs((2, 3, n, d), 11 + d, "bf16" if bf16 else "f32", scale=2.0)
    means, sizes = sva_block_means(to_dev(x, torch.bfloat16 if bf16 else torch.float32), block)
    means, sizes = host(means), host(sizes)
    for b in range(2):
        for h in range(3):
            wm, ws = oracle.block_means(x[b, h], block)
            assert (sizes[b, h] == ws).all()
            if bf16:
                assert np.array_equal(means[b, h], wm)
            else:
                ulp = np.spacing(np.abs(wm).astype(np.float32))
                assert (np.abs(means[b, h] - wm) <= ulp).all()


def _threshold_case(seed, nq, nk, d, with_cand):
    rng = np.random.default_rng(seed)
    cq = rng.standard_normal((2, 2, nq, d)).astype(np.float32)
    ck = rng.standard_normal((2, 2, nk, d)).astype(np.float32)
    sq = rng.integers(0, 4, (2, 2, nq)).astype(np.int32)
    sk = rng.integers(0, 4, (2, 2, nk)).astype(np.int32)
    sq[..., 0] = 5                              # at least one non-empty query block
    cand = (rng.random((nq, nk)) < 0.3) if with_cand else None
    return cq, ck, sq, sk, cand


@pytest.mark.parametrize("with_cand", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_select_threshold_matches_oracle(d, with_cand):
    nq, nk = 37, 301
    cq, ck, sq, sk, cand = _threshold_case(5 + d + with_cand, nq, nk, d, with_cand)
    scale = float(np.float32(1 / math.sqrt(d)))
    dcand = None if cand is None else to_dev(cand.astype(np.uint8), torch.uint8)
    near_ties = 0
    for theta in [-1e30, -1.0, 0.0, 0.5, 1.0, 2.0, 1e30]:
        mask, count, idx = sva_select_threshold(to_dev(cq), to_dev(sq, torch.int32), to_dev(ck),
                                                to_dev(sk, torch.int32), scale, theta, dcand)
        mask, count, idx = host(mask), host(count), host(idx)
        _check_ell(mask, count, idx)
        for b in range(2):
            for h in range(2):
                s = oracle.centroid_scores(cq[b, h], ck[b, h], scale)
                r = oracle.threshold_select(s, sq[b, h], sk[b, h], theta, cand)
                for i in range(nq):
                    if r.margin[i] < 1e-9:
                        near_ties += 1
                        continue
                    assert np.array_equal(mask[b, h, i].astype(bool), r.mask[i]), (theta, b, h, i)
                if theta >= 1e30:   # safeguard only: every non-empty row with an eligible key keeps one
                    assert (count[b, h] <= 1).all()
    assert near_ties <= 2, near_ties


@pytest.fixture(scope="module")
def static_tensors():
    # the 5 s clip's mixture-of-Gaussians tokens (block means then carry the
    # content) on uniform 128-token blocks
    cfg = synth.CONFIGS["5s"].with_(heads=2)
    x = synth.video_qkv(cfg)
    return cfg, x


def _sampled_rows(n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, 1, 127, 128, n - 1], rng.integers(0, n, 40)]))


def test_static_ratio_layer_end_to_end(static_tensors):
    cfg, x = static_tensors
    ratios = [0.75, 0.5, 0.25]
    mask, count, idx = sva_radial_mask(cfg.n, cfg.H * cfg.W, cfg.block, 2, 8, ratios, 1, cfg.heads,
                                       device())
    off = to_dev(np.broadcast_to(synth.uniform_offsets(cfg.n, cfg.block),
                                 (1, cfg.heads, cfg.n_blocks + 1)).copy(), torch.int32)
    t = {k: to_dev(v, torch.bfloat16) for k, v in x.items()}
    scale = float(np.float32(1 / math.sqrt(cfg.d)))
    o, _ = sva_block_sparse_attn(t["q"], t["k"], t["v"], off, off, count, idx, scale)
    o = host(o)
    want = oracle.static_ratio_mask(cfg.n, cfg.H * cfg.W, cfg.block, 2, 8, ratios)
    rows = _sampled_rows(cfg.n, 1)
    for h in range(cfg.heads):
        ro, _ = oracle.block_sparse_attention(x["q"][0, h], x["k"][0, h], x["v"][0, h], want,
                                              cfg.block, np.float32(scale), rows=rows)
        check_attention(o[0, h, rows], ro, True, f"static ratio head {h}")


def test_dynamic_threshold_layer_end_to_end(static_tensors):
    cfg, x = static_tensors
    t = {k: to_dev(v, torch.bfloat16) for k, v in x.items()}
    scale = float(np.float32(1 / math.sqrt(cfg.d)))
    cand_all, _, _ = sva_radial_mask(cfg.n, cfg.H * cfg.W, cfg.block, 2, 8, [1.0, 1.0, 1.0], 1, 1,
                                     device())
    cand = cand_all[0, 0].contiguous()
    mq, sq = sva_block_means(t["q"], cfg.block)
    mk, sk = sva_block_means(t["k"], cfg.block)
    cand_o = oracle.radial_candidates(cfg.n, cfg.H * cfg.W, cfg.block, 2, 8)
    # theta at the 60th percentile of head 0's candidate proxies (oracle side)
    oq0, _ = oracle.block_means(x["q"][0, 0], cfg.block)
    ok0, _ = oracle.block_means(x["k"][0, 0], cfg.block)
    theta = float(np.quantile(oracle.centroid_scores(oq0, ok0, scale)[cand_o], 0.6))
    mask, count, idx = sva_select_threshold(mq, sq, mk, sk, scale, theta, cand)
    off = to_dev(np.broadcast_to(synth.uniform_offsets(cfg.n, cfg.block),
                                 (1, cfg.heads, cfg.n_blocks + 1)).copy(), torch.int32)
    o, _ = sva_block_sparse_attn(t["q"], t["k"], t["v"], off, off, count, idx, scale)
    o, mask = host(o), host(mask).astype(bool)
    assert np.array_equal(host(cand).astype(bool), cand_o)
    rows = _sampled_rows(cfg.n, 2)
    density = []
    for h in range(cfg.heads):
        oq, nq_ = oracle.block_means(x["q"][0, h], cfg.block)
        ok_, nk_ = oracle.block_means(x["k"][0, h], cfg.block)
        r = oracle.threshold_select(oracle.centroid_scores(oq, ok_, scale), nq_, nk_, theta, cand_o)
        firm = r.margin >= 1e-9
        assert firm.mean() > 0.99
        assert np.array_equal(mask[0, h][firm], r.mask[firm]), f"head {h}"
        assert (mask[0, h] <= cand_o).all()
        density.append(r.mask.mean())
        ro, _ = oracle.block_sparse_attention(x["q"][0, h], x["k"][0, h], x["v"][0, h], mask[0, h],
                                              cfg.block, np.float32(scale), rows=rows)
        check_attention(o[0, h, rows], ro, True, f"dynamic threshold head {h}")
    # a real filter: fewer pairs than the candidate set, at least one per row
    assert 0 < np.mean(density) < cand_o.mean()


def test_radial_layer_equals_manual_calls(static_tensors):
    cfg, x = static_tensors
    t = {k: to_dev(v, torch.bfloat16) for k, v in x.items()}
    scale = float(np.float32(1 / math.sqrt(cfg.d)))
    hw = cfg.H * cfg.W
    off = to_dev(np.broadcast_to(synth.uniform_offsets(cfg.n, cfg.block),
                                 (1, cfg.heads, cfg.n_blocks + 1)).copy(), torch.int32)
    # static
    layer = RadialSparseAttention(1, cfg.heads, cfg.n, cfg.d, hw, cfg.block, "static",
                                  ratios=(0.75, 0.5, 0.25), device=device())
    o1 = layer(t["q"], t["k"], t["v"]).clone()
    _, count, idx = sva_radial_mask(cfg.n, hw, cfg.block, 2, 8, [0.75, 0.5, 0.25], 1, cfg.heads,
                                    device())
    o2, _ = sva_block_sparse_attn(t["q"], t["k"], t["v"], off, off, count, idx, scale)
    assert torch.equal(o1, o2)
    # dynamic
    theta = 2.0
    layer = RadialSparseAttention(1, cfg.heads, cfg.n, cfg.d, hw, cfg.block, "dynamic",
                                  theta=theta, device=device())
    o1 = layer(t["q"], t["k"], t["v"]).clone()
    cand, _, _ = sva_radial_mask(cfg.n, hw, cfg.block, 2, 8, [1.0, 1.0, 1.0], 1, 1, device())
    mq, sq = sva_block_means(t["q"], cfg.block)
    mk, sk = sva_block_means(t["k"], cfg.block)
    _, count, idx = sva_select_threshold(mq, sq, mk, sk, scale, theta, cand[0, 0].contiguous())
    o2, _ = sva_block_sparse_attn(t["q"], t["k"], t["v"], off, off, count, idx, scale)
    assert torch.equal(o1, o2)
    assert 0 < layer.kept_pairs() < cfg.heads * cfg.n * cfg.n


def test_svg2_layer_with_threshold_tiny():
    # k-means clusters, then DynamicRad's threshold on the centroid logits in
    # place of top-p; the oracle decides on the layer's own fp32 centroids
    cfg = synth.CONFIGS["tiny"]
    x = synth.video_qkv(cfg)
    iq = synth.gather_init(x["q"], synth.kmeans_init_indices(cfg, "q", cfg.cq))
    ik = synth.gather_init(x["k"], synth.kmeans_init_indices(cfg, "k", cfg.ck))
    layer = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, cfg.cq, cfg.ck, cfg.iters, cfg.top_p,
                                 dtype=torch.float32, device=device(), theta=0.0)
    t = {k: to_dev(v) for k, v in x.items()}
    o = host(layer(t["q"], t["k"], t["v"], to_dev(iq), to_dev(ik)))
    cq, ck = host(layer.cent_q), host(layer.cent_k)
    sq, sk = host(layer.sizes_q), host(layer.sizes_k)
    aq, ak = host(layer.assign_q), host(layer.assign_k)
    mask = host(layer.mask).astype(bool)
    for h in range(cfg.heads):
        r = oracle.threshold_select(oracle.centroid_scores(cq[0, h], ck[0, h], layer.scale),
                                    sq[0, h], sk[0, h], 0.0)
        assert (r.margin >= 1e-9).all()
        assert np.array_equal(mask[0, h], r.mask)
        ro, _ = oracle.cluster_sparse_attention(x["q"][0, h], x["k"][0, h], x["v"][0, h], aq[0, h],
                                                ak[0, h], r.mask, np.float32(layer.scale))
        check_attention(o[0, h], ro, False, f"head {h}")
