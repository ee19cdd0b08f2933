"""GPU parity of sva_kmeans against the fp64 Lloyd oracle.

Lockstep: each GPU iteration (iters=1, centroids in/out) is compared with the
oracle's assignment step on the GPU's input centroids (exact, except rows whose
fp64 top-2 margin is below 1e-5, which are counted) and the oracle's update
step on the GPU's assignment (the GPU sums in fp64 and rounds the mean to
fp32 once, so centroids agree to an ulp of fp32).  Chained runs (10 iterations
on each side) report how many assignments a near-tie cascade changed.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from parity import TIE, assign_parity, device, host, to_dev
from sparse_attention_long_head_amd import sva_check_mfma_rounding, sva_kmeans

pytestmark = pytest.mark.gpu


def _lockstep(x, init, c, iters, dtype, heads=None):
    """x float32 [1, H, n, d] (exact values); returns tie-mismatch count."""
    dev = device()
    xt = to_dev(x, dtype)
    cent = to_dev(init.astype(np.float32))
    ties = 0
    n_ref = torch.zeros(1, dtype=torch.int32, device=dev)
    heads = range(x.shape[1]) if heads is None else heads
    for it in range(iters):
        before = host(cent).astype(np.float64)
        _, assign, sizes = sva_kmeans(xt, c, 1, cent, n_refined=n_ref)
        a, sz, after = host(assign), host(sizes), host(cent)
        for h in heads:
            xh = x[0, h].astype(np.float64)
            ref_a, margin = oracle.assign_step(xh, before[0, h])
            ties += assign_parity(a[0, h], ref_a, margin, f"iter {it} head {h}")
            assert np.array_equal(sz[0, h], np.bincount(a[0, h], minlength=c))
            ref_mu, _ = oracle.update_step(xh, a[0, h].astype(np.int64), before[0, h])
            np.testing.assert_allclose(after[0, h], ref_mu, rtol=2.4e-7, atol=1e-9,
                                       err_msg=f"iter {it} head {h}")
    return ties, int(n_ref.item())


def _lockstep_chained(x, init, c, iters, heads=None, first=2):
    """Iterations first..iters of one chained bf16 run, each in lockstep with
    the oracle.  Iteration k after the first takes the candidate path (the
    clusters within twice the radius of each token's previous cluster); the
    centroids entering it come from a (k-1)-iteration call on the same input,
    which the determinism of the library makes the chained run's own state."""
    xt = to_dev(x, torch.bfloat16)
    heads = range(x.shape[1]) if heads is None else heads
    ties = 0
    for k in range(first, iters + 1):
        cent = to_dev(init.astype(np.float32))
        sva_kmeans(xt, c, k - 1, cent)
        before = host(cent).astype(np.float64)
        cent = to_dev(init.astype(np.float32))
        _, assign, sizes = sva_kmeans(xt, c, k, cent)
        a, sz, after = host(assign), host(sizes), host(cent)
        for h in heads:
            xh = x[0, h].astype(np.float64)
            ref_a, margin = oracle.assign_step(xh, before[0, h])
            ties += assign_parity(a[0, h], ref_a, margin, f"iter {k} head {h}")
            assert np.array_equal(sz[0, h], np.bincount(a[0, h], minlength=c))
            ref_mu, _ = oracle.update_step(xh, a[0, h].astype(np.int64), before[0, h])
            np.testing.assert_allclose(after[0, h], ref_mu, rtol=2.4e-7, atol=1e-9,
                                       err_msg=f"iter {k} head {h}")
    return ties


def test_tiny_config_lockstep_fp32():
    cfg = synth.CONFIGS["tiny"]
    x = synth.video_qkv(cfg)
    for name, c in (("q", cfg.cq), ("k", cfg.ck)):
        init = synth.gather_init(x[name], synth.kmeans_init_indices(cfg, name, c))
        ties, _ = _lockstep(x[name], init, c, cfg.iters, torch.float32)
        assert ties == 0


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("c", [1, 37, 90, 128, 300, 1100])
def test_small_video_lockstep_bf16(d, c):
    cfg = synth.CONFIGS["5s"].with_(T=3, heads=2, d=d)      # 4,680 tokens, ragged tile tail
    x = synth.video_qkv(cfg)["k"]
    init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "k", c))
    ties, refined = _lockstep(x, init, c, 4, torch.bfloat16)
    assert ties <= 2


def test_mfma_accumulation_model():
    """The hardware model the k-means error bound assumes: the bf16 MFMA
    accumulates in fp32 and loses at most one unit in the last place per
    addition (2^-23), whatever the order of its additions."""
    assert sva_check_mfma_rounding() == [1] * 8


def test_many_slices_few_tokens():
    """More slices than compute units with one 64-token tile each (ragged):
    one workgroup per slice in the resident-table pass."""
    cfg = synth.CONFIGS["5s"].with_(T=1, H=6, W=13, heads=300, d=64)   # 78 tokens
    x = synth.video_qkv(cfg)["q"]
    init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "q", 20))
    ties, _ = _lockstep(x, init, 20, 2, torch.bfloat16)
    assert ties <= 2


@pytest.mark.parametrize("w,d", [(5, 128), (64, 64), (65, 128), (128, 128)])
def test_resident_pass_tile_edges(w, d):
    """Slices of fewer than one 64-token tile, exactly one or two tiles, and one
    token past a tile (the resident-table pass, C <= 128)."""
    cfg = synth.CONFIGS["5s"].with_(T=1, H=1, W=w, heads=5, d=d)
    x = synth.video_qkv(cfg)["q"]
    c = min(3, w)
    init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "q", c))
    ties, _ = _lockstep(x, init, c, 2, torch.bfloat16)
    assert ties == 0


def test_pair_path_with_duplicate_centroids():
    # 1,100 clusters (35 centroid tiles: the two-candidate path is on) with one
    # centroid doubled and one tripled, in different tiles and at the same row
    # of a tile (bit-equal w with equal row bits): rows nearest a doubled
    # centroid are two-candidate rows that tie exactly (the lower id wins),
    # rows nearest the tripled one have three candidates (refine pass)
    cfg = synth.CONFIGS["5s"].with_(T=2, heads=2)             # 3,120 tokens
    x = synth.video_qkv(cfg)["k"]
    c = 1100
    init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "k", c)).copy()
    for h in range(2):
        init[0, h, 32 + 7] = init[0, h, 7]                    # same row of tiles 0 and 1
        init[0, h, 96 + 20] = init[0, h, 20]
        init[0, h, 160 + 20] = init[0, h, 20]
        init[0, h, 250] = init[0, h, 77]                      # another row, another tile
    n_ref = torch.zeros(1, dtype=torch.int32, device=device())
    cent = to_dev(init.astype(np.float32))
    _, assign, _ = sva_kmeans(to_dev(x, torch.bfloat16), c, 1, cent, n_refined=n_ref)
    a = host(assign)
    ties = 0
    for h in range(2):
        ref, margin = oracle.assign_step(x[0, h].astype(np.float64), init[0, h].astype(np.float64))
        ties += assign_parity(a[0, h], ref, margin, f"head {h}")
        # the duplicates tie exactly: the lowest id must win on the GPU too
        dup = np.isin(ref, [7, 20, 77])
        assert dup.sum() >= 3, "the duplicated clusters must own some rows"
        assert np.array_equal(a[0, h][dup], ref[dup]), (h, np.flatnonzero(a[0, h][dup] != ref[dup]))
        assert not np.isin(a[0, h], [32 + 7, 96 + 20, 160 + 20, 250]).any()
    assert ties <= 2
    assert int(n_ref.item()) > 0


def test_empty_cluster_keeps_centroid_and_c_equals_n():
    dev = device()
    rng = np.random.default_rng(0)
    x = synth.round_bf16(rng.standard_normal((1, 1, 64, 128)).astype(np.float32))
    init = np.stack([x[0, 0, :5], x[0, 0, :5]]).reshape(1, 1, 10, 128)   # 5 duplicates
    init[0, 0, 9] = 100.0                                                 # and a far one
    cent = to_dev(init)
    _, a, s = sva_kmeans(to_dev(x, torch.bfloat16), 10, 1, cent)
    s = host(s)[0, 0]
    assert (s[5:] == 0).all()          # duplicates lose every tie; the far one is empty
    np.testing.assert_array_equal(host(cent)[0, 0, 5:], init[0, 0, 5:])
    # c == n with each row its own initial centroid: every row keeps itself
    cent = to_dev(x.copy())
    _, a, s = sva_kmeans(to_dev(x, torch.bfloat16), 64, 2, cent)
    assert np.array_equal(host(a)[0, 0], np.arange(64))


def test_chained_ten_iterations_tiny_exact():
    cfg = synth.CONFIGS["tiny"]
    x = synth.video_qkv(cfg)
    for name, c in (("q", cfg.cq), ("k", cfg.ck)):
        idx = synth.kmeans_init_indices(cfg, name, c)
        init = synth.gather_init(x[name], idx)
        cent = to_dev(init)
        _, a, s = sva_kmeans(to_dev(x[name]), c, cfg.iters, cent)
        for h in range(cfg.heads):
            r = oracle.kmeans(x[name][0, h].astype(np.float64), init[0, h].astype(np.float64),
                              cfg.iters)
            assert np.array_equal(host(a)[0, h], r.assign)
            np.testing.assert_allclose(host(cent)[0, h], r.centroids, rtol=1e-6, atol=1e-7)


def test_deterministic_bf16():
    cfg = synth.CONFIGS["5s"].with_(T=2, heads=3)
    x = synth.video_qkv(cfg)["q"]
    init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "q", 50))
    xt = to_dev(x, torch.bfloat16)
    c1, c2 = to_dev(init), to_dev(init)
    _, a1, _ = sva_kmeans(xt, 50, 5, c1)
    _, a2, _ = sva_kmeans(xt, 50, 5, c2)
    assert torch.equal(a1, a2) and torch.equal(c1, c2)


@pytest.fixture(scope="module")
def video_5s():
    cfg = synth.CONFIGS["5s"]
    return cfg, synth.video_qkv(cfg)


@pytest.mark.parametrize("name", ["q", "k"])
def test_full_size_lockstep_two_iterations(video_5s, name):
    """32,760 tokens x 40 heads, C_q = 100 / C_k = 500, every head checked."""
    cfg, x = video_5s
    c = cfg.cq if name == "q" else cfg.ck
    init = synth.gather_init(x[name], synth.kmeans_init_indices(cfg, name, c))
    ties, refined = _lockstep(x[name], init, c, 2, torch.bfloat16)
    print(f"\n{name}: tie mismatches {ties}, rows re-decided in fp64 {refined} "
          f"({refined / (2 * cfg.heads * cfg.n):.3%})")
    assert ties <= 10


def test_warm_start_lockstep_bf16():
    """The centroid cache (Sparse VideoGen2, section 2.c): the next denoising
    step's k-means starts from this step's GPU centroids; every warm iteration
    matches the oracle's Lloyd step in lockstep."""
    cfg = synth.CONFIGS["5s"].with_(T=3, heads=2)
    x0 = synth.video_qkv(cfg)["k"]
    delta = synth.denoise_direction(cfg, "k")
    c = 300
    init = synth.gather_init(x0, synth.kmeans_init_indices(cfg, "k", c))
    cent = to_dev(init)
    sva_kmeans(to_dev(x0, torch.bfloat16), c, cfg.iters, cent)
    warm = host(cent)
    x1 = synth.at_denoise_step(x0, delta, 1, 0.05)
    ties, _ = _lockstep(x1, warm, c, 3, torch.bfloat16)
    assert ties <= 2


def test_layer_warm_start_equals_explicit_init():
    from sparse_attention_long_head_amd import SparseVideoAttention
    cfg = synth.CONFIGS["5s"].with_(T=3, heads=2)
    x = synth.video_qkv(cfg)
    dq, dk = synth.denoise_direction(cfg, "q"), synth.denoise_direction(cfg, "k")
    iq = to_dev(synth.gather_init(x["q"], synth.kmeans_init_indices(cfg, "q", 40)))
    ik = to_dev(synth.gather_init(x["k"], synth.kmeans_init_indices(cfg, "k", 200)))
    t0 = {n: to_dev(x[n], torch.bfloat16) for n in "qkv"}
    t1 = {"q": to_dev(synth.at_denoise_step(x["q"], dq, 1, 0.05), torch.bfloat16),
          "k": to_dev(synth.at_denoise_step(x["k"], dk, 1, 0.05), torch.bfloat16), "v": t0["v"]}
    a = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, 40, 200, 10, 0.9, device=device(),
                             iters_warm=3)
    with pytest.raises(ValueError):
        a(t0["q"], t0["k"], t0["v"])                      # nothing cached yet
    a(t0["q"], t0["k"], t0["v"], iq, ik)
    cq, ck = a.cent_q.clone(), a.cent_k.clone()
    o_warm = a(t1["q"], t1["k"], t1["v"]).clone()      # warm: 3 iterations from the cache
    b = SparseVideoAttention(1, cfg.heads, cfg.n, cfg.d, 40, 200, 3, 0.9, device=device())
    o_cold = b(t1["q"], t1["k"], t1["v"], cq, ck)
    assert torch.equal(o_warm, o_cold)
    assert torch.equal(a.assign_k, b.assign_k) and torch.equal(a.cent_q, b.cent_q)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("c", [1, 37, 90, 128, 300, 1100])
def test_candidate_path_lockstep_bf16(d, c):
    """Iterations 2-4 run over the candidate clusters of each token's previous
    cluster (one to 35 centroid tiles, lists of every size up to a fallback
    to all clusters when a list overflows)."""
    cfg = synth.CONFIGS["5s"].with_(T=3, heads=2, d=d)      # 4,680 tokens, ragged tail
    x = synth.video_qkv(cfg)["k"]
    init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "k", c))
    assert _lockstep_chained(x, init, c, 4) <= 2


def test_candidate_path_wide_radius_and_few_tokens():
    """Centre scale 1 (clusters overlap, long candidate lists and fallbacks)
    and slices of 5 / 65 tokens (one partial group, a group past a tile)."""
    cfg = synth.CONFIGS["5s"].with_(T=2, heads=2, alpha=1.0)
    x = synth.video_qkv(cfg)["q"]
    init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "q", 200))
    assert _lockstep_chained(x, init, 200, 3) <= 2
    for w in (5, 65):
        cfg = synth.CONFIGS["5s"].with_(T=1, H=1, W=w, heads=3)
        x = synth.video_qkv(cfg)["k"]
        c = min(4, w)
        init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "k", c))
        assert _lockstep_chained(x, init, c, 3) == 0


def test_candidate_path_duplicate_centroids():
    """Exact ties on the candidate path.  Two blocks of 64 identical rows far
    from the rest of the data, one with a doubled and one with a tripled
    initial centroid on it: each block's cluster keeps exactly its block, its
    mean never moves, and the empty copies keep their centroids, so every
    iteration sees bit-equal distances that must go to the lowest id."""
    cfg = synth.CONFIGS["5s"].with_(T=2, heads=2)             # 3,120 tokens
    x = synth.video_qkv(cfg)["k"].copy()
    c = 600
    rng = np.random.default_rng(11)
    for h in range(2):
        for r0 in (100, 1500):
            far = synth.round_bf16((40.0 * rng.standard_normal(cfg.d)).astype(np.float32))
            x[0, h, r0:r0 + 64] = far
    init = synth.gather_init(x, synth.kmeans_init_indices(cfg, "k", c)).copy()
    for h in range(2):
        init[0, h, 7] = init[0, h, 32 + 7] = x[0, h, 100]          # doubled, same tile row
        init[0, h, 20] = init[0, h, 96 + 20] = init[0, h, 160 + 20] = x[0, h, 1500]
    assert _lockstep_chained(x, init, c, 4) <= 2
    cent = to_dev(init.astype(np.float32))
    _, a, s = sva_kmeans(to_dev(x, torch.bfloat16), c, 4, cent)
    a = host(a)
    for h in range(2):
        assert (a[0, h, 100:164] == 7).all() and (a[0, h, 1500:1564] == 20).all()
    assert not np.isin(a, [32 + 7, 96 + 20, 160 + 20]).any()


@pytest.mark.parametrize("name", ["q", "k"])
def test_full_size_candidate_iteration_lockstep(video_5s, name):
    """Iteration 2 at 32,760 tokens x 40 heads, every head: the first
    iteration that runs over candidates."""
    cfg, x = video_5s
    c = cfg.cq if name == "q" else cfg.ck
    init = synth.gather_init(x[name], synth.kmeans_init_indices(cfg, name, c))
    ties = _lockstep_chained(x[name], init, c, 2)
    print(f"\n{name}: iteration 2 tie mismatches {ties}")
    assert ties <= 10


@pytest.mark.parametrize("name", ["q", "k"])
def test_full_size_chained_ten_iterations(video_5s, name):
    """Each side runs its own 10 iterations from the same initial centroids
    (no lockstep): a near tie decided differently changes later centroids, so
    the final assignments may differ in a cascade.  Counted and bounded on 8
    of the 40 heads."""
    cfg, x = video_5s
    c = cfg.cq if name == "q" else cfg.ck
    heads = (0, 5, 10, 15, 20, 25, 30, 35)
    init = synth.gather_init(x[name], synth.kmeans_init_indices(cfg, name, c))
    cent = to_dev(init)
    _, a, _ = sva_kmeans(to_dev(x[name], torch.bfloat16), c, cfg.iters, cent)
    a = host(a)
    diff = 0
    for h in heads:
        r = oracle.kmeans(x[name][0, h].astype(np.float64), init[0, h].astype(np.float64),
                          cfg.iters)
        diff += int((a[0, h] != r.assign).sum())
    print(f"\n{name}: rows that differ after 10 chained iterations {diff} of "
          f"{len(heads) * cfg.n}")
    assert diff <= 0.002 * len(heads) * cfg.n
