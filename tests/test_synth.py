"""Checks of the seeded input generator (CPU only)."""
import numpy as np

import synth


def test_deterministic_and_head_subsets_agree():
    cfg = synth.CONFIGS["tiny"]
    a = synth.video_qkv(cfg)
    b = synth.video_qkv(cfg, heads=(1,))
    for n in "qkv":
        assert a[n].shape == (1, 2, 256, 64)
        assert np.array_equal(a[n][:, 1:], b[n])
    c = synth.video_qkv(cfg)
    assert all(np.array_equal(a[n], c[n]) for n in "qkv")


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0],
                 np.float32)
    got = synth.round_bf16(x)
    assert got.tolist() == [1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0, -2.5, 0.0]
    cfg = synth.CONFIGS["5s"].with_(T=2, heads=1)
    q = synth.video_qkv(cfg)["q"]
    assert np.array_equal(synth.round_bf16(q), q)


def test_static_mask_exact_count_and_radial_subset():
    cfg = synth.CONFIGS["static"]
    nb = cfg.n_blocks
    assert nb == 256
    for sp, tiles in ((0.8, 13107), (0.85, 9830)):
        m = synth.static_block_mask(cfg, sp)
        assert m.sum() == tiles
        radial = synth.radial_block_keep(cfg.n, cfg.H * cfg.W, cfg.block)
        assert (m[radial]).all()
        assert np.diag(m).all()


def test_radial_rule_by_loops():
    n, hw, block = 32760, 1560, 128
    keep = synth.radial_block_keep(n, hw, block)
    for a in range(0, 256, 17):
        for b in range(256):
            ta, tb = (a * block) // hw, (b * block) // hw
            sa, sb = (a * block % hw) // block, (b * block % hw) // block
            dt, ds = abs(ta - tb), abs(sa - sb)
            assert keep[a, b] == (dt <= 2 and ds <= (8 >> dt))


def test_init_indices_distinct_sorted():
    cfg = synth.CONFIGS["tiny"]
    idx = synth.kmeans_init_indices(cfg, "k", 37)
    for h in range(cfg.heads):
        row = idx[0, h]
        assert (np.diff(row) > 0).all() and row[0] >= 0 and row[-1] < cfg.n


def test_ell_encoding():
    m = np.array([[1, 0, 1], [0, 0, 0], [0, 1, 1]], bool)
    cnt, idx = synth.mask_to_ell(m)
    assert cnt.tolist() == [2, 0, 2]
    assert idx.tolist() == [[0, 2, -1], [-1, -1, -1], [1, 2, -1]]


def test_uniform_offsets_ragged_tail():
    off = synth.uniform_offsets(300, 128)
    assert off.tolist() == [0, 128, 256, 300]


def test_denoise_steps_are_a_fixed_drift():
    cfg = synth.CONFIGS["5s"].with_(T=2, heads=2)
    x0 = synth.video_qkv(cfg)["q"]
    d1 = synth.denoise_direction(cfg, "q")
    d2 = synth.denoise_direction(cfg, "q", heads=(1,))
    assert np.array_equal(d1[:, 1:], d2)                 # stateless per head
    assert np.array_equal(synth.at_denoise_step(x0, d1, 0, 0.05), x0)
    x2 = synth.at_denoise_step(x0, d1, 2, 0.05, dtype="f32")
    np.testing.assert_allclose(x2 - x0, 0.1 * d1, atol=1e-5)
    assert abs(float(d1.std()) - 1.0) < 0.01
