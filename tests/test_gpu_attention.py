"""GPU parity of sva_full_attn and sva_block_sparse_attn against the fp64 oracle.

Tolerance derivation (bf16 inputs, fp32 accumulation): logits are exact
products summed in fp32 (relative error ~1e-6); P is rounded to bf16 before the
PV product (relative 2^-9 per weight, averaging out over the kept keys); the
output rounds to bf16 (half an ulp: up to 2^-9 relative, i.e. ~1.6e-2 absolute
for |O| near 2..4 and ~1.1e-3 mean for N(0,1)-sized outputs).  The contract
bounds are max-abs 2e-2 and mean-abs 2e-3 in bf16 mode and 1e-4 in fp32 mode;
LSE is checked to 1e-3 (bf16) / 1e-5 (fp32) absolute.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from parity import (check_attention, check_lse, device, host, rand_inputs, to_dev)
from sparse_attention_long_head_amd import (sva_block_sparse_attn, sva_block_sparse_attn_perm,
                                          sva_full_attn, sva_set_debug_checks)

pytestmark = pytest.mark.gpu


def _tdtype(bf16):
    return torch.bfloat16 if bf16 else torch.float32


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("nq,nk", [(256, 256), (300, 333), (1, 1), (129, 5), (1000, 64)])
def test_full_attention(bf16, d, nq, nk):
    h = 2
    dt = "bf16" if bf16 else "f32"
    q = rand_inputs((1, h, nq, d), 1, dt)
    k = rand_inputs((1, h, nk, d), 2, dt)
    v = rand_inputs((1, h, nk, d), 3, dt)
    scale = 1.0 / math.sqrt(d)
    o, lse = sva_full_attn(to_dev(q, _tdtype(bf16)), to_dev(k, _tdtype(bf16)),
                           to_dev(v, _tdtype(bf16)), scale, want_lse=True)
    o, lse = host(o), host(lse)
    for hh in range(h):
        ro, rl = oracle.full_attention(q[0, hh], k[0, hh], v[0, hh], np.float32(scale))
        check_attention(o[0, hh], ro, bf16, f"head {hh}")
        check_lse(lse[0, hh], rl, 1e-3 if bf16 else 1e-5)


def test_full_attention_fp32_output_of_bf16_inputs():
    q, k, v = (rand_inputs((1, 1, 700, 128), s) for s in (4, 5, 6))
    o, _ = sva_full_attn(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16),
                         to_dev(v, torch.bfloat16), 1 / math.sqrt(128), o_dtype=torch.float32)
    ro, _ = oracle.full_attention(q[0, 0], k[0, 0], v[0, 0], np.float32(1 / math.sqrt(128)))
    err = np.abs(host(o)[0, 0] - ro)
    # without the final bf16 rounding only the kernel's own error remains
    assert err.max() < 4e-3 and err.mean() < 3e-4, (err.max(), err.mean())


def _uniform_case(n, block, heads, seed, density, bf16, d):
    rng = np.random.default_rng(seed)
    nb = -(-n // block)
    masks = rng.random((heads, nb, nb)) < density
    masks[:, np.arange(nb), np.arange(nb)] = True
    masks[0, nb - 1, :] = False          # one query block keeps nothing
    dt = "bf16" if bf16 else "f32"
    q, k, v = (rand_inputs((1, heads, n, d), seed + i, dt) for i in range(3))
    off = np.tile(synth.uniform_offsets(n, block), (1, heads, 1))
    cnt, idx = synth.mask_to_ell(masks[None])
    return q, k, v, masks, off, cnt, idx


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_uniform_blocks_ragged(bf16, d):
    n, block, heads = 1000, 128, 3
    q, k, v, masks, off, cnt, idx = _uniform_case(n, block, heads, 11, 0.4, bf16, d)
    T = _tdtype(bf16)
    scale = 1 / math.sqrt(d)
    o, lse = sva_block_sparse_attn(to_dev(q, T), to_dev(k, T), to_dev(v, T),
                                   to_dev(off, torch.int32), to_dev(off, torch.int32),
                                   to_dev(cnt, torch.int32), to_dev(idx, torch.int32), scale,
                                   want_lse=True)
    o, lse = host(o), host(lse)
    for h in range(heads):
        ro, rl = oracle.block_sparse_attention(q[0, h], k[0, h], v[0, h], masks[h], block,
                                               np.float32(scale))
        check_attention(o[0, h], ro, bf16, f"head {h}")
        check_lse(lse[0, h], rl, 1e-3 if bf16 else 1e-5)
    # the query block that keeps nothing: O = 0, LSE = -inf
    assert (o[0, 0, 896:] == 0).all() and np.isneginf(lse[0, 0, 896:]).all()


def _random_partition(n, nb, rng, extreme=True):
    cuts = np.sort(rng.integers(0, n + 1, nb - 1))
    if extreme and nb > 4:
        cuts[0] = cuts[1]            # an empty block
        cuts[2] = max(cuts[1], cuts[3] - 1)   # often a 1-row block
    off = np.concatenate([[0], cuts, [n]]).astype(np.int32)
    return off


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_variable_blocks(bf16, seed):
    rng = np.random.default_rng(seed)
    heads, d, nq, nk, nqb, nkb = 2, 128, 777, 901, 9, 23
    dt = "bf16" if bf16 else "f32"
    q = rand_inputs((1, heads, nq, d), 20 + seed, dt)
    k = rand_inputs((1, heads, nk, d), 30 + seed, dt)
    v = rand_inputs((1, heads, nk, d), 40 + seed, dt)
    qoff = np.stack([_random_partition(nq, nqb, rng) for _ in range(heads)])[None]
    koff = np.stack([_random_partition(nk, nkb, rng) for _ in range(heads)])[None]
    masks = rng.random((1, heads, nqb, nkb)) < 0.35
    masks[0, 0, 1] = False
    cnt, idx = synth.mask_to_ell(masks)
    T = _tdtype(bf16)
    scale = 1 / math.sqrt(d)
    o, lse = sva_block_sparse_attn(to_dev(q, T), to_dev(k, T), to_dev(v, T),
                                   to_dev(qoff, torch.int32), to_dev(koff, torch.int32),
                                   to_dev(cnt, torch.int32), to_dev(idx, torch.int32), scale,
                                   want_lse=True)
    o, lse = host(o), host(lse)
    for h in range(heads):
        aq = np.repeat(np.arange(nqb), np.diff(qoff[0, h]))
        ak = np.repeat(np.arange(nkb), np.diff(koff[0, h]))
        ro, rl = oracle.cluster_sparse_attention(q[0, h], k[0, h], v[0, h], aq, ak, masks[0, h],
                                                 np.float32(scale))
        check_attention(o[0, h], ro, bf16, f"head {h}")
        check_lse(lse[0, h], rl, 1e-3 if bf16 else 1e-5)


def test_many_slices_per_xcd():
    # 3 x 30 = 90 slices: up to 12 dealt to one XCD, so the work queues group
    # two slices per sort group; every slice must still be complete and exact
    rng = np.random.default_rng(21)
    b, heads, d, nq, nk, nqb, nkb = 3, 30, 64, 300, 260, 5, 7
    q = rand_inputs((b, heads, nq, d), 70, "bf16")
    k = rand_inputs((b, heads, nk, d), 71, "bf16")
    v = rand_inputs((b, heads, nk, d), 72, "bf16")
    qoff = np.stack([np.stack([_random_partition(nq, nqb, rng) for _ in range(heads)])
                     for _ in range(b)])
    koff = np.stack([np.stack([_random_partition(nk, nkb, rng) for _ in range(heads)])
                     for _ in range(b)])
    masks = rng.random((b, heads, nqb, nkb)) < 0.5
    masks[..., 0] = True
    cnt, idx = synth.mask_to_ell(masks)
    T = _tdtype(True)
    scale = 1 / math.sqrt(d)
    o, lse = sva_block_sparse_attn(to_dev(q, T), to_dev(k, T), to_dev(v, T),
                                   to_dev(qoff, torch.int32), to_dev(koff, torch.int32),
                                   to_dev(cnt, torch.int32), to_dev(idx, torch.int32), scale,
                                   want_lse=True)
    o, lse = host(o), host(lse)
    for bi in range(b):
        for h in range(heads):
            aq = np.repeat(np.arange(nqb), np.diff(qoff[bi, h]))
            ak = np.repeat(np.arange(nkb), np.diff(koff[bi, h]))
            ro, rl = oracle.cluster_sparse_attention(q[bi, h], k[bi, h], v[bi, h], aq, ak,
                                                     masks[bi, h], np.float32(scale))
            check_attention(o[bi, h], ro, True, f"slice {bi},{h}")
            check_lse(lse[bi, h], rl, 1e-3)


@pytest.mark.parametrize("bf16", [False, True])
def test_one_key_blocks_and_empty_blocks(bf16):
    # every kept key block holds one key or none: a 64-key chunk then spans 64
    # key blocks (the most it can), with empty blocks interleaved in the list
    rng = np.random.default_rng(9)
    d, nq, nk = 64, 150, 333
    sizes = np.ones(300, np.int32)
    sizes[3::7] = 0                                  # empty blocks in between
    sizes[-1] = nk - sizes[:-1].sum()                # one large block at the end
    koff = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)[None, None]
    nkb = sizes.size
    dt = "bf16" if bf16 else "f32"
    q = rand_inputs((1, 1, nq, d), 60, dt)
    k = rand_inputs((1, 1, nk, d), 61, dt)
    v = rand_inputs((1, 1, nk, d), 62, dt)
    qoff = np.array([[[0, 70, nq]]], np.int32)
    masks = np.ones((1, 1, 2, nkb), bool)
    masks[0, 0, 1] = rng.random(nkb) < 0.6
    cnt, idx = synth.mask_to_ell(masks)
    T = _tdtype(bf16)
    scale = 1 / math.sqrt(d)
    o, lse = sva_block_sparse_attn(to_dev(q, T), to_dev(k, T), to_dev(v, T),
                                   to_dev(qoff, torch.int32), to_dev(koff, torch.int32),
                                   to_dev(cnt, torch.int32), to_dev(idx, torch.int32), scale,
                                   want_lse=True)
    aq = np.repeat(np.arange(2), np.diff(qoff[0, 0]))
    ak = np.repeat(np.arange(nkb), sizes)
    ro, rl = oracle.cluster_sparse_attention(q[0, 0], k[0, 0], v[0, 0], aq, ak, masks[0, 0],
                                             np.float32(scale))
    check_attention(host(o)[0, 0], ro, bf16)
    check_lse(host(lse)[0, 0], rl, 1e-3 if bf16 else 1e-5)


@pytest.mark.parametrize("d", [64, 128])
def test_split_pairs_on_small_query_blocks(d):
    # Q blocks of at most 128 rows (so the two waves of a SIMD split each
    # chunk's keys): key lists of 5, 20 and 32 keys leave the second key half
    # empty in every chunk, others end a chunk with 1..32 keys; one query
    # block keeps nothing, one holds a single row
    rng = np.random.default_rng(33 + d)
    heads, nq = 2, 700
    qsizes = np.array([128, 1, 100, 128, 64, 33, 120, 126], np.int32)
    assert qsizes.sum() == nq
    ksizes = np.array([5, 20, 32, 1, 64, 97, 128, 3, 40, 250, 7, 33], np.int32)
    nk, nqb, nkb = int(ksizes.sum()), qsizes.size, ksizes.size
    qoff = np.tile(np.concatenate([[0], np.cumsum(qsizes)]).astype(np.int32), (1, heads, 1))
    koff = np.tile(np.concatenate([[0], np.cumsum(ksizes)]).astype(np.int32), (1, heads, 1))
    masks = rng.random((1, heads, nqb, nkb)) < 0.3
    masks[0, :, 0] = False
    masks[0, :, 0, 0] = True            # 5 keys
    masks[0, :, 1] = False
    masks[0, :, 1, 1] = True            # 20 keys, a 1-row query block
    masks[0, :, 2] = False
    masks[0, :, 2, [2, 3]] = True       # 33 keys
    masks[0, 0, 3] = False              # keeps nothing (head 0)
    cnt, idx = synth.mask_to_ell(masks)
    q = rand_inputs((1, heads, nq, d), 80, "bf16")
    k = rand_inputs((1, heads, nk, d), 81, "bf16")
    v = rand_inputs((1, heads, nk, d), 82, "bf16")
    scale = 1 / math.sqrt(d)
    T = torch.bfloat16
    o, lse = sva_block_sparse_attn(to_dev(q, T), to_dev(k, T), to_dev(v, T),
                                   to_dev(qoff, torch.int32), to_dev(koff, torch.int32),
                                   to_dev(cnt, torch.int32), to_dev(idx, torch.int32), scale,
                                   want_lse=True)
    o, lse = host(o), host(lse)
    for h in range(heads):
        aq = np.repeat(np.arange(nqb), qsizes)
        ak = np.repeat(np.arange(nkb), ksizes)
        ro, rl = oracle.cluster_sparse_attention(q[0, h], k[0, h], v[0, h], aq, ak, masks[0, h],
                                                 np.float32(scale))
        check_attention(o[0, h], ro, True, f"head {h}")
        check_lse(lse[0, h], rl, 1e-3)
    rows3 = slice(int(qoff[0, 0, 3]), int(qoff[0, 0, 4]))
    assert (o[0, 0, rows3] == 0).all() and np.isneginf(lse[0, 0, rows3]).all()


def _growing_keys(k, jumps):
    """Scale key rows so that the scores grow along the key sequence: every
    64-key chunk c is multiplied by (1 + c), and the rows listed in ``jumps``
    (row -> factor) further, rounded back to bf16."""
    k = k.copy()
    for c in range(-(-k.shape[-2] // 64)):
        k[..., 64 * c:64 * (c + 1), :] *= 1.0 + c
    for row, f in jumps.items():
        k[..., row, :] *= f
    return synth.round_bf16(k.astype(np.float32))


@pytest.mark.parametrize("mode", ["dense", "split", "perm"])
def test_rescale_when_later_chunks_score_higher(mode):
    # The running max is taken on a list's first chunk only, and again when a
    # lane's sum of P shows some P above 2^8; then the chunk is redone.  Scores
    # that grow chunk by chunk (and single keys 20x and 40x larger, whose P
    # would be ~2^90 and overflow to inf against the stale max) force that
    # path repeatedly, in the full, split (key halves) and permuted kernels.
    d, heads = 128, 2
    nq, nk = 256, 64 * 7 + 13
    q = rand_inputs((1, heads, nq, d), 90, "bf16")
    k = _growing_keys(rand_inputs((1, heads, nk, d), 91, "bf16"), {200: 20.0, 5 * 64 + 17: 40.0})
    v = rand_inputs((1, heads, nk, d), 92, "bf16")
    scale = 1 / math.sqrt(d)
    T = torch.bfloat16
    if mode == "dense":
        o, lse = sva_full_attn(to_dev(q, T), to_dev(k, T), to_dev(v, T), scale, want_lse=True)
        refs = [oracle.full_attention(q[0, h], k[0, h], v[0, h], np.float32(scale))
                for h in range(heads)]
    else:
        # two 128-row query blocks (split mode) or one 256-row block (perm),
        # every key in one block that both keep
        qs = [128, 128] if mode == "split" else [256]
        qoff = np.tile(np.concatenate([[0], np.cumsum(qs)]).astype(np.int32), (1, heads, 1))
        koff = np.tile(np.array([0, nk], np.int32), (1, heads, 1))
        masks = np.ones((1, heads, len(qs), 1), bool)
        cnt, idx = synth.mask_to_ell(masks)
        args = (to_dev(qoff, torch.int32), to_dev(koff, torch.int32), to_dev(cnt, torch.int32),
                to_dev(idx, torch.int32), scale)
        if mode == "split":
            o, lse = sva_block_sparse_attn(to_dev(q, T), to_dev(k, T), to_dev(v, T), *args,
                                           want_lse=True)
        else:
            rng = np.random.default_rng(93)
            pq = np.stack([rng.permutation(nq) for _ in range(heads)])[None].astype(np.int32)
            pk = np.stack([rng.permutation(nk) for _ in range(heads)])[None].astype(np.int32)
            o, lse = sva_block_sparse_attn_perm(to_dev(q, T), to_dev(k, T), to_dev(v, T),
                                                to_dev(pq, torch.int32), to_dev(pk, torch.int32),
                                                *args, want_lse=True)
        refs = [oracle.full_attention(q[0, h], k[0, h], v[0, h], np.float32(scale))
                for h in range(heads)]
    o, lse = host(o), host(lse)
    for h in range(heads):
        check_attention(o[0, h], refs[h][0], True, f"{mode} head {h}")
        check_lse(lse[0, h], refs[h][1], 1e-3 * max(1.0, float(np.abs(refs[h][1]).max()) / 100))


def test_kept_list_longer_than_one_lds_segment():
    # 1300 two-key blocks, all kept: the kept list is walked in several segments
    rng = np.random.default_rng(5)
    d, nq, nkb = 128, 200, 1300
    nk = 2 * nkb
    q = rand_inputs((1, 1, nq, d), 50)
    k = rand_inputs((1, 1, nk, d), 51)
    v = rand_inputs((1, 1, nk, d), 52)
    qoff = np.array([[[0, 77, nq]]], np.int32)
    koff = (2 * np.arange(nkb + 1, dtype=np.int32))[None, None]
    masks = np.ones((1, 1, 2, nkb), bool)
    masks[0, 0, 1] = rng.random(nkb) < 0.85
    cnt, idx = synth.mask_to_ell(masks)
    scale = 1 / math.sqrt(d)
    o, _ = sva_block_sparse_attn(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16),
                                 to_dev(v, torch.bfloat16), to_dev(qoff, torch.int32),
                                 to_dev(koff, torch.int32), to_dev(cnt, torch.int32),
                                 to_dev(idx, torch.int32), scale)
    aq = np.repeat(np.arange(2), np.diff(qoff[0, 0]))
    ak = np.repeat(np.arange(nkb), 2)
    ro, _ = oracle.cluster_sparse_attention(q[0, 0], k[0, 0], v[0, 0], aq, ak, masks[0, 0],
                                            np.float32(scale))
    check_attention(host(o)[0, 0], ro, True)


def test_deterministic():
    q, k, v, masks, off, cnt, idx = _uniform_case(1500, 128, 2, 3, 0.3, True, 128)
    args = [to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16),
            to_dev(off, torch.int32), to_dev(off, torch.int32), to_dev(cnt, torch.int32),
            to_dev(idx, torch.int32), 0.088]
    a, _ = sva_block_sparse_attn(*args)
    b, _ = sva_block_sparse_attn(*args)
    assert torch.equal(a, b)


@pytest.mark.parametrize("bf16", [False, True])
def test_nan_reaches_exactly_the_rows_that_read_it(bf16):
    """The NaN rule on the GPU (both kernels; bf16 here also runs the split
    mode): a NaN in a query row, in a kept K row or in an element of a kept V row
    puts NaN exactly where the oracle has it (all of O_n and LSE_n, all of O_n
    and LSE_n, O_n[c] only), and every other output is bitwise the clean run's.
    A key block that no query block keeps may hold NaN in K and V: nothing
    reads it."""
    n, block, heads, d = 1000, 128, 3, 128
    q, k, v, masks, off, cnt, idx = _uniform_case(n, block, heads, 11, 0.4, bf16, d)
    masks[1, :, 5] = False                   # head 1: key block 5 kept by nobody
    cnt, idx = synth.mask_to_ell(masks[None])
    T = _tdtype(bf16)
    scale = 1 / math.sqrt(d)

    def run(qq, kk, vv):
        o, lse = sva_block_sparse_attn(to_dev(qq, T), to_dev(kk, T), to_dev(vv, T),
                                       to_dev(off, torch.int32), to_dev(off, torch.int32),
                                       to_dev(cnt, torch.int32), to_dev(idx, torch.int32),
                                       scale, want_lse=True)
        return host(o), host(lse)

    o0, l0 = run(q, k, v)
    qn, kn, vn = q.copy(), k.copy(), v.copy()
    kn[0, 0, 300, 5] = np.nan                # head 0: one K element (key block 2)
    vn[0, 1, 450, 7] = np.nan                # head 1: one V element (key block 3)
    kn[0, 1, 640:768] = np.nan               # head 1: the unkept key block
    vn[0, 1, 640:768] = np.nan
    qn[0, 2, 777, 0] = np.nan                # head 2: one query element
    o, lse = run(qn, kn, vn)
    for h in range(heads):
        ro, rl = oracle.block_sparse_attention(qn[0, h], kn[0, h], vn[0, h], masks[h], block,
                                               np.float32(scale))
        nan_o, nan_l = np.isnan(ro), np.isnan(rl)
        assert nan_o.any() and (~nan_o).any(), h
        assert np.array_equal(np.isnan(o[0, h]), nan_o), h
        assert np.array_equal(np.isnan(lse[0, h]), nan_l), h
        assert np.array_equal(o[0, h][~nan_o], o0[0, h][~nan_o]), h
        assert np.array_equal(lse[0, h][~nan_l], l0[0, h][~nan_l]), h


def test_debug_checks_catch_bad_device_indices():
    """Debug mode: a call whose device arrays break the layout's preconditions
    is refused with SVA_EINVAL naming the violation, and the attention is not
    launched; a valid call gives the same bits as without the checks.  Every
    violation used here would stay inside the buffers even if the attention
    were launched (ranges of negative length are skipped, ids and rows one past
    the end land in the next slice)."""
    n, block, heads, d = 1000, 128, 3, 128
    q, k, v, masks, off, cnt, idx = _uniform_case(n, block, heads, 5, 0.4, True, d)
    masks[1, 0, :] = True                    # head 1, block 0 keeps every key block
    cnt, idx = synth.mask_to_ell(masks[None])
    nb = masks.shape[-1]
    qd, kd, vd = (to_dev(x, torch.bfloat16) for x in (q, k, v))
    scale = 1 / math.sqrt(d)

    def call(qoff, koff, c, i, perm=None):
        if perm is None:
            return sva_block_sparse_attn(qd, kd, vd, to_dev(qoff, torch.int32),
                                         to_dev(koff, torch.int32), to_dev(c, torch.int32),
                                         to_dev(i, torch.int32), scale)[0]
        return sva_block_sparse_attn_perm(qd, kd, vd, to_dev(perm, torch.int32),
                                          to_dev(np.tile(np.arange(n), (1, heads, 1)),
                                                 torch.int32),
                                          to_dev(qoff, torch.int32), to_dev(koff, torch.int32),
                                          to_dev(c, torch.int32), to_dev(i, torch.int32),
                                          scale)[0]

    ref = call(off, off, cnt, idx)
    sva_set_debug_checks(True)
    try:
        assert torch.equal(call(off, off, cnt, idx), ref)
        bad_q = off.copy()
        bad_q[0, 0, 2] = 100                 # block 1 = [128, 100): not monotone
        bad_k = off.copy()
        bad_k[0, 2, 2] = 320                 # head 2: key block 1 = [128, 320),
        bad_k[0, 2, 3] = 300                 # block 2 = [320, 300), block 3 = [300, 384)
        bad_c = cnt.copy()
        bad_c[0, 1, 0] = nb + 1              # more than the row's stride holds
        bad_i = idx.copy()
        bad_i[0, 0, 3, 0] = nb               # a kept id past the last key block
        bad_p = np.tile(np.arange(n), (1, heads, 1)).astype(np.int32)
        bad_p[0, 0, 17] = n                  # a query row past the slice
        for args, perm, what in [((bad_q, off, cnt, idx), None, "q_offsets"),
                                 ((off, bad_k, cnt, idx), None, "k_offsets"),
                                 ((off, off, bad_c, idx), None, "kept_count"),
                                 ((off, off, cnt, bad_i), None, "kept_idx"),
                                 ((off, off, cnt, idx), bad_p, "q_perm")]:
            with pytest.raises(RuntimeError, match=what):
                call(*args, perm=perm)
        with pytest.raises(RuntimeError, match="q_offsets.*kept_idx"):
            call(bad_q, off, cnt, bad_i)
        assert torch.equal(call(off, off, cnt, idx), ref)   # nothing sticks
    finally:
        sva_set_debug_checks(False)


@pytest.fixture(scope="module")
def static_full():
    """The static-mask workload at full size: 32,760 tokens x 40 heads, d=128,
    i.i.d. N(0,1) bf16, radial + random mask at 80% sparsity (shared by heads)."""
    cfg = synth.CONFIGS["static"]
    x = synth.video_qkv(cfg)
    mask = synth.static_block_mask(cfg)
    return cfg, x, mask


def _sample_rows(n, rng, k=24):
    fixed = [0, 1, 127, 128, 255, n // 2, n - 121, n - 120, n - 1]
    return np.unique(np.concatenate([fixed, rng.integers(0, n, k)]))


def test_static_config_full_size_sampled(static_full):
    cfg, x, mask = static_full
    dev = device()
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in "qkv")
    off = np.tile(synth.uniform_offsets(cfg.n, cfg.block), (1, cfg.heads, 1))
    cnt, idx = synth.mask_to_ell(np.broadcast_to(mask, (1, cfg.heads) + mask.shape))
    scale = 1 / math.sqrt(cfg.d)
    o, lse = sva_block_sparse_attn(q, k, v, to_dev(off, torch.int32), to_dev(off, torch.int32),
                                   to_dev(cnt, torch.int32), to_dev(idx, torch.int32), scale,
                                   want_lse=True)
    o, lse = host(o), host(lse)
    rng = np.random.default_rng(0)
    for h in (0, 17, 39):
        rows = _sample_rows(cfg.n, rng)
        ro, rl = oracle.block_sparse_attention(x["q"][0, h], x["k"][0, h], x["v"][0, h], mask,
                                               cfg.block, np.float32(scale), rows=rows)
        check_attention(o[0, h, rows], ro, True, f"static head {h}")
        check_lse(lse[0, h, rows], rl, 1e-3)


def test_dense_full_size_sampled(static_full):
    cfg, x, _ = static_full
    dev = device()
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(torch.bfloat16) for n in "qkv")
    scale = 1 / math.sqrt(cfg.d)
    o, _ = sva_full_attn(q, k, v, scale)
    o = host(o)
    rng = np.random.default_rng(1)
    for h in (3, 38):
        rows = _sample_rows(cfg.n, rng, 8)
        ro, _ = oracle.full_attention(x["q"][0, h], x["k"][0, h], x["v"][0, h],
                                      np.float32(scale), rows=rows)
        check_attention(o[0, h, rows], ro, True, f"dense head {h}")


@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_fused_permutation_equals_gather_attend_scatter(bf16, d):
    # sva_block_sparse_attn_perm on original-order tensors must equal, bit for
    # bit, gathering q[q_perm], k[k_perm], v[k_perm], sva_block_sparse_attn and
    # scattering the output back; and it must match the oracle in original
    # coordinates
    rng = np.random.default_rng(7 + d)
    heads, nq, nk, nqb, nkb = 2, 701, 866, 11, 29
    dt = "bf16" if bf16 else "f32"
    q = rand_inputs((1, heads, nq, d), 70, dt)
    k = rand_inputs((1, heads, nk, d), 71, dt)
    v = rand_inputs((1, heads, nk, d), 72, dt)
    qoff = np.stack([_random_partition(nq, nqb, rng) for _ in range(heads)])[None]
    koff = np.stack([_random_partition(nk, nkb, rng) for _ in range(heads)])[None]
    qperm = np.stack([rng.permutation(nq) for _ in range(heads)])[None].astype(np.int32)
    kperm = np.stack([rng.permutation(nk) for _ in range(heads)])[None].astype(np.int32)
    masks = rng.random((1, heads, nqb, nkb)) < 0.4
    cnt, idx = synth.mask_to_ell(masks)
    T = _tdtype(bf16)
    scale = 1 / math.sqrt(d)
    dq, dk, dv = to_dev(q, T), to_dev(k, T), to_dev(v, T)
    dqp, dkp = to_dev(qperm, torch.int32), to_dev(kperm, torch.int32)
    lists = (to_dev(qoff, torch.int32), to_dev(koff, torch.int32), to_dev(cnt, torch.int32),
             to_dev(idx, torch.int32))
    o_f, lse_f = sva_block_sparse_attn_perm(dq, dk, dv, dqp, dkp, *lists, scale, want_lse=True)
    gq = torch.gather(dq, 2, dqp.long()[..., None].expand(-1, -1, -1, d))
    gk = torch.gather(dk, 2, dkp.long()[..., None].expand(-1, -1, -1, d))
    gv = torch.gather(dv, 2, dkp.long()[..., None].expand(-1, -1, -1, d))
    o_p, lse_p = sva_block_sparse_attn(gq, gk, gv, *lists, scale, want_lse=True)
    o_ref = torch.empty_like(o_p).scatter_(2, dqp.long()[..., None].expand(-1, -1, -1, d), o_p)
    lse_ref = torch.empty_like(lse_p).scatter_(2, dqp.long(), lse_p)
    assert torch.equal(o_f, o_ref)
    assert torch.equal(lse_f, lse_ref)
    o_f, lse_f = host(o_f), host(lse_f)
    for h in range(heads):
        # cluster id of each ORIGINAL row: permuted position -> block
        aq = np.empty(nq, np.int64)
        aq[qperm[0, h]] = np.repeat(np.arange(nqb), np.diff(qoff[0, h]))
        ak = np.empty(nk, np.int64)
        ak[kperm[0, h]] = np.repeat(np.arange(nkb), np.diff(koff[0, h]))
        ro, rl = oracle.cluster_sparse_attention(q[0, h], k[0, h], v[0, h], aq, ak, masks[0, h],
                                                 np.float32(scale))
        check_attention(o_f[0, h], ro, bf16, f"head {h}")
        check_lse(lse_f[0, h], rl, 1e-3 if bf16 else 1e-5)
