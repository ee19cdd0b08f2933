"""The C ABI on the host (no GPU needed): the library builds and loads, exports
every entry point include/sva.h declares, and rejects bad arguments with the
documented status before launching anything."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from sparse_attention_long_head_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from sparse_attention_long_head_amd import build
        build.build()
    _lib.lib()
    return _lib


def _declared():
    with open(os.path.join(ROOT, "include", "sva.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(sva_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 13
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sva_\w+)", out))
    for n in names:
        assert n in exported, n
        assert n in L.SIGNATURES, f"binding lacks {n}"
    assert L.lib().sva_abi_version() == 1


P = ctypes.c_void_p(256)   # a non-NULL dummy: nothing may be dereferenced before validation


def test_rounding_check_validation(L):
    assert L.lib().sva_check_mfma_rounding(None, None) == 1   # SVA_EINVAL, nothing launched
    assert "NULL" in L.last_error()


def test_kmeans_validation(L):
    lib = L.lib()
    ws = lib.sva_kmeans_workspace_bytes(1, 2, 1000, 128, 10)
    assert ws > 0
    cases = [
        ((None, 1, 1, 2, 1000, 128, 10, 3, P, P, P, None, P, ws, None), L.SVA_EINVAL),
        ((P, 7, 1, 2, 1000, 128, 10, 3, P, P, P, None, P, ws, None), L.SVA_EINVAL),
        ((P, 1, 1, 2, 1000, 96, 10, 3, P, P, P, None, P, ws, None), L.SVA_EUNSUPPORTED),
        ((P, 1, 1, 2, 1000, 128, 0, 3, P, P, P, None, P, ws, None), L.SVA_EINVAL),
        ((P, 1, 1, 2, 1000, 128, 1001, 3, P, P, P, None, P, ws, None), L.SVA_EINVAL),
        ((P, 1, 1, 2, 1000, 128, 10, 0, P, P, P, None, P, ws, None), L.SVA_EINVAL),
        ((P, 1, 1, 2, 1000, 128, 10, 3, P, P, P, None, P, ws - 1, None), L.SVA_EWORKSPACE),
        ((P, 1, 1, 2, 1000, 128, 10, 3, P, P, P, None, None, ws, None), L.SVA_EINVAL),
        ((P, 1, 0, 2, 1000, 128, 10, 3, P, P, P, None, P, ws, None), L.SVA_EINVAL),
        ((P, 1, 1, 70000, 1000, 128, 10, 3, P, P, P, None, P, ws, None), L.SVA_EUNSUPPORTED),
    ]
    for args, want in cases:
        assert lib.sva_kmeans(*args) == want, args
        assert L.last_error().startswith("sva_kmeans")


def test_cluster_spread_validation(L):
    lib = L.lib()
    ok = [P, 1, 1, 2, 1000, 128, 10, P, P, P, None]
    for i, bad, want in [(0, None, L.SVA_EINVAL), (1, 9, L.SVA_EINVAL), (4, 0, L.SVA_EINVAL),
                         (5, 96, L.SVA_EUNSUPPORTED), (6, 0, L.SVA_EINVAL),
                         (6, 1001, L.SVA_EINVAL), (7, None, L.SVA_EINVAL),
                         (8, None, L.SVA_EINVAL), (9, None, L.SVA_EINVAL)]:
        args = list(ok)
        args[i] = bad
        assert lib.sva_cluster_spread(*args) == want, (i, bad)
    assert L.last_error().startswith("sva_cluster_spread")


def test_permute_validation(L):
    lib = L.lib()
    ws = lib.sva_permute_workspace_bytes(1, 1, 100, 7)
    src = (ctypes.c_void_p * 2)(256, 512)
    bad = (ctypes.c_void_p * 2)(256, None)
    assert lib.sva_permute(P, 7, 1, 1, 100, 128, 1, P, P, 3, src, src, P, ws, None) == L.SVA_EINVAL
    assert lib.sva_permute(P, 0, 1, 1, 100, 128, 1, P, P, 1, src, src, P, ws, None) == L.SVA_EINVAL
    assert lib.sva_permute(P, 7, 1, 1, 100, 128, 1, P, P, 2, src, bad, P, ws, None) == L.SVA_EINVAL
    assert lib.sva_permute(P, 7, 1, 1, 100, 32, 1, P, P, 1, src, src, P, ws, None) \
        == L.SVA_EUNSUPPORTED
    assert lib.sva_permute(P, 7, 1, 1, 100, 128, 1, P, P, 1, src, src, P, ws - 4, None) \
        == L.SVA_EWORKSPACE
    assert lib.sva_permute(P, 20000, 1, 1, 30000, 128, 1, P, P, 0, None, None, P, 1 << 30,
                           None) == L.SVA_EUNSUPPORTED


def test_select_validation(L):
    lib = L.lib()
    ok = (P, P, 10, P, P, 20, 1, 2, 128, 0.1, 0.9, P, P, P, None, 0, None)
    for i, bad, want in [(10, 0.0, L.SVA_EINVAL), (10, 1.5, L.SVA_EINVAL),
                         (10, float("nan"), L.SVA_EINVAL), (5, 5000, L.SVA_EUNSUPPORTED),
                         (8, 64 + 1, L.SVA_EUNSUPPORTED), (0, None, L.SVA_EINVAL),
                         (9, float("inf"), L.SVA_EINVAL)]:
        args = list(ok)
        args[i] = bad
        assert lib.sva_select_blocks(*args) == want, (i, bad)


def test_dynamicrad_validation(L):
    lib = L.lib()
    ok = (P, P, 10, P, P, 20, 1, 2, 128, 0.1, 0.5, None, P, P, P, None)
    for i, bad, want in [(0, None, L.SVA_EINVAL), (2, 0, L.SVA_EINVAL), (5, 5000, L.SVA_EUNSUPPORTED),
                         (8, 96, L.SVA_EUNSUPPORTED), (9, float("inf"), L.SVA_EINVAL),
                         (10, float("nan"), L.SVA_EINVAL), (14, None, L.SVA_EINVAL)]:
        args = list(ok)
        args[i] = bad
        assert lib.sva_select_threshold(*args) == want, (i, bad)
    ratios = (ctypes.c_float * 3)(1.0, 0.5, 0.25)
    bad_ratios = (ctypes.c_float * 3)(1.0, 1.5, 0.25)
    rp = ctypes.cast(ratios, ctypes.c_void_p)
    ok = [32760, 1560, 128, 2, 8, rp, 1, 2, P, P, P, None]
    for i, bad, want in [(0, 0, L.SVA_EINVAL), (1, 0, L.SVA_EINVAL), (2, 0, L.SVA_EINVAL),
                         (3, -1, L.SVA_EINVAL), (3, 16, L.SVA_EINVAL), (4, -1, L.SVA_EINVAL),
                         (5, None, L.SVA_EINVAL),
                         (5, ctypes.cast(bad_ratios, ctypes.c_void_p), L.SVA_EINVAL),
                         (1, 1 << 30, L.SVA_EUNSUPPORTED), (8, None, L.SVA_EINVAL)]:
        args = list(ok)
        args[i] = bad
        assert lib.sva_radial_mask(*args) == want, (i, bad)
    ok = [P, 1, 1, 2, 1000, 128, 64, P, P, None]
    for i, bad, want in [(0, None, L.SVA_EINVAL), (1, 7, L.SVA_EINVAL), (4, 0, L.SVA_EINVAL),
                         (5, 32, L.SVA_EUNSUPPORTED), (6, 0, L.SVA_EINVAL), (8, None, L.SVA_EINVAL)]:
        args = list(ok)
        args[i] = bad
        assert lib.sva_block_means(*args) == want, (i, bad)
    assert "sva_block_means" in L.last_error()


def test_attention_validation(L):
    lib = L.lib()
    ws = lib.sva_attn_workspace_bytes(1, 2, 1000, 8)
    ok = [P, P, P, 1, 1, 2, 1000, 1000, 128, P, 8, P, 8, P, P, 8, 0.1, P, 1, None, P, ws, None]
    for i, bad, want in [(0, None, L.SVA_EINVAL), (3, 5, L.SVA_EINVAL), (8, 80, L.SVA_EUNSUPPORTED),
                         (10, 0, L.SVA_EINVAL), (10, 1001, L.SVA_EINVAL), (12, 0, L.SVA_EINVAL),
                         (15, 0, L.SVA_EINVAL), (16, float("nan"), L.SVA_EINVAL),
                         (16, -0.125, L.SVA_EINVAL), (16, float("-inf"), L.SVA_EINVAL),
                         (18, 9, L.SVA_EINVAL), (21, ws - 1, L.SVA_EWORKSPACE),
                         (13, None, L.SVA_EINVAL)]:
        args = list(ok)
        args[i] = bad
        assert lib.sva_block_sparse_attn(*args) == want, (i, bad)
    assert lib.sva_full_attn(P, P, P, 1, 1, 2, 10, 10, 64, float("inf"), P, 1, None, None, 0,
                             None) == L.SVA_EINVAL
    assert lib.sva_full_attn(P, P, P, 1, 1, 2, 10, 10, 64, -1.0, P, 1, None, None, 0,
                             None) == L.SVA_EINVAL
    assert ">= 0" in L.last_error()
    assert lib.sva_unpermute(P, None, 1, 1, 1, 10, 64, P, None) == L.SVA_EINVAL
    assert "sva_unpermute" in L.last_error()


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from sparse_attention_long_head_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.lib()


def test_valid_call_without_gpu_returns_hip_error(L):
    """Arguments that pass validation, on a host with no GPU: the launch fails
    and the call returns SVA_EHIP with HIP's message.  (With a GPU visible the
    dummy pointers would be dereferenced, so the test only runs without one.)"""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: dummy device pointers must not be launched on")
    lib = L.lib()
    assert lib.sva_unpermute(P, P, 1, 1, 2, 10, 64, P, None) == L.SVA_EHIP
    msg = L.last_error()
    assert msg.startswith("sva_unpermute") and "device" in msg.lower(), msg
    ws = lib.sva_full_attn_workspace_bytes(1, 2, 100)
    assert lib.sva_full_attn(P, P, P, 1, 1, 2, 100, 100, 128, 0.088, P, 1, None, P, ws,
                             None) == L.SVA_EHIP
    assert L.last_error().startswith("sva_full_attn")


def test_noalloc_attention_rejects_a_schedule_beyond_its_scratch(L):
    """The static-scratch entry point refuses a schedule larger than its 8 MiB
    before any HIP call (so this runs without a GPU)."""
    lib = L.lib()
    need = lib.sva_attn_workspace_bytes(1, 4096, 32760, 256)
    assert need > 8 << 20
    st = lib.sva_block_sparse_attn_noalloc(P, P, P, 1, 1, 4096, 32760, 32760, 128, P, 256, P, 256,
                                           P, P, 256, 0.088, P, 1, None, None)
    assert st == L.SVA_EWORKSPACE
    assert "static scratch" in L.last_error()
    assert lib.sva_block_sparse_attn_noalloc(P, P, P, 1, 1, 2, 1000, 1000, 128, P, 8, P, 0, P, P,
                                             8, 0.088, P, 1, None, None) == L.SVA_EINVAL


def test_gather_slices_validation(L):
    lib = L.lib()
    assert lib.sva_gather_slices(None, P, P, 2, 4096, 0, None) == L.SVA_EINVAL
    assert lib.sva_gather_slices(P, P, None, 2, 4096, 0, None) == L.SVA_EINVAL
    assert lib.sva_gather_slices(P, P, P, -1, 4096, 0, None) == L.SVA_EINVAL
    assert lib.sva_gather_slices(P, P, P, 2, 4100, 0, None) == L.SVA_EINVAL   # not 16-byte pieces
    assert lib.sva_gather_slices(P, P, P, 2, 0, 0, None) == L.SVA_EINVAL
    assert lib.sva_gather_slices(ctypes.c_void_p(264), P, P, 2, 4096, 0, None) == L.SVA_EINVAL
    assert lib.sva_gather_slices(P, P, P, 2, 4096, 2, None) == L.SVA_EINVAL
    assert L.last_error().startswith("sva_gather_slices")


def test_debug_checks_switch(L):
    """sva_set_debug_checks only sets a flag: host validation still runs first
    (a bad argument is rejected before any device work), and on a host with no
    GPU a valid call in debug mode fails in its check with SVA_EHIP."""
    import torch
    lib = L.lib()
    assert lib.sva_set_debug_checks(1) == L.SVA_OK
    try:
        ws = lib.sva_attn_workspace_bytes(1, 2, 1000, 8)
        ok = [P, P, P, 1, 1, 2, 1000, 1000, 128, P, 8, P, 8, P, P, 8, 0.1, P, 1, None, P, ws, None]
        bad = list(ok)
        bad[10] = 0
        assert lib.sva_block_sparse_attn(*bad) == L.SVA_EINVAL
        if torch.cuda.device_count() == 0:
            assert lib.sva_block_sparse_attn(*ok) == L.SVA_EHIP
            assert L.last_error().startswith("sva_block_sparse_attn")
    finally:
        assert lib.sva_set_debug_checks(0) == L.SVA_OK


def test_value_arrays_must_be_16_byte_aligned(L):
    """Value arrays are read in 16-byte pieces: a misaligned one is refused on
    the host with SVA_EINVAL before anything is launched."""
    lib = L.lib()
    M = ctypes.c_void_p(264)   # 8 bytes past a 16-byte boundary
    ws = lib.sva_attn_workspace_bytes(1, 2, 1000, 8)
    ok = [P, P, P, 1, 1, 2, 1000, 1000, 128, P, 8, P, 8, P, P, 8, 0.1, P, 1, None, P, ws, None]
    for i in (0, 1, 2, 17):               # q, k, v, o
        args = list(ok)
        args[i] = M
        assert lib.sva_block_sparse_attn(*args) == L.SVA_EINVAL, i
        assert "16-byte aligned" in L.last_error()
    kws = lib.sva_kmeans_workspace_bytes(1, 2, 1000, 128, 10)
    assert lib.sva_kmeans(M, 1, 1, 2, 1000, 128, 10, 3, P, P, P, None, P, kws, None) == L.SVA_EINVAL
    assert lib.sva_kmeans(P, 1, 1, 2, 1000, 128, 10, 3, M, P, P, None, P, kws, None) == L.SVA_EINVAL
    assert lib.sva_select_blocks(M, P, 4, P, P, 4, 1, 2, 128, 0.1, 0.9, P, P, P, None, 0,
                                 None) == L.SVA_EINVAL
    assert lib.sva_block_means(M, 1, 1, 2, 1000, 128, 128, P, P, None) == L.SVA_EINVAL
    assert lib.sva_unpermute(M, P, 1, 1, 2, 10, 64, P, None) == L.SVA_EINVAL
