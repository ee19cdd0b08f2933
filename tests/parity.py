"""Shared helpers of the GPU parity tests (not a test module).

Tolerances (from the target contract; the derivation is in the attention test
docstrings): attention output in bf16 mode max-abs <= 2e-2 and mean-abs <= 2e-3
against fp64; in fp32 mode max-abs <= 1e-4.  Integer outputs (assignments,
permutations, masks) must match exactly except where the oracle's own fp64
decision margin is below a stated tie threshold; such rows are counted.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import synth

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_MAX = 1e-4
TIE = 1e-5


def device() -> torch.device:
    if not torch.cuda.is_available():
        pytest.fail("GPU parity tests need a visible gfx950 GPU")
    return torch.device("cuda:0")


def to_dev(a: np.ndarray, dtype=torch.float32) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(device()).to(dtype)


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def rand_inputs(shape, seed, dtype="bf16", scale=1.0) -> np.ndarray:
    """Seeded N(0, scale^2) values, bf16-representable when dtype == "bf16"."""
    x = (scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)
    return synth.round_bf16(x) if dtype == "bf16" else x


def check_attention(o: np.ndarray, ref: np.ndarray, bf16: bool, what: str = "") -> dict:
    err = np.abs(o.astype(np.float64) - ref)
    stats = dict(max=float(err.max()), mean=float(err.mean()))
    if os.environ.get("SVA_PARITY_REPORT"):    # print the margins (run pytest with -s)
        print(f"[parity] {what or 'attention'}: max-abs {stats['max']:.3g}, "
              f"mean-abs {stats['mean']:.3g}")
    if bf16:
        assert stats["max"] <= BF16_MAX and stats["mean"] <= BF16_MEAN, (what, stats)
    else:
        assert stats["max"] <= F32_MAX, (what, stats)
    return stats


def check_lse(lse: np.ndarray, ref: np.ndarray, tol: float, what: str = "") -> None:
    inf = np.isneginf(ref)
    assert (np.isneginf(lse) == inf).all(), what
    if (~inf).any():
        err = np.abs(lse[~inf] - ref[~inf]).max()
        assert err <= tol, (what, err)


def assign_parity(gpu: np.ndarray, ref: np.ndarray, margin: np.ndarray, what: str = "") -> int:
    """Exact except where the fp64 margin is below TIE; returns the tie mismatch count."""
    mism = gpu != ref
    bad = mism & (margin >= TIE)
    assert not bad.any(), (what, int(bad.sum()), np.flatnonzero(bad)[:10])
    return int(mism.sum())
