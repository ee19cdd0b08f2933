"""Seeded synthetic inputs for the block-sparse video attention path.

This module is shared by the fp64 oracle (``oracle/``) and the HIP path's tests
and benchmark.  It holds none of the method's arithmetic: it only draws the
latent Q/K/V activations of a video diffusion transformer layer, the k-means
initial row indices, and the static radial block mask that is fed *to* the
attention kernel as an input.  Everything is a deterministic function of the
config and its seed.

Workloads (token grids from the long-video post's VRAM-wall figures: about
32.7K tokens for 5 s, 65.5K for 10 s and about 200K for 30 s of video):

* ``tiny``   -- 4x8x8 grid, 2 heads, d=64, fp32.  Small enough for brute force.
* ``5s``     -- 21x30x52 grid (32,760 tokens), 40 heads, d=128, bf16.
* ``static`` -- same shape as ``5s``; i.i.d. N(0,1) tensors and a fixed
  radial + random block mask at a fixed sparsity (DynamicRad's static-ratio
  mode, "Methodology, a. unified candidate set and dual-mode selection").
* ``10s``    -- 41x30x52 grid (63,960 tokens), 40 heads.
* ``30s``    -- 125x30x52 grid (195,000 tokens), 12 heads.

Generator recipe (per video, per tensor X in {Q, K, V}, per head):

1. A spatial Voronoi partition of the (t, y, x) grid into M regions: M seed
   points uniform in [0,T)x[0,H)x[0,W); every token goes to the nearest seed
   (Euclidean, grid units; ties to the lowest seed index).  One partition per
   video, shared by all heads and by Q, K and V.
2. Per-region centres mu ~ alpha_X * N(0, I_d), alpha_V = 1.
3. A per-frame Gaussian random-walk drift of the centres, step sigma = drift,
   zero at t = 0 (the "feature drift" of DynamicRad's BO proxy task).
4. i.i.d. N(0, noise^2) per element; X = mu + drift + noise.
5. Rounded to bf16 (round to nearest even) for bf16 configs; fp32 otherwise.

Token order is t-major: n = (t*H + y)*W + x.

Denoising-step sequences (for the centroid cache, Sparse VideoGen2 explainer,
technical summary section 2.c): the tensors at step s are
X_s = round(X_0 + s * step_drift * Delta), with one seeded direction field
Delta ~ N(0, 1) per element, so consecutive steps differ by a small, fixed
perturbation while the cluster structure stays put.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np

STREAMS = ("voronoi", "centres_q", "centres_k", "centres_v", "drift", "noise", "init", "pad",
           "denoise")


@dataclass(frozen=True)
class VideoConfig:
    name: str
    batch: int
    heads: int
    d: int
    dtype: str            # "f32" or "bf16"
    T: int
    H: int
    W: int
    centres: int          # M, mixture components (0 = i.i.d. N(0,1) tensors)
    noise: float
    drift: float
    block: int
    cq: int
    ck: int
    iters: int
    top_p: float
    seed: int
    alpha: float = 1.0            # centre scale for Q and K (1.0 = the literal recipe)
    static_sparsity: Optional[float] = None   # static-mask config only

    @property
    def n(self) -> int:
        return self.T * self.H * self.W

    @property
    def n_blocks(self) -> int:
        return -(-self.n // self.block)

    def with_(self, **kw) -> "VideoConfig":
        return dataclasses.replace(self, **kw)


# Centre scale that puts the 5 s workload at about 85% sparsity under top-p 0.9
# (oracle, heads 0/13/26/39: densities 0.139/0.149/0.142/0.159;
# the literal alpha = 1 gives densities near 0.68).
CALIBRATED_ALPHA = 1.75

CONFIGS: Dict[str, VideoConfig] = {
    "tiny": VideoConfig("tiny", 1, 2, 64, "f32", 4, 8, 8, 8, 0.3, 0.0, 32, 4, 4, 10, 0.9, seed=0),
    "5s": VideoConfig("5s", 1, 40, 128, "bf16", 21, 30, 52, 64, 0.3, 0.05, 128, 100, 500, 10, 0.9,
                      seed=1, alpha=CALIBRATED_ALPHA),
    "static": VideoConfig("static", 1, 40, 128, "bf16", 21, 30, 52, 0, 1.0, 0.0, 128, 0, 0, 0, 0.0,
                          seed=2, static_sparsity=0.8),
    "10s": VideoConfig("10s", 1, 40, 128, "bf16", 41, 30, 52, 128, 0.3, 0.05, 128, 200, 1000, 10,
                       0.9, seed=3, alpha=CALIBRATED_ALPHA),
    "30s": VideoConfig("30s", 1, 12, 128, "bf16", 125, 30, 52, 256, 0.3, 0.05, 128, 400, 2000, 10,
                       0.9, seed=4, alpha=CALIBRATED_ALPHA),
}


# ----------------------------------------------------------------------------
# seeding helpers
# ----------------------------------------------------------------------------
def _stream(seed: int, name: str) -> np.random.SeedSequence:
    root = np.random.SeedSequence(seed)
    idx = STREAMS.index(name)
    return np.random.SeedSequence(entropy=root.entropy, spawn_key=root.spawn_key + (idx,))


def _child(ss: np.random.SeedSequence, *key: int) -> np.random.Generator:
    """Stateless child generator: the same (stream, key) always gives the same numbers."""
    return np.random.default_rng(np.random.SeedSequence(entropy=ss.entropy,
                                                        spawn_key=ss.spawn_key + tuple(key)))


# ----------------------------------------------------------------------------
# bf16 rounding (input preparation: both paths consume the rounded values)
# ----------------------------------------------------------------------------
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (NaN kept quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + rounding) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 array -> float32 array holding the nearest-even bf16 values."""
    return bf16_values(bf16_bits(x))


# ----------------------------------------------------------------------------
# generator pieces
# ----------------------------------------------------------------------------
def voronoi_regions(cfg: VideoConfig, batch_index: int = 0) -> np.ndarray:
    """Region id of every token, int32 [N], t-major token order."""
    rng = _child(_stream(cfg.seed, "voronoi"), batch_index)
    m = cfg.centres
    seeds = rng.uniform(low=0.0, high=1.0, size=(m, 3)) * np.array([cfg.T, cfg.H, cfg.W], float)
    t, y, x = np.meshgrid(np.arange(cfg.T), np.arange(cfg.H), np.arange(cfg.W), indexing="ij")
    pts = np.stack([t.ravel(), y.ravel(), x.ravel()], axis=1).astype(np.float64)
    region = np.empty(pts.shape[0], dtype=np.int32)
    step = 16384
    for s in range(0, pts.shape[0], step):
        diff = pts[s:s + step, None, :] - seeds[None, :, :]
        dist = np.einsum("nmk,nmk->nm", diff, diff)
        region[s:s + step] = np.argmin(dist, axis=1)   # first minimum = lowest index
    return region


def _tensor_head(cfg: VideoConfig, which: int, b: int, h: int, region: Optional[np.ndarray],
                 alpha: float) -> np.ndarray:
    """One head of one tensor (which: 0=Q, 1=K, 2=V) as float32 [N, d] before rounding."""
    n, d = cfg.n, cfg.d
    key = (which, b, h)
    noise_rng = _child(_stream(cfg.seed, "noise"), *key)
    if cfg.centres == 0:                       # i.i.d. N(0, noise^2)
        return (cfg.noise * noise_rng.standard_normal((n, d), dtype=np.float32)).astype(np.float32)
    cname = ("centres_q", "centres_k", "centres_v")[which]
    mu = alpha * _child(_stream(cfg.seed, cname), b, h).standard_normal((cfg.centres, d))
    frame = np.arange(n) // (cfg.H * cfg.W)
    if cfg.drift > 0.0 and cfg.T > 1:
        steps = cfg.drift * _child(_stream(cfg.seed, "drift"), *key).standard_normal(
            (cfg.T - 1, cfg.centres, d))
        walk = np.concatenate([np.zeros((1, cfg.centres, d)), np.cumsum(steps, axis=0)], axis=0)
        base = (mu[None, :, :] + walk)[frame, region]          # [N, d] float64
    else:
        base = mu[region]
    x = base.astype(np.float32)
    x += cfg.noise * noise_rng.standard_normal((n, d), dtype=np.float32)
    return x


def video_qkv(cfg: VideoConfig, heads: Optional[Tuple[int, ...]] = None,
              alpha: Optional[float] = None) -> Dict[str, np.ndarray]:
    """Q, K, V as float32 arrays [batch, len(heads), N, d] holding the exact values
    both paths consume (bf16-representable for bf16 configs)."""
    heads = tuple(range(cfg.heads)) if heads is None else tuple(heads)
    a = cfg.alpha if alpha is None else alpha
    out = {}
    for which, name in enumerate("qkv"):
        arr = np.empty((cfg.batch, len(heads), cfg.n, cfg.d), dtype=np.float32)
        for b in range(cfg.batch):
            region = voronoi_regions(cfg, b) if cfg.centres > 0 else None
            for j, h in enumerate(heads):
                x = _tensor_head(cfg, which, b, h, region, a if which < 2 else 1.0)
                arr[b, j] = round_bf16(x) if cfg.dtype == "bf16" else x
        out[name] = arr
    return out


def denoise_direction(cfg: VideoConfig, which: str,
                      heads: Optional[Tuple[int, ...]] = None) -> np.ndarray:
    """The drift direction Delta of one tensor across denoising steps, float32
    [batch, len(heads), N, d], i.i.d. N(0, 1)."""
    heads = tuple(range(cfg.heads)) if heads is None else tuple(heads)
    w = {"q": 0, "k": 1, "v": 2}[which]
    out = np.empty((cfg.batch, len(heads), cfg.n, cfg.d), dtype=np.float32)
    for b in range(cfg.batch):
        for j, h in enumerate(heads):
            rng = _child(_stream(cfg.seed, "denoise"), w, b, h)
            out[b, j] = rng.standard_normal((cfg.n, cfg.d), dtype=np.float32)
    return out


def at_denoise_step(x0: np.ndarray, delta: np.ndarray, step: int, step_drift: float,
                    dtype: str = "bf16") -> np.ndarray:
    """X_s = X_0 + s * step_drift * Delta, evaluated in float32 and rounded like
    the config's tensors (the exact values both paths consume)."""
    x = (x0 + np.float32(step * step_drift) * delta).astype(np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def kmeans_init_indices(cfg: VideoConfig, which: str, c: int,
                        heads: Optional[Tuple[int, ...]] = None) -> np.ndarray:
    """Initial centroid row indices: c distinct rows per (batch, head), sorted ascending.
    int64 [batch, len(heads), c].  which is "q" or "k"."""
    heads = tuple(range(cfg.heads)) if heads is None else tuple(heads)
    if not 1 <= c <= cfg.n:
        raise ValueError("need 1 <= c <= n")
    w = {"q": 0, "k": 1}[which]
    out = np.empty((cfg.batch, len(heads), c), dtype=np.int64)
    for b in range(cfg.batch):
        for j, h in enumerate(heads):
            rng = _child(_stream(cfg.seed, "init"), w, b, h)
            out[b, j] = np.sort(rng.choice(cfg.n, size=c, replace=False))
    return out


def gather_init(x: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Initial centroids = the chosen rows, float32 [batch, heads, c, d]."""
    b_, h_, c = idx.shape
    out = np.empty((b_, h_, c, x.shape[-1]), dtype=np.float32)
    for b in range(b_):
        for h in range(h_):
            out[b, h] = x[b, h, idx[b, h]]
    return out


# ----------------------------------------------------------------------------
# static radial + random block mask (an input of the attention kernel)
# ----------------------------------------------------------------------------
def radial_block_keep(n: int, hw: int, block: int) -> np.ndarray:
    """Radial locality candidate set over uniform token blocks (bool [nb, nb]).

    Block b spans tokens [block*b, block*b + block); its frame is
    floor(block*b / hw) and its spatial window index floor((block*b mod hw) / block).
    A query block keeps a key block when their frames differ by dt <= 2 and their
    window indices by at most 8 >> dt (the window halves per frame of distance).
    """
    nb = -(-n // block)
    start = np.arange(nb) * block
    t = start // hw
    s = (start % hw) // block
    dt = np.abs(t[:, None] - t[None, :])
    ds = np.abs(s[:, None] - s[None, :])
    return (dt <= 2) & (ds <= (8 >> np.minimum(dt, 3)))


def static_block_mask(cfg: VideoConfig, sparsity: Optional[float] = None) -> np.ndarray:
    """Radial candidate set padded with seeded uniformly random tiles until exactly
    round((1 - sparsity) * nb^2) tiles are kept.  One mask shared by all heads."""
    sp = cfg.static_sparsity if sparsity is None else sparsity
    nb = cfg.n_blocks
    keep = radial_block_keep(cfg.n, cfg.H * cfg.W, cfg.block)
    target = int(round((1.0 - sp) * nb * nb))
    have = int(keep.sum())
    if have > target:
        raise ValueError(f"radial set alone keeps {have} tiles > target {target}")
    free = np.flatnonzero(~keep.ravel())
    rng = _child(_stream(cfg.seed, "pad"), int(round(sp * 1e6)))
    extra = rng.choice(free, size=target - have, replace=False)
    flat = keep.ravel().copy()
    flat[extra] = True
    return flat.reshape(nb, nb)


def uniform_offsets(n: int, block: int) -> np.ndarray:
    """Block boundaries 0, block, 2*block, ..., n (the last block may be short)."""
    nb = -(-n // block)
    return np.minimum(np.arange(nb + 1, dtype=np.int64) * block, n).astype(np.int32)


def mask_to_ell(mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """bool [..., nq, nk] -> (kept_count int32 [..., nq], kept_idx int32 [..., nq, nk]) with
    ascending kept column ids first and -1 padding.  Pure re-encoding of an input mask."""
    m = np.asarray(mask, dtype=bool)
    count = m.sum(axis=-1).astype(np.int32)
    nk = m.shape[-1]
    cols = np.where(m, np.arange(nk, dtype=np.int32), np.int32(nk))
    idx = np.sort(cols, axis=-1)
    idx = np.where(idx == nk, -1, idx).astype(np.int32)
    return count, idx
