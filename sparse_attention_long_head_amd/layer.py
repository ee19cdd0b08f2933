"""One SVG2-form sparse attention layer as a sequence of libsva calls.

Sparse VideoGen2 explainer, technical summary section 2: k-means of Q and K
(2.a), permutation so that clusters are contiguous (2.a), centroid top-p
(2.b), attention over the kept blocks (2.c), inverse permutation (2.a).

With ``fuse_permutation`` (the default) the permutation never materialises:
the sort only produces the permutation and the block offsets, and the
attention kernel reads Q, K and V rows through the permutation and writes O
(and the LSE) back to the original token order, so there is no gather of Q, K,
V and no unpermute pass.  The result equals the unfused sequence bit for bit.

``SparseVideoAttention`` owns every buffer the layer needs (allocated once,
through torch), so ``forward`` only enqueues the library calls: it allocates
nothing and never synchronises.  The clustering and permutation of Q run on a
side stream concurrently with those of K and V on the current stream (the two
are independent until the selection); the current stream waits for the side
stream before the selection, so to a caller the layer is ordered on the
current stream like any other op.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np
import torch

from . import _lib as L


class SparseVideoAttention:
    def __init__(self, batch: int, heads: int, n: int, d: int, cq: int, ck: int, iters: int,
                 top_p: float, dtype: torch.dtype = torch.bfloat16, device="cuda",
                 scale: Optional[float] = None, want_lse: bool = False,
                 fuse_permutation: bool = True, theta: Optional[float] = None,
                 iters_warm: Optional[int] = None, out: Optional[torch.Tensor] = None):
        self.shape = (batch, heads, n, d)
        # centroid cache (Sparse VideoGen2, section 2.c): a call without
        # initial centroids starts from the previous call's final ones and runs
        # iters_warm Lloyd iterations instead of iters
        self.iters_warm = iters if iters_warm is None else iters_warm
        self.cached = False
        self.fused = fuse_permutation
        # theta given: DynamicRad's dynamic threshold on the centroid logits
        # replaces the cumulative top-p (the same candidates: all cluster pairs)
        self.theta = theta
        self.cq, self.ck, self.iters, self.top_p = cq, ck, iters, top_p
        # a float32-representable scale, so the fp64 selection and the fp32
        # attention kernels use the identical value
        self.scale = float(np.float32(1.0 / math.sqrt(d) if scale is None else scale))
        dev = torch.device(device)
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        self.cent_q = torch.empty((batch, heads, cq, d), **f32)
        self.cent_k = torch.empty((batch, heads, ck, d), **f32)
        self.assign_q = torch.empty((batch, heads, n), **i32)
        self.assign_k = torch.empty((batch, heads, n), **i32)
        self.sizes_q = torch.empty((batch, heads, cq), **i32)
        self.sizes_k = torch.empty((batch, heads, ck), **i32)
        self.perm_q = torch.empty((batch, heads, n), **i32)
        self.perm_k = torch.empty((batch, heads, n), **i32)
        self.off_q = torch.empty((batch, heads, cq + 1), **i32)
        self.off_k = torch.empty((batch, heads, ck + 1), **i32)
        # cluster-ordered copies of Q, K, V and O: only the unfused path has them
        perm_buf = (lambda: None) if self.fused else (
            lambda: torch.empty(self.shape, dtype=dtype, device=dev))
        self.q_p, self.k_p, self.v_p, self.o_p = perm_buf(), perm_buf(), perm_buf(), perm_buf()
        self.mask = torch.empty((batch, heads, cq, ck), dtype=torch.uint8, device=dev)
        self.kept_count = torch.empty((batch, heads, cq), **i32)
        self.kept_idx = torch.empty((batch, heads, cq, ck), **i32)
        # the output: a caller-provided contiguous buffer (e.g. a head range of a
        # larger output) or one of our own
        if out is not None:
            if tuple(out.shape) != self.shape or not out.is_contiguous() or out.dtype != dtype:
                raise ValueError("out must be a contiguous tensor of the layer's shape and dtype")
            self.o = out
        else:
            self.o = torch.empty(self.shape, dtype=dtype, device=dev)
        # LSE per query row: in original token order when fused, else of the
        # permuted rows (row i belongs to token perm_q[i])
        self.lse = torch.empty((batch, heads, n), **f32) if want_lse else None
        lib = L.lib()
        km = max(lib.sva_kmeans_workspace_bytes(batch, heads, n, d, cq),
                 lib.sva_kmeans_workspace_bytes(batch, heads, n, d, ck))
        pm = max(lib.sva_permute_workspace_bytes(batch, heads, n, cq),
                 lib.sva_permute_workspace_bytes(batch, heads, n, ck))
        at = lib.sva_attn_workspace_bytes(batch, heads, n, cq)
        self.ws = torch.empty(max(km, pm, at, 1), dtype=torch.uint8, device=dev)
        # the Q clustering runs on a side stream with a workspace of its own
        self.ws_q = torch.empty(max(km, pm, 1), dtype=torch.uint8, device=dev)
        self.side = torch.cuda.Stream(device=dev)

    # the individual stages, so callers (and the benchmark) can time them
    def kmeans(self, q, k, init_q, init_k):
        self.cent_q.copy_(init_q)
        self.cent_k.copy_(init_k)
        L.sva_kmeans(q, self.cq, self.iters, self.cent_q, self.assign_q, self.sizes_q, ws=self.ws)
        L.sva_kmeans(k, self.ck, self.iters, self.cent_k, self.assign_k, self.sizes_k, ws=self.ws)
        self.cached = True

    def _sort_q(self, q, ws):
        L.sva_permute(self.assign_q, self.cq, [] if self.fused else [q], self.perm_q, self.off_q,
                      None if self.fused else [self.q_p], ws=ws)

    def _sort_kv(self, k, v, ws):
        L.sva_permute(self.assign_k, self.ck, [] if self.fused else [k, v], self.perm_k,
                      self.off_k, None if self.fused else [self.k_p, self.v_p], ws=ws)

    def permute(self, q, k, v):
        self._sort_q(q, self.ws)
        self._sort_kv(k, v, self.ws)

    def select(self):
        if self.theta is None:
            L.sva_select_blocks(self.cent_q, self.sizes_q, self.cent_k, self.sizes_k, self.scale,
                                self.top_p, self.mask, self.kept_count, self.kept_idx)
        else:
            L.sva_select_threshold(self.cent_q, self.sizes_q, self.cent_k, self.sizes_k,
                                   self.scale, self.theta, None, self.mask, self.kept_count,
                                   self.kept_idx)

    def attend(self, q=None, k=None, v=None):
        """Attention over the kept blocks; the fused path needs the original
        q, k, v (the unfused one reads its permuted copies)."""
        if self.fused:
            if q is None or k is None or v is None:
                raise ValueError("attend: the fused path needs the original q, k and v")
            L.sva_block_sparse_attn_perm(q, k, v, self.perm_q, self.perm_k, self.off_q,
                                         self.off_k, self.kept_count, self.kept_idx, self.scale,
                                         o=self.o, lse=self.lse, ws=self.ws)
        else:
            L.sva_block_sparse_attn(self.q_p, self.k_p, self.v_p, self.off_q, self.off_k,
                                    self.kept_count, self.kept_idx, self.scale, o=self.o_p,
                                    lse=self.lse, ws=self.ws)

    def unpermute(self):
        """Inverse permutation of the output (nothing to do when fused)."""
        if not self.fused:
            L.sva_unpermute(self.o_p, self.perm_q, self.o)

    def cluster(self, q, k, v, init_q=None, init_k=None):
        """k-means and permutation of Q (side stream) and of K, V (current
        stream), concurrently; returns with the current stream ordered after
        both.  Without init_q / init_k the previous call's centroids seed the
        clustering (warm start)."""
        cold = init_q is not None
        if cold != (init_k is not None):
            raise ValueError("give both init_q and init_k, or neither (warm start)")
        if not cold and not self.cached:
            raise ValueError("a warm start needs a previous call")
        iters = self.iters if cold else self.iters_warm
        cur = torch.cuda.current_stream(self.ws.device)
        self.side.wait_stream(cur)
        with torch.cuda.stream(self.side):
            if cold:
                self.cent_q.copy_(init_q)
            L.sva_kmeans(q, self.cq, iters, self.cent_q, self.assign_q, self.sizes_q,
                         ws=self.ws_q)
            self._sort_q(q, self.ws_q)
        if cold:
            self.cent_k.copy_(init_k)
        L.sva_kmeans(k, self.ck, iters, self.cent_k, self.assign_k, self.sizes_k, ws=self.ws)
        self._sort_kv(k, v, self.ws)
        cur.wait_stream(self.side)
        self.cached = True

    def forward(self, q, k, v, init_q=None, init_k=None) -> torch.Tensor:
        self.cluster(q, k, v, init_q, init_k)
        self.select()
        self.attend(q, k, v)
        self.unpermute()
        return self.o

    __call__ = forward

    def kept_pairs(self) -> int:
        """(query, key) pairs the mask allows; synchronises (host read-back)."""
        sq = self.sizes_q.cpu().numpy().astype(np.int64)
        sk = self.sizes_k.cpu().numpy().astype(np.int64)
        m = self.mask.cpu().numpy().astype(np.int64)
        return int(np.einsum("bhi,bhij,bhj->", sq, m, sk))


class RadialSparseAttention:
    """DynamicRad-style block-sparse attention on uniform token blocks
    (DynamicRad explainer, technical summary section 2.a).

    One radial candidate set over blocks of ``block`` consecutive tokens of the
    frame-major grid (hw tokens per frame), and one of two exclusive modes:

    * ``"static"`` (throughput-first): per temporal distance dt, a fixed share
      ``ratios[dt]`` of the candidates, nearest first.  The mask depends on the
      geometry only, so it is built once here; ``forward`` is attention alone.
    * ``"dynamic"`` (quality-first): block means of Q and K as proxies, pairs of
      the candidate set whose proxy logit reaches ``theta`` are kept, and a
      query block left empty keeps its best candidate.  ``forward`` runs block
      means -> threshold -> attention.

    Buffers are allocated once; ``forward`` allocates nothing and never
    synchronises.
    """

    def __init__(self, batch: int, heads: int, n: int, d: int, hw: int, block: int = 128,
                 mode: str = "static", ratios=(1.0, 1.0, 1.0), dt_max: int = 2, window0: int = 8,
                 theta: Optional[float] = None, dtype: torch.dtype = torch.bfloat16,
                 device="cuda", scale: Optional[float] = None, want_lse: bool = False):
        if mode not in ("static", "dynamic"):
            raise ValueError("mode must be 'static' or 'dynamic'")
        if mode == "dynamic" and theta is None:
            raise ValueError("the dynamic mode needs theta")
        self.shape = (batch, heads, n, d)
        self.mode, self.theta, self.block = mode, theta, block
        self.scale = float(np.float32(1.0 / math.sqrt(d) if scale is None else scale))
        dev = torch.device(device)
        nb = -(-n // block)
        self.nb = nb
        off = torch.clamp(torch.arange(nb + 1, dtype=torch.int32, device=dev) * block, max=n)
        self.off = off.expand(batch, heads, nb + 1).contiguous()
        if mode == "static":
            self.mask, self.kept_count, self.kept_idx = L.sva_radial_mask(
                n, hw, block, dt_max, window0, list(ratios), batch, heads, dev)
        else:
            cand, _, _ = L.sva_radial_mask(n, hw, block, dt_max, window0, [1.0] * (dt_max + 1),
                                           1, 1, dev)
            self.cand = cand[0, 0].contiguous()
            f32 = dict(dtype=torch.float32, device=dev)
            i32 = dict(dtype=torch.int32, device=dev)
            self.mean_q = torch.empty((batch, heads, nb, d), **f32)
            self.mean_k = torch.empty((batch, heads, nb, d), **f32)
            self.size_q = torch.empty((batch, heads, nb), **i32)
            self.size_k = torch.empty((batch, heads, nb), **i32)
            self.mask = torch.empty((batch, heads, nb, nb), dtype=torch.uint8, device=dev)
            self.kept_count = torch.empty((batch, heads, nb), **i32)
            self.kept_idx = torch.empty((batch, heads, nb, nb), **i32)
        self.o = torch.empty(self.shape, dtype=dtype, device=dev)
        self.lse = (torch.empty((batch, heads, n), dtype=torch.float32, device=dev)
                    if want_lse else None)
        lib = L.lib()
        self.ws = torch.empty(max(lib.sva_attn_workspace_bytes(batch, heads, n, nb), 1),
                              dtype=torch.uint8, device=dev)

    def select(self, q, k):
        """Dynamic mode: block means and the threshold selection (no-op when static)."""
        if self.mode == "dynamic":
            L.sva_block_means(q, self.block, self.mean_q, self.size_q)
            L.sva_block_means(k, self.block, self.mean_k, self.size_k)
            L.sva_select_threshold(self.mean_q, self.size_q, self.mean_k, self.size_k, self.scale,
                                   self.theta, self.cand, self.mask, self.kept_count,
                                   self.kept_idx)

    def attend(self, q, k, v):
        L.sva_block_sparse_attn(q, k, v, self.off, self.off, self.kept_count, self.kept_idx,
                                self.scale, o=self.o, lse=self.lse, ws=self.ws)

    def forward(self, q, k, v) -> torch.Tensor:
        self.select(q, k)
        self.attend(q, k, v)
        return self.o

    __call__ = forward

    def kept_pairs(self) -> int:
        """(query, key) token pairs the mask allows; synchronises."""
        sizes = (self.off[0, 0, 1:] - self.off[0, 0, :-1]).cpu().numpy().astype(np.int64)
        m = self.mask.cpu().numpy().astype(np.int64)
        return int(np.einsum("i,bhij,j->", sizes, m, sizes))


def strided_rows(x: torch.Tensor, c: int) -> torch.Tensor:
    """Initial centroids for a calibration run: rows floor(i * n / c) of every
    slice of x [b, h, n, d], as fp32 [b, h, c, d] (no random numbers, so a
    calibration is reproducible)."""
    n = x.shape[2]
    idx = (torch.arange(c, device=x.device, dtype=torch.int64) * n) // c
    return x[:, :, idx, :].float().contiguous()


def choose_clusters(x: torch.Tensor, ladder, iters: int, delta: float = 0.1):
    """Per-head cluster count: the smallest C of ``ladder`` whose k-means
    objective J(C) is within (1 + delta) of the objective at the largest C
    (the point past which more clusters stop fitting the content better).
    Each candidate runs ``iters`` Lloyd iterations from strided rows; the
    objectives come from sva_cluster_spread.  Returns (list of C per head,
    [len(ladder), heads] array of J / T, T being each head's scatter).  Batch 1."""
    ladder = sorted(int(c) for c in ladder)
    b, h, n, d = x.shape
    if b != 1:
        raise ValueError("choose_clusters: batch 1 only")
    dev = x.device
    J = np.zeros((len(ladder), h))
    T = np.zeros(h)
    assign = torch.empty((b, h, n), dtype=torch.int32, device=dev)
    for i, c in enumerate(ladder):
        cent = strided_rows(x, c)
        sizes = torch.empty((b, h, c), dtype=torch.int32, device=dev)
        L.sva_kmeans(x, c, iters, cent, assign, sizes)
        sp = L.sva_cluster_spread(x, c, cent, assign).cpu().numpy()[0]
        J[i] = sp[:, 0]
        T = sp[:, 1]
    chosen = []
    for j in range(h):
        ok = [i for i in range(len(ladder)) if J[i, j] <= (1.0 + delta) * J[-1, j]]
        chosen.append(ladder[ok[0]])
    return chosen, J / np.maximum(T, 1e-300)[None, :]


class AdaptiveSparseVideoAttention:
    """The SVG2 layer with its own (C_q, C_k) per head.  Heads with equal counts
    form one group, wherever they sit, that runs as one ``SparseVideoAttention``:
    a group of consecutive heads works on views of its head range and writes
    straight into that range of the output; any other group's heads are packed
    into buffers of their own (sva_gather_slices) and its output scattered back.
    Batch 1 (a head of a [1, H, n, d] tensor is one contiguous slice)."""

    def __init__(self, heads: int, n: int, d: int, cq_per_head, ck_per_head, iters: int,
                 top_p: float, dtype: torch.dtype = torch.bfloat16, device="cuda", **kw):
        cq_per_head, ck_per_head = list(cq_per_head), list(ck_per_head)
        if len(cq_per_head) != heads or len(ck_per_head) != heads:
            raise ValueError("one C_q and one C_k per head")
        dev = torch.device(device)
        self.o = torch.empty((1, heads, n, d), dtype=dtype, device=dev)
        order = {}
        for h, key in enumerate(zip(cq_per_head, ck_per_head)):
            order.setdefault(key, []).append(h)
        self.groups = []          # (heads, layer)
        self._packs = []          # None for a head range, else (idx, q, k, v, o) buffers
        for (cq, ck), hs in order.items():
            g = len(hs)
            if hs == list(range(hs[0], hs[0] + g)):
                layer = SparseVideoAttention(1, g, n, d, cq, ck, iters, top_p, dtype=dtype,
                                             device=dev, out=self.o[:, hs[0]:hs[0] + g], **kw)
                pack = None
            else:
                po = torch.empty((1, g, n, d), dtype=dtype, device=dev)
                layer = SparseVideoAttention(1, g, n, d, cq, ck, iters, top_p, dtype=dtype,
                                             device=dev, out=po, **kw)
                idx = torch.tensor(hs, dtype=torch.int32, device=dev)
                pack = (idx, *(torch.empty((1, g, n, d), dtype=dtype, device=dev)
                               for _ in range(3)), po)
            self.groups.append((hs, layer))
            self._packs.append(pack)

    def forward(self, q, k, v, init_q=None, init_k=None) -> torch.Tensor:
        """init_q / init_k: one initial-centroid tensor per group ([1, g, C, d],
        the group's heads in ascending order), or None for a warm start from the
        previous call."""
        for gi, ((hs, layer), pack) in enumerate(zip(self.groups, self._packs)):
            iq = None if init_q is None else init_q[gi]
            ik = None if init_k is None else init_k[gi]
            if pack is None:
                h0, h1 = hs[0], hs[0] + len(hs)
                layer(q[:, h0:h1], k[:, h0:h1], v[:, h0:h1], iq, ik)
            else:
                idx, pq, pk, pv, po = pack
                for src, dst in ((q, pq), (k, pk), (v, pv)):
                    L.sva_gather_slices(src[0], idx, dst[0])
                layer(pq, pk, pv, iq, ik)
                L.sva_gather_slices(po[0], idx, self.o[0], scatter=True)
        return self.o

    __call__ = forward

    def kept_pairs(self) -> int:
        return sum(layer.kept_pairs() for _, layer in self.groups)
