"""ctypes binding of libsva (include/sva.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the HIP stream, workspaces are torch byte tensors, and a
non-OK status raises ``RuntimeError(sva_last_error())``.  Every step of the
computation runs in the library's HIP kernels; there is no fallback, and
loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsva.so")

SVA_OK, SVA_EINVAL, SVA_EUNSUPPORTED, SVA_EWORKSPACE, SVA_EHIP = range(5)
SVA_F32, SVA_BF16 = 0, 1

_P = ctypes.c_void_p
_I = ctypes.c_int32
_Z = ctypes.c_size_t
_D = ctypes.c_double
_F = ctypes.c_float

# name -> (restype, argtypes); mirrors include/sva.h
SIGNATURES = {
    "sva_last_error": (ctypes.c_char_p, []),
    "sva_abi_version": (_I, []),
    "sva_set_debug_checks": (_I, [_I]),
    "sva_kmeans_workspace_bytes": (_Z, [_I, _I, _I, _I, _I]),
    "sva_kmeans": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _Z, _P]),
    "sva_cluster_spread": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "sva_permute_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "sva_permute": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _I, _P, _P, _P, _Z, _P]),
    "sva_select_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "sva_select_blocks": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _D, _D, _P, _P, _P, _P, _Z,
                               _P]),
    "sva_select_threshold": (_I, [_P, _P, _I, _P, _P, _I, _I, _I, _I, _D, _D, _P, _P, _P, _P,
                                  _P]),
    "sva_radial_mask": (_I, [_I, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P, _P]),
    "sva_block_means": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "sva_attn_workspace_bytes": (_Z, [_I, _I, _I, _I]),
    "sva_block_sparse_attn": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _P, _I, _P, _P,
                                   _I, _F, _P, _I, _P, _P, _Z, _P]),
    "sva_block_sparse_attn_noalloc": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _I, _P, _I,
                                           _P, _P, _I, _F, _P, _I, _P, _P]),
    "sva_block_sparse_attn_perm": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _I, _P,
                                        _I, _P, _P, _I, _F, _P, _I, _P, _P, _Z, _P]),
    "sva_unpermute": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "sva_gather_slices": (_I, [_P, _P, _P, _I, ctypes.c_int64, _I, _P]),
    "sva_full_attn_workspace_bytes": (_Z, [_I, _I, _I]),
    "sva_full_attn": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _P, _I, _P, _P, _Z, _P]),
    "sva_check_mfma_rounding": (_I, [_P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def last_error() -> str:
    return lib().sva_last_error().decode()


def sva_set_debug_checks(on: bool) -> None:
    """Turn the device-side precondition checks of the block-sparse calls on
    or off (process-wide; each checked call waits for its check kernel)."""
    _check(lib().sva_set_debug_checks(1 if on else 0), "sva_set_debug_checks")


def _check(status: int, name: str) -> None:
    if status != SVA_OK:
        raise RuntimeError(f"{name} failed (status {status}): {last_error()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libsva must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SVA_BF16
    if t.dtype == torch.float32:
        return SVA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _workspace(nbytes: int, like: torch.Tensor, ws: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if ws is not None:
        if ws.numel() * ws.element_size() < nbytes:
            raise ValueError(f"workspace of {ws.numel() * ws.element_size()} bytes < {nbytes}")
        return ws, ws.numel() * ws.element_size()
    buf = torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    return buf, nbytes


# ---------------------------------------------------------------------------
# entry points, same names as the C ABI
# ---------------------------------------------------------------------------
def sva_kmeans(x: torch.Tensor, c: int, iters: int, centroids: torch.Tensor,
               assign: Optional[torch.Tensor] = None, sizes: Optional[torch.Tensor] = None,
               n_refined: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None):
    """k-means of x [B, H, N, D]; centroids [B, H, c, D] fp32 is updated in place.
    Returns (centroids, assign int32 [B, H, N], sizes int32 [B, H, c])."""
    b, h, n, d = x.shape
    if assign is None:
        assign = torch.empty((b, h, n), dtype=torch.int32, device=x.device)
    if sizes is None:
        sizes = torch.empty((b, h, c), dtype=torch.int32, device=x.device)
    need = lib().sva_kmeans_workspace_bytes(b, h, n, d, c)
    w, wb = _workspace(need, x, ws)
    _check(lib().sva_kmeans(_ptr(x), _dtype_code(x), b, h, n, d, c, iters, _ptr(centroids),
                            _ptr(assign), _ptr(sizes), _ptr(n_refined), _ptr(w), wb, _stream(x)),
           "sva_kmeans")
    return centroids, assign, sizes


def sva_cluster_spread(x: torch.Tensor, c: int, centroids: torch.Tensor, assign: torch.Tensor,
                       out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Per slice (J, T): the k-means objective and the scatter about the mean,
    fp64 [b, h, 2]."""
    b, h, n, d = x.shape
    if out is None:
        out = torch.empty((b, h, 2), dtype=torch.float64, device=x.device)
    _check(lib().sva_cluster_spread(_ptr(x), _dtype_code(x), b, h, n, d, c, _ptr(centroids),
                                    _ptr(assign), _ptr(out), _stream(x)), "sva_cluster_spread")
    return out


def sva_permute(assign: torch.Tensor, c: int, tensors: Sequence[torch.Tensor] = (),
                perm: Optional[torch.Tensor] = None, offsets: Optional[torch.Tensor] = None,
                outs: Optional[Sequence[torch.Tensor]] = None, ws: Optional[torch.Tensor] = None):
    """Stable sort of rows by cluster.  Returns (perm, offsets, [permuted tensors])."""
    b, h, n = assign.shape
    if perm is None:
        perm = torch.empty((b, h, n), dtype=torch.int32, device=assign.device)
    if offsets is None:
        offsets = torch.empty((b, h, c + 1), dtype=torch.int32, device=assign.device)
    tensors = list(tensors)
    if outs is None:
        outs = [torch.empty_like(t) for t in tensors]
    d = tensors[0].shape[-1] if tensors else 0
    dt = _dtype_code(tensors[0]) if tensors else SVA_BF16
    src = (ctypes.c_void_p * max(1, len(tensors)))(*[t.data_ptr() for t in tensors])
    dst = (ctypes.c_void_p * max(1, len(outs)))(*[t.data_ptr() for t in outs])
    need = lib().sva_permute_workspace_bytes(b, h, n, c)
    w, wb = _workspace(need, assign, ws)
    _check(lib().sva_permute(_ptr(assign), c, b, h, n, d, dt, _ptr(perm), _ptr(offsets),
                             len(tensors), ctypes.cast(src, _P), ctypes.cast(dst, _P), _ptr(w), wb,
                             _stream(assign)), "sva_permute")
    return perm, offsets, list(outs)


def sva_select_blocks(cent_q: torch.Tensor, size_q: torch.Tensor, cent_k: torch.Tensor,
                      size_k: torch.Tensor, scale: float, top_p: float,
                      mask: Optional[torch.Tensor] = None,
                      kept_count: Optional[torch.Tensor] = None,
                      kept_idx: Optional[torch.Tensor] = None):
    """Top-p over centroid scores.  Returns (mask u8, kept_count, kept_idx)."""
    b, h, cq, d = cent_q.shape
    ck = cent_k.shape[2]
    dev = cent_q.device
    if mask is None:
        mask = torch.empty((b, h, cq, ck), dtype=torch.uint8, device=dev)
    if kept_count is None:
        kept_count = torch.empty((b, h, cq), dtype=torch.int32, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((b, h, cq, ck), dtype=torch.int32, device=dev)
    _check(lib().sva_select_blocks(_ptr(cent_q), _ptr(size_q), cq, _ptr(cent_k), _ptr(size_k),
                                   ck, b, h, d, float(scale), float(top_p), _ptr(mask),
                                   _ptr(kept_count), _ptr(kept_idx), None, 0, _stream(cent_q)),
           "sva_select_blocks")
    return mask, kept_count, kept_idx


def sva_select_threshold(cent_q: torch.Tensor, size_q: torch.Tensor, cent_k: torch.Tensor,
                         size_k: torch.Tensor, scale: float, theta: float,
                         cand: Optional[torch.Tensor] = None,
                         mask: Optional[torch.Tensor] = None,
                         kept_count: Optional[torch.Tensor] = None,
                         kept_idx: Optional[torch.Tensor] = None):
    """Global threshold on proxy logits (top pair kept if a row ends empty).
    Returns (mask u8, kept_count, kept_idx)."""
    b, h, nq, d = cent_q.shape
    nk = cent_k.shape[2]
    dev = cent_q.device
    if cand is not None and tuple(cand.shape) != (nq, nk):
        raise ValueError(f"cand must be [{nq}, {nk}] uint8")
    if mask is None:
        mask = torch.empty((b, h, nq, nk), dtype=torch.uint8, device=dev)
    if kept_count is None:
        kept_count = torch.empty((b, h, nq), dtype=torch.int32, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((b, h, nq, nk), dtype=torch.int32, device=dev)
    _check(lib().sva_select_threshold(_ptr(cent_q), _ptr(size_q), nq, _ptr(cent_k), _ptr(size_k),
                                      nk, b, h, d, float(scale), float(theta), _ptr(cand),
                                      _ptr(mask), _ptr(kept_count), _ptr(kept_idx),
                                      _stream(cent_q)), "sva_select_threshold")
    return mask, kept_count, kept_idx


def sva_radial_mask(n: int, hw: int, block: int, dt_max: int, window0: int, ratios,
                    batch: int, heads: int, device, mask: Optional[torch.Tensor] = None,
                    kept_count: Optional[torch.Tensor] = None,
                    kept_idx: Optional[torch.Tensor] = None):
    """Radial candidate set with a static ratio per temporal distance (uniform
    blocks).  Returns (mask u8 [b,h,nb,nb], kept_count, kept_idx)."""
    nb = -(-n // block)
    dev = torch.device(device)
    if len(ratios) != dt_max + 1:
        raise ValueError("one ratio per temporal distance 0..dt_max")
    r = (ctypes.c_float * (dt_max + 1))(*[float(x) for x in ratios])
    if mask is None:
        mask = torch.empty((batch, heads, nb, nb), dtype=torch.uint8, device=dev)
    if kept_count is None:
        kept_count = torch.empty((batch, heads, nb), dtype=torch.int32, device=dev)
    if kept_idx is None:
        kept_idx = torch.empty((batch, heads, nb, nb), dtype=torch.int32, device=dev)
    _check(lib().sva_radial_mask(n, hw, block, dt_max, window0, ctypes.cast(r, _P), batch, heads,
                                 _ptr(mask), _ptr(kept_count), _ptr(kept_idx), _stream(mask)),
           "sva_radial_mask")
    return mask, kept_count, kept_idx


def sva_block_means(x: torch.Tensor, block: int, means: Optional[torch.Tensor] = None,
                    sizes: Optional[torch.Tensor] = None):
    """Mean of every uniform block of rows.  Returns (means fp32 [b,h,nb,d], sizes int32)."""
    b, h, n, d = x.shape
    nb = -(-n // block)
    if means is None:
        means = torch.empty((b, h, nb, d), dtype=torch.float32, device=x.device)
    if sizes is None:
        sizes = torch.empty((b, h, nb), dtype=torch.int32, device=x.device)
    _check(lib().sva_block_means(_ptr(x), _dtype_code(x), b, h, n, d, block, _ptr(means),
                                 _ptr(sizes), _stream(x)), "sva_block_means")
    return means, sizes


def sva_block_sparse_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          q_offsets: torch.Tensor, k_offsets: torch.Tensor,
                          kept_count: torch.Tensor, kept_idx: torch.Tensor, scale: float,
                          o: Optional[torch.Tensor] = None, o_dtype=None,
                          lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                          ws: Optional[torch.Tensor] = None):
    """Attention over the kept blocks.  Returns (o, lse or None)."""
    b, h, nq, d = q.shape
    nk = k.shape[2]
    nqb = q_offsets.shape[-1] - 1
    nkb = k_offsets.shape[-1] - 1
    if o is None:
        o = torch.empty((b, h, nq, d), dtype=o_dtype or q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
    need = lib().sva_attn_workspace_bytes(b, h, nq, nqb)
    w, wb = _workspace(need, q, ws)
    _check(lib().sva_block_sparse_attn(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), b, h, nq, nk, d,
                                       _ptr(q_offsets), nqb, _ptr(k_offsets), nkb,
                                       _ptr(kept_count), _ptr(kept_idx), kept_idx.shape[-1],
                                       float(scale), _ptr(o), _dtype_code(o), _ptr(lse), _ptr(w),
                                       wb, _stream(q)), "sva_block_sparse_attn")
    return o, lse


def sva_block_sparse_attn_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  q_offsets: torch.Tensor, k_offsets: torch.Tensor,
                                  kept_count: torch.Tensor, kept_idx: torch.Tensor, scale: float,
                                  o: torch.Tensor, lse: Optional[torch.Tensor] = None):
    """sva_block_sparse_attn with the library's static schedule scratch: the
    caller provides o (and lse, optional); nothing is allocated."""
    b, h, nq, d = q.shape
    nk = k.shape[2]
    _check(lib().sva_block_sparse_attn_noalloc(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), b, h,
                                               nq, nk, d, _ptr(q_offsets),
                                               q_offsets.shape[-1] - 1, _ptr(k_offsets),
                                               k_offsets.shape[-1] - 1, _ptr(kept_count),
                                               _ptr(kept_idx), kept_idx.shape[-1], float(scale),
                                               _ptr(o), _dtype_code(o), _ptr(lse), _stream(q)),
           "sva_block_sparse_attn_noalloc")
    return o, lse


def sva_block_sparse_attn_perm(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                               q_perm: torch.Tensor, k_perm: torch.Tensor,
                               q_offsets: torch.Tensor, k_offsets: torch.Tensor,
                               kept_count: torch.Tensor, kept_idx: torch.Tensor, scale: float,
                               o: Optional[torch.Tensor] = None, o_dtype=None,
                               lse: Optional[torch.Tensor] = None, want_lse: bool = False,
                               ws: Optional[torch.Tensor] = None):
    """Attention over the kept blocks with the permutation fused in: q, k, v, o, lse in
    original token order, blocks over the permuted order.  Returns (o, lse or None)."""
    b, h, nq, d = q.shape
    nk = k.shape[2]
    nqb = q_offsets.shape[-1] - 1
    nkb = k_offsets.shape[-1] - 1
    if o is None:
        o = torch.empty((b, h, nq, d), dtype=o_dtype or q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
    need = lib().sva_attn_workspace_bytes(b, h, nq, nqb)
    w, wb = _workspace(need, q, ws)
    _check(lib().sva_block_sparse_attn_perm(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), b, h, nq, nk, d, _ptr(q_perm), _ptr(k_perm),
        _ptr(q_offsets), nqb, _ptr(k_offsets), nkb, _ptr(kept_count), _ptr(kept_idx),
        kept_idx.shape[-1], float(scale), _ptr(o), _dtype_code(o), _ptr(lse), _ptr(w), wb,
        _stream(q)), "sva_block_sparse_attn_perm")
    return o, lse


def sva_check_mfma_rounding(device=None) -> list:
    """Flags (8 ints) of the on-device accumulation check; all 1 on hardware
    whose bf16 MFMA accumulates with a 24-bit significand, at most one unit
    in the last place lost per addition (the k-means error bound's model)."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    flags = torch.full((8,), -1, dtype=torch.int32, device=dev)
    _check(lib().sva_check_mfma_rounding(_ptr(flags), _stream(flags)), "sva_check_mfma_rounding")
    return flags.cpu().tolist()


def sva_unpermute(o_perm: torch.Tensor, perm: torch.Tensor, o: Optional[torch.Tensor] = None):
    b, h, n, d = o_perm.shape
    if o is None:
        o = torch.empty_like(o_perm)
    _check(lib().sva_unpermute(_ptr(o_perm), _ptr(perm), _dtype_code(o_perm), b, h, n, d, _ptr(o),
                               _stream(o_perm)), "sva_unpermute")
    return o


def sva_gather_slices(src: torch.Tensor, idx: torch.Tensor, dst: torch.Tensor,
                      scatter: bool = False):
    """Whole leading-dimension slices: dst[i] = src[idx[i]] (gather), or
    dst[idx[i]] = src[i] (scatter).  src and dst are contiguous with equal
    slice shapes; idx is an int32 device tensor."""
    if not (src.is_contiguous() and dst.is_contiguous()):
        raise ValueError("tensors passed to libsva must be contiguous")
    if src.shape[1:] != dst.shape[1:] or src.dtype != dst.dtype:
        raise ValueError("src and dst slices must have one shape and dtype")
    if idx.dtype != torch.int32 or idx.device != src.device:
        raise ValueError("idx must be an int32 tensor on the tensors' device")
    slice_bytes = src[0].numel() * src.element_size()
    _check(lib().sva_gather_slices(_ptr(src), _ptr(dst), _ptr(idx), idx.numel(), slice_bytes,
                                   1 if scatter else 0, _stream(src)), "sva_gather_slices")
    return dst


def sva_full_attn(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float,
                  o: Optional[torch.Tensor] = None, o_dtype=None,
                  lse: Optional[torch.Tensor] = None, want_lse: bool = False):
    b, h, nq, d = q.shape
    nk = k.shape[2]
    if o is None:
        o = torch.empty((b, h, nq, d), dtype=o_dtype or q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((b, h, nq), dtype=torch.float32, device=q.device)
    _check(lib().sva_full_attn(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), b, h, nq, nk, d,
                               float(scale), _ptr(o), _dtype_code(o), _ptr(lse), None, 0,
                               _stream(q)), "sva_full_attn")
    return o, lse
