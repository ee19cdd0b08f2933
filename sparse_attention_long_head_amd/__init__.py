"""MI355X-native content-adaptive block-sparse attention for video DiT latents.

The compute lives in ``libsva.so`` (hand-written HIP for gfx950, C ABI in
``include/sva.h``); this package is its ctypes binding plus a layer object
that sequences the calls.  Importing it does not load the library; the first
call does, and raises if it has not been built.
"""
from ._lib import (  # noqa: F401
    SVA_BF16, SVA_F32, LIB_PATH, lib, last_error,
    sva_kmeans, sva_permute, sva_select_blocks, sva_block_sparse_attn,
    sva_block_sparse_attn_perm, sva_block_sparse_attn_noalloc, sva_unpermute, sva_full_attn,
    sva_gather_slices, sva_set_debug_checks,
    sva_select_threshold,
    sva_check_mfma_rounding, sva_cluster_spread,
    sva_radial_mask, sva_block_means,
)
from .layer import (RadialSparseAttention, SparseVideoAttention,  # noqa: F401
                    AdaptiveSparseVideoAttention, choose_clusters, strided_rows)
