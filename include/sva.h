/*
 * sva.h -- C ABI of libsva, content-adaptive block-sparse self-attention over
 * the frame x height x width latent tokens of a video diffusion transformer,
 * for AMD Instinct MI355X (gfx950).
 *
 * The layer follows Sparse VideoGen2 (gist.science explainer of
 * arXiv 2505.18875, technical summary section 2, "Methodology"):
 *   sva_kmeans            k-means of Q and of K per head            (section 2.a)
 *   sva_permute           make every cluster contiguous             (section 2.a)
 *   sva_select_blocks     centroid scores + cumulative top-p        (section 2.b)
 *   sva_block_sparse_attn attention over the kept blocks only       (section 2.c)
 *   sva_unpermute         inverse permutation of the output         (section 2.a)
 * plus the dense baseline sva_full_attn (full 3-D attention, the "VRAM wall" of
 * the long-video blog, atlascloud.ai, "Why long video is hard").  DynamicRad's
 * two selection modes (DynamicRad explainer, arXiv 2604.20470, technical
 * summary section 2.a) work on uniform token blocks and feed the same
 * attention with uniform offsets:
 *   sva_radial_mask       radial candidate set + static ratio per temporal distance
 *   sva_block_means       block means, the proxies of the dynamic mode
 *   sva_select_threshold  global threshold on proxy logits, top pair kept if empty
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are [batch][heads][n][d], row-major, d fastest, contiguous.
 *   "bh" below is batch*heads; per-(b,h) arrays are laid out [bh][...].
 * - All tensor / array pointers are DEVICE pointers owned by the caller.  The
 *   library never allocates, never frees and never synchronises.  Scratch
 *   memory is the caller's `ws` buffer of `ws_bytes` bytes; its size comes
 *   from the matching *_workspace_bytes() query (0 means none is needed, and
 *   then ws may be NULL).  The workspace holds no state between calls.
 * - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *   call only enqueues work on that stream and returns.
 * - dtype codes: SVA_F32 (IEEE fp32) or SVA_BF16 (bfloat16).  Supported head
 *   dims are 64 and 128.
 * - Value arrays (Q, K, V, O, x, centroids and their permuted copies) are
 *   read and written in 16-byte pieces and must be 16-byte aligned (any
 *   allocation from hipMalloc or torch is); a misaligned one is refused with
 *   SVA_EINVAL.  Index arrays and LSE need only their natural alignment.
 * - Errors: every argument is validated on the host before anything is
 *   launched.  A failed check returns SVA_EINVAL / SVA_EUNSUPPORTED /
 *   SVA_EWORKSPACE and launches nothing; a HIP launch failure returns
 *   SVA_EHIP.  sva_last_error() then gives a message (thread-local; valid
 *   until the next call on the same thread).  Device-side preconditions
 *   (monotone offsets, in-range indices) are documented per call; they are
 *   checked on the device only in the debug mode of sva_set_debug_checks.
 * - Results are deterministic: identical inputs give bitwise-identical
 *   outputs.  Calls on different streams may overlap if their buffers differ.
 */
#ifndef SVA_H
#define SVA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SVA_OK = 0,
  SVA_EINVAL = 1,        /* bad argument (null pointer, size out of range) */
  SVA_EUNSUPPORTED = 2,  /* valid but not implemented (e.g. d not 64/128)  */
  SVA_EWORKSPACE = 3,    /* ws_bytes smaller than the workspace query       */
  SVA_EHIP = 4           /* a HIP runtime call failed                       */
};

enum { SVA_F32 = 0, SVA_BF16 = 1 };

/* Message for the last non-OK status returned on this thread ("" if none). */
const char *sva_last_error(void);

/* ABI version of this header (bumped on any signature change). */
int32_t sva_abi_version(void);

/* Debug mode (process-wide, off by default).  While on, every block-sparse
 * attention call (sva_block_sparse_attn, _perm, _noalloc) first runs a check
 * kernel on its stream over the device arrays the call reads, waits for it,
 * and returns SVA_EINVAL without launching the attention if any of these
 * preconditions of the block layout (Sparse VideoGen2, section 2.c: the
 * kernel over blocks of varying size) fails:
 *   q_offsets / k_offsets of each slice monotone, from >= 0 to <= n_q / n_k;
 *   kept_count in [0, min(kept_stride, n_kblocks)];
 *   each listed kept_idx in [0, n_kblocks) (at most kept_stride read per row);
 *   q_perm / k_perm entries in [0, n_q) / [0, n_k).
 * The message names the violated ones.  The check synchronises the stream, so
 * debug mode is for testing, not for graph capture or timed runs.  It uses a
 * static device word per GPU (no allocation); overlapping checked calls on
 * one GPU may report each other's violations.  on = 0 turns it off.
 * Returns SVA_OK. */
int32_t sva_set_debug_checks(int32_t on);

/* ---------------------------------------------------------------------------
 * sva_kmeans -- Lloyd k-means of every (b,h) slice of x, independently.
 * Sparse VideoGen2, technical summary section 2.a (Q and K are clustered into
 * C_q and C_k clusters); section 2.c (centroid cache: the previous step's
 * centroids seed this one, so the initial centroids are an input).
 *
 *   x          [bh][n][d], dtype SVA_BF16 or SVA_F32 (read only)
 *   c          clusters per slice, 1 <= c <= min(n, 16384)
 *   iters      Lloyd iterations, >= 1 (exactly this many; no early stop)
 *   centroids  [bh][c][d] fp32.  IN: initial centroids.  OUT: the means of the
 *              final assignment (an empty cluster keeps its previous value).
 *   assign     [bh][n] int32 OUT: cluster of every row in the last iteration,
 *              argmin of squared Euclidean distance, ties to the lowest index.
 *   sizes      [bh][c] int32 OUT: rows per cluster in the final assignment.
 *   n_refined  optional [1] int32 device counter (may be NULL): incremented by
 *              the number of rows whose assignment was re-decided in fp64
 *              because the fast MFMA distances could not separate the best
 *              two clusters.  The caller zeroes it.
 * Decisions are exact: the fast path carries a rigorous error bound and every
 * row inside it is re-decided with fp64 distances.
 * ------------------------------------------------------------------------ */
size_t sva_kmeans_workspace_bytes(int32_t batch, int32_t heads, int32_t n, int32_t d, int32_t c);
int32_t sva_kmeans(const void *x, int32_t dtype, int32_t batch, int32_t heads, int32_t n,
                   int32_t d, int32_t c, int32_t iters, float *centroids, int32_t *assign,
                   int32_t *sizes, int32_t *n_refined, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * sva_cluster_spread -- how tightly a clustering fits each slice, the input of
 * a per-head choice of the cluster count (Sparse VideoGen2, section 2.b: the
 * kept density follows the content; the pages give no rule for C itself, so
 * the caller's rule decides from these two numbers).  Per (b,h) slice, in fp64
 * with a fixed summation order (deterministic):
 *   spread[2 bh]     J = sum over rows of ||x - centroids[assign[row]]||^2
 *                        (the k-means objective)
 *   spread[2 bh + 1] T = sum over rows of ||x - mean||^2, the slice's scatter
 *                        (computed as sum ||x||^2 - ||sum x||^2 / n)
 *
 *   x          [bh][n][d], dtype SVA_BF16 or SVA_F32
 *   c          clusters, 1 <= c <= n; centroids [bh][c][d] fp32
 *   assign     [bh][n] int32 in [0, c) (ids outside are clamped into it)
 *   spread     [bh][2] fp64 OUT, DEVICE memory owned by the caller
 * ------------------------------------------------------------------------ */
int32_t sva_cluster_spread(const void *x, int32_t dtype, int32_t batch, int32_t heads, int32_t n,
                           int32_t d, int32_t c, const float *centroids, const int32_t *assign,
                           double *spread, void *stream);

/* ---------------------------------------------------------------------------
 * sva_permute -- semantic-aware permutation (Sparse VideoGen2, section 2.a).
 * A stable counting sort of the rows of each slice by cluster id: clusters in
 * ascending id, rows of a cluster in ascending original index.
 *
 *   assign     [bh][n] int32 cluster ids in [0, c); an id outside that range
 *              is clamped into it on the device (no error is reported, and
 *              no memory outside the arguments is touched)
 *   perm       [bh][n] int32 OUT: perm[i] = original row of permuted row i
 *   offsets    [bh][c+1] int32 OUT: cluster j is permuted rows
 *              [offsets[j], offsets[j+1]); offsets[c] = n
 *   n_tensors  0, 1 or 2 tensors to gather (e.g. Q alone, or K and V)
 *   src, dst   HOST arrays of n_tensors DEVICE pointers, each [bh][n][d] of
 *              `dtype`; dst[t][i] = src[t][perm[i]].  src and dst must not
 *              overlap.
 * ------------------------------------------------------------------------ */
size_t sva_permute_workspace_bytes(int32_t batch, int32_t heads, int32_t n, int32_t c);
int32_t sva_permute(const int32_t *assign, int32_t c, int32_t batch, int32_t heads, int32_t n,
                    int32_t d, int32_t dtype, int32_t *perm, int32_t *offsets, int32_t n_tensors,
                    const void *const *src, void *const *dst, void *ws, size_t ws_bytes,
                    void *stream);

/* ---------------------------------------------------------------------------
 * sva_select_blocks -- centroid-based top-p (Sparse VideoGen2, section 2.b),
 * with DynamicRad's rule that a block never ends empty (section 2.a).
 * For each (b,h) and each Q cluster i with size_q[i] > 0, in fp64:
 *   S_ij = (cent_q_i . cent_k_j) * scale
 *   P_ij = size_k[j] exp(S_ij - max) / sum over non-empty K clusters
 *   order non-empty K clusters by descending P (ties: ascending j) and keep
 *   the shortest prefix whose cumulative sum is >= top_p (top_p >= 1 keeps
 *   every non-empty K cluster).  Empty Q clusters keep nothing.
 *
 *   cent_q [bh][cq][d] fp32, size_q [bh][cq] int32; likewise cent_k, size_k
 *   cq, ck     1 <= cq, 1 <= ck <= 4096;  0 < top_p <= 1
 *   scale, top_p are doubles: the cut is decided in fp64
 *   mask       [bh][cq][ck] uint8 OUT (1 = kept)
 *   kept_count [bh][cq] int32 OUT
 *   kept_idx   [bh][cq][ck] int32 OUT: the kept K ids in ascending order,
 *              then -1 padding (this compact list is what attention walks)
 * ------------------------------------------------------------------------ */
size_t sva_select_workspace_bytes(int32_t batch, int32_t heads, int32_t cq, int32_t ck);
int32_t sva_select_blocks(const float *cent_q, const int32_t *size_q, int32_t cq,
                          const float *cent_k, const int32_t *size_k, int32_t ck, int32_t batch,
                          int32_t heads, int32_t d, double scale, double top_p, uint8_t *mask,
                          int32_t *kept_count, int32_t *kept_idx, void *ws, size_t ws_bytes,
                          void *stream);

/* ---------------------------------------------------------------------------
 * sva_select_threshold -- DynamicRad's dynamic-threshold ("quality-first")
 * mode (DynamicRad explainer, technical summary section 2.a): pre-softmax
 * logits as importance proxies, one global threshold, and a block that ends
 * empty keeps its top-scoring pair.  For each (b,h) and each query block i
 * with size_q[i] > 0, in fp64:
 *   S_ij = (cent_q_i . cent_k_j) * scale    (the same arithmetic as
 *                                            sva_select_blocks)
 *   eligible: size_k[j] > 0 and (cand == NULL or cand[i][j] != 0)
 *   keep every eligible j with S_ij >= theta; if none, keep the eligible j of
 *   largest S_ij (ties: lowest j); if nothing is eligible, keep nothing.
 * Query blocks with size_q[i] == 0 keep nothing.
 *
 *   cent_q [bh][nq][d] fp32, size_q [bh][nq] int32 (block means and sizes
 *              from sva_block_means, or k-means centroids and sizes)
 *   cent_k [bh][nk][d] fp32, size_k [bh][nk] int32
 *   nq <= 65535, nk <= 4096; scale finite; theta any non-NaN value
 *   cand       [nq][nk] uint8, DEVICE, shared by every slice, or NULL (all
 *              pairs are candidates), e.g. a radial set from sva_radial_mask
 *   mask, kept_count, kept_idx  OUT as in sva_select_blocks
 * ------------------------------------------------------------------------ */
int32_t sva_select_threshold(const float *cent_q, const int32_t *size_q, int32_t nq,
                             const float *cent_k, const int32_t *size_k, int32_t nk,
                             int32_t batch, int32_t heads, int32_t d, double scale, double theta,
                             const uint8_t *cand, uint8_t *mask, int32_t *kept_count,
                             int32_t *kept_idx, void *stream);

/* ---------------------------------------------------------------------------
 * sva_radial_mask -- DynamicRad's radial locality candidate set with its
 * static-ratio ("throughput-first") selection (DynamicRad explainer,
 * technical summary section 2.a: attention fades with spatial and temporal
 * distance; the static mode keeps a fixed share of the candidates chosen by
 * temporal distance, with no content scoring).  The mask depends on geometry
 * only, so every slice gets the same one.
 *
 * Uniform blocks of `block` consecutive tokens (the last may be short),
 * nb = ceil(n / block); token order is frame-major with hw tokens per frame.
 * Block b lies in frame t_b = (block*b) / hw at window s_b = ((block*b) % hw)
 * / block.  Candidates: dt = |t_a - t_b| <= dt_max and |s_a - s_b| <=
 * window0 >> dt.  For query block a and each dt, of the n candidates at that
 * distance the first ceil(ratios[dt] * n) in (|s_a - s_b|, b) order are kept
 * (ceil evaluated in fp64 on the float ratio).  ratios of 1 keep the whole
 * candidate set.
 *
 *   n, hw, block  >= 1;  0 <= dt_max <= 15;  window0 >= 0
 *   ratios     HOST float[dt_max + 1], each in [0, 1]
 *   mask       [bh][nb][nb] uint8 OUT
 *   kept_count [bh][nb] int32 OUT
 *   kept_idx   [bh][nb][nb] int32 OUT: kept key blocks ascending, then -1
 *              (pass kept_stride = nb and uniform offsets to the attention)
 * Rejected with SVA_EUNSUPPORTED when the 2*dt_max+1 frames around a block
 * hold more than 8192 blocks.
 * ------------------------------------------------------------------------ */
int32_t sva_radial_mask(int32_t n, int32_t hw, int32_t block, int32_t dt_max, int32_t window0,
                        const float *ratios, int32_t batch, int32_t heads, uint8_t *mask,
                        int32_t *kept_count, int32_t *kept_idx, void *stream);

/* ---------------------------------------------------------------------------
 * sva_block_means -- the mean of every uniform block of rows, the proxy of a
 * block for sva_select_threshold (DynamicRad explainer, section 2.a).
 *   x      [bh][n][d] of dtype; block >= 1; nb = ceil(n / block)
 *   means  [bh][nb][d] fp32 OUT: rows summed in fp64 in row order, divided by
 *          the row count, rounded to fp32
 *   sizes  [bh][nb] int32 OUT: rows per block (block, the last may be short)
 * ------------------------------------------------------------------------ */
int32_t sva_block_means(const void *x, int32_t dtype, int32_t batch, int32_t heads, int32_t n,
                        int32_t d, int32_t block, float *means, int32_t *sizes, void *stream);

/* ---------------------------------------------------------------------------
 * sva_block_sparse_attn -- attention over the kept blocks only (Sparse
 * VideoGen2, section 2.c: dynamic block sizes, contiguous Q computed densely,
 * K/V of the kept blocks gathered).  For every query row r of Q block i:
 *   O[r]   = sum over keys n' of the kept K blocks of softmax(q_r.k_n' * scale) v_n'
 *   LSE[r] = log sum exp(q_r.k_n' * scale)
 * A row whose block keeps no key gets O = 0 and LSE = -inf.
 *
 *   q [bh][n_q][d], k and v [bh][n_k][d]: dtype SVA_BF16 (bf16 MFMA, fp32
 *              accumulation) or SVA_F32 (fp32 throughout)
 *   q_offsets  [bh][n_qblocks+1] int32, monotone, q_offsets[0] = 0,
 *              q_offsets[n_qblocks] = n_q (device precondition)
 *   k_offsets  [bh][n_kblocks+1] int32, likewise over n_k
 *   kept_count [bh][n_qblocks] int32 in [0, n_kblocks]
 *   kept_idx   [bh][n_qblocks][kept_stride] int32; the first kept_count
 *              entries are distinct K block ids in [0, n_kblocks)
 *   scale      logit scale, finite and >= 0 (1/sqrt(d) for standard
 *              attention); a negative scale is rejected with SVA_EINVAL
 *   o          [bh][n_q][d] OUT, o_dtype SVA_BF16 or SVA_F32
 *   lse        [bh][n_q] fp32 OUT, natural log; may be NULL
 * ------------------------------------------------------------------------ */
size_t sva_attn_workspace_bytes(int32_t batch, int32_t heads, int32_t n_q, int32_t n_qblocks);
int32_t sva_block_sparse_attn(const void *q, const void *k, const void *v, int32_t dtype,
                              int32_t batch, int32_t heads, int32_t n_q, int32_t n_k, int32_t d,
                              const int32_t *q_offsets, int32_t n_qblocks,
                              const int32_t *k_offsets, int32_t n_kblocks,
                              const int32_t *kept_count, const int32_t *kept_idx,
                              int32_t kept_stride, float scale, void *o, int32_t o_dtype,
                              float *lse, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------------
 * sva_block_sparse_attn_noalloc -- sva_block_sparse_attn for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): no workspace argument; the work
 * schedule lives in a static device array of 8 MiB per GPU, held by the
 * library until the process ends.  The call allocates and frees nothing.
 * Arguments, results and errors are those of sva_block_sparse_attn, plus:
 *   SVA_EWORKSPACE  the schedule (sva_attn_workspace_bytes(batch, heads, n_q,
 *                   n_qblocks)) exceeds 8 MiB; nothing is launched
 * Every call on one GPU uses that GPU's array: calls that overlap on one GPU
 * (different streams, different threads) race and must be ordered by the
 * caller.  Each call rewrites every part of the array it reads.
 * ------------------------------------------------------------------------ */
int32_t sva_block_sparse_attn_noalloc(const void *q, const void *k, const void *v,
                                      int32_t dtype, int32_t batch, int32_t heads, int32_t n_q,
                                      int32_t n_k, int32_t d, const int32_t *q_offsets,
                                      int32_t n_qblocks, const int32_t *k_offsets,
                                      int32_t n_kblocks, const int32_t *kept_count,
                                      const int32_t *kept_idx, int32_t kept_stride, float scale,
                                      void *o, int32_t o_dtype, float *lse, void *stream);

/* ------------------------------------------------------------------------
 * sva_block_sparse_attn_perm -- the same attention with the permutation
 * fused into its loads and stores (Sparse VideoGen2, section 2.a: the
 * permutation only makes each cluster contiguous; section 2.c: sparse loading
 * of the kept K/V).  q, k, v, o and lse stay in ORIGINAL token order; the
 * blocks are ranges of the PERMUTED order, as sva_permute returns them:
 *
 *   q_perm     [bh][n_q] int32: q_perm[i] = original row of permuted query
 *              row i (a permutation of [0, n_q); device precondition)
 *   k_perm     [bh][n_k] int32: likewise for the key/value rows
 *
 * Every other argument is as for sva_block_sparse_attn.  The result equals
 * sva_block_sparse_attn on the gathered tensors q[q_perm], k[k_perm],
 * v[k_perm] followed by sva_unpermute, bit for bit; it writes o and lse at
 * the original rows, and skips both gathers and the unpermutation.
 * ------------------------------------------------------------------------ */
int32_t sva_block_sparse_attn_perm(const void *q, const void *k, const void *v, int32_t dtype,
                                   int32_t batch, int32_t heads, int32_t n_q, int32_t n_k,
                                   int32_t d, const int32_t *q_perm, const int32_t *k_perm,
                                   const int32_t *q_offsets, int32_t n_qblocks,
                                   const int32_t *k_offsets, int32_t n_kblocks,
                                   const int32_t *kept_count, const int32_t *kept_idx,
                                   int32_t kept_stride, float scale, void *o, int32_t o_dtype,
                                   float *lse, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * sva_unpermute -- o[perm[i]] = o_perm[i] per slice (Sparse VideoGen2,
 * section 2.a: the permuted result is mapped back to token order).
 *   o_perm, o  [bh][n][d] of dtype (must not overlap); perm [bh][n] int32, a
 *   permutation of [0, n) (device precondition).
 * ------------------------------------------------------------------------ */
int32_t sva_unpermute(const void *o_perm, const int32_t *perm, int32_t dtype, int32_t batch,
                      int32_t heads, int32_t n, int32_t d, void *o, void *stream);

/* ---------------------------------------------------------------------------
 * sva_gather_slices -- moves whole (b, h) slices between a tensor and a packed
 * one, so that heads that share their cluster counts (one C_q and C_k per
 * head: the density follows the content, Sparse VideoGen2, section 2.b) run as
 * one group of consecutive slices:
 *   scatter = 0:  dst slice i = src slice idx[i]  (gather into the pack)
 *   scatter = 1:  dst slice idx[i] = src slice i  (scatter back)
 *   src, dst     device memory, 16-byte aligned, must not overlap
 *   idx          [n_idx] int32 DEVICE array of slice indices; the caller
 *                guarantees they lie in the tensor and (scatter) are distinct
 *   slice_bytes  bytes per slice, a positive multiple of 16
 * Returns SVA_EINVAL for a bad argument, SVA_EHIP if the launch fails;
 * asynchronous on stream.
 * ------------------------------------------------------------------------ */
int32_t sva_gather_slices(const void *src, void *dst, const int32_t *idx, int32_t n_idx,
                          int64_t slice_bytes, int32_t scatter, void *stream);

/* ---------------------------------------------------------------------------
 * sva_full_attn -- dense softmax attention over all keys (density 1.0), the
 * baseline the sparse layer is measured against.  Same kernels and the same
 * numerics as sva_block_sparse_attn with a single block holding every key.
 * Arguments as in sva_block_sparse_attn.
 * ------------------------------------------------------------------------ */
size_t sva_full_attn_workspace_bytes(int32_t batch, int32_t heads, int32_t n_q);
int32_t sva_full_attn(const void *q, const void *k, const void *v, int32_t dtype, int32_t batch,
                      int32_t heads, int32_t n_q, int32_t n_k, int32_t d, float scale, void *o,
                      int32_t o_dtype, float *lse, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------
 * sva_check_mfma_rounding -- checks on the current GPU the model of the
 * hardware that sva_kmeans's error bound assumes: the 32x32x16 bf16
 * matrix-multiply instruction accumulates its products and the value it is
 * seeded with in fp32 (24-bit significand), each addition losing at most one
 * unit in the last place, in any order.  Eight cases with known answers:
 * four whose every partial sum is exact in fp32 (they must come out exact)
 * and four that need rounding (they must land within one unit per addition).
 *
 *   flags   [8] int32 device memory, OUT: 1 where the case meets the model,
 *           0 otherwise.  The caller owns it.
 * Returns SVA_EINVAL for a NULL flags, SVA_EHIP if the launch fails;
 * asynchronous on stream like the other calls.
 * ------------------------------------------------------------------------ */
int32_t sva_check_mfma_rounding(int32_t *flags, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SVA_H */
