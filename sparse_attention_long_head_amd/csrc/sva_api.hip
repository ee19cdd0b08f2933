// extern "C" entry points of libsva: host-side validation, workspace carving
// and kernel dispatch.  Nothing here allocates, frees or synchronises (except
// the opt-in debug checks of device preconditions, which wait for their
// check kernel); every host check runs before the first launch, so a rejected
// call launches nothing.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <atomic>
#include <string>

#include "../../include/sva.h"
#include "sva_internal.h"

namespace {

thread_local std::string g_err;
std::atomic<bool> g_debug_checks{false};   // sva_set_debug_checks

int32_t fail(int32_t code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int32_t ok() {
  g_err.clear();
  return SVA_OK;
}

int32_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(SVA_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool dtype_ok(int32_t t) { return t == SVA_F32 || t == SVA_BF16; }
int32_t elem_bytes(int32_t t) { return t == SVA_F32 ? 4 : 2; }

// shared shape checks; returns SVA_OK or an error status (message set)
int32_t check_slices(const char *fn, int32_t batch, int32_t heads, int32_t n) {
  if (batch < 1 || heads < 1) return fail(SVA_EINVAL, "%s: batch and heads must be >= 1", fn);
  if (static_cast<long long>(batch) * heads > 65535)
    return fail(SVA_EUNSUPPORTED, "%s: batch*heads must be <= 65535", fn);
  if (n < 1) return fail(SVA_EINVAL, "%s: n must be >= 1 (got %d)", fn, n);
  return SVA_OK;
}

int32_t check_d(const char *fn, int32_t d) {
  if (d != 64 && d != 128)
    return fail(SVA_EUNSUPPORTED, "%s: head dim %d not supported (64 or 128)", fn, d);
  return SVA_OK;
}

// value arrays (tensors, centroids) are read and written in 16-byte pieces
int32_t check_a16(const char *fn, const char *what, const void *p) {
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0)
    return fail(SVA_EINVAL, "%s: %s must be 16-byte aligned", fn, what);
  return SVA_OK;
}

int32_t check_ws(const char *fn, size_t need, const void *ws, size_t ws_bytes) {
  if (ws_bytes < need)
    return fail(SVA_EWORKSPACE, "%s: workspace of %zu bytes given, %zu needed", fn, ws_bytes, need);
  if (need > 0 && ws == nullptr) return fail(SVA_EINVAL, "%s: ws is NULL", fn);
  return SVA_OK;
}

#define SVA_TRY(expr)                    \
  do {                                   \
    const int32_t st_ = (expr);          \
    if (st_ != SVA_OK) return st_;       \
  } while (0)

}  // namespace

extern "C" {

const char *sva_last_error(void) { return g_err.c_str(); }

int32_t sva_abi_version(void) { return 1; }

// ---------------------------------------------------------------------------
size_t sva_kmeans_workspace_bytes(int32_t batch, int32_t heads, int32_t n, int32_t d, int32_t c) {
  if (batch < 1 || heads < 1 || n < 1 || c < 1 || (d != 64 && d != 128)) return 0;
  return sva::kmeans_ws_bytes(batch * heads, n, d, c);
}

int32_t sva_kmeans(const void *x, int32_t dtype, int32_t batch, int32_t heads, int32_t n,
                   int32_t d, int32_t c, int32_t iters, float *centroids, int32_t *assign,
                   int32_t *sizes, int32_t *n_refined, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "sva_kmeans";
  if (!x || !centroids || !assign || !sizes)
    return fail(SVA_EINVAL, "%s: x, centroids, assign and sizes must be non-NULL", fn);
  SVA_TRY(check_a16(fn, "x", x));
  SVA_TRY(check_a16(fn, "centroids", centroids));
  if (!dtype_ok(dtype)) return fail(SVA_EINVAL, "%s: bad dtype %d", fn, dtype);
  SVA_TRY(check_slices(fn, batch, heads, n));
  SVA_TRY(check_d(fn, d));
  if (c < 1 || c > n) return fail(SVA_EINVAL, "%s: need 1 <= c <= n (c=%d, n=%d)", fn, c, n);
  if (c > sva::kMaxClustersSort)
    return fail(SVA_EUNSUPPORTED, "%s: c=%d exceeds %d", fn, c, sva::kMaxClustersSort);
  if (iters < 1) return fail(SVA_EINVAL, "%s: iters must be >= 1", fn);
  SVA_TRY(check_ws(fn, sva::kmeans_ws_bytes(batch * heads, n, d, c), ws, ws_bytes));
  sva::KmeansArgs a{x, dtype, batch * heads, n, d, c, iters, centroids, assign, sizes, n_refined, ws};
  return hip_status(sva::launch_kmeans(a, static_cast<hipStream_t>(stream)), fn);
}

int32_t sva_cluster_spread(const void *x, int32_t dtype, int32_t batch, int32_t heads, int32_t n,
                           int32_t d, int32_t c, const float *centroids, const int32_t *assign,
                           double *spread, void *stream) {
  const char *fn = "sva_cluster_spread";
  if (!x || !centroids || !assign || !spread)
    return fail(SVA_EINVAL, "%s: x, centroids, assign and spread must be non-NULL", fn);
  SVA_TRY(check_a16(fn, "x", x));
  SVA_TRY(check_a16(fn, "centroids", centroids));
  if (!dtype_ok(dtype)) return fail(SVA_EINVAL, "%s: bad dtype %d", fn, dtype);
  SVA_TRY(check_slices(fn, batch, heads, n));
  SVA_TRY(check_d(fn, d));
  if (c < 1 || c > n) return fail(SVA_EINVAL, "%s: need 1 <= c <= n (c=%d, n=%d)", fn, c, n);
  return hip_status(sva::launch_cluster_spread(x, dtype, batch * heads, n, d, c, centroids, assign,
                                               spread, static_cast<hipStream_t>(stream)),
                    fn);
}

// ---------------------------------------------------------------------------
size_t sva_permute_workspace_bytes(int32_t batch, int32_t heads, int32_t n, int32_t c) {
  if (batch < 1 || heads < 1 || n < 1 || c < 1) return 0;
  return sva::sort_ws_bytes(batch * heads, n, c);
}

int32_t sva_permute(const int32_t *assign, int32_t c, int32_t batch, int32_t heads, int32_t n,
                    int32_t d, int32_t dtype, int32_t *perm, int32_t *offsets, int32_t n_tensors,
                    const void *const *src, void *const *dst, void *ws, size_t ws_bytes,
                    void *stream) {
  const char *fn = "sva_permute";
  if (!assign || !perm || !offsets)
    return fail(SVA_EINVAL, "%s: assign, perm and offsets must be non-NULL", fn);
  SVA_TRY(check_slices(fn, batch, heads, n));
  if (c < 1 || c > n) return fail(SVA_EINVAL, "%s: need 1 <= c <= n (c=%d, n=%d)", fn, c, n);
  if (c > sva::kMaxClustersSort)
    return fail(SVA_EUNSUPPORTED, "%s: c=%d exceeds %d", fn, c, sva::kMaxClustersSort);
  if (n_tensors < 0 || n_tensors > 2) return fail(SVA_EINVAL, "%s: n_tensors must be 0, 1 or 2", fn);
  if (n_tensors > 0) {
    if (!dtype_ok(dtype)) return fail(SVA_EINVAL, "%s: bad dtype %d", fn, dtype);
    SVA_TRY(check_d(fn, d));
    if (!src || !dst) return fail(SVA_EINVAL, "%s: src and dst arrays must be non-NULL", fn);
    for (int t = 0; t < n_tensors; ++t) {
      if (!src[t] || !dst[t]) return fail(SVA_EINVAL, "%s: tensor pointer %d is NULL", fn, t);
      SVA_TRY(check_a16(fn, "every tensor", src[t]));
      SVA_TRY(check_a16(fn, "every tensor", dst[t]));
    }
  }
  SVA_TRY(check_ws(fn, sva::sort_ws_bytes(batch * heads, n, c), ws, ws_bytes));
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int bh = batch * heads;
  hipError_t e = sva::launch_cluster_sort(assign, bh, n, c, perm, offsets, nullptr, ws, s);
  for (int t = 0; t < n_tensors && e == hipSuccess; ++t)
    e = sva::launch_gather_rows(src[t], dst[t], perm, bh, n, d * elem_bytes(dtype), 0, s);
  return hip_status(e, fn);
}

int32_t sva_gather_slices(const void *src, void *dst, const int32_t *idx, int32_t n_idx,
                          int64_t slice_bytes, int32_t scatter, void *stream) {
  const char *fn = "sva_gather_slices";
  if (!src || !dst || !idx) return fail(SVA_EINVAL, "%s: src, dst and idx must be non-NULL", fn);
  if (n_idx < 0 || n_idx > 65535)
    return fail(SVA_EINVAL, "%s: need 0 <= n_idx <= 65535 (n_idx=%d)", fn, n_idx);
  if (slice_bytes <= 0 || slice_bytes % 16 != 0)
    return fail(SVA_EINVAL, "%s: slice_bytes must be a positive multiple of 16", fn);
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return fail(SVA_EINVAL, "%s: src and dst must be 16-byte aligned", fn);
  if (scatter != 0 && scatter != 1) return fail(SVA_EINVAL, "%s: scatter must be 0 or 1", fn);
  return hip_status(sva::launch_move_slices(src, dst, idx, n_idx, slice_bytes, scatter,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

// ---------------------------------------------------------------------------
size_t sva_select_workspace_bytes(int32_t, int32_t, int32_t, int32_t) { return 0; }

int32_t sva_select_blocks(const float *cent_q, const int32_t *size_q, int32_t cq,
                          const float *cent_k, const int32_t *size_k, int32_t ck, int32_t batch,
                          int32_t heads, int32_t d, double scale, double top_p, uint8_t *mask,
                          int32_t *kept_count, int32_t *kept_idx, void *ws, size_t ws_bytes,
                          void *stream) {
  const char *fn = "sva_select_blocks";
  (void)ws;
  (void)ws_bytes;
  if (!cent_q || !size_q || !cent_k || !size_k || !mask || !kept_count || !kept_idx)
    return fail(SVA_EINVAL, "%s: NULL pointer argument", fn);
  SVA_TRY(check_a16(fn, "cent_q", cent_q));
  SVA_TRY(check_a16(fn, "cent_k", cent_k));
  SVA_TRY(check_slices(fn, batch, heads, 1));
  SVA_TRY(check_d(fn, d));
  if (cq < 1 || ck < 1) return fail(SVA_EINVAL, "%s: cq and ck must be >= 1", fn);
  if (ck > sva::kMaxSelectK)
    return fail(SVA_EUNSUPPORTED, "%s: ck=%d exceeds %d", fn, ck, sva::kMaxSelectK);
  if (!(top_p > 0.0 && top_p <= 1.0))
    return fail(SVA_EINVAL, "%s: top_p must be in (0, 1] (got %g)", fn, top_p);
  if (!isfinite(scale)) return fail(SVA_EINVAL, "%s: scale must be finite", fn);
  sva::SelectArgs a{cent_q, cent_k, size_q, size_k, batch * heads, cq, ck, d, scale, top_p,
                    mask, kept_count, kept_idx};
  return hip_status(sva::launch_select(a, static_cast<hipStream_t>(stream)), fn);
}

int32_t sva_select_threshold(const float *cent_q, const int32_t *size_q, int32_t nq,
                             const float *cent_k, const int32_t *size_k, int32_t nk,
                             int32_t batch, int32_t heads, int32_t d, double scale, double theta,
                             const uint8_t *cand, uint8_t *mask, int32_t *kept_count,
                             int32_t *kept_idx, void *stream) {
  const char *fn = "sva_select_threshold";
  if (!cent_q || !size_q || !cent_k || !size_k || !mask || !kept_count || !kept_idx)
    return fail(SVA_EINVAL, "%s: NULL pointer argument", fn);
  SVA_TRY(check_a16(fn, "cent_q", cent_q));
  SVA_TRY(check_a16(fn, "cent_k", cent_k));
  SVA_TRY(check_slices(fn, batch, heads, 1));
  SVA_TRY(check_d(fn, d));
  if (nq < 1 || nk < 1) return fail(SVA_EINVAL, "%s: nq and nk must be >= 1", fn);
  if (nq > 65535) return fail(SVA_EUNSUPPORTED, "%s: nq=%d exceeds 65535", fn, nq);
  if (nk > sva::kMaxSelectK)
    return fail(SVA_EUNSUPPORTED, "%s: nk=%d exceeds %d", fn, nk, sva::kMaxSelectK);
  if (!isfinite(scale)) return fail(SVA_EINVAL, "%s: scale must be finite", fn);
  if (isnan(theta)) return fail(SVA_EINVAL, "%s: theta is NaN", fn);
  sva::ThresholdArgs a{cent_q, cent_k, size_q, size_k, batch * heads, nq, nk, d, scale, theta,
                       cand, mask, kept_count, kept_idx};
  return hip_status(sva::launch_select_threshold(a, static_cast<hipStream_t>(stream)), fn);
}

int32_t sva_radial_mask(int32_t n, int32_t hw, int32_t block, int32_t dt_max, int32_t window0,
                        const float *ratios, int32_t batch, int32_t heads, uint8_t *mask,
                        int32_t *kept_count, int32_t *kept_idx, void *stream) {
  const char *fn = "sva_radial_mask";
  if (!ratios || !mask || !kept_count || !kept_idx)
    return fail(SVA_EINVAL, "%s: NULL pointer argument", fn);
  SVA_TRY(check_slices(fn, batch, heads, n));
  if (hw < 1 || block < 1) return fail(SVA_EINVAL, "%s: hw and block must be >= 1", fn);
  if (dt_max < 0 || dt_max > sva::kMaxRadialDt)
    return fail(SVA_EINVAL, "%s: dt_max must be in [0, %d] (got %d)", fn, sva::kMaxRadialDt, dt_max);
  if (window0 < 0) return fail(SVA_EINVAL, "%s: window0 must be >= 0", fn);
  sva::RadialParams p{};
  p.n = n;
  p.hw = hw;
  p.block = block;
  p.nb = static_cast<int32_t>((static_cast<long long>(n) + block - 1) / block);
  p.dt_max = dt_max;
  p.window0 = window0;
  for (int t = 0; t <= dt_max; ++t) {
    if (!(ratios[t] >= 0.f && ratios[t] <= 1.f))
      return fail(SVA_EINVAL, "%s: ratios[%d] must be in [0, 1] (got %g)", fn, t, ratios[t]);
    p.ratio[t] = ratios[t];
  }
  const long long span = (2LL * dt_max + 1) * (hw / block + 2) + 1;
  if (span > sva::kMaxRadialRow)
    return fail(SVA_EUNSUPPORTED, "%s: %lld candidate blocks per row exceed %d", fn, span,
                sva::kMaxRadialRow);
  if (static_cast<long long>(batch) * heads * p.nb * p.nb > (1LL << 40))
    return fail(SVA_EUNSUPPORTED, "%s: mask too large", fn);
  return hip_status(sva::launch_radial_mask(p, batch * heads, mask, kept_count, kept_idx,
                                            static_cast<hipStream_t>(stream)), fn);
}

int32_t sva_block_means(const void *x, int32_t dtype, int32_t batch, int32_t heads, int32_t n,
                        int32_t d, int32_t block, float *means, int32_t *sizes, void *stream) {
  const char *fn = "sva_block_means";
  if (!x || !means || !sizes) return fail(SVA_EINVAL, "%s: NULL pointer argument", fn);
  SVA_TRY(check_a16(fn, "x", x));
  if (!dtype_ok(dtype)) return fail(SVA_EINVAL, "%s: bad dtype %d", fn, dtype);
  SVA_TRY(check_slices(fn, batch, heads, n));
  SVA_TRY(check_d(fn, d));
  if (block < 1) return fail(SVA_EINVAL, "%s: block must be >= 1", fn);
  return hip_status(sva::launch_block_means(x, dtype, batch * heads, n, d, block, means, sizes,
                                            static_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
static int32_t check_attn(const char *fn, const void *q, const void *k, const void *v,
                          int32_t dtype, int32_t batch, int32_t heads, int32_t n_q, int32_t n_k,
                          int32_t d, float scale, const void *o, int32_t o_dtype) {
  if (!q || !k || !v || !o) return fail(SVA_EINVAL, "%s: q, k, v and o must be non-NULL", fn);
  SVA_TRY(check_a16(fn, "q", q));
  SVA_TRY(check_a16(fn, "k", k));
  SVA_TRY(check_a16(fn, "v", v));
  SVA_TRY(check_a16(fn, "o", o));
  if (!dtype_ok(dtype) || !dtype_ok(o_dtype))
    return fail(SVA_EINVAL, "%s: bad dtype (%d) or o_dtype (%d)", fn, dtype, o_dtype);
  SVA_TRY(check_slices(fn, batch, heads, n_q));
  if (n_k < 1) return fail(SVA_EINVAL, "%s: n_k must be >= 1", fn);
  SVA_TRY(check_d(fn, d));
  // the bf16 kernel's running max is taken on the raw scores and scaled
  // afterwards, which is the max of the scaled scores only for scale >= 0
  if (!isfinite(scale) || scale < 0.f)
    return fail(SVA_EINVAL, "%s: scale must be finite and >= 0 (got %g)", fn, scale);
  return SVA_OK;
}

size_t sva_attn_workspace_bytes(int32_t batch, int32_t heads, int32_t n_q, int32_t n_qblocks) {
  if (batch < 1 || heads < 1 || n_q < 1 || n_qblocks < 1) return 0;
  return sva::attn_ws_bytes(batch * heads, n_q, n_qblocks);
}

static int32_t block_sparse(const char *fn, const void *q, const void *k, const void *v,
                            int32_t dtype, int32_t batch, int32_t heads, int32_t n_q, int32_t n_k,
                            int32_t d, const int32_t *q_perm, const int32_t *k_perm,
                            const int32_t *q_offsets, int32_t n_qblocks,
                            const int32_t *k_offsets, int32_t n_kblocks,
                            const int32_t *kept_count, const int32_t *kept_idx,
                            int32_t kept_stride, float scale, void *o, int32_t o_dtype,
                            float *lse, void *ws, size_t ws_bytes, void *stream,
                            bool static_ws = false) {
  SVA_TRY(check_attn(fn, q, k, v, dtype, batch, heads, n_q, n_k, d, scale, o, o_dtype));
  if (!q_offsets || !k_offsets || !kept_count || !kept_idx)
    return fail(SVA_EINVAL, "%s: offsets and kept lists must be non-NULL", fn);
  if (n_qblocks < 1 || n_qblocks > n_q)
    return fail(SVA_EINVAL, "%s: need 1 <= n_qblocks <= n_q", fn);
  if (n_kblocks < 1 || n_kblocks > n_k)
    return fail(SVA_EINVAL, "%s: need 1 <= n_kblocks <= n_k", fn);
  if (kept_stride < 1) return fail(SVA_EINVAL, "%s: kept_stride must be >= 1", fn);
  const long long items = static_cast<long long>(batch) * heads * ((n_q + 127) / 128 + n_qblocks);
  if (items > 0x7ffffff0LL) return fail(SVA_EUNSUPPORTED, "%s: problem too large for one launch", fn);
  const size_t need = sva::attn_ws_bytes(batch * heads, n_q, n_qblocks);
  if (static_ws) {
    if (need > sva::kStaticAttnScratch)
      return fail(SVA_EWORKSPACE,
                  "%s: the work schedule needs %zu bytes, more than the %zu-byte static scratch "
                  "(use sva_block_sparse_attn with a workspace)",
                  fn, need, sva::kStaticAttnScratch);
    hipError_t e = hipSuccess;
    ws = sva::attn_static_scratch(&e);
    if (ws == nullptr) return hip_status(e, fn);
    ws_bytes = sva::kStaticAttnScratch;
  } else {
    SVA_TRY(check_ws(fn, need, ws, ws_bytes));
  }
  sva::AttnArgs a{q, k, v, o, lse, q_offsets, k_offsets, kept_count, kept_idx, q_perm, k_perm,
                  kept_stride, batch * heads, n_q, n_k, d, n_qblocks, n_kblocks, dtype, o_dtype,
                  0, scale, ws};
  if (g_debug_checks.load()) {
    int32_t bits = 0;
    hipError_t e = sva::attn_debug_check(a, static_cast<hipStream_t>(stream), &bits);
    if (e != hipSuccess) return hip_status(e, fn);
    if (bits != 0)
      return fail(SVA_EINVAL,
                  "%s: debug check: device preconditions violated:%s%s%s%s%s%s", fn,
                  bits & sva::kDebugQOffsets ? " q_offsets not monotone in [0, n_q]" : "",
                  bits & sva::kDebugKOffsets ? " k_offsets not monotone in [0, n_k]" : "",
                  bits & sva::kDebugKeptCount ? " kept_count outside [0, min(kept_stride, n_kblocks)]" : "",
                  bits & sva::kDebugKeptIdx ? " kept_idx outside [0, n_kblocks)" : "",
                  bits & sva::kDebugQPerm ? " q_perm outside [0, n_q)" : "",
                  bits & sva::kDebugKPerm ? " k_perm outside [0, n_k)" : "");
  }
  return hip_status(sva::launch_attention(a, static_cast<hipStream_t>(stream)), fn);
}

int32_t sva_set_debug_checks(int32_t on) {
  g_debug_checks.store(on != 0);
  return SVA_OK;
}

int32_t sva_block_sparse_attn(const void *q, const void *k, const void *v, int32_t dtype,
                              int32_t batch, int32_t heads, int32_t n_q, int32_t n_k, int32_t d,
                              const int32_t *q_offsets, int32_t n_qblocks,
                              const int32_t *k_offsets, int32_t n_kblocks,
                              const int32_t *kept_count, const int32_t *kept_idx,
                              int32_t kept_stride, float scale, void *o, int32_t o_dtype,
                              float *lse, void *ws, size_t ws_bytes, void *stream) {
  return block_sparse("sva_block_sparse_attn", q, k, v, dtype, batch, heads, n_q, n_k, d,
                      nullptr, nullptr, q_offsets, n_qblocks, k_offsets, n_kblocks, kept_count,
                      kept_idx, kept_stride, scale, o, o_dtype, lse, ws, ws_bytes, stream);
}

int32_t sva_block_sparse_attn_noalloc(const void *q, const void *k, const void *v,
                                      int32_t dtype, int32_t batch, int32_t heads, int32_t n_q,
                                      int32_t n_k, int32_t d, const int32_t *q_offsets,
                                      int32_t n_qblocks, const int32_t *k_offsets,
                                      int32_t n_kblocks, const int32_t *kept_count,
                                      const int32_t *kept_idx, int32_t kept_stride, float scale,
                                      void *o, int32_t o_dtype, float *lse, void *stream) {
  return block_sparse("sva_block_sparse_attn_noalloc", q, k, v, dtype, batch, heads, n_q, n_k, d,
                      nullptr, nullptr, q_offsets, n_qblocks, k_offsets, n_kblocks, kept_count,
                      kept_idx, kept_stride, scale, o, o_dtype, lse, nullptr, 0, stream, true);
}

int32_t sva_block_sparse_attn_perm(const void *q, const void *k, const void *v, int32_t dtype,
                                   int32_t batch, int32_t heads, int32_t n_q, int32_t n_k,
                                   int32_t d, const int32_t *q_perm, const int32_t *k_perm,
                                   const int32_t *q_offsets, int32_t n_qblocks,
                                   const int32_t *k_offsets, int32_t n_kblocks,
                                   const int32_t *kept_count, const int32_t *kept_idx,
                                   int32_t kept_stride, float scale, void *o, int32_t o_dtype,
                                   float *lse, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "sva_block_sparse_attn_perm";
  if (!q_perm || !k_perm) return fail(SVA_EINVAL, "%s: q_perm and k_perm must be non-NULL", fn);
  return block_sparse(fn, q, k, v, dtype, batch, heads, n_q, n_k, d, q_perm, k_perm, q_offsets,
                      n_qblocks, k_offsets, n_kblocks, kept_count, kept_idx, kept_stride, scale,
                      o, o_dtype, lse, ws, ws_bytes, stream);
}

size_t sva_full_attn_workspace_bytes(int32_t, int32_t, int32_t) { return 0; }

int32_t sva_full_attn(const void *q, const void *k, const void *v, int32_t dtype, int32_t batch,
                      int32_t heads, int32_t n_q, int32_t n_k, int32_t d, float scale, void *o,
                      int32_t o_dtype, float *lse, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "sva_full_attn";
  (void)ws;
  (void)ws_bytes;
  SVA_TRY(check_attn(fn, q, k, v, dtype, batch, heads, n_q, n_k, d, scale, o, o_dtype));
  sva::AttnArgs a{q, k, v, o, lse, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                  batch * heads, n_q, n_k, d, 1, 1, dtype, o_dtype, 1, scale, nullptr};
  return hip_status(sva::launch_attention(a, static_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
int32_t sva_check_mfma_rounding(int32_t *flags, void *stream) {
  const char *fn = "sva_check_mfma_rounding";
  if (!flags) return fail(SVA_EINVAL, "%s: NULL pointer argument", fn);
  return hip_status(sva::launch_mfma_rounding_check(flags, static_cast<hipStream_t>(stream)), fn);
}

// ---------------------------------------------------------------------------
int32_t sva_unpermute(const void *o_perm, const int32_t *perm, int32_t dtype, int32_t batch,
                      int32_t heads, int32_t n, int32_t d, void *o, void *stream) {
  const char *fn = "sva_unpermute";
  if (!o_perm || !perm || !o) return fail(SVA_EINVAL, "%s: NULL pointer argument", fn);
  SVA_TRY(check_a16(fn, "o_perm", o_perm));
  SVA_TRY(check_a16(fn, "o", o));
  if (!dtype_ok(dtype)) return fail(SVA_EINVAL, "%s: bad dtype %d", fn, dtype);
  SVA_TRY(check_slices(fn, batch, heads, n));
  SVA_TRY(check_d(fn, d));
  return hip_status(sva::launch_gather_rows(o_perm, o, perm, batch * heads, n,
                                            d * elem_bytes(dtype), 1,
                                            static_cast<hipStream_t>(stream)),
                    fn);
}

}  // extern "C"
