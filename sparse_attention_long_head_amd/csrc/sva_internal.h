// Internal declarations shared by the libsva HIP sources (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sva {

// ---------------------------------------------------------------------------
// vector types for MFMA operands / accumulators and 16-byte memory moves
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);   // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// 32x32x16 bf16 MFMA: D = A(32x16) * B(16x32) + C, fp32 accumulate.
// Operand layout (wave64): lane l holds A[l%32][8*(l/32) .. +8] and
// B[8*(l/32) .. +8][l%32]; the accumulator element i of lane l is
// C[8*(i/4) + 4*(l/32) + (i%4)][l%32].
__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// row index (0..31) held by accumulator element i of a lane in half h
__device__ __forceinline__ constexpr int acc_row(int i, int h) { return 8 * (i / 4) + 4 * h + (i % 4); }

// ---------------------------------------------------------------------------
// launchers (host side, defined in the .hip files).  All return hipError_t of
// the launch and take the stream to enqueue on.
// ---------------------------------------------------------------------------
struct AttnArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  const int32_t *q_off, *k_off, *kept_count, *kept_idx;
  const int32_t *q_perm, *k_perm;   // NULL, or permuted row -> original row (fused permutation)
  int32_t kept_stride;
  int32_t bh, n_q, n_k, d, nqb, nkb;
  int32_t dtype, o_dtype;     // SVA_F32 / SVA_BF16
  int32_t dense;              // 1: one block holding every key (sva_full_attn)
  float scale;
  void *ws;                   // schedule scratch (sparse only)
};
size_t attn_ws_bytes(int32_t bh, int32_t n_q, int32_t nqb);
hipError_t launch_attention(const AttnArgs &a, hipStream_t s);
// the static schedule scratch of the no-allocation entry point: its device
// address on the current device (looked up once per device), or NULL with *err
constexpr size_t kStaticAttnScratch = size_t{8} << 20;
void *attn_static_scratch(hipError_t *err);
// debug checks of the block-sparse calls' device preconditions: *bits = the
// violated ones (0: none); synchronises the stream
enum : int32_t {
  kDebugQOffsets = 1, kDebugKOffsets = 2, kDebugKeptCount = 4, kDebugKeptIdx = 8,
  kDebugQPerm = 16, kDebugKPerm = 32
};
hipError_t attn_debug_check(const AttnArgs &a, hipStream_t s, int32_t *bits);

struct KmeansArgs {
  const void *x;
  int32_t dtype, bh, n, d, c, iters;
  float *centroids;
  int32_t *assign, *sizes, *n_refined;
  void *ws;
};
size_t kmeans_ws_bytes(int32_t bh, int32_t n, int32_t d, int32_t c);
hipError_t launch_kmeans(const KmeansArgs &a, hipStream_t s);
hipError_t launch_cluster_spread(const void *x, int32_t dtype, int32_t bh, int32_t n, int32_t d,
                                 int32_t c, const float *cent, const int32_t *assign,
                                 double *out, hipStream_t s);

// stable counting sort of rows by cluster id (shared by k-means and permute);
// `clear`, if not NULL, holds bh ints that the sort sets to zero; `seg`, if
// not NULL, [bh][n] receives the cluster id of every sorted position
size_t sort_ws_bytes(int32_t bh, int32_t n, int32_t c);
hipError_t launch_cluster_sort(const int32_t *assign, int32_t bh, int32_t n, int32_t c,
                               int32_t *perm, int32_t *offsets, int32_t *sizes, void *ws,
                               hipStream_t s, int32_t *clear = nullptr, int32_t *seg = nullptr);
hipError_t launch_gather_rows(const void *src, void *dst, const int32_t *perm, int32_t bh,
                              int32_t n, int32_t row_bytes, int32_t scatter, hipStream_t s);

struct SelectArgs {
  const float *cent_q, *cent_k;
  const int32_t *size_q, *size_k;
  int32_t bh, cq, ck, d;
  double scale, top_p;
  uint8_t *mask;
  int32_t *kept_count, *kept_idx;
};
hipError_t launch_select(const SelectArgs &a, hipStream_t s);

struct ThresholdArgs {
  const float *cent_q, *cent_k;
  const int32_t *size_q, *size_k;
  int32_t bh, nq, nk, d;
  double scale, theta;
  const uint8_t *cand;   // [nq][nk] shared by all slices, or nullptr
  uint8_t *mask;
  int32_t *kept_count, *kept_idx;
};
hipError_t launch_select_threshold(const ThresholdArgs &a, hipStream_t s);

constexpr int kMaxRadialDt = 15;        // largest temporal distance of the radial set
constexpr int kMaxRadialRow = 8192;     // LDS capacity for one query block's kept list
struct RadialParams {
  int32_t n, hw, block, nb, dt_max, window0;
  float ratio[kMaxRadialDt + 1];
};
hipError_t launch_radial_mask(const RadialParams &p, int32_t bh, uint8_t *mask,
                              int32_t *kept_count, int32_t *kept_idx, hipStream_t s);
hipError_t launch_block_means(const void *x, int32_t dtype, int32_t bh, int32_t n, int32_t d,
                              int32_t block, float *means, int32_t *sizes, hipStream_t s);

hipError_t launch_fill_i32(int32_t *p, int32_t value, size_t count, hipStream_t s);
hipError_t launch_move_slices(const void *src, void *dst, const int32_t *idx, int32_t n_idx,
                              long long slice_bytes, int32_t scatter, hipStream_t s);

// compute units of the current device (persistent grids); 256 if the query fails
int device_cus();

// the accumulate-path rounding check of the bf16 MFMA (flags[kMfmaChecks])
constexpr int kMfmaChecks = 8;
hipError_t launch_mfma_rounding_check(int32_t *flags, hipStream_t s);

constexpr int kMaxClustersSort = 16384;   // LDS counter capacity of the sort
constexpr int kMaxSelectK = 4096;         // LDS sort capacity of top-p selection

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace sva
