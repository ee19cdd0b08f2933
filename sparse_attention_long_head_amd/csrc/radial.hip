// DynamicRad's radial candidate set and static-ratio mask, and block means
// (the proxies of its dynamic-threshold mode), for gfx950.  DynamicRad
// explainer, technical summary section 2.a: one radial locality candidate set
// (block attention fades with spatial and temporal distance) and two modes;
// the static-ratio mode keeps a fixed share of the candidates per temporal
// distance with no content scoring.
//
// Uniform blocks of `block` consecutive tokens on the frame-major token grid:
// block b starts at token block*b, lies in frame t_b = (block*b) / hw and at
// window index s_b = ((block*b) % hw) / block.  (a, b) is a candidate when
// dt = |t_a - t_b| <= dt_max and |s_a - s_b| <= window0 >> dt.  The static
// ratio keeps, for each query block and each dt, the first ceil(r[dt] * n)
// of the n candidates at that distance in (|s_a - s_b|, b) order.
#include <math.h>

#include "../../include/sva.h"
#include "sva_internal.h"

namespace sva {
namespace {

constexpr int kRadThreads = 256;

__device__ __forceinline__ long long first_block(long long frame, int hw, int block) {
  return (frame * hw + block - 1) / block;   // first block starting in the frame
}

// One workgroup per query block: wave 0 walks the blocks of frames
// t_a - dt_max .. t_a + dt_max (the only ones that can be candidates) and
// builds the ascending kept list; then every thread writes the row for every
// slice (the mask does not depend on content, so all slices share it).
__global__ __launch_bounds__(kRadThreads) void radial_kernel(RadialParams p, int bh,
                                                             uint8_t *__restrict__ mask,
                                                             int32_t *__restrict__ kept_count,
                                                             int32_t *__restrict__ kept_idx) {
  __shared__ int32_t sKept[kMaxRadialRow];
  __shared__ int32_t sCnt;
  const int a = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const long long start_a = static_cast<long long>(a) * p.block;
  const int ta = static_cast<int>(start_a / p.hw);
  const int sa = static_cast<int>((start_a % p.hw) / p.block);
  const long long b_lo = first_block(max(0, ta - p.dt_max), p.hw, p.block);
  const long long b_hi = min(static_cast<long long>(p.nb),
                             first_block(static_cast<long long>(ta) + p.dt_max + 1, p.hw, p.block));
  if (tid < 64) {
    int cnt = 0;
    for (long long base = b_lo; base < b_hi; base += 64) {
      const long long b = base + lane;
      bool keep = false;
      if (b < b_hi) {
        const long long sb0 = b * p.block;
        const int tb = static_cast<int>(sb0 / p.hw);
        const int sb = static_cast<int>((sb0 % p.hw) / p.block);
        const int dt = abs(ta - tb), ds = abs(sa - sb);
        if (dt <= p.dt_max && ds <= (p.window0 >> dt)) {
          // rank of b among the candidates at distance dt, and their number
          int n = 0, rank = 0;
          for (int side = 0; side < (dt == 0 ? 1 : 2); ++side) {
            const int f = side == 0 ? ta - dt : ta + dt;
            if (f < 0) continue;
            const long long f_lo = first_block(f, p.hw, p.block);
            const long long f_hi = min(static_cast<long long>(p.nb), first_block(f + 1LL, p.hw, p.block));
            for (long long b2 = f_lo; b2 < f_hi; ++b2) {
              const int s2 = static_cast<int>(((b2 * p.block) % p.hw) / p.block);
              const int ds2 = abs(sa - s2);
              if (ds2 <= (p.window0 >> dt)) {
                ++n;
                if (ds2 < ds || (ds2 == ds && b2 < b)) ++rank;
              }
            }
          }
          const int k = static_cast<int>(ceil(static_cast<double>(p.ratio[dt]) * n));
          keep = rank < k;
        }
      }
      const uint64_t bal = __ballot(keep);
      if (keep) sKept[cnt + __popcll(bal & ((1ull << lane) - 1))] = static_cast<int32_t>(b);
      cnt += __popcll(bal);
    }
    if (lane == 0) sCnt = cnt;
  }
  __syncthreads();
  const int cnt = sCnt;
  for (int s = 0; s < bh; ++s) {
    const size_t row = static_cast<size_t>(s) * p.nb + a;
    uint8_t *mrow = mask + row * p.nb;
    int32_t *irow = kept_idx + row * p.nb;
    for (int j = tid; j < p.nb; j += kRadThreads) {
      mrow[j] = 0;
      irow[j] = j < cnt ? sKept[j] : -1;
    }
    __syncthreads();   // the zeros land before the kept flags of this row
    for (int j = tid; j < cnt; j += kRadThreads) mrow[sKept[j]] = 1;
    if (tid == 0) kept_count[row] = cnt;
  }
}

// Block means: a thread owns one 16-byte piece of the row (8 bf16 or 4 fp32
// columns) of one block and adds the block's rows into fp64 accumulators in
// row order, eight rows' loads in flight; the sum divided by the row count is
// stored as fp32.  A workgroup of kMeanThr threads covers kMeanThr / pieces
// consecutive blocks of one slice.
constexpr int kMeanThr = 256;
template <typename T, int D>
__global__ __launch_bounds__(kMeanThr) void block_means_kernel(
    const T *__restrict__ x, int n, int block, int nb, float *__restrict__ means,
    int32_t *__restrict__ sizes) {
  constexpr int EPT = 16 / sizeof(T);          // columns per thread
  constexpr int PPR = D / EPT;                 // threads per block (pieces per row)
  constexpr int BPW = kMeanThr / PPR;          // blocks per workgroup
  constexpr int U = 8;                         // rows in flight
  const int s = blockIdx.y, tid = threadIdx.x;
  const int b = blockIdx.x * BPW + tid / PPR, pc = tid % PPR;
  if (b >= nb) return;
  const int r0 = b * block, r1 = min(n, r0 + block);
  const u32x4 *src = reinterpret_cast<const u32x4 *>(x + (static_cast<size_t>(s) * n + r0) * D) + pc;
  double acc[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) acc[e] = 0.0;
  for (int r = r0; r < r1; r += U) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)   // (clamped: every load is in the block, all U in flight)
      v[u] = src[static_cast<size_t>(min(r + u, r1 - 1) - r0) * PPR];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = r + u < r1;   // rows past the block add +0 (no branch, so the loads stay ahead)
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        float f;
        if constexpr (sizeof(T) == 2) f = bf16_bits_to_f32(static_cast<uint16_t>(v[u][e >> 1] >> (16 * (e & 1))));
        else f = __uint_as_float(v[u][e]);
        acc[e] += in ? static_cast<double>(f) : 0.0;
      }
    }
  }
  float *out = means + (static_cast<size_t>(s) * nb + b) * D + pc * EPT;
#pragma unroll
  for (int e = 0; e < EPT; ++e) out[e] = static_cast<float>(acc[e] / (r1 - r0));
  if (pc == 0) sizes[static_cast<size_t>(s) * nb + b] = r1 - r0;
}

}  // namespace

hipError_t launch_radial_mask(const RadialParams &p, int32_t bh, uint8_t *mask,
                              int32_t *kept_count, int32_t *kept_idx, hipStream_t s) {
  hipLaunchKernelGGL(radial_kernel, dim3(p.nb), dim3(kRadThreads), 0, s, p, bh, mask, kept_count,
                     kept_idx);
  return hipGetLastError();
}

hipError_t launch_block_means(const void *x, int32_t dtype, int32_t bh, int32_t n, int32_t d,
                              int32_t block, float *means, int32_t *sizes, hipStream_t s) {
  const int nb = (n + block - 1) / block;
  // blocks per workgroup: kMeanThr / (d / columns per thread)
  auto grid = [&](int cols) { return dim3((nb + kMeanThr / (d / cols) - 1) / (kMeanThr / (d / cols)), bh); };
#define SVA_MEANS(T, DD, COLS)                                                              \
  hipLaunchKernelGGL((block_means_kernel<T, DD>), grid(COLS), dim3(kMeanThr), 0, s,          \
                     static_cast<const T *>(x), n, block, nb, means, sizes)
  if (dtype == SVA_BF16) {
    if (d == 128) SVA_MEANS(uint16_t, 128, 8);
    else SVA_MEANS(uint16_t, 64, 8);
  } else {
    if (d == 128) SVA_MEANS(float, 128, 4);
    else SVA_MEANS(float, 64, 4);
  }
#undef SVA_MEANS
  return hipGetLastError();
}

}  // namespace sva
