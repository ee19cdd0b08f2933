// Centroid-based top-p block selection for gfx950 (Sparse VideoGen2 explainer,
// technical summary section 2.b; DynamicRad explainer, section 2.a: a block
// never ends empty).
//
// One workgroup per (slice, Q cluster), all arithmetic in fp64:
//   scores S_j = (mu_q . mu_k_j) * scale over the K clusters;
//   P_j = size_k_j exp(S_j - max) / sum over non-empty K clusters (the mass the
//   Q centroid's softmax gives cluster j when its keys are replaced by its
//   centroid);
//   bitonic sort in LDS by (P descending, id ascending), empty clusters last;
//   block scan of the sorted P; keep the shortest prefix reaching top_p;
//   write the u8 mask row and the ascending list of kept ids (the compact list
//   the attention kernel walks, so no wave ever touches a skipped block).
// Integer outputs depend on fp64 comparisons only, and every reduction and
// scan has a fixed order, so results are deterministic.
#include <math.h>

#include "../../include/sva.h"
#include "sva_internal.h"

namespace sva {
namespace {

constexpr int kThreads = 256;
constexpr int kCap = kMaxSelectK;
constexpr int kPer = kCap / kThreads;   // entries per thread in the scans

__device__ __forceinline__ bool before(double ka, int ia, double kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ double block_reduce_max(double v, double *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = fmax(r, red[w]);
  __syncthreads();
  return r;
}

__device__ double block_reduce_sum(double v, double *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  double r = 0.0;
  for (int w = 0; w < kThreads / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

__device__ int block_reduce_isum(int v, int *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = 0;
  for (int w = 0; w < kThreads / 64; ++w) r += red[w];
  __syncthreads();
  return r;
}

__device__ int block_reduce_imin(int v, int *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int r = red[0];
  for (int w = 1; w < kThreads / 64; ++w) r = min(r, red[w]);
  __syncthreads();
  return r;
}

// sum over d of q[d] * k[d] in fp64, one fma per term in ascending d; the
// fp32 row is read in 16-byte pieces, eight at a time
template <int D>
__device__ __forceinline__ double centroid_dot(const double *q, const float *k) {
  const f32x4 *k4 = reinterpret_cast<const f32x4 *>(k);
  double s = 0.0;
#pragma unroll 1   // (unrolled, the compiler keeps all of q in registers across j)
  for (int p0 = 0; p0 < D / 4; p0 += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = k4[p0 + u];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) s = fma(q[4 * (p0 + u) + e], static_cast<double>(v[u][e]), s);
  }
  return s;
}

template <int D>
__global__ __launch_bounds__(kThreads) void select_kernel(
    const float *__restrict__ cent_q, const int32_t *__restrict__ size_q,
    const float *__restrict__ cent_k, const int32_t *__restrict__ size_k, int cq, int ck, int ckp,
    double scale, double top_p, uint8_t *__restrict__ mask, int32_t *__restrict__ kept_count,
    int32_t *__restrict__ kept_idx) {
  // sort arrays sized by the launch for ckp keys (not the kCap maximum), so
  // small C_k leaves room for more workgroups per CU
  extern __shared__ __attribute__((aligned(16))) unsigned char s_sel[];
  double *key = reinterpret_cast<double *>(s_sel);              // [ckp]
  int32_t *idx = reinterpret_cast<int32_t *>(key + ckp);         // [ckp]
  uint8_t *mk = reinterpret_cast<uint8_t *>(idx + ckp);          // [ck]
  __shared__ double sq[D];
  __shared__ double red[kThreads / 64];
  __shared__ int ired[kThreads / 64];

  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  uint8_t *mrow = mask + (static_cast<size_t>(bh) * cq + i) * ck;
  int32_t *irow = kept_idx + (static_cast<size_t>(bh) * cq + i) * ck;
  const int32_t *szk = size_k + static_cast<size_t>(bh) * ck;
  if (size_q[static_cast<size_t>(bh) * cq + i] == 0) {
    for (int j = tid; j < ck; j += kThreads) {
      mrow[j] = 0;
      irow[j] = -1;
    }
    if (tid == 0) kept_count[static_cast<size_t>(bh) * cq + i] = 0;
    return;
  }
  if (tid < D) sq[tid] = static_cast<double>(cent_q[(static_cast<size_t>(bh) * cq + i) * D + tid]);
  __syncthreads();

  // scores and max over non-empty K clusters
  double lmax = -INFINITY;
  int lvalid = 0;
  for (int j = tid; j < ck; j += kThreads) {
    const double s = centroid_dot<D>(sq, cent_k + (static_cast<size_t>(bh) * ck + j) * D) * scale;
    key[j] = s;
    if (szk[j] > 0) {
      lmax = fmax(lmax, s);
      ++lvalid;
    }
  }
  const double smax = block_reduce_max(lmax, red);
  const int n_valid = block_reduce_isum(lvalid, ired);
  double lsum = 0.0;
  for (int j = tid; j < ck; j += kThreads) {
    const double w = szk[j] > 0 ? static_cast<double>(szk[j]) * exp(key[j] - smax) : 0.0;
    key[j] = w;
    lsum += w;
  }
  const double total = block_reduce_sum(lsum, red);
  for (int j = tid; j < ckp; j += kThreads) {
    if (j < ck) {
      key[j] = szk[j] > 0 ? key[j] / total : -1.0;
      idx[j] = j;
    } else {
      key[j] = -2.0;
      idx[j] = 0x7fffffff;
    }
  }
  __syncthreads();

  // bitonic sort: (P descending, id ascending)
  for (int k = 2; k <= ckp; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int t = tid; t < ckp; t += kThreads) {
        const int u = t ^ j;
        if (u > t) {
          const bool want_t_first = (t & k) == 0;
          const bool t_first = before(key[t], idx[t], key[u], idx[u]);
          if (want_t_first != t_first) {
            const double kt = key[t];
            key[t] = key[u];
            key[u] = kt;
            const int it = idx[t];
            idx[t] = idx[u];
            idx[u] = it;
          }
        }
      }
      __syncthreads();
    }

  // inclusive scan of sorted P over the valid prefix, then the cut
  const int per = (ckp + kThreads - 1) / kThreads;
  const int s0 = min(ckp, tid * per), s1 = min(ckp, s0 + per);
  double seg = 0.0;
  for (int e = s0; e < s1; ++e)
    if (e < n_valid) seg += key[e];
  // exclusive scan of segment sums (fixed order)
  double x = seg;
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  double run = x - seg;
  for (int w = 0; w < wave; ++w) run += red[w];
  int first = 0x7fffffff;
  for (int e = s0; e < s1 && e < n_valid; ++e) {
    run += key[e];
    if (first == 0x7fffffff && run >= top_p) first = e;
  }
  __syncthreads();
  const int hit = block_reduce_imin(first, ired);
  int m = n_valid;
  if (top_p < 1.0 && hit != 0x7fffffff) m = hit + 1;

  for (int j = tid; j < ck; j += kThreads) mk[j] = 0;
  __syncthreads();
  for (int e = tid; e < m; e += kThreads) mk[idx[e]] = 1;
  __syncthreads();
  // ascending compaction of the kept ids
  const int cper = (ck + kThreads - 1) / kThreads;
  const int c0 = min(ck, tid * cper), c1 = min(ck, c0 + cper);
  int cnt = 0;
  for (int j = c0; j < c1; ++j) cnt += mk[j];
  int xi = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(xi, o);
    if (lane >= o) xi += y;
  }
  if (lane == 63) ired[wave] = xi;
  __syncthreads();
  int pos = xi - cnt;
  for (int w = 0; w < wave; ++w) pos += ired[w];
  for (int j = c0; j < c1; ++j) {
    mrow[j] = mk[j];
    if (mk[j]) irow[pos++] = j;
  }
  for (int j = m + tid; j < ck; j += kThreads) irow[j] = -1;
  if (tid == 0) kept_count[static_cast<size_t>(bh) * cq + i] = m;
}

// DynamicRad's dynamic-threshold mode: one workgroup per (slice, query
// block), fp64 proxies S_j = (mu_q . mu_k_j) * scale computed exactly as in
// the top-p kernel; eligible pairs (non-empty key block, inside the candidate
// set) with S_j >= theta are kept; a non-empty query block left with none keeps
// its eligible argmax (ties: lower j).
template <int D>
__global__ __launch_bounds__(kThreads) void threshold_kernel(
    const float *__restrict__ cent_q, const int32_t *__restrict__ size_q,
    const float *__restrict__ cent_k, const int32_t *__restrict__ size_k, int nq, int nk,
    double scale, double theta, const uint8_t *__restrict__ cand, uint8_t *__restrict__ mask,
    int32_t *__restrict__ kept_count, int32_t *__restrict__ kept_idx) {
  __shared__ uint8_t mk[kCap];
  __shared__ double sq[D];
  __shared__ double red[kThreads / 64];
  __shared__ int ired[kThreads / 64];

  const int i = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  uint8_t *mrow = mask + (static_cast<size_t>(bh) * nq + i) * nk;
  int32_t *irow = kept_idx + (static_cast<size_t>(bh) * nq + i) * nk;
  const int32_t *szk = size_k + static_cast<size_t>(bh) * nk;
  if (size_q[static_cast<size_t>(bh) * nq + i] == 0) {
    for (int j = tid; j < nk; j += kThreads) {
      mrow[j] = 0;
      irow[j] = -1;
    }
    if (tid == 0) kept_count[static_cast<size_t>(bh) * nq + i] = 0;
    return;
  }
  if (tid < D) sq[tid] = static_cast<double>(cent_q[(static_cast<size_t>(bh) * nq + i) * D + tid]);
  __syncthreads();

  int lkept = 0;
  double best = -INFINITY;
  int best_j = 0x7fffffff;
  for (int j = tid; j < nk; j += kThreads) {
    const double s = centroid_dot<D>(sq, cent_k + (static_cast<size_t>(bh) * nk + j) * D) * scale;
    const bool elig = szk[j] > 0 && (cand == nullptr || cand[static_cast<size_t>(i) * nk + j] != 0);
    const bool keep = elig && s >= theta;
    mk[j] = keep ? 1 : 0;
    lkept += keep ? 1 : 0;
    if (elig && (best_j == 0x7fffffff || s > best || (s == best && j < best_j))) {
      best = s;
      best_j = j;
    }
  }
  int total = block_reduce_isum(lkept, ired);
  if (total == 0) {   // the safeguard: argmax over eligible pairs, lower id on ties
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const double ob = __shfl_xor(best, o);
      const int oj = __shfl_xor(best_j, o);
      if (oj != 0x7fffffff && (best_j == 0x7fffffff || ob > best || (ob == best && oj < best_j))) {
        best = ob;
        best_j = oj;
      }
    }
    if (lane == 0) {
      red[wave] = best;
      ired[wave] = best_j;
    }
    __syncthreads();
    double b = red[0];
    int bj = ired[0];
    for (int w = 1; w < kThreads / 64; ++w)
      if (ired[w] != 0x7fffffff && (bj == 0x7fffffff || red[w] > b || (red[w] == b && ired[w] < bj))) {
        b = red[w];
        bj = ired[w];
      }
    __syncthreads();
    if (bj != 0x7fffffff) {
      if (tid == 0) mk[bj] = 1;
      total = 1;
    }
  }
  __syncthreads();
  // ascending compaction of the kept ids
  const int cper = (nk + kThreads - 1) / kThreads;
  const int c0 = min(nk, tid * cper), c1 = min(nk, c0 + cper);
  int cnt = 0;
  for (int j = c0; j < c1; ++j) cnt += mk[j];
  int xi = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(xi, o);
    if (lane >= o) xi += y;
  }
  if (lane == 63) ired[wave] = xi;
  __syncthreads();
  int pos = xi - cnt;
  for (int w = 0; w < wave; ++w) pos += ired[w];
  for (int j = c0; j < c1; ++j) {
    mrow[j] = mk[j];
    if (mk[j]) irow[pos++] = j;
  }
  for (int j = total + tid; j < nk; j += kThreads) irow[j] = -1;
  if (tid == 0) kept_count[static_cast<size_t>(bh) * nq + i] = total;
}

}  // namespace

hipError_t launch_select_threshold(const ThresholdArgs &a, hipStream_t s) {
  const dim3 grid(a.nq, a.bh);
  if (a.d == 128)
    hipLaunchKernelGGL(threshold_kernel<128>, grid, dim3(kThreads), 0, s, a.cent_q, a.size_q,
                       a.cent_k, a.size_k, a.nq, a.nk, a.scale, a.theta, a.cand, a.mask,
                       a.kept_count, a.kept_idx);
  else
    hipLaunchKernelGGL(threshold_kernel<64>, grid, dim3(kThreads), 0, s, a.cent_q, a.size_q,
                       a.cent_k, a.size_k, a.nq, a.nk, a.scale, a.theta, a.cand, a.mask,
                       a.kept_count, a.kept_idx);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs &a, hipStream_t s) {
  int ckp = 1;
  while (ckp < a.ck) ckp <<= 1;
  const dim3 grid(a.cq, a.bh);
  const size_t lds = static_cast<size_t>(ckp) * (8 + 4) + align_up(static_cast<size_t>(a.ck), 16);
  if (a.d == 128)
    hipLaunchKernelGGL(select_kernel<128>, grid, dim3(kThreads), lds, s, a.cent_q, a.size_q,
                       a.cent_k, a.size_k, a.cq, a.ck, ckp, a.scale, a.top_p, a.mask, a.kept_count, a.kept_idx);
  else
    hipLaunchKernelGGL(select_kernel<64>, grid, dim3(kThreads), lds, s, a.cent_q, a.size_q,
                       a.cent_k, a.size_k, a.cq, a.ck, ckp, a.scale, a.top_p, a.mask, a.kept_count, a.kept_idx);
  return hipGetLastError();
}

}  // namespace sva
