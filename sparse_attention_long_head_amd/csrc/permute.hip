// Semantic-aware permutation for gfx950 (Sparse VideoGen2 explainer, technical
// summary section 2.a: tokens are reordered so that every cluster is one
// contiguous range).
//
// A stable counting sort of the rows of each (b,h) slice by cluster id, in
// three passes, followed by 16-byte-per-lane row gathers:
//   1. hist_rank: per tile of 2048 rows, every row's rank among the rows of the
//      same cluster earlier in the tile (wave ballots over the key bits give
//      the equal-key mask; the 4 waves of a step add to LDS counters in order)
//      and the tile's cluster histogram, stored cluster-major.
//   2. scan_rows: one wave per cluster: the exclusive scan of its row of tile
//      counts (the cluster's first permuted row of each tile, relative to the
//      cluster) and the cluster's size, in parallel over every (slice, cluster).
//   3. scan_totals: per slice, the exclusive scan of the cluster sizes gives the
//      cluster offsets (and the sizes when asked).
//   4. scatter: perm[offset(cluster) + base(cluster, tile) + rank] = row.
// Integer work only, so the result is exact and deterministic.
#include "../../include/sva.h"
#include "sva_internal.h"

namespace sva {
namespace {

constexpr int kThreads = 256;
constexpr int kTile = 2048;
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kThreads) void sort_hist_rank_kernel(
    const int32_t *__restrict__ assign, int n, int c, int tiles, int nbits,
    int32_t *__restrict__ hist, int32_t *__restrict__ rank) {
  extern __shared__ int32_t cnt[];
  const int tile = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < c; i += kThreads) cnt[i] = 0;
  __syncthreads();
  const int32_t *a = assign + static_cast<size_t>(bh) * n;
  int32_t *rk = rank + static_cast<size_t>(bh) * n;
  const int t0 = tile * kTile, t1 = min(n, t0 + kTile);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = t0; base < t1; base += kThreads) {
    const int i = base + tid;
    const bool valid = i < t1;
    // ids outside [0, c) are clamped, so no input can index outside the tables
    const int key = valid ? min(max(a[i], 0), c - 1) : 0;
    uint64_t eq = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = (key >> b) & 1;
      const uint64_t m = __ballot(bit);
      eq &= bit ? m : ~m;
    }
    const int r_in = __popcll(eq & lt);
    const int n_eq = __popcll(eq);
    for (int w = 0; w < kThreads / 64; ++w) {
      if (wave == w && valid) {
        rk[i] = cnt[key] + r_in;
        if (r_in == 0) cnt[key] += n_eq;   // one leader per key in this wave
      }
      __syncthreads();
    }
  }
  int32_t *hh = hist + static_cast<size_t>(bh) * c * tiles;
  for (int cl = tid; cl < c; cl += kThreads) hh[static_cast<size_t>(cl) * tiles + tile] = cnt[cl];
}

// one wave per (slice, cluster): row [cluster][0, tiles) of the histogram
// -> base (exclusive, relative to the cluster) and the row total, which goes
// to offsets[cluster] for scan_totals to turn into the cluster's offset
__global__ __launch_bounds__(kThreads) void sort_scan_rows_kernel(
    const int32_t *__restrict__ hist, int c, int tiles, int32_t *__restrict__ base,
    int32_t *__restrict__ offsets) {
  const int cl = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6), bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  if (cl >= c) return;   // wave-uniform
  const size_t row = (static_cast<size_t>(bh) * c + cl) * tiles;
  int carry = 0;
  for (int t0 = 0; t0 < tiles; t0 += 64) {
    const int t = t0 + lane;
    const int v = t < tiles ? hist[row + t] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (t < tiles) base[row + t] = carry + x - v;
    carry += __shfl(x, 63);
  }
  if (lane == 0) offsets[static_cast<size_t>(bh) * (c + 1) + cl] = carry;
}

// per slice: offsets[0, c) holds the cluster sizes; replaced in place by their
// exclusive scan (4 consecutive clusters per thread per round), offsets[c] = n
__global__ __launch_bounds__(kScanThreads) void sort_scan_totals_kernel(
    int n, int c, int32_t *__restrict__ offsets, int32_t *__restrict__ sizes,
    int32_t *__restrict__ clear) {
  __shared__ int32_t wsum[kScanThreads / 64];
  const int bh = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t *off = offsets + static_cast<size_t>(bh) * (c + 1);
  int32_t *sz = sizes != nullptr ? sizes + static_cast<size_t>(bh) * c : nullptr;
  int carry = 0;
  for (int r0 = 0; r0 < c; r0 += 4 * kScanThreads) {
    const int e0 = r0 + 4 * tid;
    int v[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[j] = e0 + j < c ? off[e0 + j] : 0;
      sum += v[j];
    }
    int x = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int run = carry + x - sum, tot = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) {
      run += w < wave ? wsum[w] : 0;
      tot += wsum[w];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (e0 + j < c) {
        if (sz != nullptr) sz[e0 + j] = v[j];
        off[e0 + j] = run;
        run += v[j];
      }
    carry += tot;
    __syncthreads();   // wsum is reused by the next round
  }
  if (tid == 0) {
    off[c] = n;
    if (clear != nullptr) clear[bh] = 0;   // a per-slice counter of the caller
  }
}

__global__ __launch_bounds__(kThreads) void sort_scatter_kernel(
    const int32_t *__restrict__ assign, const int32_t *__restrict__ rank,
    const int32_t *__restrict__ base, const int32_t *__restrict__ offsets, int n, int c,
    int tiles, int32_t *__restrict__ perm, int32_t *__restrict__ seg) {
  const int bh = blockIdx.y;
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i >= n) return;
  const size_t row = static_cast<size_t>(bh) * n + i;
  const int key = min(max(assign[row], 0), c - 1);   // as in hist_rank
  const int pos = offsets[static_cast<size_t>(bh) * (c + 1) + key] +
                  base[(static_cast<size_t>(bh) * c + key) * tiles + i / kTile] + rank[row];
  perm[static_cast<size_t>(bh) * n + pos] = i;
  if (seg != nullptr) seg[static_cast<size_t>(bh) * n + pos] = key;
}

// dst row r <- src row perm[r] (gather), or dst row perm[r] <- src row r
// (scatter), per slice; a row is 2^lcpr 16-byte pieces, one piece per thread
__global__ __launch_bounds__(kThreads) void move_rows_kernel(const u32x4 *__restrict__ src,
                                                             u32x4 *__restrict__ dst,
                                                             const int32_t *__restrict__ perm,
                                                             int n, int lcpr, int scatter) {
  const int bh = blockIdx.y;
  const int r = blockIdx.x * (kThreads >> lcpr) + (threadIdx.x >> lcpr);
  if (r >= n) return;
  const int part = threadIdx.x & ((1 << lcpr) - 1);
  const size_t slice = static_cast<size_t>(bh) * n;
  const size_t other = slice + perm[slice + r];
  const size_t self = slice + r;
  if (scatter) dst[(other << lcpr) + part] = src[(self << lcpr) + part];
  else dst[(self << lcpr) + part] = src[(other << lcpr) + part];
}

// whole slices of 16-byte pieces: packed slice i <-> slice idx[i]; one
// grid row per packed slice, grid-stride over its pieces
__global__ __launch_bounds__(kThreads) void move_slices_kernel(const u32x4 *__restrict__ src,
                                                               u32x4 *__restrict__ dst,
                                                               const int32_t *__restrict__ idx,
                                                               long long pieces, int scatter) {
  const long long i = blockIdx.y;
  const long long other = idx[i];
  const u32x4 *s = src + (scatter ? i : other) * pieces;
  u32x4 *d = dst + (scatter ? other : i) * pieces;
  for (long long p = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x; p < pieces;
       p += static_cast<long long>(gridDim.x) * kThreads)
    d[p] = s[p];
}

__global__ void fill_i32_kernel(int32_t *p, int32_t value, size_t count) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < count;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = value;
}

int bits_for(int c) {
  int b = 0;
  while ((1 << b) < c) ++b;
  return b;
}

}  // namespace

size_t sort_ws_bytes(int32_t bh, int32_t n, int32_t c) {
  const size_t tiles = (static_cast<size_t>(n) + kTile - 1) / kTile;
  const size_t hist = align_up(static_cast<size_t>(bh) * c * tiles * 4, 256);
  const size_t rank = align_up(static_cast<size_t>(bh) * n * 4, 256);
  return 2 * hist + rank;
}

hipError_t launch_cluster_sort(const int32_t *assign, int32_t bh, int32_t n, int32_t c,
                               int32_t *perm, int32_t *offsets, int32_t *sizes, void *ws,
                               hipStream_t s, int32_t *clear, int32_t *seg) {
  const int tiles = (n + kTile - 1) / kTile;
  const size_t hist_bytes = align_up(static_cast<size_t>(bh) * c * tiles * 4, 256);
  int32_t *hist = static_cast<int32_t *>(ws);
  int32_t *base = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + hist_bytes);
  int32_t *rank = reinterpret_cast<int32_t *>(static_cast<char *>(ws) + 2 * hist_bytes);
  hipLaunchKernelGGL(sort_hist_rank_kernel, dim3(tiles, bh), dim3(kThreads),
                     static_cast<size_t>(c) * 4, s, assign, n, c, tiles, bits_for(c), hist, rank);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sort_scan_rows_kernel, dim3((c + kThreads / 64 - 1) / (kThreads / 64), bh),
                     dim3(kThreads), 0, s, hist, c, tiles, base, offsets);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sort_scan_totals_kernel, dim3(bh), dim3(kScanThreads), 0, s, n, c, offsets,
                     sizes, clear);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(sort_scatter_kernel, dim3((n + kThreads - 1) / kThreads, bh),
                     dim3(kThreads), 0, s, assign, rank, base, offsets, n, c, tiles, perm, seg);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *src, void *dst, const int32_t *perm, int32_t bh,
                              int32_t n, int32_t row_bytes, int32_t scatter, hipStream_t s) {
  if (static_cast<long long>(bh) * n == 0) return hipSuccess;
  int lcpr = 0;
  while ((16 << lcpr) < row_bytes) ++lcpr;      // row_bytes is 16 * 2^lcpr
  const int rows_per_blk = kThreads >> lcpr;
  hipLaunchKernelGGL(move_rows_kernel, dim3((n + rows_per_blk - 1) / rows_per_blk, bh),
                     dim3(kThreads), 0, s, static_cast<const u32x4 *>(src),
                     static_cast<u32x4 *>(dst), perm, n, lcpr, scatter);
  return hipGetLastError();
}

hipError_t launch_move_slices(const void *src, void *dst, const int32_t *idx, int32_t n_idx,
                              long long slice_bytes, int32_t scatter, hipStream_t s) {
  if (n_idx == 0) return hipSuccess;
  const long long pieces = slice_bytes / 16;
  const long long want = (pieces + kThreads - 1) / kThreads;
  const int gx = static_cast<int>(want < 512 ? want : 512);
  hipLaunchKernelGGL(move_slices_kernel, dim3(gx, n_idx), dim3(kThreads), 0, s,
                     static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst), idx, pieces,
                     scatter);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int32_t value, size_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  size_t want = (count + 255) / 256;
  const int grid = static_cast<int>(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(fill_i32_kernel, dim3(grid), dim3(256), 0, s, p, value, count);
  return hipGetLastError();
}

}  // namespace sva
