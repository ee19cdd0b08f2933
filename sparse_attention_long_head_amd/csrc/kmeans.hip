// Lloyd k-means of Q and K per head for gfx950 (Sparse VideoGen2 explainer,
// technical summary section 2.a: Q and K are clustered independently before
// attention; section 2.c: the previous step's centroids seed the next step).
//
// One iteration = assign -> refine -> stable counting sort -> mean.
//
// assign (bf16 inputs): argmin_c ||x - c||^2 = argmax_c w_c with
//   w_c = x.c - ||c||^2 / 2.  The dot products run on 32x32x16 bf16 MFMA with
//   clusters on the accumulator rows and tokens on lanes; the accumulator
//   starts at -||c||^2/2, so no VALU op is spent on it.  x is exactly bf16 and
//   every fp32 centroid is split into bf16 hi + lo (residual <= 2^-16 |c|).
//   Each lane keeps the best and second-best w of its clusters (max + med3)
//   and the best index; the two lane halves merge.  Every w carries a rigorous
//   error bound E (split residual + fp32 accumulation of 2d exact products and
//   the start value + final rounding, from ||x|| and max ||c||).  A row whose
//   best two w are more than 2E apart is decided; any other row is queued
//   with the threshold best - 2E.
// refine: queued rows run through the same MFMA loop; every cluster with
//   w >= threshold (a set that provably holds the true argmin) goes to an LDS
//   candidate list; one wave per candidate computes the exact fp64 distance,
//   and the smallest distance wins, ties to the lowest index.  Assignments
//   therefore equal exact-arithmetic ones.
// assign (fp32 inputs): plain fp64 distances for every cluster.
// sort: the counting sort of permute.hip gives every cluster's rows in
//   ascending token order (and clears the per-slice counters for the next
//   iteration).
// mean: one workgroup per cluster sums its rows in that fixed order in fp64
//   and rounds the mean to fp32 once, so results are deterministic; an empty
//   cluster keeps its centroid.  The same kernel splits the new centroids
//   into hi/lo bf16 and computes -||c||^2/2 and max ||c|| for the next assign.
#include <math.h>

#include "../../include/sva.h"
#include "sva_internal.h"

namespace sva {
namespace {

constexpr int kThreads = 256;
constexpr int kNT = 3;                          // 32-token tiles per wave
constexpr int kTokTile = kNT * 32 * (kThreads / 64);   // tokens per workgroup (384)
constexpr int kCandCap = 3072;                  // refine candidates staged per batch

template <int D>
__device__ __forceinline__ int cswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

struct KmLayout {
  size_t chi, clo, nh, ctl, flags, perm, offsets, sort, total;
};

// ctl holds 2*bh ints: queue counters [0, bh) and max-norm bits [bh, 2bh)
KmLayout km_layout(int32_t bh, int32_t n, int32_t d, int32_t c) {
  const size_t cpad = (static_cast<size_t>(c) + 31) / 32 * 32;
  KmLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off += align_up(bytes, 256);
    return at;
  };
  L.chi = take(static_cast<size_t>(bh) * cpad * d * 2);
  L.clo = take(static_cast<size_t>(bh) * cpad * d * 2);
  L.nh = take(static_cast<size_t>(bh) * cpad * 4);
  L.ctl = take(static_cast<size_t>(bh) * 2 * 4);
  L.flags = take(static_cast<size_t>(bh) * n * 8);
  L.perm = take(static_cast<size_t>(bh) * n * 4);
  L.offsets = take(static_cast<size_t>(bh) * (c + 1) * 4);
  L.sort = take(sort_ws_bytes(bh, n, c));
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// MFMA assignment (REFINE = false) and fp64 refinement of queued rows (true)
// ---------------------------------------------------------------------------
template <int D, bool REFINE>
__global__ __launch_bounds__(kThreads, 2) void km_assign_mfma_kernel(
    const uint16_t *__restrict__ x, int n, int c, int cpad, const uint16_t *__restrict__ chi,
    const uint16_t *__restrict__ clo, const float *__restrict__ nh,
    const int32_t *__restrict__ ctl, const float *__restrict__ cent,
    int32_t *__restrict__ assign, int2 *__restrict__ flags, int32_t *__restrict__ qcount,
    int32_t *__restrict__ n_refined, int nbh, int tph) {
  constexpr int NS = D / 16;
  constexpr int KCH = D / 8;                 // 16-byte chunks per centroid row
  constexpr int CPT = KCH / 4;               // chunks per thread per tile load
  constexpr int CC = REFINE ? kCandCap : 1;
  constexpr int TS = REFINE ? kTokTile : 1;
  __shared__ __attribute__((aligned(16))) uint16_t sC[2][2][32 * D];
  __shared__ __attribute__((aligned(16))) float sN[2][32];
  __shared__ int32_t s_cand[CC];
  __shared__ double s_dist[CC];
  __shared__ unsigned long long s_bestd[TS];
  __shared__ int32_t s_bestc[TS];
  __shared__ int32_t s_tok[TS];
  __shared__ int32_t s_over[TS];
  __shared__ int32_t s_ncand;

  // Workgroups are dispatched round-robin over the 8 XCDs; slices are dealt
  // to XCDs the same way, so all tiles of a slice run on one XCD and its
  // centroids stay in that XCD's L2.  tph = token tiles per slice.
  const int xcd = blockIdx.x & 7, k8 = blockIdx.x >> 3;
  const int bh = xcd + 8 * (k8 / tph);
  const int tile = k8 % tph;
  if (bh >= nbh) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int ntl = cpad / 32;
  const uint16_t *xb = x + static_cast<size_t>(bh) * n * D;
  const int ntok = REFINE ? ctl[bh] : n;
  const float cm = __int_as_float(ctl[nbh + bh]);
  const int step = tph * kTokTile;

  // tile loader: thread -> (split, row, quarter of the row)
  const int ld_split = tid >> 7, ld_row = (tid >> 2) & 31, ld_part = tid & 3;
  const uint16_t *ld_src = (ld_split ? clo : chi) + (static_cast<size_t>(bh) * cpad + ld_row) * D;
  u32x4 creg[CPT];
  float nreg = 0.f;
  auto load_tile = [&](int ct) {
    const u32x4 *src = reinterpret_cast<const u32x4 *>(ld_src + static_cast<size_t>(ct) * 32 * D) +
                       ld_part * CPT;
#pragma unroll
    for (int i = 0; i < CPT; ++i) creg[i] = src[i];
    if (tid < 32) nreg = nh[static_cast<size_t>(bh) * cpad + ct * 32 + tid];
  };
  auto store_tile = [&](int buf) {
    uint16_t *dst = sC[buf][ld_split] + ld_row * D;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int ch = ld_part * CPT + i;
      *reinterpret_cast<u32x4 *>(dst + ((ch ^ cswz<D>(ld_row)) * 8)) = creg[i];
    }
    if (tid < 32) sN[buf][tid] = nreg;
  };

  // main pass: one tile of tokens per workgroup; refine: grid-stride over the queue
  for (int base = tile * kTokTile; base < ntok; base = REFINE ? base + step : ntok) {
    int tok[kNT];
    bool tv[kNT];
    float thr[kNT];
    bf16x8 xf[kNT][NS];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const int slot = wave * (kNT * 32) + nt * 32 + col;
      const int idx = base + slot;
      tv[nt] = idx < ntok;
      tok[nt] = idx;
      thr[nt] = 0.f;
      if (REFINE && tv[nt]) {
        const int2 e = flags[static_cast<size_t>(bh) * n + idx];
        tok[nt] = e.x;
        thr[nt] = __int_as_float(e.y);
      }
      const uint16_t *row = xb + static_cast<size_t>(tv[nt] ? tok[nt] : 0) * D + h * 8;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const u32x4 raw = tv[nt] ? *reinterpret_cast<const u32x4 *>(row + s * 16) : u32x4{0, 0, 0, 0};
        xf[nt][s] = __builtin_bit_cast(bf16x8, raw);
      }
      if constexpr (REFINE) {
        if (h == 0) {
          s_tok[slot] = tv[nt] ? tok[nt] : -1;
          s_over[slot] = 0;
          s_bestd[slot] = ~0ull;
          s_bestc[slot] = 0x7fffffff;
        }
      }
    }
    if constexpr (REFINE) {
      if (tid == 0) s_ncand = 0;
    }
    // error bound of w per token: 2E (main pass)
    float two_e[kNT];
    if constexpr (!REFINE) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        float p = 0.f;
#pragma unroll
        for (int s = 0; s < NS; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float f = static_cast<float>(xf[nt][s][j]);
            p = fmaf(f, f, p);
          }
        p += __shfl_xor(p, 32);
        const float nx = sqrtf(p) * (1.f + 0x1p-10f);
        const float e = 0x1p-25f * cm * cm + 0x1p-16f * nx * cm +
                        (2.f * D) * 0x1p-23f * (0.5f * cm * cm + 1.02f * nx * cm);
        two_e[nt] = 2.f * 1.25f * e;
      }
    }

    float b1[kNT], b2[kNT];
    int i1[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      b1[nt] = -INFINITY;
      b2[nt] = -INFINITY;
      i1[nt] = 0;
    }

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int ct = 0; ct < ntl; ++ct) {
      const int buf = ct & 1;
      if (ct + 1 < ntl) load_tile(ct + 1);
      f32x16 cinit;   // -||c||^2/2 of the lane's 16 cluster rows
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 q4 = *reinterpret_cast<const f32x4 *>(&sN[buf][8 * g + 4 * h]);
#pragma unroll
        for (int j = 0; j < 4; ++j) cinit[4 * g + j] = q4[j];
      }
      f32x16 acc[kNT];
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
              sC[buf][sp] + col * D + (((2 * s + h) ^ cswz<D>(col)) * 8));
#pragma unroll
          for (int nt = 0; nt < kNT; ++nt)
            acc[nt] = mfma32x32x16(a, xf[nt][s], (sp == 0 && s == 0) ? cinit : acc[nt]);
        }
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int cl = ct * 32 + acc_row(i, h);
          const float w = acc[nt][i];
          if constexpr (!REFINE) {
            const bool gt = w > b1[nt];
            b2[nt] = __builtin_amdgcn_fmed3f(b1[nt], b2[nt], w);
            b1[nt] = fmaxf(b1[nt], w);
            i1[nt] = gt ? cl : i1[nt];
          } else {
            if (tv[nt] && cl < c && w >= thr[nt]) {
              const int slot = wave * (kNT * 32) + nt * 32 + col;
              const int k = atomicAdd(&s_ncand, 1);
              if (k < kCandCap) s_cand[k] = (slot << 14) | cl;
              else s_over[slot] = 1;
            }
          }
        }
      if (ct + 1 < ntl) store_tile(buf ^ 1);
      __syncthreads();
    }

    if constexpr (!REFINE) {
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const float ob1 = __shfl_xor(b1[nt], 32), ob2 = __shfl_xor(b2[nt], 32);
        const int oi1 = __shfl_xor(i1[nt], 32);
        const bool other = ob1 > b1[nt] || (ob1 == b1[nt] && oi1 < i1[nt]);
        const float nb1 = fmaxf(b1[nt], ob1);
        const int ni1 = other ? oi1 : i1[nt];
        const float nb2 = fmaxf(fminf(b1[nt], ob1), fmaxf(b2[nt], ob2));
        if (h == 0 && tv[nt]) {
          if (nb1 - nb2 > two_e[nt]) {
            assign[static_cast<size_t>(bh) * n + tok[nt]] = ni1;
          } else {
            const int q = atomicAdd(&qcount[bh], 1);
            flags[static_cast<size_t>(bh) * n + q] = int2{tok[nt], __float_as_int(nb1 - two_e[nt])};
          }
        }
      }
    } else {
      // exact fp64 distance of every candidate, one lane per candidate (rows read
      // as 16-byte pieces, summed in ascending dimension order)
      const int ncand = min(s_ncand, kCandCap);
      for (int j = tid; j < ncand; j += kThreads) {
        const int e = s_cand[j];
        const int slot = e >> 14, cl = e & 0x3fff;
        const u32x4 *xr = reinterpret_cast<const u32x4 *>(xb + static_cast<size_t>(s_tok[slot]) * D);
        const f32x4 *cr = reinterpret_cast<const f32x4 *>(cent + (static_cast<size_t>(bh) * c + cl) * D);
        double dist = 0.0;
#pragma unroll 4
        for (int q = 0; q < D / 8; ++q) {
          const u32x4 xv = xr[q];
          const f32x4 c0 = cr[2 * q], c1 = cr[2 * q + 1];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float xf32 = bf16_bits_to_f32(static_cast<uint16_t>(xv[t >> 1] >> (16 * (t & 1))));
            const float cf32 = t < 4 ? c0[t] : c1[t - 4];
            const double df = static_cast<double>(xf32) - static_cast<double>(cf32);
            dist = fma(df, df, dist);
          }
        }
        s_dist[j] = dist;
        atomicMin(&s_bestd[slot], static_cast<unsigned long long>(__double_as_longlong(dist)));
      }
      __syncthreads();
      for (int j = tid; j < ncand; j += kThreads) {
        const int e = s_cand[j];
        const int slot = e >> 14;
        if (static_cast<unsigned long long>(__double_as_longlong(s_dist[j])) == s_bestd[slot])
          atomicMin(&s_bestc[slot], e & 0x3fff);
      }
      __syncthreads();
      int done = 0;
      for (int slot = tid; slot < kTokTile; slot += kThreads) {
        const int t = s_tok[slot];
        if (t < 0) continue;
        int best = s_bestc[slot];
        if (s_over[slot] || best == 0x7fffffff) {
          // candidate list overflowed: exact scan over every cluster
          const uint16_t *xr = xb + static_cast<size_t>(t) * D;
          double bd = INFINITY;
          best = 0;
          for (int cl = 0; cl < c; ++cl) {
            const float *cr = cent + (static_cast<size_t>(bh) * c + cl) * D;
            double dist = 0.0;
            for (int d = 0; d < D; ++d) {
              const double df = static_cast<double>(bf16_bits_to_f32(xr[d])) - static_cast<double>(cr[d]);
              dist = fma(df, df, dist);
            }
            if (dist < bd) {
              bd = dist;
              best = cl;
            }
          }
        }
        assign[static_cast<size_t>(bh) * n + t] = best;
        ++done;
      }
      if (n_refined != nullptr && done > 0) atomicAdd(n_refined, done);
      __syncthreads();
    }
  }
}

// ---------------------------------------------------------------------------
// fp64 assignment (fp32 inputs): exact distances to every cluster
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void km_assign_f64_kernel(const float *__restrict__ x,
                                                                 int n, int c,
                                                                 const float *__restrict__ cent,
                                                                 int32_t *__restrict__ assign) {
  __shared__ float sc[32 * D];
  const int bh = blockIdx.y, tid = threadIdx.x;
  const int i = blockIdx.x * kThreads + tid;
  const bool valid = i < n;
  float xr[D];
  const float *row = x + (static_cast<size_t>(bh) * n + (valid ? i : 0)) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) xr[d] = row[d];
  double best = INFINITY;
  int bi = 0;
  for (int c0 = 0; c0 < c; c0 += 32) {
    const int m = min(32, c - c0);
    __syncthreads();
    for (int e = tid; e < m * D; e += kThreads)
      sc[e] = cent[(static_cast<size_t>(bh) * c + c0) * D + e];
    __syncthreads();
    for (int j = 0; j < m; ++j) {
      double s = 0.0;
#pragma unroll
      for (int d = 0; d < D; ++d) {
        const double df = static_cast<double>(xr[d]) - static_cast<double>(sc[j * D + d]);
        s = fma(df, df, s);
      }
      if (s < best) {
        best = s;
        bi = c0 + j;
      }
    }
  }
  if (valid) assign[static_cast<size_t>(bh) * n + i] = bi;
}

// ---------------------------------------------------------------------------
// mean of every cluster in fixed (ascending token) order + next-assign prep
//   mode 0: prep only (initial centroids); 1: mean + prep; 2: mean only
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void km_mean_kernel(
    const void *__restrict__ x, int n, int c, int cpad, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, float *__restrict__ cent, uint16_t *__restrict__ chi,
    uint16_t *__restrict__ clo, float *__restrict__ nh, int32_t *__restrict__ cmax, int mode) {
  constexpr int EB = BF16 ? 2 : 4;           // element bytes
  constexpr int EPT = 16 / EB;               // elements per 16-byte piece
  constexpr int TPR = D / EPT;               // threads per row
  constexpr int RG = kThreads / TPR;         // row groups
  constexpr int U = 8;                       // rows in flight per thread
  __shared__ double part[RG * D];
  __shared__ double red[kThreads / 64];
  const int cl = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const bool real = cl < c;
  float val = 0.f;   // this thread's coordinate (tid < D) of the final centroid
  if (real && tid < D) val = cent[(static_cast<size_t>(bh) * c + cl) * D + tid];
  if (mode != 0 && real) {
    const int st = offsets[static_cast<size_t>(bh) * (c + 1) + cl];
    const int en = offsets[static_cast<size_t>(bh) * (c + 1) + cl + 1];
    const int rg = tid / TPR, pc = tid % TPR;
    double acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.0;
    const int32_t *pm = perm + static_cast<size_t>(bh) * n;
    const char *xb = static_cast<const char *>(x) + static_cast<size_t>(bh) * n * D * EB;
    for (int r0 = st + rg; r0 < en; r0 += U * RG) {
      int pr[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int r = r0 + u * RG;
        pr[u] = r < en ? pm[r] : -1;
      }
      u32x4 buf[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        buf[u] = pr[u] >= 0 ? *reinterpret_cast<const u32x4 *>(
                                  xb + (static_cast<size_t>(pr[u]) * D + pc * EPT) * EB)
                            : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (pr[u] < 0) break;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          float f;
          if constexpr (BF16) f = bf16_bits_to_f32(static_cast<uint16_t>(buf[u][e >> 1] >> (16 * (e & 1))));
          else f = __uint_as_float(buf[u][e]);
          acc[e] += static_cast<double>(f);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < EPT; ++e) part[rg * D + pc * EPT + e] = acc[e];
    __syncthreads();
    if (tid < D && en > st) {
      double s = 0.0;
      for (int g = 0; g < RG; ++g) s += part[g * D + tid];
      val = static_cast<float>(s / static_cast<double>(en - st));
      cent[(static_cast<size_t>(bh) * c + cl) * D + tid] = val;
    }
  }
  if (mode == 2) return;
  // prep for the next assignment: hi/lo split, -||c||^2/2, max ||c||
  double sq = 0.0;
  if (tid < D) {
    const __bf16 hi = static_cast<__bf16>(val);
    const __bf16 lo = static_cast<__bf16>(val - static_cast<float>(hi));
    const size_t o = (static_cast<size_t>(bh) * cpad + cl) * D + tid;
    chi[o] = __builtin_bit_cast(uint16_t, hi);
    clo[o] = __builtin_bit_cast(uint16_t, lo);
    sq = static_cast<double>(val) * static_cast<double>(val);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
  if ((tid & 63) == 0) red[tid >> 6] = sq;
  __syncthreads();
  if (tid == 0) {
    double ss = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) ss += red[w];
    nh[static_cast<size_t>(bh) * cpad + cl] = real ? static_cast<float>(-0.5 * ss) : -INFINITY;
    if (real)
      atomicMax(&cmax[bh], __float_as_int(static_cast<float>(sqrt(ss)) * (1.f + 0x1p-20f)));
  }
}

template <int D>
hipError_t run_kmeans(const KmeansArgs &a, hipStream_t s) {
  const KmLayout L = km_layout(a.bh, a.n, a.d, a.c);
  char *w = static_cast<char *>(a.ws);
  uint16_t *chi = reinterpret_cast<uint16_t *>(w + L.chi);
  uint16_t *clo = reinterpret_cast<uint16_t *>(w + L.clo);
  float *nh = reinterpret_cast<float *>(w + L.nh);
  int32_t *ctl = reinterpret_cast<int32_t *>(w + L.ctl);   // [bh] queue counts, [bh] max norms
  int2 *flags = reinterpret_cast<int2 *>(w + L.flags);
  int32_t *perm = reinterpret_cast<int32_t *>(w + L.perm);
  int32_t *offsets = reinterpret_cast<int32_t *>(w + L.offsets);
  void *sort_ws = w + L.sort;
  const int cpad = (a.c + 31) / 32 * 32;
  const bool bf16 = a.dtype == SVA_BF16;
  const int tph = (a.n + kTokTile - 1) / kTokTile;
  const dim3 tok_grid(8 * tph * ((a.bh + 7) / 8));
  hipError_t e;
#define SVA_CHECK(x)               \
  do {                             \
    e = (x);                       \
    if (e != hipSuccess) return e; \
  } while (0)

  auto mean = [&](int mode) -> hipError_t {
    const dim3 grid(mode == 2 ? a.c : cpad, a.bh);
    if (bf16)
      hipLaunchKernelGGL((km_mean_kernel<D, true>), grid, dim3(kThreads), 0, s, a.x, a.n, a.c,
                         cpad, perm, offsets, a.centroids, chi, clo, nh, ctl + a.bh, mode);
    else
      hipLaunchKernelGGL((km_mean_kernel<D, false>), grid, dim3(kThreads), 0, s, a.x, a.n, a.c,
                         cpad, perm, offsets, a.centroids, chi, clo, nh, ctl + a.bh, mode);
    return hipGetLastError();
  };

  if (bf16) {
    SVA_CHECK(launch_fill_i32(ctl, 0, 2 * static_cast<size_t>(a.bh), s));
    SVA_CHECK(mean(0));
  }
  for (int it = 0; it < a.iters; ++it) {
    const bool last = it + 1 == a.iters;
    if (bf16) {
      hipLaunchKernelGGL((km_assign_mfma_kernel<D, false>), tok_grid, dim3(kThreads), 0, s,
                         static_cast<const uint16_t *>(a.x), a.n, a.c, cpad, chi, clo, nh, ctl,
                         a.centroids, a.assign, flags, ctl, a.n_refined, a.bh, tph);
      SVA_CHECK(hipGetLastError());
      hipLaunchKernelGGL((km_assign_mfma_kernel<D, true>), tok_grid, dim3(kThreads), 0, s,
                         static_cast<const uint16_t *>(a.x), a.n, a.c, cpad, chi, clo, nh, ctl,
                         a.centroids, a.assign, flags, ctl, a.n_refined, a.bh, tph);
      SVA_CHECK(hipGetLastError());
    } else {
      hipLaunchKernelGGL((km_assign_f64_kernel<D>), dim3((a.n + kThreads - 1) / kThreads, a.bh),
                         dim3(kThreads), 0, s, static_cast<const float *>(a.x), a.n, a.c,
                         a.centroids, a.assign);
      SVA_CHECK(hipGetLastError());
    }
    // the sort's scan clears both per-slice counters for the next iteration
    SVA_CHECK(launch_cluster_sort(a.assign, a.bh, a.n, a.c, perm, offsets,
                                  last ? a.sizes : nullptr, sort_ws, s, bf16 ? ctl : nullptr));
    SVA_CHECK(mean((bf16 && !last) ? 1 : 2));
  }
#undef SVA_CHECK
  return hipSuccess;
}

}  // namespace

size_t kmeans_ws_bytes(int32_t bh, int32_t n, int32_t d, int32_t c) {
  return km_layout(bh, n, d, c).total;
}

hipError_t launch_kmeans(const KmeansArgs &a, hipStream_t s) {
  return a.d == 128 ? run_kmeans<128>(a, s) : run_kmeans<64>(a, s);
}

}  // namespace sva
