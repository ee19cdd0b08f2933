// Lloyd k-means of Q and K per head for gfx950 (Sparse VideoGen2 explainer,
// technical summary section 2.a: Q and K are clustered independently before
// attention; section 2.c: the previous step's centroids seed the next step).
//
// One iteration = assign -> refine -> stable counting sort -> mean.
//
// assign (bf16 inputs): argmin_c ||x - c||^2 = argmin_c (||c||^2 - 2 x.c).  The
//   dot products run on 32x32x16 bf16 MFMA with clusters on the accumulator
//   rows and tokens on lanes: x is exactly bf16, and each fp32 centroid is
//   split into bf16 hi + lo (residual <= 2^-16 |c|).  Every lane keeps the
//   best and second-best value of its clusters; the two lane halves merge.
//   The value of every cluster carries a rigorous error bound E (split
//   residual + fp32 accumulation of 2d exact products + final roundings, from
//   ||x|| and max ||c||).  A row whose best two values are more than 2E apart
//   is decided; any other row is queued with the threshold best + 2E.
// refine: the queued rows run through the same MFMA loop again, and every
//   cluster whose value is within the threshold (a set that provably holds
//   the true argmin) gets its exact fp64 distance; the smallest wins, ties to
//   the lowest index.  Assignments therefore equal exact-arithmetic ones.
// assign (fp32 inputs): plain fp64 distances for every cluster.
// sort: the counting sort of permute.hip gives every cluster's rows in
//   ascending token order.
// mean: one workgroup per cluster sums its rows in that fixed order in fp64
//   and rounds the mean to fp32 once, so results are deterministic; an empty
//   cluster keeps its centroid.  The same kernel splits the new centroids
//   into hi/lo bf16 and computes ||c||^2 and max ||c|| for the next assign.
#include <math.h>

#include "../../include/sva.h"
#include "sva_internal.h"

namespace sva {
namespace {

constexpr int kThreads = 256;
constexpr int kTokTile = 256;   // tokens per assign workgroup (4 waves x 64)

template <int D>
__device__ __forceinline__ int cswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

struct KmLayout {
  size_t chi, clo, cn2, cmax, flags, flag_cnt, perm, offsets, sort, total;
};

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
  L.cn2 = take(static_cast<size_t>(bh) * cpad * 4);
  L.cmax = take(static_cast<size_t>(bh) * 4);
  L.flags = take(static_cast<size_t>(bh) * n * 8);
  L.flag_cnt = take(static_cast<size_t>(bh) * 4);
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
    const uint16_t *__restrict__ clo, const float *__restrict__ cn2,
    const uint32_t *__restrict__ cmax, const float *__restrict__ cent,
    int32_t *__restrict__ assign, int2 *__restrict__ flags, int32_t *__restrict__ flag_cnt,
    int32_t *__restrict__ n_refined) {
  constexpr int NS = D / 16;
  constexpr int NT = 2;                      // 32-token tiles per wave
  constexpr int KCH = D / 8;                 // 16-byte chunks per centroid row
  constexpr int CPT = KCH / 4;               // chunks per thread per tile load
  __shared__ __attribute__((aligned(16))) uint16_t sC[2][2][32 * D];
  __shared__ __attribute__((aligned(16))) float sN[2][32];

  const int bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int ntl = cpad / 32;
  const uint16_t *xb = x + static_cast<size_t>(bh) * n * D;
  const int ntok = REFINE ? flag_cnt[bh] : n;
  // main pass: one tile per workgroup; refine: grid-stride over the queue
  const int step = gridDim.x * kTokTile;
  const float cm = __uint_as_float(cmax[bh]);

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
    if (tid < 32) nreg = cn2[static_cast<size_t>(bh) * cpad + ct * 32 + tid];
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

  for (int base = blockIdx.x * kTokTile; base < ntok; base = REFINE ? base + step : ntok) {
    int tok[NT];
    bool tv[NT];
    float thr[NT];
    bf16x8 xf[NT][NS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int idx = base + wave * 64 + nt * 32 + col;
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
    }
    // error bound per token (main pass only)
    float two_e[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
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
      const float e = (4.f * D * 0x1p-23f * 1.02f + 2.f * 0x1p-16f) * nx * cm +
                      0x1p-22f * (cm * cm + 2.f * nx * cm);
      two_e[nt] = 2.f * 1.25f * e;
    }

    float b1[NT], b2[NT];
    int i1[NT];
    double bd[NT];
    int bi[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      b1[nt] = INFINITY;
      b2[nt] = INFINITY;
      i1[nt] = 0;
      bd[nt] = INFINITY;
      bi[nt] = 0;
    }

    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int ct = 0; ct < ntl; ++ct) {
      const int buf = ct & 1;
      if (ct + 1 < ntl) load_tile(ct + 1);
      f32x16 acc[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[nt][i] = 0.f;
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
              sC[buf][sp] + col * D + (((2 * s + h) ^ cswz<D>(col)) * 8));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[nt] = mfma32x32x16(a, xf[nt][s], acc[nt]);
        }
      float cn[16];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 q4 = *reinterpret_cast<const f32x4 *>(&sN[buf][8 * g + 4 * h]);
        cn[4 * g + 0] = q4[0];
        cn[4 * g + 1] = q4[1];
        cn[4 * g + 2] = q4[2];
        cn[4 * g + 3] = q4[3];
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int cl = ct * 32 + acc_row(i, h);
          const float val = fmaf(-2.f, acc[nt][i], cn[i]);
          if constexpr (!REFINE) {
            if (val < b1[nt]) {
              b2[nt] = b1[nt];
              b1[nt] = val;
              i1[nt] = cl;
            } else {
              b2[nt] = fminf(b2[nt], val);
            }
          } else {
            if (tv[nt] && cl < c && val <= thr[nt]) {
              const uint16_t *xr = xb + static_cast<size_t>(tok[nt]) * D;
              const float *cr = cent + (static_cast<size_t>(bh) * c + cl) * D;
              double dist = 0.0;
              for (int d = 0; d < D; ++d) {
                const double df = static_cast<double>(bf16_bits_to_f32(xr[d])) -
                                  static_cast<double>(cr[d]);
                dist = fma(df, df, dist);
              }
              if (dist < bd[nt] || (dist == bd[nt] && cl < bi[nt])) {
                bd[nt] = dist;
                bi[nt] = cl;
              }
            }
          }
        }
      if (ct + 1 < ntl) store_tile(buf ^ 1);
      __syncthreads();
    }

#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      if constexpr (!REFINE) {
        const float ob1 = __shfl_xor(b1[nt], 32), ob2 = __shfl_xor(b2[nt], 32);
        const int oi1 = __shfl_xor(i1[nt], 32);
        const bool other = ob1 < b1[nt] || (ob1 == b1[nt] && oi1 < i1[nt]);
        const float nb1 = fminf(b1[nt], ob1);
        const int ni1 = other ? oi1 : i1[nt];
        const float nb2 = fminf(fmaxf(b1[nt], ob1), fminf(b2[nt], ob2));
        if (h == 0 && tv[nt]) {
          if (nb2 - nb1 > two_e[nt]) {
            assign[static_cast<size_t>(bh) * n + tok[nt]] = ni1;
          } else {
            const int slot = atomicAdd(&flag_cnt[bh], 1);
            flags[static_cast<size_t>(bh) * n + slot] =
                int2{tok[nt], __float_as_int(nb1 + two_e[nt])};
          }
        }
      } else {
        const double od = __shfl_xor(bd[nt], 32);
        const int oi = __shfl_xor(bi[nt], 32);
        if (od < bd[nt] || (od == bd[nt] && oi < bi[nt])) {
          bd[nt] = od;
          bi[nt] = oi;
        }
        if (h == 0 && tv[nt]) {
          assign[static_cast<size_t>(bh) * n + tok[nt]] = bi[nt];
          if (n_refined != nullptr) atomicAdd(n_refined, 1);
        }
      }
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
    uint16_t *__restrict__ clo, float *__restrict__ cn2, uint32_t *__restrict__ cmax, int mode) {
  constexpr int EB = BF16 ? 2 : 4;           // element bytes
  constexpr int EPT = 16 / EB;               // elements per 16-byte piece
  constexpr int TPR = D / EPT;               // threads per row
  constexpr int RG = kThreads / TPR;         // rows in flight per pass
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
    for (int r0 = st + rg; r0 < en; r0 += 4 * RG) {
      u32x4 buf[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int r = r0 + u * RG;
        buf[u] = r < en ? *reinterpret_cast<const u32x4 *>(
                              xb + (static_cast<size_t>(pm[r]) * D + pc * EPT) * EB)
                        : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (r0 + u * RG >= en) break;
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
  // prep for the next assignment: hi/lo split, ||c||^2, max ||c||
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
    cn2[static_cast<size_t>(bh) * cpad + cl] = real ? static_cast<float>(ss) : INFINITY;
    if (real)
      atomicMax(&cmax[bh], __float_as_uint(static_cast<float>(sqrt(ss)) * (1.f + 0x1p-20f)));
  }
}

template <int D>
hipError_t run_kmeans(const KmeansArgs &a, hipStream_t s) {
  const KmLayout L = km_layout(a.bh, a.n, a.d, a.c);
  char *w = static_cast<char *>(a.ws);
  uint16_t *chi = reinterpret_cast<uint16_t *>(w + L.chi);
  uint16_t *clo = reinterpret_cast<uint16_t *>(w + L.clo);
  float *cn2 = reinterpret_cast<float *>(w + L.cn2);
  uint32_t *cmax = reinterpret_cast<uint32_t *>(w + L.cmax);
  int2 *flags = reinterpret_cast<int2 *>(w + L.flags);
  int32_t *flag_cnt = reinterpret_cast<int32_t *>(w + L.flag_cnt);
  int32_t *perm = reinterpret_cast<int32_t *>(w + L.perm);
  int32_t *offsets = reinterpret_cast<int32_t *>(w + L.offsets);
  void *sort_ws = w + L.sort;
  const int cpad = (a.c + 31) / 32 * 32;
  const bool bf16 = a.dtype == SVA_BF16;
  const dim3 tok_grid((a.n + kTokTile - 1) / kTokTile, a.bh);
  const int rg = a.n / 4096 < 1 ? 1 : (a.n / 4096 > 64 ? 64 : a.n / 4096);
  hipError_t e;
#define SVA_CHECK(x)            \
  do {                          \
    e = (x);                    \
    if (e != hipSuccess) return e; \
  } while (0)
#define SVA_LAUNCHED() SVA_CHECK(hipGetLastError())

  auto mean = [&](int mode) -> hipError_t {
    if (bf16)
      hipLaunchKernelGGL((km_mean_kernel<D, true>), dim3(mode == 2 ? a.c : cpad, a.bh),
                         dim3(kThreads), 0, s, a.x, a.n, a.c, cpad, perm, offsets, a.centroids,
                         chi, clo, cn2, cmax, mode);
    else
      hipLaunchKernelGGL((km_mean_kernel<D, false>), dim3(mode == 2 ? a.c : cpad, a.bh),
                         dim3(kThreads), 0, s, a.x, a.n, a.c, cpad, perm, offsets, a.centroids,
                         chi, clo, cn2, cmax, mode);
    return hipGetLastError();
  };

  if (bf16) {
    SVA_CHECK(launch_fill_i32(reinterpret_cast<int32_t *>(cmax), 0, a.bh, s));
    SVA_CHECK(mean(0));
  }
  for (int it = 0; it < a.iters; ++it) {
    const bool last = it + 1 == a.iters;
    if (bf16) {
      SVA_CHECK(launch_fill_i32(flag_cnt, 0, a.bh, s));
      hipLaunchKernelGGL((km_assign_mfma_kernel<D, false>), tok_grid, dim3(kThreads), 0, s,
                         static_cast<const uint16_t *>(a.x), a.n, a.c, cpad, chi, clo, cn2, cmax,
                         a.centroids, a.assign, flags, flag_cnt, a.n_refined);
      SVA_LAUNCHED();
      hipLaunchKernelGGL((km_assign_mfma_kernel<D, true>), dim3(rg, a.bh), dim3(kThreads), 0, s,
                         static_cast<const uint16_t *>(a.x), a.n, a.c, cpad, chi, clo, cn2, cmax,
                         a.centroids, a.assign, flags, flag_cnt, a.n_refined);
      SVA_LAUNCHED();
    } else {
      hipLaunchKernelGGL((km_assign_f64_kernel<D>), tok_grid, dim3(kThreads), 0, s,
                         static_cast<const float *>(a.x), a.n, a.c, a.centroids, a.assign);
      SVA_LAUNCHED();
    }
    SVA_CHECK(launch_cluster_sort(a.assign, a.bh, a.n, a.c, perm, offsets, last ? a.sizes : nullptr,
                                  sort_ws, s));
    if (bf16 && !last) SVA_CHECK(launch_fill_i32(reinterpret_cast<int32_t *>(cmax), 0, a.bh, s));
    SVA_CHECK(mean((bf16 && !last) ? 1 : 2));
  }
#undef SVA_LAUNCHED
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
