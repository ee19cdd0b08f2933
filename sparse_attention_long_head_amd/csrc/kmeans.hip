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
//   every fp32 centroid is split into bf16 hi + lo: hi and lo are
//   round-to-nearest conversions and c - hi is exact in fp32, so each element's
//   residual is at most 2^-18 of it.
//   Each lane keeps the three best w of its clusters (max + two med3) and the
//   tiles of the best two; the two lane halves merge.  Every w carries a rigorous
//   error bound E (split residual + fp32 accumulation of 2d exact products and
//   the start value + final rounding, from ||x|| and max ||c||).  Each
//   addition inside and between the MFMAs is taken to lose at most one unit
//   in the last place of fp32 (2^-23 of its operands' magnitude) in any
//   order: the seed's addition rounds to nearest even, but the additions
//   among an MFMA's products do not (-2^25 + 2^25 + 3 gives 2), so no
//   round-to-nearest half-unit is assumed.  sva_check_mfma_rounding checks
//   this model on the device.  A row whose
//   best two w are more than 2E apart is decided.  A row whose third-best w
//   is more than 2E below its best has exactly two candidates (no other
//   cluster can be the argmin): it goes to the pair list of its token tile
//   and is settled by two fp64 distances.  Any other row is queued with the
//   threshold best - 2E (each token tile writes its queued rows to the front
//   of a region of its own and its pairs to the back; a join kernel
//   concatenates the queue parts in tile order, so there are no atomics and
//   the queue order is deterministic).
// pair: d/8 lanes per listed row compute the exact fp64 distances to its two
//   candidates; the smaller wins, ties to the lower index.
// refine: queued rows run through the same MFMA loop; every cluster with
//   w >= threshold (a set that provably holds the true argmin) goes to an LDS
//   candidate list; one wave per candidate computes the exact fp64 distance,
//   and the smallest distance wins, ties to the lowest index.  Assignments
//   therefore equal exact-arithmetic ones.
// assign (fp32 inputs): plain fp64 distances for every cluster.
// sort: the counting sort of permute.hip gives every cluster's rows in
//   ascending token order (and clears the per-slice queue lengths for the next
//   iteration).
// mean: one wave (small clusters) or four (large ones) per cluster sum its
//   rows in that fixed order in fp64 and round the mean to fp32 once, so
//   results are deterministic; an empty cluster keeps its centroid.  The same kernel splits the new centroids
//   into hi/lo bf16 and computes -||c||^2/2 for the next assign (whose
//   workgroups take max ||c|| of their slice from it).
#include <float.h>
#include <math.h>

#include <type_traits>

#include "../../include/sva.h"
#include "sva_internal.h"
#include "lds_pipe.h"

namespace sva {
namespace {

constexpr int kThreads = 256;
constexpr int kNT = 3;                          // 32-token tiles per wave
constexpr int kTokTile = kNT * 32 * (kThreads / 64);   // tokens per workgroup (384)
constexpr int kCandCap = 3072;                  // refine candidates staged per batch
constexpr int kResTok = 64;                     // tokens per tile of the resident pass
constexpr int kResWaves = 8;                    // waves per workgroup of the resident pass
constexpr int kResTiles = 4;                    // centroid tiles (of 32) it holds per slice

// p + the sum of squares of 8 bf16 values: each square is exact in fp32, each
// addition rounds once (the values are widened by moving their bits, so the
// arithmetic is explicit: plain fp32 multiply-adds)
__device__ __forceinline__ float bf16x8_sumsq(bf16x8 v, float p) {
  const u32x4 u = __builtin_bit_cast(u32x4, v);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float lo = __uint_as_float(u[j] << 16), hi = __uint_as_float(u[j] & 0xffff0000u);
    p = fmaf(lo, lo, p);
    p = fmaf(hi, hi, p);
  }
  return p;
}

template <int D>
__device__ __forceinline__ int cswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

constexpr int kCandWaves = 4;                   // waves per workgroup of the candidate pass
constexpr int kCandTok = 32 * kCandWaves;       // sorted positions per workgroup (128)
constexpr int kNbrMaxC = 4096;                  // largest C of the candidate path

struct KmLayout {
  size_t chi, clo, nh, ctl, flags, tflags, tcount, pcount, perm, seg, offsets, rad, nbr, tun,
      sort, total;
};

// ctl holds the bh refine-queue lengths
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
  L.ctl = take(static_cast<size_t>(bh) * 4);
  L.flags = take(static_cast<size_t>(bh) * n * 8);
  L.tflags = take(static_cast<size_t>(bh) * n * 8);
  L.tcount = take(static_cast<size_t>(bh) * ((n + kResTok - 1) / kResTok) * 4);   // any pass
  L.pcount = take(static_cast<size_t>(bh) * ((n + kCandTok - 1) / kCandTok) * 4);
  L.perm = take(static_cast<size_t>(bh) * n * 4);
  L.seg = take(static_cast<size_t>(bh) * n * 4);
  L.offsets = take(static_cast<size_t>(bh) * (c + 1) * 4);
  L.rad = take(static_cast<size_t>(bh) * cpad * 4);
  // neighbour rows [bh][cpad][cpad/32] and tile unions [bh][tiles][cpad/32]
  // (candidate path, C <= kNbrMaxC)
  const size_t nw = c <= kNbrMaxC ? cpad / 32 : 0;
  L.nbr = take(static_cast<size_t>(bh) * cpad * nw * 4);
  L.tun = take(static_cast<size_t>(bh) * ((n + kCandTok - 1) / kCandTok) * nw * 4);
  L.sort = take(sort_ws_bytes(bh, n, c));
  L.total = off;
  return L;
}

// ---------------------------------------------------------------------------
// MFMA assignment, main pass.  A workgroup holds kTokTile tokens of one slice
// in registers (MFMA B operands) and streams the slice's centroid tiles (32
// clusters, hi and lo split, plus their -||c||^2/2) through a three-stage LDS
// ring filled by direct global->LDS copies two tiles ahead; one partial vmcnt
// wait and one barrier per tile.
// ---------------------------------------------------------------------------
template <int D, bool PAIRS>
__global__ __launch_bounds__(kThreads, 2) void km_assign_main_kernel(
    const uint16_t *__restrict__ x, int n, int c, int cpad, const uint16_t *__restrict__ chi,
    const uint16_t *__restrict__ clo, const float *__restrict__ nh,
    int32_t *__restrict__ assign, int2 *__restrict__ tflags, int32_t *__restrict__ tcount,
    int32_t *__restrict__ pcount, int nbh, int tph) {
  constexpr int NS = D / 16;
  constexpr int NT = kNT;
  constexpr int PPR = D / 8;                          // 16-byte pieces per centroid row
  constexpr int RPI = 64 / PPR;                       // rows per 1 KB wave copy
  constexpr int BPS = 32 / RPI;                       // wave copies per split per tile
  constexpr int CPW = 2 * BPS / (kThreads / 64);      // wave copies per wave per tile
  static_assert(CPW >= 1 && CPW < 15, "copy split");
  constexpr int kSplitB = 32 * D * 2;                 // bytes of one split of a tile
  constexpr int kStageB = 2 * kSplitB;
  __shared__ __attribute__((aligned(16))) uint16_t sC[3][2][32 * D];
  __shared__ __attribute__((aligned(16))) float sN[3][64];   // [32, 64): copy padding
  __shared__ int32_t s_wq[kThreads / 64];
  __shared__ int32_t s_wp[kThreads / 64];
  __shared__ float s_nhmin[kThreads / 64];

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
  const size_t cbase = static_cast<size_t>(bh) * cpad;

  // copy geometry: wave copy j of a tile fills LDS bytes [1 KB * blk, +1 KB) of
  // split blk / BPS (blk = wave * CPW + j); lane l fills physical piece l % PPR
  // of row RPI * (blk % BPS) + l / PPR, i.e. the row's logical piece
  // (l % PPR) ^ swizzle(row).  Each wave also copies the tile's 32 -||c||^2/2.
  const int cp_rsub = lane / PPR, cp_piece = lane % PPR;
  auto issue_tile = [&](int ct, auto st) {
    constexpr int S = decltype(st)::value;
    const int t = ct < ntl ? ct : 0;                  // past the end: reload tile 0
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int blk = wave * CPW + j;
      const int sp = blk / BPS, rb = blk % BPS;
      const int r = rb * RPI + cp_rsub;
      const size_t goff = (cbase + t * 32 + r) * D + ((cp_piece ^ cswz<D>(r)) << 3);
      const uint16_t *src = (sp ? clo : chi) + goff;
      uint16_t *dst = &sC[S][sp][rb * RPI * D];
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
    {   // every wave copies the same 32 values (no branch, uniform copy counts);
        // lanes 32-63 repeat them into the padding
      const float *src = nh + cbase + t * 32 + (lane & 31);
      float *dst = &sN[S][0];
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 4, 0, 0);
    }
  };

  // ring prologue first: the compiler's wait for the token registers below
  // covers every load in flight (it cannot order plain loads against
  // global->LDS copies), so the copies are issued before anything it waits for
  issue_tile(0, std::integral_constant<int, 0>{});
  issue_tile(1, std::integral_constant<int, 1>{});
  asm volatile("" ::: "memory");

  // this workgroup's tokens: B operands of 32x32x16 MFMAs, lane holds
  // x[token][16 s + 8 h .. +8] of its token column
  int tok[NT];
  bool tv[NT];
  bf16x8 xf[NT][NS];
  const int base = tile * kTokTile;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    tok[nt] = base + wave * (NT * 32) + nt * 32 + col;
    tv[nt] = tok[nt] < n;
    // columns past the end load row n-1 unconditionally (a conditional load
    // makes the compiler wait for it at the branch join); their results are
    // never used
    const uint16_t *row = xb + static_cast<size_t>(tv[nt] ? tok[nt] : n - 1) * D + h * 8;
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2)
      xf[nt][s2] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(row + s2 * 16));
  }
  // -||c||^2/2 of the slice's real clusters, for max ||c||
  float mn = 0.f;
  for (int j0 = 0; j0 < c; j0 += 4 * kThreads) {
    float v4[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int j = j0 + k * kThreads + tid;
      v4[k] = j < c ? nh[cbase + j] : 0.f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) mn = fminf(mn, v4[k]);
  }

  // per-wave minimum of -||c||^2/2, read after the barriers below
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mn = fminf(mn, __shfl_xor(mn, off));
  if (lane == 0) s_nhmin[wave] = mn;

  // ||x|| bound per token: bf16 pair dot products (exact products, fp32
  // sums); the 2^-60 covers products below the fp32 normal range if flushed
  float nx[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float p = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) p = bf16x8_sumsq(xf[nt][s2], p);
    p += __shfl_xor(p, 32);
    nx[nt] = sqrtf(p) * (1.f + 0x1p-10f) + 0x1p-60f;
  }

  // LDS byte addresses of this lane's A fragments (centroid row col, piece
  // 2s+h) and -||c||^2/2 values in stage 0, split 0
  uint32_t ka[NS];
  const uint32_t sc0 = lds_offset(&sC[0][0][0]);
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) ka[s2] = sc0 + col * D * 2 + (((2 * s2 + h) ^ cswz<D>(col)) << 4);
  const uint32_t na = lds_offset(&sN[0][0]) + 16 * h;

  // the three best w of the lane's clusters; each value's row within its tile
  // rides in its 4 low mantissa bits, the tiles of the best two in t1, t2
  float b1[NT], b2[NT], b3[NT];
  int t1[NT], t2[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    b1[nt] = -INFINITY;
    b2[nt] = -INFINITY;
    b3[nt] = -INFINITY;
    t1[nt] = 0;
    t2[nt] = 0;
  }

  auto step = [&](auto st, int ct) {
    constexpr int S = decltype(st)::value;
    // tile ct has landed once only tile ct+1's copies are outstanding; after
    // the barrier every wave's copies of tile ct are in LDS and every wave is
    // done with tile ct-1, whose stage tile ct+2 then refills
    wait_vmcnt<CPW + 1>();
    lds_barrier();
    issue_tile(ct + 2, std::integral_constant<int, (S + 2) % 3>{});
    f32x4 n4[4];                                      // -||c||^2/2 of the lane's 16 rows
    lds_read_f32x4x4<S * 256, 32>(n4, na);
    f32x16 cinit;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) cinit[4 * g + j] = n4[g][j];
    f32x16 acc[NT];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
      bf16x8 af[NS];
      if (sp == 0) lds_read_frags<S * kStageB>(af, ka);
      else lds_read_frags<S * kStageB + kSplitB>(af, ka);
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[nt] = mfma32x32x16(af[s2], xf[nt][s2], (sp == 0 && s2 == 0) ? cinit : acc[nt]);
    }
    // w with its accumulator index i (0..15) in the 4 low mantissa bits: one
    // and-or, and max / med3 then carry the index along (the change of w,
    // below 2^-19 |w|, is part of the error bound).  Inserting we into
    // b1 >= b2 >= b3: b3 = med3(b2, b3, we), b2 = med3(b1, b2, we), b1 = max.
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float p1 = b1[nt], p2 = b2[nt];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float we = __int_as_float((__float_as_int(acc[nt][i]) & ~15) | i);
        if constexpr (PAIRS) b3[nt] = __builtin_amdgcn_fmed3f(b2[nt], b3[nt], we);
        b2[nt] = __builtin_amdgcn_fmed3f(b1[nt], b2[nt], we);
        b1[nt] = __builtin_elementwise_maximum(b1[nt], we);
      }
      // the second best is the old one, the demoted old best, or from this
      // tile (a bit-equal value from another tile makes b3 == b2, and such a
      // row is never settled from t2)
      const bool new1 = b1[nt] != p1;
      if constexpr (PAIRS) t2[nt] = b2[nt] == p2 ? t2[nt] : ((new1 && b2[nt] == p1) ? t1[nt] : ct);
      t1[nt] = new1 ? ct : t1[nt];
    }
  };
  for (int ct = 0; ct < ntl; ct += 3) {
    step(std::integral_constant<int, 0>{}, ct);
    if (ct + 1 < ntl) step(std::integral_constant<int, 1>{}, ct + 1);
    if (ct + 2 < ntl) step(std::integral_constant<int, 2>{}, ct + 2);
  }
  wait_vmcnt<0>();   // the copies past the end land before the workgroup ends

  // error bound E of every w of a token (split residual of the centroid, fp32
  // accumulation of 2d exact products and the start value, final rounding,
  // index bits), from ||x|| and the slice's max ||c|| (with margin)
  float nhmin = 0.f;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) nhmin = fminf(nhmin, s_nhmin[w]);
  const float cm = sqrtf(-2.f * nhmin) * (1.f + 0x1p-20f);
  // decided rows are assigned; queued rows are compacted, in wave and lane
  // order, to the front of this tile's region of the slice's queue area
  // (tflags), pair rows (token, best, second; cluster ids below 2^16) to its
  // back, with their counts in tcount and pcount
  bool queued[NT], paired[NT];
  uint64_t qm[NT], pm[NT];
  int thr_bits[NT], pair_ids[NT];
  int wq = 0, wp = 0;
  const bool pairs_ok = PAIRS && c <= 65536;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float e = 0x1p-25f * cm * cm + 0x1p-18f * nx[nt] * cm +
                    (2.f * D) * 0x1p-23f * (0.5f * cm * cm + 1.02f * nx[nt] * cm) +
                    0x1p-19f * (nx[nt] * cm + 0.5f * cm * cm);
    const float two_e = 2.f * 1.25f * e;
    const int i1 = t1[nt] * 32 + acc_row(__float_as_int(b1[nt]) & 15, h);
    const int i2 = t2[nt] * 32 + acc_row(__float_as_int(b2[nt]) & 15, h);
    const float ob1 = __shfl_xor(b1[nt], 32), ob2 = __shfl_xor(b2[nt], 32);
    const float ob3 = __shfl_xor(b3[nt], 32);
    const int oi1 = __shfl_xor(i1, 32), oi2 = __shfl_xor(i2, 32);
    const bool other = ob1 > b1[nt] || (ob1 == b1[nt] && oi1 < i1);
    const float nb1 = fmaxf(b1[nt], ob1);
    const int ival = other ? oi1 : i1;
    // second best: the smaller of the two bests or the larger of the two
    // seconds; third best of the six (each lane's three sorted)
    const float lo1 = fminf(b1[nt], ob1), hi2 = fmaxf(b2[nt], ob2);
    const float nb2 = fmaxf(lo1, hi2);
    const int ival2 = lo1 >= hi2 ? (other ? i1 : oi1) : (b2[nt] >= ob2 ? i2 : oi2);
    const float nb3 = fmaxf(fmaxf(fminf(b1[nt], ob2), fminf(b2[nt], ob1)), fmaxf(b3[nt], ob3));
    const bool decided = nb1 - nb2 > two_e;
    const bool two = !decided && pairs_ok && nb1 - nb3 > two_e;
    if (h == 0 && tv[nt] && decided) assign[static_cast<size_t>(bh) * n + tok[nt]] = ival;
    queued[nt] = h == 0 && tv[nt] && !decided && !two;
    paired[nt] = h == 0 && tv[nt] && two;
    thr_bits[nt] = __float_as_int(nb1 - two_e);
    pair_ids[nt] = (ival << 16) | ival2;
    qm[nt] = __ballot(queued[nt]);
    pm[nt] = __ballot(paired[nt]);
    wq += __popcll(qm[nt]);
    wp += __popcll(pm[nt]);
  }
  if (lane == 0) {
    s_wq[wave] = wq;
    s_wp[wave] = wp;
  }
  __syncthreads();
  int q = base, p = 0, tot = 0, ptot = 0;
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    q += w < wave ? s_wq[w] : 0;
    p += w < wave ? s_wp[w] : 0;
    tot += s_wq[w];
    ptot += s_wp[w];
  }
  // the region's last row: pair k sits at [last - k]
  const int last = base + min(kTokTile, n - base) - 1;
  const uint64_t lt = (1ull << lane) - 1;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (queued[nt])
      tflags[static_cast<size_t>(bh) * n + q + __popcll(qm[nt] & lt)] = int2{tok[nt], thr_bits[nt]};
    if (paired[nt])
      tflags[static_cast<size_t>(bh) * n + last - (p + __popcll(pm[nt] & lt))] =
          int2{tok[nt], pair_ids[nt]};
    q += __popcll(qm[nt]);
    p += __popcll(pm[nt]);
  }
  if (tid == 0) {
    tcount[static_cast<size_t>(bh) * tph + tile] = tot;
    pcount[static_cast<size_t>(bh) * tph + tile] = ptot;
  }
}

// ---------------------------------------------------------------------------
// MFMA assignment, main pass with the centroid table resident (at most
// kResTiles tiles of 32 clusters).  A slice's whole table (hi and lo splits
// plus -||c||^2/2) fits in LDS, so a persistent workgroup loads it once and
// its waves then run with no barrier: wave w takes the 64-token tiles
// t0 + w, t0 + w + 8, ... of the workgroup's range [t0, t1), loading the next
// tile's rows into a second register buffer while the current tile's MFMAs
// run.  A range never covers more than two consecutive slices (the grid has
// at least one workgroup per slice), and both tables are loaded up front.
// Arithmetic, error bound and queue rows are those of the streaming pass;
// each 64-token tile has its own queue region and count.
// ---------------------------------------------------------------------------
// v from lane l ^ 32: permlane32_swap exchanges lanes 32-63 of its first
// operand with lanes 0-31 of its second
__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

template <int D, int NTL>
__global__ __launch_bounds__(64 * kResWaves, 1) void km_assign_res_kernel(
    const uint16_t *__restrict__ x, int n, int c, int cpad, const uint16_t *__restrict__ chi,
    const uint16_t *__restrict__ clo, const float *__restrict__ nh,
    int32_t *__restrict__ assign, int2 *__restrict__ tflags, int32_t *__restrict__ tcount,
    int nbh, int tph) {
  constexpr int NS = D / 16;
  constexpr int PPR = D / 8;                       // 16-byte pieces per centroid row
  constexpr int ROWS = NTL * 32;
  constexpr int kSplitB = ROWS * D * 2;            // bytes of one split of a slot
  constexpr int kThr = 64 * kResWaves;
  __shared__ __attribute__((aligned(16))) uint16_t sC[2][2][ROWS * D];
  __shared__ __attribute__((aligned(16))) float sN[2][ROWS];
  __shared__ float s_min[2][kResWaves];
  __shared__ float s_cm[2];

  const long long tt = static_cast<long long>(nbh) * tph;
  const int t0 = static_cast<int>(tt * blockIdx.x / gridDim.x);
  const int t1 = static_cast<int>(tt * (blockIdx.x + 1) / gridDim.x);
  if (t0 >= t1) return;   // uniform over the workgroup
  const int s0 = t0 / tph, ns = (t1 - 1) / tph - s0 + 1;   // 1 or 2 slices
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar tile bookkeeping
  const int h = lane >> 5, col = lane & 31;

  // the tile's rows: B operands of 32x32x16 MFMAs, lane holds
  // x[token][16 s + 8 h .. +8] of token base + 32 nt + col
  auto load = [&](bf16x8 (&xf)[2][NS], int t) {
    const int sl = t / tph, base = (t % tph) * kResTok;
    const uint16_t *xb = x + static_cast<size_t>(sl) * n * D;
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int tok = min(base + nt * 32 + col, n - 1);
      const uint16_t *row = xb + static_cast<size_t>(tok) * D + h * 8;
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2)
        xf[nt][s2] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(row + s2 * 16));
    }
  };

  // the first tile's rows are in flight while the tables load (a wave with
  // no tile loads its range's first tile and leaves after the barriers)
  int gt = t0 + wave;
  bf16x8 xa[2][NS], xb[2][NS];
  load(xa, gt < t1 ? gt : t0);

  // both tables, k-major: piece p = 2 s + h (dimensions 8p .. 8p+7) of row r
  // sits at 16-byte slot (s * ROWS + r) * 2 + h of its split, so a wave's
  // fragment read for one k-step is 1 KB of consecutive bytes.  Thread idx
  // fills slot idx (consecutive lanes, consecutive LDS bytes).
  for (int k = 0; k < ns; ++k) {
    const size_t cbase = static_cast<size_t>(s0 + k) * cpad;
    for (int idx = tid; idx < 2 * ROWS * PPR; idx += kThr) {
      const int sp = idx / (ROWS * PPR), slot = idx % (ROWS * PPR);
      const int hh = slot & 1, r = (slot >> 1) % ROWS, s2 = (slot >> 1) / ROWS;
      const u32x4 v = *reinterpret_cast<const u32x4 *>((sp ? clo : chi) + (cbase + r) * D +
                                                       (2 * s2 + hh) * 8);
      *reinterpret_cast<u32x4 *>(&sC[k][sp][slot * 8]) = v;
    }
    float mn = 0.f;
    for (int j = tid; j < ROWS; j += kThr) {
      const float v = nh[cbase + j];
      sN[k][j] = v;
      if (j < c) mn = fminf(mn, v);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mn = fminf(mn, __shfl_xor(mn, off));
    if (lane == 0) s_min[k][wave] = mn;
  }
  __syncthreads();
  // each slot's bound: max ||c|| of the slice's real clusters (with margin)
  if (tid < 2) {
    float m = 0.f;
#pragma unroll
    for (int w = 0; w < kResWaves; ++w) m = fminf(m, tid < ns ? s_min[tid][w] : 0.f);
    s_cm[tid] = sqrtf(-2.f * m) * (1.f + 0x1p-20f);
  }
  __syncthreads();

  if (gt >= t1) return;   // wave-uniform; no barrier follows

  auto tile_pass = [&](const bf16x8 (&xf)[2][NS], int t) {
    const int sl = t / tph, tile = t % tph, k = sl - s0;
    const int base = tile * kResTok;
    // LDS byte address of this lane's A fragment (row col, piece h) of k-step
    // 0 in the slot's split 0, tile 0; k-step s is ROWS * 32 bytes further
    const uint32_t ka = lds_offset(&sC[k][0][0]) + (col * 2 + h) * 16;
    const uint32_t na = lds_offset(&sN[k][0]) + 16 * h;
    float b1[2], b2[2];
    int t1r[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      b1[nt] = -INFINITY;
      b2[nt] = -INFINITY;
      t1r[nt] = 0;
    }
    f32x16 acc[2];
    auto ctile = [&](auto ctc) {
      constexpr int ct = decltype(ctc)::value;
      f32x4 n4[4];                                  // -||c||^2/2 of the lane's 16 rows
      lds_read_f32x4x4<ct * 128, 32>(n4, na);
      f32x16 cinit;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) cinit[4 * g + j] = n4[g][j];
      // hi split for both token groups, then the lo split group by group, so
      // that the first group's argmax tracking below runs under the second
      // group's MFMAs
      bf16x8 af[NS];
      lds_read_frags_strided<ct * 1024, ROWS * 32>(af, ka);
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[nt] = mfma32x32x16(af[s2], xf[nt][s2], s2 == 0 ? cinit : acc[nt]);
      lds_read_frags_strided<kSplitB + ct * 1024, ROWS * 32>(af, ka);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int s2 = 0; s2 < NS; ++s2) acc[nt] = mfma32x32x16(af[s2], xf[nt][s2], acc[nt]);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const float p1 = b1[nt];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float we = __int_as_float((__float_as_int(acc[nt][i]) & ~15) | i);
          b2[nt] = __builtin_amdgcn_fmed3f(b1[nt], b2[nt], we);
          b1[nt] = __builtin_elementwise_maximum(b1[nt], we);
        }
        t1r[nt] = b1[nt] != p1 ? ct : t1r[nt];
        // the tracking happens here: otherwise the compiler sinks it to the
        // decisions and keeps every tile's accumulators alive until then
        asm volatile("" : "+v"(b1[nt]), "+v"(b2[nt]), "+v"(t1r[nt]));
      }
      // schedule: the first group's lo MFMAs, then the second group's, each
      // followed by an equal share of the first group's tracking; nothing
      // moves across tiles (register budget)
      __builtin_amdgcn_sched_group_barrier(0x008, NS, 0);
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 48 / NS, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    ctile(std::integral_constant<int, 0>{});
    if constexpr (NTL > 1) ctile(std::integral_constant<int, 1>{});
    if constexpr (NTL > 2) ctile(std::integral_constant<int, 2>{});
    if constexpr (NTL > 3) ctile(std::integral_constant<int, 3>{});
    // decisions, as in the streaming pass; queued rows compacted in lane order
    const float cm = s_cm[k];
    bool queued[2];
    uint64_t qm[2];
    int thr_bits[2], tok[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      tok[nt] = base + nt * 32 + col;
      const bool tv = tok[nt] < n;
      // ||x||^2 (exact products, fp32 sums); the 2^-60 covers products
      // below the fp32 normal range if they are flushed
      float p = 0.f;
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) p = bf16x8_sumsq(xf[nt][s2], p);
      p += xor32(p);
      const float nx = sqrtf(p) * (1.f + 0x1p-10f) + 0x1p-60f;
      const float e = 0x1p-25f * cm * cm + 0x1p-18f * nx * cm +
                      (2.f * D) * 0x1p-23f * (0.5f * cm * cm + 1.02f * nx * cm) +
                      0x1p-19f * (nx * cm + 0.5f * cm * cm);
      const float two_e = 2.f * 1.25f * e;
      const int i1 = t1r[nt] * 32 + acc_row(__float_as_int(b1[nt]) & 15, h);
      const float ob1 = xor32(b1[nt]), ob2 = xor32(b2[nt]);
      const int oi1 = __float_as_int(xor32(__int_as_float(i1)));
      const bool other = ob1 > b1[nt] || (ob1 == b1[nt] && oi1 < i1);
      const float nb1 = fmaxf(b1[nt], ob1);
      const float nb2 = fmaxf(fminf(b1[nt], ob1), fmaxf(b2[nt], ob2));
      const bool decided = nb1 - nb2 > two_e;
      if (h == 0 && tv && decided) assign[static_cast<size_t>(sl) * n + tok[nt]] = other ? oi1 : i1;
      queued[nt] = h == 0 && tv && !decided;
      thr_bits[nt] = __float_as_int(nb1 - two_e);
      qm[nt] = __ballot(queued[nt]);
    }
    // rank among the queued lanes below this one
    auto below = [](uint64_t m) {
      return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                       __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
    };
    const size_t region = static_cast<size_t>(sl) * n + base;
    if (queued[0]) tflags[region + below(qm[0])] = int2{tok[0], thr_bits[0]};
    if (queued[1]) tflags[region + __popcll(qm[0]) + below(qm[1])] = int2{tok[1], thr_bits[1]};
    if (lane == 0) tcount[static_cast<size_t>(sl) * tph + tile] = __popcll(qm[0]) + __popcll(qm[1]);
  };

  // two register buffers in turn; past the range end the current tile is
  // loaded again (a cache hit) so the loads stay unconditional
  for (;;) {
    int nx = gt + kResWaves;
    load(xb, nx < t1 ? nx : gt);
    tile_pass(xa, gt);
    if (nx >= t1) break;
    gt = nx;
    nx = gt + kResWaves;
    load(xa, nx < t1 ? nx : gt);
    tile_pass(xb, gt);
    if (nx >= t1) break;
    gt = nx;
  }
}

// ---------------------------------------------------------------------------
// pair rows: the rows listed at the back of a token tile's region (one
// workgroup per tile, as the main pass), D/8 lanes per row (each lane 8 consecutive dimensions); exact fp64 squared distances
// to the two candidates, each lane's 8 terms added in ascending dimension
// order and the lanes' partial sums then in a fixed butterfly; the smaller
// distance wins, ties to the lower index.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void km_pair_kernel(
    const uint16_t *__restrict__ x, int n, int c, const float *__restrict__ cent,
    const int2 *__restrict__ tflags, const int32_t *__restrict__ pcount,
    int32_t *__restrict__ assign, int32_t *__restrict__ n_refined, int nbh, int tph) {
  const int xcd = blockIdx.x & 7, k8 = blockIdx.x >> 3;
  const int bh = xcd + 8 * (k8 / tph);
  const int tile = k8 % tph;
  if (bh >= nbh) return;
  constexpr int LPR = D / 8;                 // lanes per row
  constexpr int RPW = 64 / LPR;              // rows per wave pass
  constexpr int RPB = RPW * (kThreads / 64); // rows per workgroup pass
  const int np = pcount[static_cast<size_t>(bh) * tph + tile];
  const int base = tile * kTokTile;
  const int last = base + min(kTokTile, n - base) - 1;
  const uint16_t *xb = x + static_cast<size_t>(bh) * n * D;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR;                // this lane's 8 dimensions
  const int rw = wave * RPW + lane / LPR;    // this lane's row within a pass
  for (int k0 = 0; k0 < np; k0 += RPB) {
    const int k = k0 + rw;
    const bool live = k < np;                // uniform over the row's lanes
    const int2 e = tflags[static_cast<size_t>(bh) * n + last - (live ? k : 0)];
    const int ids[2] = {(e.y >> 16) & 0xffff, e.y & 0xffff};
    const u32x4 xv = reinterpret_cast<const u32x4 *>(xb + static_cast<size_t>(e.x) * D)[sub];
    double dist[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const f32x4 *cr = reinterpret_cast<const f32x4 *>(cent + (static_cast<size_t>(bh) * c + ids[r]) * D);
      const f32x4 c0 = cr[2 * sub], c1 = cr[2 * sub + 1];
      double s = 0.0;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const float xf32 = bf16_bits_to_f32(static_cast<uint16_t>(xv[t >> 1] >> (16 * (t & 1))));
        const float cf32 = t < 4 ? c0[t] : c1[t - 4];
        const double df = static_cast<double>(xf32) - static_cast<double>(cf32);
        s = fma(df, df, s);
      }
#pragma unroll
      for (int o = LPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
      dist[r] = s;
    }
    if (live && sub == 0) {
      const bool second = dist[1] < dist[0] || (dist[1] == dist[0] && ids[1] < ids[0]);
      assign[static_cast<size_t>(bh) * n + e.x] = second ? ids[1] : ids[0];
    }
  }
  if (n_refined != nullptr && threadIdx.x == 0 && np > 0) atomicAdd(n_refined, np);
}

// ---------------------------------------------------------------------------
// fp64 refinement of the queued rows: the queued rows run through the same
// MFMA loop (centroid tiles staged through registers into two LDS buffers);
// every cluster with w >= the row's threshold goes to an LDS candidate list,
// one lane per candidate computes the exact fp64 distance, and the smallest
// distance wins, ties to the lowest index.  Grid-stride over the slice's
// queue, 32 rows per wave.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads, 2) void km_refine_kernel(
    const uint16_t *__restrict__ x, int n, int c, int cpad, const uint16_t *__restrict__ chi,
    const uint16_t *__restrict__ clo, const float *__restrict__ nh,
    const int32_t *__restrict__ qcount, const float *__restrict__ cent,
    int32_t *__restrict__ assign, const int2 *__restrict__ flags,
    int32_t *__restrict__ n_refined, int nbh, int tph) {
  constexpr int NS = D / 16;
  constexpr int KCH = D / 8;                 // 16-byte chunks per centroid row
  constexpr int CPT = KCH / 4;               // chunks per thread per tile load
  constexpr int CC = kCandCap;
  constexpr int NT = 1;                      // 32 queued rows per wave
  constexpr int TOKT = NT * 32 * (kThreads / 64);
  constexpr int TS = TOKT;
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
  const int ntok = qcount[bh];
  const int step = tph * TOKT;

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

  for (int base = tile * TOKT; base < ntok; base += step) {
    int tok[NT];
    bool tv[NT];
    float thr[NT];
    bf16x8 xf[NT][NS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int slot = wave * (NT * 32) + nt * 32 + col;
      const int idx = base + slot;
      tv[nt] = idx < ntok;
      tok[nt] = idx;
      thr[nt] = 0.f;
      if (tv[nt]) {
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
      if (h == 0) {
        s_tok[slot] = tv[nt] ? tok[nt] : -1;
        s_over[slot] = 0;
        s_bestd[slot] = ~0ull;
        s_bestc[slot] = 0x7fffffff;
      }
    }
    if (tid == 0) s_ncand = 0;

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
      f32x16 acc[NT];
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
#pragma unroll
        for (int s = 0; s < NS; ++s) {
          const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
              sC[buf][sp] + col * D + (((2 * s + h) ^ cswz<D>(col)) * 8));
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[nt] = mfma32x32x16(a, xf[nt][s], (sp == 0 && s == 0) ? cinit : acc[nt]);
        }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int cl = ct * 32 + acc_row(i, h);
          const float w = acc[nt][i];
          if (tv[nt] && cl < c && w >= thr[nt]) {
            const int slot = wave * (NT * 32) + nt * 32 + col;
            const int k = atomicAdd(&s_ncand, 1);
            if (k < kCandCap) s_cand[k] = (slot << 14) | cl;
            else s_over[slot] = 1;
          }
        }
      if (ct + 1 < ntl) store_tile(buf ^ 1);
      __syncthreads();
    }

    {
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
      for (int slot = tid; slot < TOKT; slot += kThreads) {
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
// refine queue of a slice: the per-tile regions of tflags (rt rows apart)
// joined in tile order into flags[0, total); total goes to qcount[slice].  A
// workgroup takes kJoinTiles consecutive tiles: it adds up the counts of the
// slice's earlier tiles, scans its own counts in one wave, and its threads
// then copy the tiles' rows together; the workgroup with the last tile writes
// the total.
// ---------------------------------------------------------------------------
constexpr int kJoinTiles = 64;
__global__ __launch_bounds__(kThreads) void km_queue_join_kernel(
    const int2 *__restrict__ tflags, const int32_t *__restrict__ tcount, int n, int tph, int rt,
    int2 *__restrict__ flags, int32_t *__restrict__ qcount) {
  __shared__ int32_t s_off[kJoinTiles + 1];
  __shared__ int32_t s_part[kThreads / 64];
  const int bh = blockIdx.y, t0 = blockIdx.x * kJoinTiles;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t *cnt = tcount + static_cast<size_t>(bh) * tph;
  int pre = 0;
  for (int u = tid; u < t0; u += kThreads) pre += cnt[u];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) pre += __shfl_xor(pre, o);
  if (lane == 0) s_part[wave] = pre;
  __syncthreads();
  if (wave == 0) {
    int base = 0;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) base += s_part[w];
    const int c = t0 + lane < tph ? cnt[t0 + lane] : 0;
    int v = c;   // inclusive scan over the 64 lanes
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(v, o);
      if (lane >= o) v += y;
    }
    s_off[lane] = base + v - c;
    if (lane == 63) s_off[kJoinTiles] = base + v;
  }
  __syncthreads();
  // the block's rows in output order: row e belongs to the last tile j with
  // s_off[j] <= e (binary search; tiles past the slice end are empty)
  const int first = s_off[0], total = s_off[kJoinTiles] - first;
  const int2 *from = tflags + static_cast<size_t>(bh) * n + static_cast<size_t>(t0) * rt;
  int2 *to = flags + static_cast<size_t>(bh) * n + first;
  for (int e = tid; e < total; e += kThreads) {
    int lo = 0;
#pragma unroll
    for (int step = kJoinTiles / 2; step > 0; step >>= 1)
      if (s_off[lo + step] - first <= e) lo += step;
    to[e] = from[static_cast<size_t>(lo) * rt + (e - (s_off[lo] - first))];
  }
  if (t0 + kJoinTiles >= tph && tid == 0) qcount[bh] = s_off[kJoinTiles];
}

// ---------------------------------------------------------------------------
// Candidate path (every iteration after the first, for C <= kNbrMaxC).  The
// assignment of the previous iteration says which cluster a each token was
// in; the mean pass of that iteration bounds R_a >= max ||x - c_a|| over those
// tokens for the new centroid c_a.  For any token x of a and any cluster j with
// ||c_a - c_j|| > 2 R_a, the triangle inequality gives ||x - c_j|| >=
// ||c_a - c_j|| - ||x - c_a|| > R_a >= ||x - c_a||, so j is strictly farther
// than a and can be neither the argmin nor tied with it.  The argmin over all
// clusters is therefore the argmin over N(a) = {j : ||c_a - c_j|| <= 2 R_a},
// which holds a itself, and over any superset of N(a).
//   km_nbr_kernel       the neighbour bit matrix: bit j of row a is set for j
//                       in N(a) (up to a rigorous error bound, always on the
//                       side of setting it)
//   km_tile_union_kernel  for each tile of kCandTok positions of the previous
//                       iteration's sorted order, the OR of the rows of the
//                       tile's clusters (a run of ids, since the order is
//                       sorted by cluster)
//   km_assign_cand_kernel  the tile's tokens against the clusters of its union,
//                       then the rows the fast path leaves undecided, in fp64
// ---------------------------------------------------------------------------

// Neighbour bits.  A workgroup takes kNbrWaves tiles of 32 clusters a of a
// slice (one per wave, held as MFMA B operands, hi and lo split) and streams
// every tile of 32 clusters j through two LDS buffers (direct global->LDS
// copies, swizzled as in the main pass).  The Gram block G = hi_j.hi_a +
// lo_j.hi_a + hi_j.lo_a runs on MFMA (clusters j on the accumulator rows, the
// lane's cluster a on its column), D = ||c_a||^2 + ||c_j||^2 - 2 G, and bit j
// is cleared only if D - errD > 4 R_a^2, with errD a rigorous bound of
// |D - ||c_a - c_j||^2|:
// * the split leaves c = hi + lo + res with |res| <= 2^-18 |c| per element, so
//   the three dropped products (lo.lo and the two res terms) are below
//   3.1 * 2^-18 |c_a||c_j|;
// * the 3d accumulated products sum, in magnitude, to at most 1.03 |c_a||c_j|
//   and each addition loses at most one unit (2^-23) of that;
// * the fp32 norms (rounded from fp64), their sum and the final subtraction
//   lose at most 4 * 2^-24 (|c_a|^2 + |c_j|^2);
// all with a 1.25 margin.
constexpr int kNbrWaves = 4;
constexpr int kNbrJt = 4;                       // tiles of clusters j per workgroup
template <int D>
__global__ __launch_bounds__(64 * kNbrWaves) void km_nbr_kernel(
    const uint16_t *__restrict__ chi, const uint16_t *__restrict__ clo,
    const float *__restrict__ nh, const float *__restrict__ rad, int c, int cpad,
    uint32_t *__restrict__ nbr) {
  constexpr int NS = D / 16;
  constexpr int PPR = D / 8;                        // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;                     // rows per 1 KB wave copy
  constexpr int BPS = 32 / RPI;                     // wave copies per split per tile
  constexpr int CPW = 2 * BPS / kNbrWaves;          // wave copies per wave per tile
  static_assert(CPW >= 1 && CPW < 8, "copy split");
  constexpr int kSplitB = 32 * D * 2;
  constexpr int kBufB = 2 * kSplitB;
  __shared__ __attribute__((aligned(16))) uint16_t sJ[2][2][32 * D];   // [buffer][split]
  __shared__ __attribute__((aligned(16))) float sNj[2][64];            // [32, 64): padding
  const int bh = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int nw = cpad / 32;
  const int jt0 = blockIdx.y * kNbrJt, jt1 = min(nw, jt0 + kNbrJt);
  const size_t cb = static_cast<size_t>(bh) * cpad;
  const int a0 = (blockIdx.x * kNbrWaves + wave) * 32;
  const bool wave_ok = a0 < cpad;                  // wave-uniform
  const int a = wave_ok ? a0 + col : col;
  bf16x8 bh_[NS], bl_[NS];
  {
    const uint16_t *pa = chi + (cb + a) * D + h * 8, *pb = clo + (cb + a) * D + h * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bh_[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(pa + s * 16));
      bl_[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(pb + s * 16));
    }
  }
  const float na = -2.f * nh[cb + a];
  const float r = rad[cb + a];
  const float lim = 4.f * r * r * (1.f + 0x1p-20f);
  const int cp_rsub = lane / PPR, cp_piece = lane % PPR;
  auto issue = [&](int jt, int b) {
    {
      const float *src = nh + cb + jt * 32 + (lane & 31);
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)&sNj[b][0], 4, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int blk = wave * CPW + j;
      const int sp = blk / BPS, rb = blk % BPS;
      const int rr = rb * RPI + cp_rsub;
      const size_t goff = (cb + jt * 32 + rr) * D + ((cp_piece ^ cswz<D>(rr)) << 3);
      const uint16_t *src = (sp ? clo : chi) + goff;
      uint16_t *dst = &sJ[b][sp][rb * RPI * D];
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
  };
  uint32_t ka[NS];
  const uint32_t sj0 = lds_offset(&sJ[0][0][0]);
#pragma unroll
  for (int s = 0; s < NS; ++s) ka[s] = sj0 + col * D * 2 + (((2 * s + h) ^ cswz<D>(col)) << 4);
  const uint32_t nja = lds_offset(&sNj[0][0]) + 16 * h;
  constexpr float kG = 2.f * (3.1f * 0x1p-18f + 3.f * D * 0x1p-23f * 1.03f);
  auto compute = [&](auto bufc, int jt) {
    constexpr int B = decltype(bufc)::value;
    f32x4 n4[4];
    lds_read_f32x4x4<B * 256, 32>(n4, nja);
    f32x16 g;
#pragma unroll
    for (int i = 0; i < 16; ++i) g[i] = 0.f;
    bf16x8 ah[NS], al[NS];
    lds_read_frags<B * kBufB>(ah, ka);
    lds_read_frags<B * kBufB + kSplitB>(al, ka);
#pragma unroll
    for (int s = 0; s < NS; ++s) g = mfma32x32x16(ah[s], bh_[s], g);
#pragma unroll
    for (int s = 0; s < NS; ++s) g = mfma32x32x16(al[s], bh_[s], g);
#pragma unroll
    for (int s = 0; s < NS; ++s) g = mfma32x32x16(ah[s], bl_[s], g);
    uint32_t bits = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = acc_row(i, h);
      const float nj = -2.f * n4[i >> 2][i & 3];
      const float dd = (na + nj) - 2.f * g[i];
      const float err = 1.25f * (kG * sqrtf(na * nj) + 0x1p-22f * (na + nj));
      const int j = jt * 32 + row;
      const bool need = j < c && (j == a || dd - err <= lim);
      bits |= need ? (1u << row) : 0u;
    }
    bits |= __shfl_xor(bits, 32);                      // both halves: all 32 rows
    if (wave_ok && h == 0 && a < c) nbr[(cb + a) * nw + jt] = bits;
  };
  issue(jt0, 0);
  if (jt0 + 1 < jt1) issue(jt0 + 1, 1);
  for (int jt = jt0; jt < jt1; ++jt) {
    const int b = (jt - jt0) & 1;
    if (jt + 1 < jt1) wait_vmcnt<CPW + 1>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (b) compute(std::integral_constant<int, 1>{}, jt);
    else compute(std::integral_constant<int, 0>{}, jt);
    if (jt + 2 < jt1) {
      lds_barrier();                                   // every wave is done with buffer b
      issue(jt + 2, b);
    }
  }
}

// Tile unions: word w of tile t = OR of word w of the rows of the tile's
// clusters a0 .. a1 (the clusters of its first and last sorted positions).
__global__ __launch_bounds__(64) void km_tile_union_kernel(
    const int32_t *__restrict__ seg, const uint32_t *__restrict__ nbr, int n, int c, int cpad,
    int tph, uint32_t *__restrict__ tun) {
  const int tile = blockIdx.x, bh = blockIdx.y, lane = threadIdx.x;
  const int nw = cpad / 32;
  const int base = tile * kCandTok, last = min(n, base + kCandTok) - 1;
  const int32_t *sg = seg + static_cast<size_t>(bh) * n;
  const int a0 = min(max(sg[base], 0), c - 1), a1 = min(max(sg[last], 0), c - 1);
  const uint32_t *rows = nbr + static_cast<size_t>(bh) * cpad * nw;
  for (int w = lane; w < nw; w += 64) {
    uint32_t m = 0;
    for (int a = a0; a <= a1; ++a) m |= rows[static_cast<size_t>(a) * nw + w];
    tun[(static_cast<size_t>(bh) * tph + tile) * nw + w] = m;
  }
}

// The union of a tile as ascending ids in LDS, from word `m` of its bit mask
// held by thread m's index (threads nw and above hold 0); returns its size
// (ids past cap are not stored).  All kThr threads must call it.
template <int kThr>
__device__ int tile_union_ids(uint32_t m, int32_t *ids, int cap, int32_t *wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int cnt = __popc(m);
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  lds_barrier();
  int pre = 0, nu = 0;
#pragma unroll
  for (int w = 0; w < kThr / 64; ++w) {
    pre += w < wave ? wsum[w] : 0;
    nu += wsum[w];
  }
  int k = pre + incl - cnt;
  for (uint32_t b = m; b; b &= b - 1, ++k)
    if (k < cap) ids[k] = 32 * tid + __builtin_ctz(b);
  lds_barrier();
  return nu;
}

// Assign pass over candidates.  A workgroup takes kCandTok consecutive
// positions of the previous iteration's sorted order, one group of 32 tokens
// per wave held as MFMA B operands.  The tile's union (ascending ids; every
// cluster when it is too large) is gathered 32 clusters at a time ("virtual
// tiles": hi and lo split, swizzled as in the main pass) into two LDS buffers
// by direct global->LDS copies, the next tile's copies in flight while a tile
// is computed.  Every value's tracking, error bound and decision (decided /
// two candidates / queued) are those of km_assign_main_kernel, the tile of a
// value being its virtual tile.  The pass then settles its own undecided rows
// in fp64 (pair rows over their two clusters, queued rows over the slots
// their per-tile candidate masks kept).
constexpr int kUnionCap = 1024;                 // union ids held in LDS (more: every cluster)
// union tiles whose candidate masks the candidate pass keeps: 16 (8 KB of LDS)
// up to 16 tiles of clusters, 32 above (16 KB; two workgroups per CU)
constexpr int kMaskTilesSmall = 16, kMaskTilesLarge = 32;
template <int D, int kMaskTiles>
__global__ __launch_bounds__(64 * kCandWaves) void km_assign_cand_kernel(
    const uint16_t *__restrict__ x, int n, int c, int cpad, const uint16_t *__restrict__ chi,
    const uint16_t *__restrict__ clo, const float *__restrict__ nh,
    const float *__restrict__ cent, const int32_t *__restrict__ perm,
    const uint32_t *__restrict__ tun, int32_t *__restrict__ assign,
    int32_t *__restrict__ n_refined, int nbh, int tph) {
  constexpr int NS = D / 16;
  constexpr int kThr = 64 * kCandWaves;
  constexpr int PPR = D / 8;                        // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;                     // rows per 1 KB wave copy
  constexpr int BPS = 32 / RPI;                     // wave copies per split per tile
  constexpr int CPW = 2 * BPS / kCandWaves;         // wave copies per wave per tile
  static_assert(CPW >= 1 && CPW < 8, "copy split");
  constexpr int kSplitB = 32 * D * 2;
  constexpr int kBufB = 2 * kSplitB;
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][2][32 * D];   // [buffer][split]
  __shared__ __attribute__((aligned(16))) float sN[2][64];   // [32, 64): copy padding
  __shared__ int32_t sU[kUnionCap];
  __shared__ int32_t s_wsum[kCandWaves];
  __shared__ int32_t s_wq[kCandWaves], s_wp[kCandWaves];
  __shared__ int2 sRow[kCandTok];             // undecided rows: queued first, pairs last
  // per virtual tile (the first kMaskTiles) and token, each lane half's
  // candidate slots: those whose value reached the half's running best - 2E
  __shared__ uint16_t sCm[kMaskTiles][kCandTok][2];
  const int xcd = blockIdx.x & 7, k8 = blockIdx.x >> 3;
  const int bh = xcd + 8 * (k8 / tph);
  const int tile = k8 % tph;
  if (bh >= nbh) return;   // uniform over the workgroup
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const size_t cb = static_cast<size_t>(bh) * cpad;
  const int nw = cpad / 32;
  const uint16_t *xb = x + static_cast<size_t>(bh) * n * D;
  int32_t *as = assign + static_cast<size_t>(bh) * n;
  const int base = tile * kCandTok;
  const int last = base + min(kCandTok, n - base) - 1;

  // the tile's union mask (loaded first: loads complete in order, and this one
  // is waited for before the token rows are needed); this wave's 32 tokens as
  // B operands, in flight while the union is compacted (the barriers below
  // wait for LDS only)
  const uint32_t m_own = tid < nw ? tun[(static_cast<size_t>(bh) * tph + tile) * nw + tid] : 0u;
  // max ||c|| of the slice (with margin), as in the main pass: eight
  // independent loads per lane at a time
  float mn = 0.f;
  for (int j0 = 0; j0 < c; j0 += 8 * 64) {
    float v8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + u * 64 + lane;
      v8[u] = j < c ? nh[cb + j] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) mn = fminf(mn, v8[u]);
  }
  const int p = base + wave * 32 + col;
  const bool tv = p < n;
  const int tok = perm[static_cast<size_t>(bh) * n + (tv ? p : last)];
  bf16x8 xf[NS];
  {
    const uint16_t *row = xb + static_cast<size_t>(tok) * D + h * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      xf[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(row + s * 16));
  }
  int nu = tile_union_ids<kThr>(m_own, sU, kUnionCap, s_wsum);
  const bool ids_all = nu > kUnionCap || nu >= c;
  if (ids_all) nu = c;
  const int nv = (nu + 31) / 32;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mn = fminf(mn, __shfl_xor(mn, o));
  const float cm = sqrtf(-2.f * mn) * (1.f + 0x1p-20f);

  // virtual tile v into buffer b: wave copy j of the tile fills LDS bytes
  // [1 KB * blk, +1 KB) of split blk / BPS; lane l fills physical piece l % PPR of
  // row RPI * (blk % BPS) + l / PPR (the row's logical piece (l % PPR) ^ swizzle);
  // each wave also copies the tile's 32 -||c||^2/2 values, so every wave has
  // CPW + 1 copies per tile in flight (padding rows are masked in compute)
  const int cp_rsub = lane / PPR, cp_piece = lane % PPR;
  auto uid = [&](int slot) { return ids_all ? min(slot, c - 1) : sU[min(slot, nu - 1)]; };
  auto issue = [&](int v, int b) {
    {
      const float *src = nh + cb + uid(v * 32 + (lane & 31));
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)&sN[b][0], 4, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const int blk = wave * CPW + j;
      const int sp = blk / BPS, rb = blk % BPS;
      const int r = rb * RPI + cp_rsub;
      const int id = uid(v * 32 + r);
      const size_t goff = (cb + id) * D + ((cp_piece ^ cswz<D>(r)) << 3);
      const uint16_t *src = (sp ? clo : chi) + goff;
      uint16_t *dst = &sA[b][sp][rb * RPI * D];
      __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void *)dst, 16, 0, 0);
    }
  };
  uint32_t ka[NS];
  const uint32_t sa0 = lds_offset(&sA[0][0][0]);
#pragma unroll
  for (int s = 0; s < NS; ++s) ka[s] = sa0 + col * D * 2 + (((2 * s + h) ^ cswz<D>(col)) << 4);
  const uint32_t na = lds_offset(&sN[0][0]) + 16 * h;

  // the error bound of this token's values (x row norm, slice max ||c||)
  float px = 0.f;
#pragma unroll
  for (int s = 0; s < NS; ++s) px = bf16x8_sumsq(xf[s], px);
  px += __shfl_xor(px, 32);
  const float nx = sqrtf(px) * (1.f + 0x1p-10f) + 0x1p-60f;
  const float e = 0x1p-25f * cm * cm + 0x1p-18f * nx * cm +
                  (2.f * D) * 0x1p-23f * (0.5f * cm * cm + 1.02f * nx * cm) +
                  0x1p-19f * (nx * cm + 0.5f * cm * cm);
  const float two_e = 2.f * 1.25f * e;

  // candidates: slots whose value reaches this lane half's best so far minus
  // 2E (a superset of those that reach the final best minus 2E, which hold
  // the argmin), kept in LDS for the first kMaskTiles virtual tiles
  float b1 = -INFINITY, b2 = -INFINITY, b3 = -INFINITY;
  int t1 = 0, t2 = 0;
  auto compute = [&](auto bufc, int v) {
    constexpr int B = decltype(bufc)::value;
    f32x4 n4[4];
    lds_read_f32x4x4<B * 256, 32>(n4, na);
    f32x16 acc;
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * g + j;
        acc[i] = v * 32 + acc_row(i, h) < nu ? n4[g][j] : -FLT_MAX;   // padding rows
      }
    bf16x8 af[NS];
    lds_read_frags<B * kBufB>(af, ka);
#pragma unroll
    for (int s = 0; s < NS; ++s) acc = mfma32x32x16(af[s], xf[s], acc);
    lds_read_frags<B * kBufB + kSplitB>(af, ka);
#pragma unroll
    for (int s = 0; s < NS; ++s) acc = mfma32x32x16(af[s], xf[s], acc);
    const float p1 = b1, p2 = b2;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float we = __int_as_float((__float_as_int(acc[i]) & ~15) | i);
      b3 = __builtin_amdgcn_fmed3f(b2, b3, we);
      b2 = __builtin_amdgcn_fmed3f(b1, b2, we);
      b1 = __builtin_elementwise_maximum(b1, we);
    }
    const bool new1 = b1 != p1;
    t2 = b2 == p2 ? t2 : ((new1 && b2 == p1) ? t1 : v);
    t1 = new1 ? v : t1;
    if (v < kMaskTiles) {   // uniform
      const float thr = b1 - two_e;
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) m |= acc[i] >= thr ? (1u << i) : 0u;
      sCm[v][wave * 32 + col][h] = static_cast<uint16_t>(m);
    }
  };

  issue(0, 0);
  if (nv > 1) issue(1, 1);
  for (int v = 0; v < nv; ++v) {
    // tile v has landed once only tile v+1's copies are outstanding (the token
    // rows, issued earlier, have landed too)
    if (v + 1 < nv) wait_vmcnt<CPW + 1>();
    else wait_vmcnt<0>();
    lds_barrier();
    if (v & 1) compute(std::integral_constant<int, 1>{}, v);
    else compute(std::integral_constant<int, 0>{}, v);
    if (v + 2 < nv) {
      lds_barrier();                                   // every wave is done with buffer v & 1
      issue(v + 2, v & 1);
    }
  }

  const int i1 = uid(t1 * 32 + acc_row(__float_as_int(b1) & 15, h));
  const int i2 = uid(t2 * 32 + acc_row(__float_as_int(b2) & 15, h));
  const float ob1 = __shfl_xor(b1, 32), ob2 = __shfl_xor(b2, 32), ob3 = __shfl_xor(b3, 32);
  const int oi1 = __shfl_xor(i1, 32), oi2 = __shfl_xor(i2, 32);
  const bool other = ob1 > b1 || (ob1 == b1 && oi1 < i1);
  const float nb1 = fmaxf(b1, ob1);
  const int ival = other ? oi1 : i1;
  const float lo1 = fminf(b1, ob1), hi2 = fmaxf(b2, ob2);
  const float nb2 = fmaxf(lo1, hi2);
  const int ival2 = lo1 >= hi2 ? (other ? i1 : oi1) : (b2 >= ob2 ? i2 : oi2);
  const float nb3 = fmaxf(fmaxf(fminf(b1, ob2), fminf(b2, ob1)), fmaxf(b3, ob3));
  const bool decided = nb1 - nb2 > two_e;
  const bool two = !decided && nb1 - nb3 > two_e;
  if (h == 0 && tv && decided) as[tok] = ival;
  const bool queued = h == 0 && tv && !decided && !two;
  const bool paired = h == 0 && tv && two;
  const uint64_t qm = __ballot(queued), pmk = __ballot(paired);
  if (lane == 0) {
    s_wq[wave] = __popcll(qm);
    s_wp[wave] = __popcll(pmk);
  }
  __syncthreads();
  int q = 0, pp = 0, nq = 0, np = 0;
#pragma unroll
  for (int w = 0; w < kCandWaves; ++w) {
    q += w < wave ? s_wq[w] : 0;
    pp += w < wave ? s_wp[w] : 0;
    nq += s_wq[w];
    np += s_wp[w];
  }
  const uint64_t lt = (1ull << lane) - 1;
  if (queued) sRow[q + __popcll(qm & lt)] = int2{tok, wave * 32 + col};
  if (paired) sRow[kCandTok - 1 - (pp + __popcll(pmk & lt))] = int2{tok, (ival << 16) | ival2};
  __syncthreads();

  // Settle the undecided rows exactly, in fp64: a pair row compares its two
  // clusters, a queued row the slots its masks kept (unions of up to
  // kMaskTiles tiles) or else every cluster of the union.  A group of 8 lanes
  // per row (D/8 dimensions per lane, each lane's terms added in ascending
  // order, the lanes in a fixed butterfly), four candidates loaded at a time;
  // the smallest distance wins, ties to the lowest id.
  constexpr int LPR = 8;                     // lanes per row
  constexpr int DPL = D / LPR;               // dimensions per lane (8 or 16)
  constexpr int XQ = DPL / 8;                // 16-byte pieces of x per lane
  constexpr int CQ = 2 * XQ;                 // 16-byte pieces of a centroid per lane
  constexpr int GPB = kThr / LPR;            // rows in flight per workgroup
  constexpr int U = 4;                       // candidates loaded at a time
  const int sub = tid % LPR, grp = tid / LPR;
  const float *cs = cent + static_cast<size_t>(bh) * c * D;
  for (int k = grp; k < nq + np; k += GPB) {   // uniform over the row's lanes
    const bool pair = k >= nq;
    const int2 e = pair ? sRow[kCandTok - 1 - (k - nq)] : sRow[k];
    const bool masked = !pair && nv <= kMaskTiles;
    // a queued row's full mask of tile t: the two halves' slots, slot i of
    // half hh being row acc_row(i, hh) of the tile
    auto tile_mask = [&](int t) {
      uint32_t m = 0;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const uint32_t mh = sCm[t][e.y][hh];
#pragma unroll
        for (int g = 0; g < 4; ++g) m |= ((mh >> (4 * g)) & 15u) << (8 * g + 4 * hh);
      }
      return m;
    };
    int nmask = 0;
    if (masked)
      for (int t = 0; t < nv; ++t) nmask += __popc(tile_mask(t));
    int cur_t = -1;
    uint32_t cur_m = 0;
    u32x4 xv[XQ];
#pragma unroll
    for (int i = 0; i < XQ; ++i)
      xv[i] = reinterpret_cast<const u32x4 *>(xb + static_cast<size_t>(e.x) * D)[sub * XQ + i];
    const int cnt = pair ? 2 : (masked ? nmask : nu);
    // called for j = 0, 1, 2, ... in order
    auto cand_id = [&](int j) {
      if (j >= cnt) return -1;
      if (pair) return j == 0 ? (e.y >> 16) & 0xffff : e.y & 0xffff;
      if (!masked) return uid(j);
      while (cur_m == 0) cur_m = tile_mask(++cur_t);   // j < cnt: a set bit remains
      const int b = __builtin_ctz(cur_m);
      cur_m &= cur_m - 1;
      return uid(cur_t * 32 + b);
    };
    double bd = INFINITY;
    int bi = 0x7fffffff;
    for (int j0 = 0; j0 < cnt; j0 += U) {
      int id[U];
      f32x4 cv[U][CQ];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        id[u] = cand_id(j0 + u);
        const f32x4 *cr = reinterpret_cast<const f32x4 *>(cs + static_cast<size_t>(id[u] >= 0 ? id[u] : 0) * D);
#pragma unroll
        for (int i = 0; i < CQ; ++i) cv[u][i] = cr[sub * CQ + i];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        double s2 = 0.0;
#pragma unroll
        for (int t = 0; t < DPL; ++t) {
          const float xf32 = bf16_bits_to_f32(static_cast<uint16_t>(xv[t >> 3][(t >> 1) & 3] >> (16 * (t & 1))));
          const float cf32 = cv[u][t >> 2][t & 3];
          const double df = static_cast<double>(xf32) - static_cast<double>(cf32);
          s2 = fma(df, df, s2);
        }
#pragma unroll
        for (int o = LPR / 2; o > 0; o >>= 1) s2 += __shfl_xor(s2, o);
        if (id[u] >= 0 && (s2 < bd || (s2 == bd && id[u] < bi))) {
          bd = s2;
          bi = id[u];
        }
      }
    }
    if (sub == 0) as[e.x] = bi;
  }
  if (n_refined != nullptr && tid == 0 && nq + np > 0) atomicAdd(n_refined, nq + np);
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
// WPC waves per cluster (1: four clusters per workgroup, for small clusters;
// 4: one cluster per workgroup, for large ones).  The cluster's rows are taken
// in batches of 64; wave w of the cluster takes batches w, w+WPC, ...  A row is
// read as TPR 16-byte pieces (one per lane) and lane group g of a wave takes
// rows g, g+RG, ... of each batch.  Each lane sums its rows in ascending
// order in fp64; lane groups and then waves are added in a fixed order, so
// the result does not depend on scheduling.
// ---------------------------------------------------------------------------
constexpr int kMeanWaves = 4;

template <int D, bool BF16, int WPC>
__global__ __launch_bounds__(64 * kMeanWaves) void km_mean_kernel(
    const void *__restrict__ x, int n, int c, int cpad, const int32_t *__restrict__ perm,
    const int32_t *__restrict__ offsets, float *__restrict__ cent, uint16_t *__restrict__ chi,
    uint16_t *__restrict__ clo, float *__restrict__ nh, float *__restrict__ rad, int mode,
    int ncl) {
  constexpr int EB = BF16 ? 2 : 4;           // element bytes
  constexpr int EPT = 16 / EB;               // elements per 16-byte piece
  constexpr int TPR = D / EPT;               // lanes per row
  constexpr int RG = 64 / TPR;               // row groups per wave
  constexpr int U = (64 / RG) < 8 ? (64 / RG) : 8;   // rows in flight per lane (8: more waves fit)
  static_assert(TPR <= 64 && 64 % TPR == 0 && (64 / RG) % U == 0, "row layout");
  static_assert(WPC == 1 || WPC == kMeanWaves, "waves per cluster");
  __shared__ double s_part[WPC > 1 ? WPC : 1][WPC > 1 ? D : 1];
  __shared__ float s_rmax[WPC > 1 ? WPC : 1][WPC > 1 ? TPR : 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wc = WPC > 1 ? wave : 0;         // this wave's rank within its cluster
  // slices in reverse launch order: the assign pass just before walked them in
  // ascending order, so the last ones it read are the likeliest still cached
  const int cl = WPC > 1 ? blockIdx.x : blockIdx.x * kMeanWaves + wave;
  const int bh = gridDim.y - 1 - blockIdx.y;
  if (cl >= ncl) return;                     // uniform over the cluster's waves
  const bool real = cl < c;
  const int g = lane / TPR, pc = lane % TPR;
  float val[EPT];                            // coordinates pc*EPT.. of the final centroid
  const size_t crow = (static_cast<size_t>(bh) * c + cl) * D + pc * EPT;
#pragma unroll
  for (int e = 0; e < EPT; ++e) val[e] = real ? cent[crow + e] : 0.f;
  // radius bound (bf16 inputs, mean + prep mode): R >= max ||x - c_new|| over
  // the cluster's rows, from the old centroid: ||x - c_new|| <= ||x - c_old|| +
  // ||c_old - c_new||.  Each lane keeps the largest sum over its EPT
  // coordinates of (x - c_old)^2 among its rows; the lanes' maxima added over
  // the TPR pieces of a row bound the largest row sum from above.
  const bool want_r = BF16 && rad != nullptr && mode == 1;
  float rmax = 0.f;
  if (mode != 0 && real) {
    const int st = offsets[static_cast<size_t>(bh) * (c + 1) + cl];
    const int en = offsets[static_cast<size_t>(bh) * (c + 1) + cl + 1];
    if (en > st) {                           // uniform over the cluster's waves
      float cold[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) cold[e] = val[e];
      double acc[EPT];
#pragma unroll
      for (int e = 0; e < EPT; ++e) acc[e] = 0.0;
      const int32_t *pm = perm + static_cast<size_t>(bh) * n;
      const char *xb = static_cast<const char *>(x) + static_cast<size_t>(bh) * n * D * EB;
      // lane j fetches the index of row r0 + j (the next batch's indices load
      // while this batch's rows are summed)
      int r0 = st + 64 * wc;
      int pidx = r0 + lane < en ? pm[r0 + lane] : -1;
      for (; r0 < en; r0 += 64 * WPC) {
        const int cur = pidx;
        const int rn = r0 + 64 * WPC + lane;
        pidx = rn < en ? pm[rn] : -1;
#pragma unroll
        for (int sb = 0; sb < 64 / RG; sb += U) {
          int pr[U];
          u32x4 buf[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            pr[u] = __shfl(cur, g + RG * (sb + u));
            buf[u] = pr[u] >= 0 ? *reinterpret_cast<const u32x4 *>(
                                      xb + (static_cast<size_t>(pr[u]) * D + pc * EPT) * EB)
                                : u32x4{0, 0, 0, 0};
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            if (pr[u] < 0) continue;
            float dd = 0.f;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
              float f;
              if constexpr (BF16) f = bf16_bits_to_f32(static_cast<uint16_t>(buf[u][e >> 1] >> (16 * (e & 1))));
              else f = __uint_as_float(buf[u][e]);
              acc[e] += static_cast<double>(f);
              const float t = f - cold[e];
              dd = fmaf(t, t, dd);
            }
            rmax = want_r ? fmaxf(rmax, dd) : rmax;
          }
        }
      }
      // combine the row groups (lanes TPR apart), then the cluster's waves
#pragma unroll
      for (int off = TPR; off < 64; off <<= 1)
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] += __shfl_xor(acc[e], off);
      if constexpr (WPC > 1) {
        if (g == 0) {
#pragma unroll
          for (int e = 0; e < EPT; ++e) s_part[wc][pc * EPT + e] = acc[e];
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          double t = s_part[0][pc * EPT + e];
#pragma unroll
          for (int w = 1; w < WPC; ++w) t += s_part[w][pc * EPT + e];
          acc[e] = t;
        }
      }
#pragma unroll
      for (int e = 0; e < EPT; ++e) val[e] = static_cast<float>(acc[e] / static_cast<double>(en - st));
      if (g == 0 && wc == 0) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) cent[crow + e] = val[e];
      }
      if (want_r) {
        // the piece's largest partial over the row groups, then the waves
#pragma unroll
        for (int off = TPR; off < 64; off <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, off));
        if constexpr (WPC > 1) {
          if (g == 0) s_rmax[wc][pc] = rmax;
          __syncthreads();
#pragma unroll
          for (int w = 0; w < WPC; ++w) rmax = fmaxf(rmax, s_rmax[w][pc]);
        }
        // sum over the pieces: R_old^2; and ||c_old - c_new||^2 likewise
        float dc = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
          const float t = cold[e] - val[e];
          dc = fmaf(t, t, dc);
        }
#pragma unroll
        for (int off = 1; off < TPR; off <<= 1) {
          rmax += __shfl_xor(rmax, off);
          dc += __shfl_xor(dc, off);
        }
        // fp32 roundings of the sums (under 2^-20 relative here) are covered
        // by the 2^-12 margins
        rmax = sqrtf(rmax * (1.f + 0x1p-12f)) + sqrtf(dc * (1.f + 0x1p-12f));
        rmax *= 1.f + 0x1p-12f;
      }
    }
  }
  if (want_r && lane == 0 && wc == 0 && cl < cpad)
    rad[static_cast<size_t>(bh) * cpad + cl] = rmax;
  if (mode == 2 || wc != 0) return;
  // prep for the next assignment (first wave of the cluster): hi/lo split,
  // -||c||^2/2
  double sq = 0.0;
  if (g == 0) {
    uint16_t hb[EPT], lb[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const __bf16 hi = static_cast<__bf16>(val[e]);
      const __bf16 lo = static_cast<__bf16>(val[e] - static_cast<float>(hi));
      hb[e] = __builtin_bit_cast(uint16_t, hi);
      lb[e] = __builtin_bit_cast(uint16_t, lo);
      sq += static_cast<double>(val[e]) * static_cast<double>(val[e]);
    }
    const size_t o = (static_cast<size_t>(bh) * cpad + cl) * D + pc * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      chi[o + e] = hb[e];
      clo[o + e] = lb[e];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
  // padding rows of the last tile start their w at -FLT_MAX: finite, so the
  // index bits the assign pass writes into w's mantissa never make a NaN
  if (lane == 0)
    nh[static_cast<size_t>(bh) * cpad + cl] = real ? static_cast<float>(-0.5 * sq) : -FLT_MAX;
}

template <int D>
hipError_t run_kmeans(const KmeansArgs &a, hipStream_t s) {
  const KmLayout L = km_layout(a.bh, a.n, a.d, a.c);
  char *w = static_cast<char *>(a.ws);
  uint16_t *chi = reinterpret_cast<uint16_t *>(w + L.chi);
  uint16_t *clo = reinterpret_cast<uint16_t *>(w + L.clo);
  float *nh = reinterpret_cast<float *>(w + L.nh);
  int32_t *ctl = reinterpret_cast<int32_t *>(w + L.ctl);   // [bh] refine-queue lengths
  int2 *flags = reinterpret_cast<int2 *>(w + L.flags);
  int2 *tflags = reinterpret_cast<int2 *>(w + L.tflags);
  int32_t *tcount = reinterpret_cast<int32_t *>(w + L.tcount);
  int32_t *pcount = reinterpret_cast<int32_t *>(w + L.pcount);
  int32_t *perm = reinterpret_cast<int32_t *>(w + L.perm);
  int32_t *seg = reinterpret_cast<int32_t *>(w + L.seg);
  int32_t *offsets = reinterpret_cast<int32_t *>(w + L.offsets);
  float *rad = reinterpret_cast<float *>(w + L.rad);
  uint32_t *nbr = reinterpret_cast<uint32_t *>(w + L.nbr);
  uint32_t *tun = reinterpret_cast<uint32_t *>(w + L.tun);
  // the candidate path for tables too large for the resident pass
  const bool cand_ok = a.c <= kNbrMaxC && (a.c + 31) / 32 > kResTiles;
  void *sort_ws = w + L.sort;
  const int cpad = (a.c + 31) / 32 * 32;
  const bool bf16 = a.dtype == SVA_BF16;
  const int tph = (a.n + kTokTile - 1) / kTokTile;
  const dim3 tok_grid(8 * tph * ((a.bh + 7) / 8));
  // candidate path: 256 sorted positions per workgroup, slices dealt to XCDs
  const int ctph = (a.n + kCandTok - 1) / kCandTok;
  const dim3 cand_grid(8 * ctph * ((a.bh + 7) / 8));
  hipError_t e;
#define SVA_CHECK(x)               \
  do {                             \
    e = (x);                       \
    if (e != hipSuccess) return e; \
  } while (0)

  // up to kResTiles centroid tiles: the resident-table main pass, one
  // workgroup per compute unit (at least one per slice), 64-token tiles
  const bool resident = cpad <= kResTiles * 32;
  const int rtph = (a.n + kResTok - 1) / kResTok;
  const long long rtiles = static_cast<long long>(a.bh) * rtph;
  const int rgrid = static_cast<int>(std::max<long long>(
      a.bh, std::min<long long>(device_cus(), (rtiles + kResWaves - 1) / kResWaves)));
#define SVA_RES(NTL)                                                                          \
  hipLaunchKernelGGL((km_assign_res_kernel<D, NTL>), dim3(rgrid), dim3(64 * kResWaves), 0, s, \
                     static_cast<const uint16_t *>(a.x), a.n, a.c, cpad, chi, clo, nh,        \
                     a.assign, tflags, tcount, a.bh, rtph)

  // clusters of 256 rows or more on average get four waves each
  const bool wide = a.n >= 256LL * a.c;
  auto mean = [&](int mode) -> hipError_t {
    const int ncl = mode == 2 ? a.c : cpad;
    const dim3 grid(wide ? ncl : (ncl + kMeanWaves - 1) / kMeanWaves, a.bh);
    const dim3 block(64 * kMeanWaves);
#define SVA_MEAN(B, W)                                                                       \
  hipLaunchKernelGGL((km_mean_kernel<D, B, W>), grid, block, 0, s, a.x, a.n, a.c, cpad, perm, \
                     offsets, a.centroids, chi, clo, nh, cand_ok ? rad : nullptr, mode, ncl)
    if (bf16) {
      if (wide) SVA_MEAN(true, kMeanWaves);
      else SVA_MEAN(true, 1);
    } else {
      if (wide) SVA_MEAN(false, kMeanWaves);
      else SVA_MEAN(false, 1);
    }
#undef SVA_MEAN
    return hipGetLastError();
  };

  if (bf16) {
    SVA_CHECK(launch_fill_i32(ctl, 0, static_cast<size_t>(a.bh), s));
    SVA_CHECK(mean(0));
  }
  for (int it = 0; it < a.iters; ++it) {
    const bool last = it + 1 == a.iters;
    if (bf16 && it > 0 && cand_ok) {
      // the tiles' unions of candidates (neighbour rows built after the
      // previous iteration's mean pass), the assignment over them, then the
      // undecided rows in fp64
      hipLaunchKernelGGL(km_tile_union_kernel, dim3(ctph, a.bh), dim3(64), 0, s, seg, nbr, a.n,
                         a.c, cpad, ctph, tun);
      SVA_CHECK(hipGetLastError());
#define SVA_CAND(MT)                                                                         \
  hipLaunchKernelGGL((km_assign_cand_kernel<D, MT>), cand_grid, dim3(64 * kCandWaves), 0, s,  \
                     static_cast<const uint16_t *>(a.x), a.n, a.c, cpad, chi, clo, nh,        \
                     a.centroids, perm, tun, a.assign, a.n_refined, a.bh, ctph)
      if (cpad / 32 > kMaskTilesSmall) SVA_CAND(kMaskTilesLarge);
      else SVA_CAND(kMaskTilesSmall);
#undef SVA_CAND
      SVA_CHECK(hipGetLastError());
    } else if (bf16) {
      // the pair path (third best tracked) pays once the refine's re-scan is
      // long: with 16 or more centroid tiles (measured break-even between 13 and 16)
      const bool pairs = cpad >= 16 * 32;
      if (resident) {
        switch (cpad / 32) {
          case 1: SVA_RES(1); break;
          case 2: SVA_RES(2); break;
          case 3: SVA_RES(3); break;
          default: SVA_RES(4); break;
        }
      } else if (pairs)
        hipLaunchKernelGGL((km_assign_main_kernel<D, true>), tok_grid, dim3(kThreads), 0, s,
                           static_cast<const uint16_t *>(a.x), a.n, a.c, cpad, chi, clo, nh,
                           a.assign, tflags, tcount, pcount, a.bh, tph);
      else
        hipLaunchKernelGGL((km_assign_main_kernel<D, false>), tok_grid, dim3(kThreads), 0, s,
                           static_cast<const uint16_t *>(a.x), a.n, a.c, cpad, chi, clo, nh,
                           a.assign, tflags, tcount, pcount, a.bh, tph);
      SVA_CHECK(hipGetLastError());
      if (pairs)
        hipLaunchKernelGGL((km_pair_kernel<D>), tok_grid, dim3(kThreads), 0, s,
                           static_cast<const uint16_t *>(a.x), a.n, a.c, a.centroids, tflags,
                           pcount, a.assign, a.n_refined, a.bh, tph);
      SVA_CHECK(hipGetLastError());
      const int jt = resident ? rtph : tph;
      hipLaunchKernelGGL(km_queue_join_kernel, dim3((jt + kJoinTiles - 1) / kJoinTiles, a.bh),
                         dim3(kThreads), 0, s, tflags, tcount, a.n, jt,
                         resident ? kResTok : kTokTile, flags, ctl);
      SVA_CHECK(hipGetLastError());
      hipLaunchKernelGGL((km_refine_kernel<D>), tok_grid, dim3(kThreads), 0, s,
                         static_cast<const uint16_t *>(a.x), a.n, a.c, cpad, chi, clo, nh, ctl,
                         a.centroids, a.assign, flags, a.n_refined, a.bh, tph);
      SVA_CHECK(hipGetLastError());
    } else {
      hipLaunchKernelGGL((km_assign_f64_kernel<D>), dim3((a.n + kThreads - 1) / kThreads, a.bh),
                         dim3(kThreads), 0, s, static_cast<const float *>(a.x), a.n, a.c,
                         a.centroids, a.assign);
      SVA_CHECK(hipGetLastError());
    }
    // the sort's scan clears the per-slice queue lengths for the next iteration
    SVA_CHECK(launch_cluster_sort(a.assign, a.bh, a.n, a.c, perm, offsets,
                                  last ? a.sizes : nullptr, sort_ws, s, bf16 ? ctl : nullptr,
                                  (bf16 && !last && cand_ok) ? seg : nullptr));
    SVA_CHECK(mean((bf16 && !last) ? 1 : 2));
    if (bf16 && !last && cand_ok) {
      hipLaunchKernelGGL((km_nbr_kernel<D>),
                         dim3((cpad / 32 + kNbrWaves - 1) / kNbrWaves,
                              (cpad / 32 + kNbrJt - 1) / kNbrJt, a.bh),
                         dim3(64 * kNbrWaves), 0, s, chi, clo, nh, rad, a.c, cpad, nbr);
      SVA_CHECK(hipGetLastError());
    }
  }
#undef SVA_CHECK
#undef SVA_RES
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Spread of a clustering, per slice: J = sum over rows of ||x - c_assign||^2
// (the k-means objective) and the scatter T = sum over rows of ||x - mean||^2,
// T taken as sum ||x||^2 - ||sum x||^2 / n.  One workgroup per slice; D/EPT
// lanes per row (EPT elements each); every lane accumulates its rows in fp64 in
// ascending order, and lanes, row groups and waves are combined in a fixed
// order, so the result is deterministic.
// ---------------------------------------------------------------------------
template <int D, bool BF16>
__global__ __launch_bounds__(kThreads) void km_spread_kernel(
    const void *__restrict__ x, int n, int c, const float *__restrict__ cent,
    const int32_t *__restrict__ assign, double *__restrict__ out) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int EPT = 16 / EB;               // elements per 16-byte piece
  constexpr int TPR = D / EPT;               // lanes per row
  constexpr int RPB = kThreads / TPR;        // rows per workgroup pass
  __shared__ double s_sum[RPB][D];
  __shared__ double s_jq[kThreads];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int pc = tid % TPR, rg = tid / TPR;
  const char *xb = static_cast<const char *>(x) + static_cast<size_t>(bh) * n * D * EB;
  const int32_t *as = assign + static_cast<size_t>(bh) * n;
  const float *cs = cent + static_cast<size_t>(bh) * c * D;
  double sx[EPT], j = 0.0, q = 0.0;
#pragma unroll
  for (int e = 0; e < EPT; ++e) sx[e] = 0.0;
  for (int r = rg; r < n; r += RPB) {
    const u32x4 v = *reinterpret_cast<const u32x4 *>(xb + (static_cast<size_t>(r) * D + pc * EPT) * EB);
    const int a = min(max(as[r], 0), c - 1);
    const float *cr = cs + static_cast<size_t>(a) * D + pc * EPT;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      float f;
      if constexpr (BF16) f = bf16_bits_to_f32(static_cast<uint16_t>(v[e >> 1] >> (16 * (e & 1))));
      else f = __uint_as_float(v[e]);
      const double df = static_cast<double>(f) - static_cast<double>(cr[e]);
      j = fma(df, df, j);
      q = fma(static_cast<double>(f), static_cast<double>(f), q);
      sx[e] += static_cast<double>(f);
    }
  }
#pragma unroll
  for (int e = 0; e < EPT; ++e) s_sum[rg][pc * EPT + e] = sx[e];
  s_jq[tid] = j;
  __syncthreads();
  // J: fixed-order sum over threads; sum ||x||^2 likewise; ||sum x||^2 from the
  // row groups' partial sums, added in order per dimension
  double jt = 0.0, qt = 0.0, s2 = 0.0;
  if (tid == 0) {
    for (int t = 0; t < kThreads; ++t) jt += s_jq[t];
  }
  __syncthreads();
  s_jq[tid] = q;
  __syncthreads();
  if (tid == 0) {
    for (int t = 0; t < kThreads; ++t) qt += s_jq[t];
    for (int dd = 0; dd < D; ++dd) {
      double col = 0.0;
      for (int g = 0; g < RPB; ++g) col += s_sum[g][dd];
      s2 += col * col;
    }
    out[2 * bh] = jt;
    out[2 * bh + 1] = qt - s2 / static_cast<double>(n);
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// The arithmetic the assign pass's error bound relies on: the 32x32x16 bf16
// MFMA accumulates with a 24-bit significand and each addition loses at most
// one unit in the last place.  One wave evaluates D = C + A.B with B all
// ones, so row r of D is C[r] + the sum of row r of A (products at k = 0, 5,
// 11).  Cases 0-3 have every partial sum exact in fp32, in any order, so
// they must come out exact; cases 4-7 need rounding and must land within one
// unit per addition of the exact value (both round-to-nearest and
// truncating results pass).  Case r's flag is 1 when it holds.
// ---------------------------------------------------------------------------
namespace {
__global__ __launch_bounds__(64) void km_mfma_rounding_kernel(int32_t *__restrict__ flags) {
  const int lane = threadIdx.x, h = lane >> 5, col = lane & 31;
  const float p23 = 0x1p23f, p24 = 0x1p24f, p25 = 0x1p25f;
  // per case: the seed C, three products (A entries), the exact result and
  // the allowed error (one unit in the last place per addition: 2 below 2^25,
  // 4 below 2^26; three additions)
  const float seed[kMfmaChecks] = {0.f, p23, -p23, 0.f, p24 + 2.f, p24, -p25, 0.f};
  const float prod[kMfmaChecks][3] = {{p23, 1.f, -p23}, {1.f, -p23, 0.f}, {p23, 1.f, 0.f},
                                      {1.f, p23, -p23}, {1.f, 0.f, 0.f},  {1.f, 1.f, 0.f},
                                      {p25, 3.f, 0.f},  {p25, 3.f, -p25}};
  const float exact[kMfmaChecks] = {1.f, 1.f, 1.f, 1.f, p24 + 3.f, p24 + 2.f, 3.f, 3.f};
  const float tol[kMfmaChecks] = {0.f, 0.f, 0.f, 0.f, 2.f * 3.f, 2.f * 3.f, 4.f * 3.f, 4.f * 3.f};
  // A fragment of this lane: row col, k = 8h .. 8h+7 (products in k = 0, 5, 11)
  bf16x8 a;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int k = 8 * h + j;
    const float v = col < kMfmaChecks ? (k == 0 ? prod[col][0] : k == 5 ? prod[col][1]
                                         : k == 11 ? prod[col][2] : 0.f) : 0.f;
    a[j] = static_cast<__bf16>(v);   // every product above is exact in bf16
  }
  bf16x8 b;
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = static_cast<__bf16>(1.f);
  f32x16 c;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = acc_row(i, h);
    c[i] = row < kMfmaChecks ? seed[row] : 0.f;
  }
  const f32x16 d = mfma32x32x16(a, b, c);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int row = acc_row(i, h);
    if (col == 0 && row < kMfmaChecks)
      flags[row] = fabsf(d[i] - exact[row]) <= tol[row] ? 1 : 0;
  }
}
}  // namespace

hipError_t launch_mfma_rounding_check(int32_t *flags, hipStream_t s) {
  hipLaunchKernelGGL(km_mfma_rounding_kernel, dim3(1), dim3(64), 0, s, flags);
  return hipGetLastError();
}

hipError_t launch_cluster_spread(const void *x, int32_t dtype, int32_t bh, int32_t n, int32_t d,
                                 int32_t c, const float *cent, const int32_t *assign,
                                 double *out, hipStream_t s) {
#define SVA_SPREAD(DD, B)                                                                     \
  hipLaunchKernelGGL((km_spread_kernel<DD, B>), dim3(bh), dim3(kThreads), 0, s, x, n, c, cent, \
                     assign, out)
  const bool b = dtype == SVA_BF16;
  if (d == 128) {
    if (b) SVA_SPREAD(128, true);
    else SVA_SPREAD(128, false);
  } else {
    if (b) SVA_SPREAD(64, true);
    else SVA_SPREAD(64, false);
  }
#undef SVA_SPREAD
  return hipGetLastError();
}

size_t kmeans_ws_bytes(int32_t bh, int32_t n, int32_t d, int32_t c) {
  return km_layout(bh, n, d, c).total;
}

hipError_t launch_kmeans(const KmeansArgs &a, hipStream_t s) {
  return a.d == 128 ? run_kmeans<128>(a, s) : run_kmeans<64>(a, s);
}

}  // namespace sva
