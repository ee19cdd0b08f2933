// Block-sparse and dense softmax attention for gfx950.
//
// Sparse VideoGen2 (explainer of arXiv 2505.18875, technical summary section
// 2.c, "customized attention kernel"): query blocks are contiguous clusters
// that are computed densely, the kept key/value clusters are gathered, and
// block sizes are dynamic, so no tile is padded to a fixed block size.
//
// Design (bf16 path):
// * A work item is up to 256 query rows of one Q block; a workgroup of 8 waves
//   takes it, each wave owning 32 query rows held in registers as the B
//   operand of S^T = K Q^T (32x32x16 bf16 MFMA).  With keys on the
//   accumulator rows and queries on lanes, every row max / row sum of the
//   online softmax is in-lane plus one exchange between the two lane halves.
// * The kept K blocks of the Q block form one virtual key sequence (their
//   row ranges concatenated); it is walked in chunks of 64 keys, so a chunk
//   may span several small clusters and only the very last chunk is partial.
//   The key row behind each virtual key comes from row-map windows of 16
//   chunks built by all threads at once in LDS.
// * A chunk's K and V rows go from HBM straight to LDS (global_load_lds,
//   16 bytes per lane, no staging registers), row-major with the 16-byte
//   pieces XOR-swizzled (K and V differently, each for its read pattern);
//   each lane picks the global piece that belongs in its LDS slot.  S^T MFMA
//   operands are conflict-free ds_read_b128 of K; the PV operand V^T comes
//   from two ds_read_b64_tr_b16 transposing reads, which hand each lane 4
//   keys of one d in exactly the key order of P^T.
// * Four LDS stages per tensor: chunks c+1 and c+2 are in flight while chunk
//   c is computed and chunk c-1's V is still read (below); one partial
//   s_waitcnt + one barrier per chunk.
// * Ping-pong: the two waves sharing a SIMD (w and w+4) run the same
//   per-chunk sequence rotated by one phase -- PV(c-1), QK(c), softmax(c)
//   against softmax(c-1), PV(c-1), QK(c) -- so one is in its MFMA phase while
//   the other runs VALU work.
// * Online softmax with a lazy rescale: the row max is taken on the first
//   chunk of a kept-list segment; after that the exponentials are taken
//   against the running max directly, and only when a lane's sum of P shows
//   some P above 2^8 is the chunk's max taken, O rescaled and the chunk
//   redone.  So P <= 32 * 2^8 and the max reduction leaves the common step.
//   P is rounded to bf16 for the PV MFMA; max, sum and O accumulate in fp32.
// * Sparse mode: one persistent workgroup per compute unit takes items from
//   per-XCD queues (slices dealt to XCDs by total cost, each XCD working
//   through its slices one at a time, longest item first within a slice) and
//   steals from the other queues when its own is empty.  Dense mode: one
//   workgroup per item, laid out so consecutive items of a head run on one
//   XCD (workgroups are dispatched round-robin over the 8 XCDs).
// * Fused permutation (PERM): Q rows, K/V rows and O/LSE rows go through the
//   permutations, so no permuted copy of any tensor is materialised.
//
// The fp32 path is a plain one-thread-per-query kernel (exact fp32, used for
// small correctness workloads).
#include <math.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "../../include/sva.h"
#include "sva_internal.h"
#include "lds_pipe.h"

namespace sva {
namespace {

constexpr int kThreads = 256;       // helper kernels
constexpr int kQTile = 256;        // query rows per work item (and per fp32 workgroup)
// bf16 attention waves per workgroup; each wave owns kQTile / waves query rows
// in 32-row MFMA tiles
template <int D>
constexpr int attn_waves() { return 8; }
constexpr int kKT = 64;           // keys per chunk
constexpr int kStages = 4;        // K/V chunk buffers in LDS (two in flight, two in use)
constexpr int kLCap = 1024;       // kept-list entries staged in LDS at a time
constexpr int kWin = 32;          // chunks per row-map window
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

struct WorkItem {
  int32_t bh, qb, row0, cost;   // cost: 64-key chunks of the item + kItemFixed
};
constexpr int kItemFixed = 3;          // per-item setup/epilogue cost, in chunk units
constexpr int kOrderThreads = 1024;    // the single workgroup that orders the work
constexpr int kOrderBuckets = 1024;    // cost buckets of the ordering sort
constexpr int kMaxOrderHeads = 4096;   // slices balanced over XCDs (more: slice % 8)

// Schedule scratch inside the attention workspace
struct SchedLayout {
  size_t items, qcost, hinfo, lists, ctl, total;
};
inline SchedLayout sched_layout(int32_t bh, int32_t n_q, int32_t nqb) {
  const size_t cap = static_cast<size_t>((n_q + kQTile - 1) / kQTile) + nqb;
  SchedLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align_up(bytes, 256);
    return at;
  };
  L.items = take(static_cast<size_t>(bh) * cap * sizeof(WorkItem));   // [bh][cap], per slice
  L.qcost = take(static_cast<size_t>(bh) * nqb * 4);                  // [bh][nqb] chunk cost
  L.hinfo = take(static_cast<size_t>(bh) * 2 * 4);                    // [bh] cost sum, items
  L.lists = take(static_cast<size_t>(bh) * cap * sizeof(WorkItem));   // per-XCD ordered lists
  L.ctl = take(32 * 4);                                               // count[8] start[8] ctr[8]
  L.total = off;
  return L;
}

// XOR swizzle of the 16-byte pieces of K row r (rows of 256 B for d=128,
// 128 B for d=64): the ds_read_b128 of an S^T operand has 16 lanes on 16
// consecutive rows at one logical piece, which this spreads over all banks.
template <int D>
__host__ __device__ constexpr int kswz(int r) {
  return D == 128 ? (r & 15) : ((r >> 1) & 7);
}

// XOR swizzle of V rows.  A ds_read_b64_tr_b16 of the PV operand has, per 32
// lanes, 4 consecutive rows x 4 logical pieces x 2 halves; moving row r's
// pieces by 4 * (r % 4) (d=128) puts the 4 rows in disjoint quarters of the
// bank space, so the 32 lanes hit 64 distinct banks.  For d=64 two rows share
// one 256-byte bank line, so the shift follows (r / 2) % 2.
template <int D>
__host__ __device__ constexpr int vswz(int r) {
  return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
}


// In-place exclusive scan of a[0..n) (n <= 4*NTHREADS) held in LDS; writes
// the total to a[n].  Must be called by all NTHREADS threads of the workgroup.
template <int NTHREADS>
__device__ void block_exclusive_scan(int32_t *a, int n, int32_t *wsum) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int v[4];
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = (4 * t + i < n) ? a[4 * t + i] : 0;
    s += v[i];
  }
  int x = s;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += wsum[w];
  int run = pre + x - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * t + i < n) a[4 * t + i] = run;
    run += v[i];
  }
  if (t == NTHREADS - 1) a[n] = run;
  __syncthreads();
}

__device__ __forceinline__ bool decode_work(const WorkItem *work, int work_cap, int n_items,
                                            int dense, int &bh, int &qb, int &row0) {
  const int nblk = gridDim.x;   // a multiple of 8
  const int w = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  if (w >= n_items) return false;
  bh = w / work_cap;
  const int slot = w - bh * work_cap;
  if (dense) {
    qb = 0;
    row0 = slot * kQTile;
    return true;
  }
  const WorkItem it = work[w];
  qb = it.qb;
  row0 = it.row0;
  return qb >= 0;
}

// Next item of a persistent workgroup (thread 0 only): the queue of the
// workgroup's XCD first, then the others (work stealing); -1 when all are
// drained.  `gone` remembers queues this workgroup found empty.
__device__ __forceinline__ int fetch_work(int32_t *ctl, int &gone) {
  const int x0 = blockIdx.x & 7;
  for (int k = 0; k < 8; ++k) {
    const int y = (x0 + k) & 7;
    if (gone & (1 << y)) continue;
    const int i = atomicAdd(&ctl[16 + y], 1);
    if (i < ctl[y]) return ctl[8 + y] + i;
    gone |= 1 << y;
  }
  return -1;
}

// ---------------------------------------------------------------------------
// schedule, sparse mode
//   cost:  one wave per Q block adds up its kept clusters' sizes L; the cost of
//          each 256-row tile of the block is ceil(L / 64) chunks + kItemFixed
//   items: per slice, one item per tile, in block order (the fp32 kernel walks
//          these directly); plus the slice's cost sum and item count
//   order: one workgroup deals slices to the 8 XCDs (largest first, each to
//          the least loaded); each XCD's queue holds its slices one after
//          another in the order they were dealt, every slice's items by
//          descending cost.  The XCD's compute units then work on one slice
//          at a time, so that slice's K/V (16.8 MB at 32,760 tokens, d = 128)
//          stays in the memory-side cache while its items run instead of
//          competing with the K/V of every other slice of the XCD; the last
//          slices still end longest processing time first.  The bf16 kernel's
//          persistent workgroups take items from these queues and steal from
//          other XCDs' queues when their own is empty
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void attn_cost_kernel(
    const int32_t *__restrict__ k_off, const int32_t *__restrict__ kept_count,
    const int32_t *__restrict__ kept_idx, int kept_stride, int nqb, int nkb,
    int32_t *__restrict__ qcost) {
  const int lane = threadIdx.x & 63;
  const int qb = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6), bh = blockIdx.y;
  if (qb >= nqb) return;                       // wave-uniform; no barriers here
  const size_t e = static_cast<size_t>(bh) * nqb + qb;
  const int kc = kept_count[e];
  const int32_t *kidx = kept_idx + e * kept_stride;
  const int32_t *koff = k_off + static_cast<size_t>(bh) * (nkb + 1);
  int L = 0;
  for (int j = lane; j < kc; j += 64) {
    const int b = kidx[j];
    L += koff[b + 1] - koff[b];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off);
  L = max(L, 0);   // offsets that break monotonicity never give a negative cost
  if (lane == 0) qcost[e] = (L + kKT - 1) / kKT + kItemFixed;
}

__global__ __launch_bounds__(kThreads) void attn_schedule_kernel(
    const int32_t *__restrict__ q_off, const int32_t *__restrict__ qcost, int nqb,
    int work_cap, int split, WorkItem *__restrict__ work, int32_t *__restrict__ hinfo) {
  __shared__ int32_t wsum[4];
  __shared__ int32_t csum[4];
  const int bh = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int32_t *off = q_off + static_cast<size_t>(bh) * (nqb + 1);
  WorkItem *out = work + static_cast<size_t>(bh) * work_cap;
  int base = 0, cost_sum = 0;
  for (int b0 = 0; b0 < nqb; b0 += kThreads) {
    const int qb = b0 + t;
    int tiles = 0, cost = 0, rows = 0;
    if (qb < nqb) {
      rows = max(0, off[qb + 1] - off[qb]);
      tiles = (rows + kQTile - 1) / kQTile;
      cost = qcost[static_cast<size_t>(bh) * nqb + qb];
    }
    // (split mode) a last item of at most half a tile takes about half the
    // chunk time
    const int rem = rows - (tiles - 1) * kQTile;
    const int cost_last = split && tiles > 0 && rem <= kQTile / 2
                              ? (cost - kItemFixed + 1) / 2 + kItemFixed
                              : cost;
    int x = tiles, cs = tiles > 0 ? (tiles - 1) * cost + cost_last : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) cs += __shfl_xor(cs, o);
    if (lane == 63) wsum[wave] = x;
    if (lane == 0) csum[wave] = cs;
    __syncthreads();
    int pre = 0, total = 0;
    for (int w = 0; w < 4; ++w) {
      if (w < wave) pre += wsum[w];
      total += wsum[w];
      cost_sum += t == 0 ? csum[w] : 0;
    }
    const int first = base + pre + x - tiles;
    for (int i = 0; i < tiles; ++i)
      if (first + i < work_cap)
        out[first + i] = WorkItem{bh, qb, i * kQTile, i == tiles - 1 ? cost_last : cost};
    base += total;
    __syncthreads();
  }
  for (int i = base + t; i < work_cap; i += kThreads) out[i] = WorkItem{bh, -1, -1, 0};
  if (t == 0) {
    hinfo[2 * bh] = cost_sum;
    hinfo[2 * bh + 1] = min(base, work_cap);
  }
}

__global__ __launch_bounds__(kOrderThreads) void attn_order_kernel(
    const WorkItem *__restrict__ work, const int32_t *__restrict__ hinfo, int nbh, int work_cap,
    WorkItem *__restrict__ lists, int32_t *__restrict__ ctl) {
  __shared__ int32_t s_x[kMaxOrderHeads];            // XCD of each slice
  __shared__ int32_t s_order[kMaxOrderHeads];        // slices by descending cost
  __shared__ int32_t s_hist[8][kOrderBuckets];       // counts, then write cursors
  __shared__ int32_t s_rank[kMaxOrderHeads];         // position among its XCD's slices
  __shared__ int32_t s_cost[kMaxOrderHeads];         // cost of each slice, by rank
  __shared__ int32_t s_cnt[8], s_start[8];
  __shared__ int32_t s_group;                        // slices per sort group
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const bool balance = nbh <= kMaxOrderHeads;
  auto xcd_of = [&](int h) { return balance ? s_x[h] : (h & 7); };
  // sort key, ascending = earlier in the queue: the slice's group (up to 8
  // groups of consecutive ranks), then the cost, descending, in kOrderBuckets/8
  // buckets (exact below 3/4 of them, then 16 chunks per bucket)
  constexpr int kCB = kOrderBuckets / 8, kExact = kCB * 3 / 4;
  auto key = [&](const WorkItem &it) {
    if (!balance) return kOrderBuckets - 1 - min(it.cost, kOrderBuckets - 1);
    const int c = it.cost < kExact ? it.cost : min(kExact + (it.cost - kExact) / 16, kCB - 1);
    return (s_rank[it.bh] / s_group) * kCB + (kCB - 1 - c);
  };
  for (int i = t; i < 8 * kOrderBuckets; i += kOrderThreads) (&s_hist[0][0])[i] = 0;
  if (balance) {
    // rank of each slice by (cost desc, index asc), then a greedy deal; the
    // costs are staged in LDS first (s_x, rewritten by the deal)
    for (int h = t; h < nbh; h += kOrderThreads) s_x[h] = hinfo[2 * h];
    __syncthreads();
    for (int h = t; h < nbh; h += kOrderThreads) {
      const int ch = s_x[h];
      int r = 0;
      for (int g = 0; g < nbh; ++g) {
        const int cg = s_x[g];
        r += (cg > ch || (cg == ch && g < h)) ? 1 : 0;
      }
      s_order[r] = h;
      s_cost[r] = ch;
    }
    __syncthreads();
    if (t == 0) {   // (serial, so it reads LDS only)
      long long load[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      int dealt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int r = 0; r < nbh; ++r) {
        const int h = s_order[r];
        int best = 0;
        for (int x = 1; x < 8; ++x) best = load[x] < load[best] ? x : best;
        s_x[h] = best;
        s_rank[h] = dealt[best]++;
        load[best] += s_cost[r];
      }
      int most = 1;
      for (int x = 0; x < 8; ++x) most = max(most, dealt[x]);
      s_group = (most + 7) / 8;
    }
  }
  __syncthreads();
  // histogram of the item keys per XCD; the first kHeld items of each thread
  // stay in registers for the scatter below
  const size_t total = static_cast<size_t>(nbh) * work_cap;
  constexpr int kHeld = 16;
  WorkItem held[kHeld];
#pragma unroll
  for (int u = 0; u < kHeld; ++u) {
    const size_t i = t + static_cast<size_t>(u) * kOrderThreads;
    held[u] = i < total ? work[i] : WorkItem{0, -1, -1, 0};
  }
#pragma unroll
  for (int u = 0; u < kHeld; ++u)
    if (held[u].qb >= 0) atomicAdd(&s_hist[xcd_of(held[u].bh)][key(held[u])], 1);
  for (size_t i = t + static_cast<size_t>(kHeld) * kOrderThreads; i < total; i += kOrderThreads) {
    const WorkItem it = work[i];
    if (it.qb < 0) continue;
    atomicAdd(&s_hist[xcd_of(it.bh)][key(it)], 1);
  }
  __syncthreads();
  // per XCD, exclusive scan in key order (wave x scans XCD x)
  if (wave < 8) {
    constexpr int PER = kOrderBuckets / 64;
    int v[PER], sum = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {           // the lane's buckets
      v[j] = s_hist[wave][lane * PER + j];
      sum += v[j];
    }
    int x = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    int run = x - sum;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      s_hist[wave][lane * PER + j] = run;
      run += v[j];
    }
    if (lane == 63) s_cnt[wave] = x;
  }
  __syncthreads();
  if (t == 0) {
    int st = 0;
    for (int x = 0; x < 8; ++x) {
      s_start[x] = st;
      st += s_cnt[x];
    }
  }
  __syncthreads();
  auto place = [&](const WorkItem &it) {
    const int x = xcd_of(it.bh);
    const int pos = atomicAdd(&s_hist[x][key(it)], 1);
    lists[s_start[x] + pos] = it;
  };
#pragma unroll
  for (int u = 0; u < kHeld; ++u)
    if (held[u].qb >= 0) place(held[u]);
  for (size_t i = t + static_cast<size_t>(kHeld) * kOrderThreads; i < total; i += kOrderThreads) {
    const WorkItem it = work[i];
    if (it.qb >= 0) place(it);
  }
  if (t < 8) {
    ctl[t] = s_cnt[t];
    ctl[8 + t] = s_start[t];
    ctl[16 + t] = 0;
  }
}

// ---------------------------------------------------------------------------
// bf16 MFMA attention
// ---------------------------------------------------------------------------
template <int D, bool OUT_F32, bool PERM, int W, bool SPLIT>
__global__ __launch_bounds__(64 * W, 1) void attn_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, void *__restrict__ o, float *__restrict__ lse,
    const int32_t *__restrict__ q_perm, const int32_t *__restrict__ k_perm,
    const int32_t *__restrict__ q_off, const int32_t *__restrict__ k_off,
    const int32_t *__restrict__ kept_count, const int32_t *__restrict__ kept_idx,
    int kept_stride, const WorkItem *__restrict__ work, int work_cap, int n_items,
    const WorkItem *__restrict__ lists, int32_t *__restrict__ ctl, int n_q, int n_k, int nqb,
    int nkb, int dense, float scale_log2) {
  constexpr int PPR = D / 8;             // 16-byte pieces per row
  constexpr int RPI = 64 / PPR;          // rows per 1 KB direct-to-LDS wave load
  constexpr int kThr = 64 * W;
  // The K/V copies of a chunk are issued by waves CW .. W-1, LPC 1 KB loads per
  // tensor each: with the fused permutation the late waves (which start each
  // step with VALU work) issue them all, in the other instantiations every
  // wave takes a share (measured: the late-wave split is 1% faster on the
  // former and 7-8% slower on the others)
  constexpr int CW = PERM ? W / 2 : 0;   // first copying wave
  constexpr int LPC = PPR / (W - CW);    // loads per copying wave per tensor per chunk
  static_assert(LPC >= 1 && PPR % (W - CW) == 0 && 2 * LPC < 16,
                "copying waves take whole 1 KB pieces");
  constexpr int NS = D / 16;             // k-steps of the S MFMA
  constexpr int ND = D / 32;             // d tiles of the O accumulator
  constexpr int kWaveRows = kQTile / W;  // query rows per wave
  constexpr int NT = kWaveRows / 32;     // 32-query tiles per wave
  constexpr float kLazy = 8.f;           // rescale only when a row max grows by > 2^8
  constexpr float kSumCap = 32.f * 256.f;  // a lane sum above this has some P > 2^kLazy

  constexpr int kStageBytes = kKT * D * 2;
  __shared__ __attribute__((aligned(16))) uint16_t sK[kStages][kKT * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kStages][kKT * D];
  __shared__ int32_t sStart[kLCap];
  __shared__ int32_t sCum[kLCap + 1];
  __shared__ int32_t sWin[2][kWin * kKT];    // row-map windows (double-buffered)
  __shared__ int32_t sPerm[kStages][kKT];  // PERM: original row of each chunk key
  __shared__ int32_t sWsum[W];

  __shared__ int32_t sNext;

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform; made scalar for the fused-permutation kernels
  // only (the other instantiations measured slower with it scalar)
  const int wave = PERM ? __builtin_amdgcn_readfirstlane(tid >> 6) : tid >> 6;
  const int h = lane >> 5, col = lane & 31;

  // one work item: rows [row0, row0 + 256) of Q block qb of slice bh
  auto item = [&](const int bh, const int qb, const int row0) {
  const int qs = dense ? 0 : q_off[static_cast<size_t>(bh) * (nqb + 1) + qb];
  const int qe = dense ? n_q : q_off[static_cast<size_t>(bh) * (nqb + 1) + qb + 1];
  // Split mode (an item of at most half the tile's rows, one 32-row query
  // tile per wave pair): the two waves that share a SIMD, w and w + W/2, take
  // the same query rows, wave w the first 32 keys of every chunk and wave
  // w + W/2 the last 32; their partial softmax states are merged at the end.
  // Each step's work per wave is then halved, so such an item runs in less
  // time than a full one instead of leaving half the waves idle.  The wave's
  // K and V fragment addresses move to its key half for the item.  (SPLIT:
  // the instantiation for Q blocks of at most kQTile / 2 rows on average; the
  // other one has none of this code, which keeps its full-item schedule.)
  const bool split = SPLIT && NT == 1 && qe - (qs + row0) <= kQTile / 2;   // uniform
  const int mt_own = split ? wave / (W / 2) : 0;                   // split: own key half
  const int rbase = qs + row0 + (split ? wave % (W / 2) : wave) * kWaveRows;
  const bool wave_active = rbase < qe;
  bool nt_active[NT];
  int myq[NT];
  bool qvalid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    nt_active[nt] = rbase + nt * 32 < qe;      // wave-uniform
    myq[nt] = rbase + nt * 32 + col;
    qvalid[nt] = myq[nt] < qe;
  }

  // source row of each lane's query: the permuted row itself, or (PERM) its
  // original row, which is also where its output goes
  int qrow_id[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if constexpr (PERM) qrow_id[nt] = qvalid[nt] ? q_perm[static_cast<size_t>(bh) * n_q + myq[nt]] : 0;
    else qrow_id[nt] = qvalid[nt] ? myq[nt] : 0;
  }
  // Q fragments: lane holds Q[query][16 s + 8 h .. +8] (B operand of S^T = K Q^T)
  bf16x8 qf[NT][NS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const uint16_t *qrow = q + (static_cast<size_t>(bh) * n_q + qrow_id[nt]) * D + h * 8;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      u32x4 raw = qvalid[nt] ? *reinterpret_cast<const u32x4 *>(qrow + s * 16) : u32x4{0, 0, 0, 0};
      qf[nt][s] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  f32x16 oacc[NT][ND];
  f32x16 sacc[NT][2];                  // scores of the chunk awaiting its softmax
  bf16x8 pb[NT][4];                    // probabilities of the chunk awaiting its PV
  const bool late = wave >= W / 2;     // runs the rotated step (see below)
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[nt][dt][i] = 0.f;
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }

  const int kc = dense ? 1 : kept_count[static_cast<size_t>(bh) * nqb + qb];
  const int32_t *kidx = kept_idx + (static_cast<size_t>(bh) * nqb + qb) * kept_stride;
  const int32_t *koff = k_off + static_cast<size_t>(bh) * (nkb + 1);
  const uint16_t *kbase = k + static_cast<size_t>(bh) * n_k * D;
  const int32_t *pbase = PERM ? k_perm + static_cast<size_t>(bh) * n_k : nullptr;
  const uint16_t *vbase = v + static_cast<size_t>(bh) * n_k * D;

  // Direct-to-LDS load geometry: wave load j writes LDS bytes [1 KB * (wave*LPW + j), +1 KB):
  // lane l fills physical piece l % PPR of row RPI*(wave*LPW + j) + l / PPR, i.e. the
  // logical piece (l % PPR) ^ swizzle(row) of that key row.
  const int ld_rsub = lane / PPR, ld_piece = lane % PPR;

  // PV operand geometry for ds_read_b64_tr_b16 (4x16 transpose per 16-lane group):
  // source lane (g, j, q) = (lane/16, (lane/4)%4, lane%4) points at key row
  // 16 ks + 4 (g/2) + j (+8 for the second read), d = 32 dt + 16 (g%2) + 4 q, so
  // result lane gets 4 keys of its own d in exactly the key order of the P^T operand.
  const int tr_g = lane >> 4, tr_j = (lane >> 2) & 3, tr_q = lane & 3;
  const int tr_row = 4 * (tr_g >> 1) + tr_j;              // + 16 ks (+ 8)
  const int tr_c0 = 2 * (tr_g & 1) + (tr_q >> 1);         // chunk within a 32-wide d tile
  const int tr_in = (tr_q & 1) * 4;                        // element within the chunk
  static_assert(vswz<D>(0) == vswz<D>(8) && vswz<D>(5) == vswz<D>(13), "+8 rows keep the V swizzle");
  const int tr_x = vswz<D>(tr_row);                        // same for +8 rows and every ks

  // LDS byte addresses of this lane's fragments in stage 0; the stage, m-tile
  // and k-step offsets are immediates of the reads.  K: piece 2s+h of row col.
  uint32_t ka[NS], va[ND];
  const uint32_t sk0 = lds_offset(&sK[0][0]), sv0 = lds_offset(&sV[0][0]);
#pragma unroll
  for (int s = 0; s < NS; ++s) ka[s] = sk0 + col * D * 2 + (((2 * s + h) ^ kswz<D>(col)) << 4);
#pragma unroll
  for (int dt = 0; dt < ND; ++dt)
    va[dt] = sv0 + tr_row * D * 2 + ((((dt << 2) | tr_c0) ^ tr_x) << 4) + tr_in * 2;

  const uint32_t split_off = static_cast<uint32_t>(mt_own) * 32 * D * 2;   // LDS bytes
#pragma unroll
  for (int s = 0; s < NS; ++s) ka[s] += split_off;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) va[dt] += split_off;
  for (int seg0 = 0; seg0 < kc; seg0 += kLCap) {
    // the segment's kept clusters as key-row ranges, empty ones dropped:
    // sStart[j] = first row, sCum[j] = virtual index of that row (exclusive scan)
    const int segn = min(kLCap, kc - seg0);
    constexpr int EPT = kLCap / kThr;     // list entries per thread
    static_assert(EPT * kThr == kLCap && EPT <= 4, "the scan covers 4 entries per thread");
    int st_r[EPT], len_r[EPT], ci[EPT];
#pragma unroll
    for (int u = 0; u < EPT; ++u) {
      const int j = tid + u * kThr;
      st_r[u] = 0;
      len_r[u] = 0;
      if (j < segn) {
        if (dense) {
          len_r[u] = n_k;
        } else {
          const int b = kidx[seg0 + j];
          st_r[u] = koff[b];
          len_r[u] = koff[b + 1] - st_r[u];
        }
      }
      sCum[j] = len_r[u] > 0 ? 1 : 0;
    }
    __syncthreads();
    block_exclusive_scan<kThr>(sCum, segn, sWsum);
#pragma unroll
    for (int u = 0; u < EPT; ++u) ci[u] = sCum[tid + u * kThr];
    const int nseg = sCum[segn];
    __syncthreads();
#pragma unroll
    for (int u = 0; u < EPT; ++u)
      if (len_r[u] > 0) {
        sStart[ci[u]] = st_r[u];
        sCum[ci[u]] = len_r[u];
      }
    __syncthreads();
    block_exclusive_scan<kThr>(sCum, nseg, sWsum);
    const int L = sCum[nseg];
    const int nch = (L + kKT - 1) / kKT;
    if (nch == 0) continue;   // uniform: L is shared

    // Row maps in windows of kWin chunks: the K row behind each virtual key
    // of the window (-1 past the end).  All threads build a window at once,
    // each for KPT consecutive keys: a branchless binary search over the range
    // starts (from the top bit of the range count) for the first, then at most
    // one range forward per further key; windows w and w+1 are
    // double-buffered, and window w+1 is built in the first step of window w.
    static_assert((kWin * kKT) % kThr == 0 && kLCap <= 1024, "window build geometry");
    constexpr int KPT = kWin * kKT / kThr;   // consecutive window keys per thread
    static_assert(KPT * kThr == kWin * kKT, "window keys split evenly over the threads");
    const int bsearch0 = 1 << (31 - __clz(max(nseg, 1)));   // top bit of nseg (uniform)
    auto build_win = [&](int w) {
      int32_t *dst = sWin[w & 1];
      const int v0 = w * (kWin * kKT) + KPT * tid;
      int lo = 0;   // the last range starting at or before v0: largest j < nseg, sCum[j] <= v0
      for (int b = bsearch0; b > 0; b >>= 1) {
        const int j = lo + b;
        const int cj = sCum[min(j, nseg)];
        lo = (j < nseg && cj <= v0) ? j : lo;
      }
#pragma unroll
      for (int u = 0; u < KPT; ++u) {
        const int v = v0 + u;
        // ranges are non-empty: the next key is in the same range or the next one
        if (u > 0 && lo + 1 < nseg && sCum[lo + 1] <= v) ++lo;
        dst[KPT * tid + u] = v < L ? sStart[lo] + (v - sCum[lo]) : -1;
      }
    };
    // PERM: the original rows of a chunk's keys reach the chunk's sPerm stage
    // in two steps: wave CW (the first copying wave) loads them into a
    // register (a plain global load, a step ahead), then stores the register
    // into the stage.  sPerm is thus an ordinary LDS array, and reading it
    // needs no wait on the K/V copies in flight.  A key past the end of the list takes the original row of the
    // chunk's first key (a kept row; row 0 of the slice when the whole chunk
    // lies past the end), so every entry of a stage is the row its copy
    // loads and the copy issue reads the stage alone, with no dependent read
    // of the row map before it.
    int pnext = 0;
    auto perm_row = [&](int c) {   // (wave CW) the original row of the lane's key of chunk c
      const bool live = c * kKT < L;   // uniform
      const int32_t *rows = sWin[(c / kWin) & 1] + (c % kWin) * kKT;
      const int rr = live ? rows[lane] : -1;
      const int r0 = live ? rows[0] : 0;
      return pbase[rr < 0 ? r0 : rr];
    };
    auto perm_load = [&](int c) {
      if constexpr (PERM) {
        if (wave == CW) pnext = perm_row(c);
      }
    };
    auto perm_store = [&](auto st) {
      if constexpr (PERM) {
        if (wave == CW) sPerm[decltype(st)::value][lane] = pnext;
      }
    };
    // the K/V source rows of this lane's copies of chunk cc (in stage st): the
    // row map, or (PERM) the stage's original rows.  Past the end of the list
    // (the chunks after the last) whole stages are refilled from key 0's row,
    // so every step issues the same number of copies.  Read a step before the
    // copies are issued, so the LDS latency hides behind that step's compute.
    struct ChunkRows {
      int phys[LPC];
    };
    auto fetch_rows = [&](auto st, int cc) {
      ChunkRows cr;
      const bool live = cc * kKT < L;   // uniform
      const int32_t *rows = sWin[(cc / kWin) & 1] + (cc % kWin) * kKT;
      const int32_t *prow = sPerm[decltype(st)::value];
      if constexpr (PERM) {
#pragma unroll
        for (int j = 0; j < LPC; ++j) cr.phys[j] = prow[RPI * ((wave - CW) * LPC + j) + ld_rsub];
      } else {
        const int dummy = live ? max(rows[0], 0) : 0;
#pragma unroll
        for (int j = 0; j < LPC; ++j) {
          const int r = RPI * ((wave - CW) * LPC + j) + ld_rsub;
          const int phys = live ? rows[r] : -1;
          cr.phys[j] = phys < 0 ? dummy : phys;
        }
      }
      return cr;
    };
    // issue the asynchronous HBM -> LDS copies of one chunk's K and V rows
    auto issue_loads = [&](auto st, const ChunkRows &cr) {
      uint16_t *dk = sK[decltype(st)::value];
      uint16_t *dv = sV[decltype(st)::value];
#pragma unroll
      for (int j = 0; j < LPC; ++j) {
        const int blk = (wave - CW) * LPC + j;
        const int r = RPI * blk + ld_rsub;
        const int phys = cr.phys[j];
        // (offsets stay in named variables: with an arithmetic expression in the
        // builtin's argument list, hipcc 7.2's host pass emits no launch stub)
        // (unsigned 32-bit byte offsets from the slice base: scalar base + vector offset)
        const uint32_t koff = static_cast<uint32_t>(phys) * (D * 2) + ((ld_piece ^ kswz<D>(r)) << 4);
        const uint32_t voff = static_cast<uint32_t>(phys) * (D * 2) + ((ld_piece ^ vswz<D>(r)) << 4);
        const char *ksrc = reinterpret_cast<const char *>(kbase) + koff;
        const char *vsrc = reinterpret_cast<const char *>(vbase) + voff;
        __builtin_amdgcn_global_load_lds(ksrc,
                                         (__attribute__((address_space(3))) void *)(dk + blk * 512),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(vsrc,
                                         (__attribute__((address_space(3))) void *)(dv + blk * 512),
                                         16, 0, 0);
      }
    };

    // prologue: row-map windows 0 and 1; (PERM) the original rows of chunks
    // 0-3 in their stages and chunk 4's loaded; chunks 0 and 1 in flight and
    // chunk 2's source rows in registers
    build_win(0);
    if (kWin < nch) build_win(1);
    __syncthreads();
    if constexpr (PERM) {
      if (wave == CW) {   // the five loads in flight together, then the four stores
        int pr[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) pr[j] = perm_row(j);
        pnext = perm_row(4);
        sPerm[0][lane] = pr[0];
        sPerm[1][lane] = pr[1];
        sPerm[2][lane] = pr[2];
        sPerm[3][lane] = pr[3];
      }
    }
    lds_barrier();
    ChunkRows nxt{};
    if (wave >= CW) {
      issue_loads(std::integral_constant<int, 0>{}, fetch_rows(std::integral_constant<int, 0>{}, 0));
      issue_loads(std::integral_constant<int, 1>{}, fetch_rows(std::integral_constant<int, 1>{}, 1));
      nxt = fetch_rows(std::integral_constant<int, 2>{}, 2);
    }

    // S^T = K Q^T for the 64 keys of the chunk in stage ST (two 32-key m-tiles)
    // x the wave's query tiles; each K fragment serves every query tile
    auto qk = [&](auto st) {
      constexpr int ST = decltype(st)::value;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        if (mt == 1 && split) break;   // split: one m-tile, the wave's key half
        bf16x8 kf[NS];
        if (mt == 0) lds_read_frags<ST * kStageBytes>(kf, ka);
        else lds_read_frags<ST * kStageBytes + 32 * D * 2>(kf, ka);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int i = 0; i < 16; ++i) sacc[nt][mt][i] = 0.f;
          if (!nt_active[nt]) continue;
#pragma unroll
          for (int s = 0; s < NS; ++s) sacc[nt][mt] = mfma32x32x16(kf[s], qf[nt][s], sacc[nt][mt]);
        }
      }
    };
    // online softmax of chunk cc: scores in sacc -> bf16 probabilities in pb,
    // running sum updated, max and O rescaled when the max grows by > 2^kLazy
    auto softmax = [&](int cc) {
      const int k0 = cc * kKT + mt_own * 32;   // key of m-tile 0, row 0
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (!nt_active[nt]) continue;
        // (split: only m-tile 0 holds scores)
        if ((cc + 1) * kKT > L) {     // partial last chunk: mask keys past the end
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            if (mt == 1 && split) break;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if (k0 + mt * 32 + acc_row(i, h) >= L) sacc[nt][mt][i] = -INFINITY;
          }
        }
        // The row max is taken on the first chunk of a kept-list segment and
        // otherwise only when a lane's probability sum exceeds 32 * 2^kLazy:
        // then some p > 2^kLazy, so the max has grown by more than 2^kLazy
        // and the chunk is redone after the rescale.  Between rescales every
        // p stays <= 32 * 2^kLazy.
        auto rescale = [&]() {
          // (maximum, not maxnum: no NaN canonicalisation, so v_maximum3 does 2
          // per op); four independent chains keep the reduction short
          float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            if (mt == 1 && split) break;
#pragma unroll
            for (int i = 0; i < 16; ++i)
              m4[i & 3] = __builtin_elementwise_maximum(m4[i & 3], sacc[nt][mt][i]);
          }
          float mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(m4[0], m4[1]),
                                                   __builtin_elementwise_maximum(m4[2], m4[3]));
          {   // both lane halves hold the same query: exchange with permlane32_swap
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx),
                                                             __float_as_uint(mx), false, false);
            mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
          }
          const float mxs = mx * scale_log2;
          if (__any(mxs > m_run[nt] + kLazy)) {
            const float m_new = fmaxf(m_run[nt], mxs);
            const float alpha = __builtin_amdgcn_exp2f(m_run[nt] - m_new);
            l_run[nt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
              for (int i = 0; i < 16; ++i) oacc[nt][dt][i] *= alpha;
            m_run[nt] = m_new;
          }
        };
        // p = 2^(s * scale_log2 - m) into pb; returns the lane's sum
        // (split: a key half may hold no key at all, the tail of the last
        // chunk; while the wave has seen no key its max stays -inf and the
        // exponent is taken against 0, giving p = 0)
        auto exps = [&]() {
          const float m_sub = m_run[nt] == -INFINITY ? 0.f : m_run[nt];
          float ps[4];   // four independent partial sums
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            if (mt == 1 && split) break;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float p = __builtin_amdgcn_exp2f(fmaf(sacc[nt][mt][i], scale_log2, -m_sub));
              ps[i & 3] = (mt == 0 && i < 4) ? p : ps[i & 3] + p;
              pb[nt][2 * mt + (i >> 3)][i & 7] = static_cast<__bf16>(p);
            }
          }
          return (ps[0] + ps[1]) + (ps[2] + ps[3]);
        };
        if (cc == 0) rescale();
        float tot = exps();
        if (cc > 0 && __builtin_expect(__any(tot > kSumCap), 0)) {
          rescale();
          tot = exps();
        }
        l_run[nt] += tot;
      }
    };
    // O^T += V^T P^T with the V rows in stage ST; the V operand (transposing
    // reads of row-major V) is shared by all query tiles
    auto pv = [&](auto st) {
      constexpr int ST = decltype(st)::value;
      if constexpr (ND == 4) {   // two k-steps per LDS round trip
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          if (kp == 1 && split) break;   // split: the wave's 32 keys only
          bf16x8 vf[2][ND];
          if (kp == 0)
            lds_read_vt2<ST * kStageBytes, ST * kStageBytes + 16 * D * 2, 8 * D * 2>(vf[0], vf[1], va);
          else
            lds_read_vt2<ST * kStageBytes + 32 * D * 2, ST * kStageBytes + 48 * D * 2, 8 * D * 2>(
                vf[0], vf[1], va);
#pragma unroll
          for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
              for (int nt = 0; nt < NT; ++nt)
                if (nt_active[nt])
                  oacc[nt][dt] = mfma32x32x16(vf[u][dt], pb[nt][2 * kp + u], oacc[nt][dt]);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          if (ks == 2 && split) break;   // split: the wave's 32 keys only
          bf16x8 vf[ND];
          if (ks == 0) lds_read_vt<ST * kStageBytes, 8 * D * 2>(vf, va);
          else if (ks == 1) lds_read_vt<ST * kStageBytes + 16 * D * 2, 8 * D * 2>(vf, va);
          else if (ks == 2) lds_read_vt<ST * kStageBytes + 32 * D * 2, 8 * D * 2>(vf, va);
          else lds_read_vt<ST * kStageBytes + 48 * D * 2, 8 * D * 2>(vf, va);
#pragma unroll
          for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
              if (nt_active[nt]) oacc[nt][dt] = mfma32x32x16(vf[dt], pb[nt][ks], oacc[nt][dt]);
        }
      }
    };

    // Step c (c = 0 .. nch; chunk c lives in stage c % 4, the body is
    // instantiated per stage).  The two waves sharing a SIMD (w, w + W/2) run
    // the same sequence -- softmax, PV, QK -- rotated against each other:
    //   waves 0 .. W/2-1:   PV(c-1), QK(c), softmax(c)
    //   waves W/2 .. W-1:   softmax(c-1), PV(c-1), QK(c)
    // so while one of them is in its MFMA phase the other is in its VALU
    // phase.  Chunk c-1's V stays in use during step c, hence four stages
    // for two chunks in flight.  Step nch only finishes chunk nch-1.
    auto step = [&](auto st, int c) {
      constexpr int S = decltype(st)::value;
      constexpr int SP = (S + kStages - 1) % kStages;   // stage of chunk c-1
      // chunk c has landed once only chunk c+1's copies are outstanding (a
      // wave that copies nothing waits for nothing); after the barrier every
      // copying wave's part of chunk c is in LDS and every wave is
      // done with chunk c-2, whose stage chunk c+2 then refills
      // (PERM: wave CW's load of chunk c+4's original rows is older than chunk
      // c+1's K/V copies, so it has landed too)
      wait_vmcnt<2 * LPC>();
      lds_barrier();
      if (c % kWin == 0 && (c / kWin + 1) * kWin < nch) build_win(c / kWin + 1);
      perm_store(st);                 // chunk c+4 (its stage is chunk c's)
      perm_load(c + 5);
      if (wave >= CW) {
        issue_loads(std::integral_constant<int, (S + 2) % kStages>{}, nxt);
        nxt = fetch_rows(std::integral_constant<int, (S + 3) % kStages>{}, c + 3);
      }

      if (wave_active) {
        if (late && c > 0) softmax(c - 1);
        if (c > 0) pv(std::integral_constant<int, SP>{});
        if (c < nch) qk(std::integral_constant<int, S>{});
        if (!late && c < nch) softmax(c);
      }
    };
    static_assert(kStages == 4, "the step loop is unrolled over four stages");
    for (int c = 0; c <= nch; c += 4) {
      step(std::integral_constant<int, 0>{}, c);
      if (c + 1 <= nch) step(std::integral_constant<int, 1>{}, c + 1);
      if (c + 2 <= nch) step(std::integral_constant<int, 2>{}, c + 2);
      if (c + 3 <= nch) step(std::integral_constant<int, 3>{}, c + 3);
    }
    wait_vmcnt<0>();   // the copies past the end must land before the stages are reused
    lds_barrier();     // the next segment reuses the LDS buffers and lists
  }
#pragma unroll
  for (int s = 0; s < NS; ++s) ka[s] -= split_off;
#pragma unroll
  for (int dt = 0; dt < ND; ++dt) va[dt] -= split_off;

  // split mode: wave w + W/2 hands its (max, sum, O) to wave w through LDS
  // (the K/V stages are free now), which merges them into its own
  if (split) {
    f32x4 *sO = reinterpret_cast<f32x4 *>(&sK[0][0]);      // [W/2][ND*4][64]
    float *sM = reinterpret_cast<float *>(&sV[0][0]);      // [W/2][2][64]
    const int pw = wave % (W / 2);
    static_assert((W / 2) * ND * 4 * 64 * 16 <= sizeof(sK) &&
                  (W / 2) * 2 * 64 * 4 <= sizeof(sV), "merge staging fits the stages");
    if (late) {
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig)
          sO[(pw * ND * 4 + dt * 4 + ig) * 64 + lane] =
              f32x4{oacc[0][dt][4 * ig], oacc[0][dt][4 * ig + 1], oacc[0][dt][4 * ig + 2],
                    oacc[0][dt][4 * ig + 3]};
      sM[(pw * 2) * 64 + lane] = m_run[0];
      sM[(pw * 2 + 1) * 64 + lane] = l_run[0];
    }
    __syncthreads();
    if (!late) {
      const float m2 = sM[(pw * 2) * 64 + lane], l2 = sM[(pw * 2 + 1) * 64 + lane];
      const float m = fmaxf(m_run[0], m2);
      const float a1 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[0] - m);
      const float a2 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m2 - m);
#pragma unroll
      for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int ig = 0; ig < 4; ++ig) {
          const f32x4 o2 = sO[(pw * ND * 4 + dt * 4 + ig) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            oacc[0][dt][4 * ig + e] = fmaf(oacc[0][dt][4 * ig + e], a1, o2[e] * a2);
        }
      l_run[0] = fmaf(l_run[0], a1, l2 * a2);
      m_run[0] = m;
    }
  }
  const bool writes = !(split && late);

  // epilogue
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    // l_tot is 0 exactly when the row saw no key (O = 0, LSE = -inf); a NaN
    // that reached the row's sum takes the other branch and stays NaN
    const float l_tot = l_run[nt] + __shfl_xor(l_run[nt], 32);
    const float inv = l_tot != 0.f ? 1.f / l_tot : 0.f;
    if (!writes || !qvalid[nt]) continue;
    const size_t orow = (static_cast<size_t>(bh) * n_q + qrow_id[nt]) * D;
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
      for (int ig = 0; ig < 4; ++ig) {
        const int d0 = dt * 32 + 8 * ig + 4 * h;
        const float o0 = oacc[nt][dt][4 * ig + 0] * inv, o1 = oacc[nt][dt][4 * ig + 1] * inv;
        const float o2 = oacc[nt][dt][4 * ig + 2] * inv, o3 = oacc[nt][dt][4 * ig + 3] * inv;
        if constexpr (OUT_F32) {
          *reinterpret_cast<f32x4 *>(static_cast<float *>(o) + orow + d0) = f32x4{o0, o1, o2, o3};
        } else {
          *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(o) + orow + d0) =
              u32x2{pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
        }
      }
    if (h == 0 && lse != nullptr)
      lse[static_cast<size_t>(bh) * n_q + qrow_id[nt]] =
          l_tot != 0.f ? (m_run[nt] + __log2f(l_tot)) * kLn2 : -INFINITY;
  }
  };

  if (dense) {   // uniform items, one per workgroup
    int bh, qb, row0;
    if (!decode_work(work, work_cap, n_items, dense, bh, qb, row0)) return;
    item(bh, qb, row0);
    return;
  }
  // sparse: persistent workgroups over the per-XCD queues
  int gone = 0;
  for (;;) {
    if (tid == 0) sNext = fetch_work(ctl, gone);
    __syncthreads();
    const int idx = sNext;
    if (idx < 0) break;                   // uniform: every thread read the same value
    const WorkItem it = lists[idx];
    // (the item is the same for every lane: keep it, and the slice bases, scalar)
    item(__builtin_amdgcn_readfirstlane(it.bh), __builtin_amdgcn_readfirstlane(it.qb),
         __builtin_amdgcn_readfirstlane(it.row0));
    __syncthreads();                      // LDS and sNext are reused by the next item
  }
}

// ---------------------------------------------------------------------------
// fp32 attention: one thread per query row, exact fp32 online softmax
// ---------------------------------------------------------------------------
template <int D, bool OUT_F32>
__global__ __launch_bounds__(kQTile) void attn_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    void *__restrict__ o, float *__restrict__ lse, const int32_t *__restrict__ q_perm,
    const int32_t *__restrict__ k_perm, const int32_t *__restrict__ q_off,
    const int32_t *__restrict__ k_off, const int32_t *__restrict__ kept_count,
    const int32_t *__restrict__ kept_idx, int kept_stride, const WorkItem *__restrict__ work,
    int work_cap, int n_items, int n_q, int n_k, int nqb, int nkb, int dense, float scale) {
  int bh, qb, row0;
  if (!decode_work(work, work_cap, n_items, dense, bh, qb, row0)) return;
  const int qs = dense ? 0 : q_off[static_cast<size_t>(bh) * (nqb + 1) + qb];
  const int qe = dense ? n_q : q_off[static_cast<size_t>(bh) * (nqb + 1) + qb + 1];
  const int myq = qs + row0 + threadIdx.x;
  const bool qvalid = myq < qe;
  float qv[D], acc[D];
  // q_perm / k_perm (may be NULL): permuted row -> original row of q, o, lse / of k, v
  const int qrow_id = q_perm == nullptr ? (qvalid ? myq : qs)
                                        : q_perm[static_cast<size_t>(bh) * n_q + (qvalid ? myq : qs)];
  const float *qrow = q + (static_cast<size_t>(bh) * n_q + qrow_id) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    qv[i] = qvalid ? qrow[i] : 0.f;
    acc[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kc = dense ? 1 : kept_count[static_cast<size_t>(bh) * nqb + qb];
  const int32_t *kidx = kept_idx + (static_cast<size_t>(bh) * nqb + qb) * kept_stride;
  const int32_t *koff = k_off + static_cast<size_t>(bh) * (nkb + 1);
  for (int j = 0; j < kc; ++j) {
    int st = 0, en = n_k;
    if (!dense) {
      const int b = kidx[j];
      st = koff[b];
      en = koff[b + 1];
    }
    for (int key = st; key < en; ++key) {
      const int kr_id = k_perm == nullptr ? key : k_perm[static_cast<size_t>(bh) * n_k + key];
      const float *kr = k + (static_cast<size_t>(bh) * n_k + kr_id) * D;
      const float *vr = v + (static_cast<size_t>(bh) * n_k + kr_id) * D;
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) s = fmaf(qv[i], kr[i], s);
      s *= scale;
      const float mn = fmaxf(m, s);
      const float a = expf(m - mn);
      const float p = expf(s - mn);
      l = l * a + p;
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = fmaf(p, vr[i], acc[i] * a);
      m = mn;
    }
  }
  if (!qvalid) return;
  const float inv = l != 0.f ? 1.f / l : 0.f;   // l = 0: no key; NaN stays NaN
  const size_t orow = (static_cast<size_t>(bh) * n_q + qrow_id) * D;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    if constexpr (OUT_F32) static_cast<float *>(o)[orow + i] = acc[i] * inv;
    else static_cast<uint16_t *>(o)[orow + i] = f32_to_bf16_bits(acc[i] * inv);
  }
  if (lse != nullptr) lse[static_cast<size_t>(bh) * n_q + qrow_id] = l != 0.f ? m + logf(l) : -INFINITY;
}

template <int D, bool OF, bool PERM, bool SPLIT>
hipError_t launch_bf16(const AttnArgs &a, const WorkItem *work, int cap, int n_items,
                       const WorkItem *lists, int32_t *ctl, int grid, hipStream_t s) {
  constexpr int kW = attn_waves<D>();
  hipLaunchKernelGGL((attn_bf16_kernel<D, OF, PERM, kW, SPLIT>), dim3(grid), dim3(64 * kW), 0, s,
                     static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
                     static_cast<const uint16_t *>(a.v), a.o, a.lse, PERM ? a.q_perm : nullptr,
                     PERM ? a.k_perm : nullptr, a.q_off, a.k_off, a.kept_count, a.kept_idx,
                     a.kept_stride, work, cap, n_items, lists, ctl, a.n_q, a.n_k, a.nqb, a.nkb,
                     a.dense, a.scale * kLog2e);
  return hipGetLastError();
}

// the split-mode instantiation serves Q blocks of at most half a tile on average
inline bool attn_split_mode(const AttnArgs &a) {
  return !a.dense && a.nqb > 0 && static_cast<long long>(a.nqb) * (kQTile / 2) >= a.n_q;
}

template <int D, bool OF>
hipError_t run_bf16(const AttnArgs &a, const WorkItem *work, int cap, int n_items,
                    const WorkItem *lists, int32_t *ctl, int grid, hipStream_t s) {
  const bool perm = a.q_perm != nullptr;
  if (attn_split_mode(a))
    return perm ? launch_bf16<D, OF, true, true>(a, work, cap, n_items, lists, ctl, grid, s)
                : launch_bf16<D, OF, false, true>(a, work, cap, n_items, lists, ctl, grid, s);
  return perm ? launch_bf16<D, OF, true, false>(a, work, cap, n_items, lists, ctl, grid, s)
              : launch_bf16<D, OF, false, false>(a, work, cap, n_items, lists, ctl, grid, s);
}

template <int D, bool OF>
hipError_t run_f32(const AttnArgs &a, const WorkItem *work, int cap, int n_items, int grid,
                   hipStream_t s) {
  hipLaunchKernelGGL((attn_f32_kernel<D, OF>), dim3(grid), dim3(kQTile), 0, s,
                     static_cast<const float *>(a.q), static_cast<const float *>(a.k),
                     static_cast<const float *>(a.v), a.o, a.lse, a.q_perm, a.k_perm, a.q_off,
                     a.k_off, a.kept_count,
                     a.kept_idx, a.kept_stride, work, cap, n_items, a.n_q, a.n_k, a.nqb, a.nkb,
                     a.dense, a.scale);
  return hipGetLastError();
}

}  // namespace

// compute units of the current device (persistent grids), cached per device
int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && cached[dev] > 0) return cached[dev];
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    cus = 256;
  if (dev < 64) cached[dev] = cus;
  return cus;
}

size_t attn_ws_bytes(int32_t bh, int32_t n_q, int32_t nqb) {
  return sched_layout(bh, n_q, nqb).total;
}

// ---------------------------------------------------------------------------
// Static schedule scratch of the no-allocation attention entry point: one
// array per GPU the library runs on, held until the process ends.  Host code
// never passes the array's name to a kernel (on the host it only stands in for
// the symbol); its device address is looked up once per device, with that
// device current, and kept.  Every call on a GPU shares that GPU's array, so
// calls that overlap on one GPU race; the schedule kernels rewrite every part
// of it they read (items, costs, queues and their counters) on each call.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kStaticAttnScratch];

void *attn_static_scratch(hipError_t *err) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *ptr[kMaxDevices] = {};
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    void *p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    ptr[dev] = p;
  }
  *err = hipSuccess;
  return ptr[dev];
}

// ---------------------------------------------------------------------------
// Debug checks of the device preconditions of the block-sparse calls (set by
// sva_set_debug_checks): one thread per (slice, Q block) checks that block's
// Q offsets, kept count and kept K block ids, one per (slice, K block) that
// block's K offsets, and grid-stride threads the permutations.  Violations set
// bits of a flag kept in a static device word per GPU (looked up like the
// static scratch); the caller clears it first and reads it back after.
// ---------------------------------------------------------------------------
static __device__ int32_t debug_flag_word[4];

__global__ __launch_bounds__(kThreads) void attn_index_check_kernel(AttnArgs a, int32_t *flag) {
  const int bh = blockIdx.y;
  const long long t = static_cast<long long>(blockIdx.x) * kThreads + threadIdx.x;
  int bits = 0;
  if (t < a.nqb) {
    const int qb = static_cast<int>(t);
    const int32_t *qo = a.q_off + static_cast<size_t>(bh) * (a.nqb + 1);
    if (qo[qb] < 0 || qo[qb] > qo[qb + 1] || qo[qb + 1] > a.n_q) bits |= kDebugQOffsets;
    const size_t e = static_cast<size_t>(bh) * a.nqb + qb;
    const int cnt = a.kept_count[e];
    if (cnt < 0 || cnt > a.kept_stride || cnt > a.nkb) bits |= kDebugKeptCount;
    const int m = min(max(cnt, 0), a.kept_stride);
    for (int j = 0; j < m; ++j) {
      const int b = a.kept_idx[e * a.kept_stride + j];
      if (b < 0 || b >= a.nkb) bits |= kDebugKeptIdx;
    }
  }
  if (t < a.nkb) {
    const int kb = static_cast<int>(t);
    const int32_t *ko = a.k_off + static_cast<size_t>(bh) * (a.nkb + 1);
    if (ko[kb] < 0 || ko[kb] > ko[kb + 1] || ko[kb + 1] > a.n_k) bits |= kDebugKOffsets;
  }
  const long long stride = static_cast<long long>(gridDim.x) * kThreads;
  if (a.q_perm != nullptr)
    for (long long i = t; i < a.n_q; i += stride) {
      const int r = a.q_perm[static_cast<size_t>(bh) * a.n_q + i];
      if (r < 0 || r >= a.n_q) bits |= kDebugQPerm;
    }
  if (a.k_perm != nullptr)
    for (long long i = t; i < a.n_k; i += stride) {
      const int r = a.k_perm[static_cast<size_t>(bh) * a.n_k + i];
      if (r < 0 || r >= a.n_k) bits |= kDebugKPerm;
    }
  if (bits) atomicOr(flag, bits);
}

__global__ void debug_flag_clear_kernel(int32_t *flag) { flag[0] = 0; }

hipError_t attn_debug_check(const AttnArgs &a, hipStream_t s, int32_t *bits) {
  static std::mutex mu;
  static int32_t *ptr[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  int32_t *flag;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
      void *p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(debug_flag_word));
      if (e != hipSuccess) return e;
      ptr[dev] = static_cast<int32_t *>(p);
    }
    flag = ptr[dev];
  }
  hipLaunchKernelGGL(debug_flag_clear_kernel, dim3(1), dim3(1), 0, s, flag);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int most = std::max(std::max(a.nqb, a.nkb), 1);
  const int gx = std::min((most + kThreads - 1) / kThreads, 1024);
  hipLaunchKernelGGL(attn_index_check_kernel, dim3(gx, a.bh), dim3(kThreads), 0, s, a, flag);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  int32_t h = 0;
  if ((e = hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, s)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(s)) != hipSuccess) return e;
  *bits = h;
  return hipSuccess;
}

hipError_t launch_attention(const AttnArgs &a, hipStream_t s) {
  int cap;
  const WorkItem *work = nullptr;
  const WorkItem *lists = nullptr;
  int32_t *ctl = nullptr;
  hipError_t e;
  if (a.dense) {
    cap = (a.n_q + kQTile - 1) / kQTile;
  } else {
    cap = (a.n_q + kQTile - 1) / kQTile + a.nqb;
    const SchedLayout L = sched_layout(a.bh, a.n_q, a.nqb);
    char *ws = static_cast<char *>(a.ws);
    WorkItem *w = reinterpret_cast<WorkItem *>(ws + L.items);
    int32_t *qcost = reinterpret_cast<int32_t *>(ws + L.qcost);
    int32_t *hinfo = reinterpret_cast<int32_t *>(ws + L.hinfo);
    WorkItem *lst = reinterpret_cast<WorkItem *>(ws + L.lists);
    ctl = reinterpret_cast<int32_t *>(ws + L.ctl);
    hipLaunchKernelGGL(attn_cost_kernel,
                       dim3((a.nqb + kThreads / 64 - 1) / (kThreads / 64), a.bh), dim3(kThreads),
                       0, s, a.k_off, a.kept_count, a.kept_idx, a.kept_stride, a.nqb, a.nkb,
                       qcost);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(attn_schedule_kernel, dim3(a.bh), dim3(kThreads), 0, s, a.q_off, qcost,
                       a.nqb, cap, a.dtype == SVA_BF16 && attn_split_mode(a) ? 1 : 0, w, hinfo);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (a.dtype == SVA_BF16) {
      hipLaunchKernelGGL(attn_order_kernel, dim3(1), dim3(kOrderThreads), 0, s, w, hinfo, a.bh,
                         cap, lst, ctl);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    work = w;
    lists = lst;
  }
  const long long n_items = static_cast<long long>(a.bh) * cap;
  const long long grid = (n_items + 7) / 8 * 8;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const bool of = a.o_dtype == SVA_F32;
  if (a.dtype == SVA_BF16) {
    // dense: one workgroup per item; sparse: one persistent workgroup per compute unit
    // (one fits per CU), at most one per item
    const int g = a.dense ? static_cast<int>(grid)
                          : static_cast<int>(std::min<long long>(device_cus(), grid));
    if (a.d == 128) return of ? run_bf16<128, true>(a, work, cap, (int)n_items, lists, ctl, g, s)
                              : run_bf16<128, false>(a, work, cap, (int)n_items, lists, ctl, g, s);
    return of ? run_bf16<64, true>(a, work, cap, (int)n_items, lists, ctl, g, s)
              : run_bf16<64, false>(a, work, cap, (int)n_items, lists, ctl, g, s);
  }
  if (a.d == 128) return of ? run_f32<128, true>(a, work, cap, (int)n_items, (int)grid, s)
                            : run_f32<128, false>(a, work, cap, (int)n_items, (int)grid, s);
  return of ? run_f32<64, true>(a, work, cap, (int)n_items, (int)grid, s)
            : run_f32<64, false>(a, work, cap, (int)n_items, (int)grid, s);
}

}  // namespace sva
