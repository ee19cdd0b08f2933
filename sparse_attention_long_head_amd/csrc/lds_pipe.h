// LDS pipeline helpers for gfx950 kernels that stream tiles from HBM into LDS
// with direct global->LDS copies (global_load_lds) kept in flight across
// barriers, and read MFMA operands back with inline-assembly ds_read blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sva_internal.h"

namespace sva {

// Wait until at most N vector-memory loads of this wave are outstanding (loads
// complete in issue order).  N < 16; expcnt and lgkmcnt are left unconstrained.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Byte offset of a __shared__ object in the workgroup's LDS (the address the
// ds_* instructions take).
__device__ __forceinline__ uint32_t lds_offset(const void *p) {
  return static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)p));
}

// MFMA operand fragments read from LDS in inline assembly.  Pipeline stages
// are filled by global->LDS copies that stay in flight across the reads of
// other stages; reads the compiler can see make it wait for every such copy
// first (vmcnt(0)), so these reads are kept out of its sight, and the caller's
// explicit vmcnt wait plus barrier at the top of each step orders them
// instead.  Each block waits for its own reads before returning (lgkmcnt(0)).
//
// Row fragments: N = 4 or 8 ds_read_b128, lane address a[s] + OFF.
template <int OFF, int N>
__device__ __forceinline__ void lds_read_frags(bf16x8 (&f)[N], const uint32_t (&a)[N]) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
  if constexpr (N == 8) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%16\n\t"
        "ds_read_b128 %1, %9 offset:%16\n\t"
        "ds_read_b128 %2, %10 offset:%16\n\t"
        "ds_read_b128 %3, %11 offset:%16\n\t"
        "ds_read_b128 %4, %12 offset:%16\n\t"
        "ds_read_b128 %5, %13 offset:%16\n\t"
        "ds_read_b128 %6, %14 offset:%16\n\t"
        "ds_read_b128 %7, %15 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]),
          "=&v"(f[6]), "=&v"(f[7])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]),
          "v"(a[7]), "i"(OFF)
        : "memory");
  } else {
    static_assert(N == 4, "4 or 8 fragments");
    asm volatile(
        "ds_read_b128 %0, %4 offset:%8\n\t"
        "ds_read_b128 %1, %5 offset:%8\n\t"
        "ds_read_b128 %2, %6 offset:%8\n\t"
        "ds_read_b128 %3, %7 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF)
        : "memory");
  }
}

// Row fragments at one lane address: N = 4 or 8 ds_read_b128 at a + OFF + STRIDE * s.
template <int OFF, int STRIDE, int N>
__device__ __forceinline__ void lds_read_frags_strided(bf16x8 (&f)[N], uint32_t a) {
  static_assert(OFF >= 0 && OFF + (N - 1) * STRIDE < 65536, "ds offset field");
  if constexpr (N == 8) {
    asm volatile(
        "ds_read_b128 %0, %8 offset:%9\n\t"
        "ds_read_b128 %1, %8 offset:%10\n\t"
        "ds_read_b128 %2, %8 offset:%11\n\t"
        "ds_read_b128 %3, %8 offset:%12\n\t"
        "ds_read_b128 %4, %8 offset:%13\n\t"
        "ds_read_b128 %5, %8 offset:%14\n\t"
        "ds_read_b128 %6, %8 offset:%15\n\t"
        "ds_read_b128 %7, %8 offset:%16\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3]), "=&v"(f[4]), "=&v"(f[5]),
          "=&v"(f[6]), "=&v"(f[7])
        : "v"(a), "i"(OFF), "i"(OFF + STRIDE), "i"(OFF + 2 * STRIDE), "i"(OFF + 3 * STRIDE),
          "i"(OFF + 4 * STRIDE), "i"(OFF + 5 * STRIDE), "i"(OFF + 6 * STRIDE),
          "i"(OFF + 7 * STRIDE)
        : "memory");
  } else {
    static_assert(N == 4, "4 or 8 fragments");
    asm volatile(
        "ds_read_b128 %0, %4 offset:%5\n\t"
        "ds_read_b128 %1, %4 offset:%6\n\t"
        "ds_read_b128 %2, %4 offset:%7\n\t"
        "ds_read_b128 %3, %4 offset:%8\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
        : "v"(a), "i"(OFF), "i"(OFF + STRIDE), "i"(OFF + 2 * STRIDE), "i"(OFF + 3 * STRIDE)
        : "memory");
  }
}

// Transposed fragments: for each of N d tiles two ds_read_b64_tr_b16 (rows +0
// and +HI of the k-step) joined into one 8-element operand.
template <int OFF, int HI, int N>
__device__ __forceinline__ void lds_read_vt(bf16x8 (&f)[N], const uint32_t (&a)[N]) {
  static_assert(OFF >= 0 && OFF + HI < 65536, "ds offset field");
  bf16x4 lo[N], hi[N];
  if constexpr (N == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %2, %9 offset:%12\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%13\n\t"
        "ds_read_b64_tr_b16 %4, %10 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %10 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %11 offset:%12\n\t"
        "ds_read_b64_tr_b16 %7, %11 offset:%13\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]),
          "=&v"(lo[3]), "=&v"(hi[3])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF), "i"(OFF + HI)
        : "memory");
  } else {
    static_assert(N == 2, "2 or 4 d tiles");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4 offset:%6\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:%7\n\t"
        "ds_read_b64_tr_b16 %2, %5 offset:%6\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1])
        : "v"(a[0]), "v"(a[1]), "i"(OFF), "i"(OFF + HI)
        : "memory");
  }
#pragma unroll
  for (int i = 0; i < N; ++i) f[i] = __builtin_shufflevector(lo[i], hi[i], 0, 1, 2, 3, 4, 5, 6, 7);
}

// Two k-steps of transposed fragments at once (offsets OFF0 and OFF1, each
// with rows +0 and +HI), for 4 d tiles: 16 reads, one wait.
template <int OFF0, int OFF1, int HI>
__device__ __forceinline__ void lds_read_vt2(bf16x8 (&f0)[4], bf16x8 (&f1)[4],
                                             const uint32_t (&a)[4]) {
  static_assert(OFF0 >= 0 && OFF1 + HI < 65536, "ds offset field");
  bf16x4 l0[4], h0[4], l1[4], h1[4];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:%20\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:%21\n\t"
      "ds_read_b64_tr_b16 %2, %17 offset:%20\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:%21\n\t"
      "ds_read_b64_tr_b16 %4, %18 offset:%20\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:%21\n\t"
      "ds_read_b64_tr_b16 %6, %19 offset:%20\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:%21\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:%22\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:%23\n\t"
      "ds_read_b64_tr_b16 %10, %17 offset:%22\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:%23\n\t"
      "ds_read_b64_tr_b16 %12, %18 offset:%22\n\t"
      "ds_read_b64_tr_b16 %13, %18 offset:%23\n\t"
      "ds_read_b64_tr_b16 %14, %19 offset:%22\n\t"
      "ds_read_b64_tr_b16 %15, %19 offset:%23\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(l0[0]), "=&v"(h0[0]), "=&v"(l0[1]), "=&v"(h0[1]), "=&v"(l0[2]), "=&v"(h0[2]),
        "=&v"(l0[3]), "=&v"(h0[3]), "=&v"(l1[0]), "=&v"(h1[0]), "=&v"(l1[1]), "=&v"(h1[1]),
        "=&v"(l1[2]), "=&v"(h1[2]), "=&v"(l1[3]), "=&v"(h1[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(OFF0), "i"(OFF0 + HI), "i"(OFF1),
        "i"(OFF1 + HI)
      : "memory");
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f0[i] = __builtin_shufflevector(l0[i], h0[i], 0, 1, 2, 3, 4, 5, 6, 7);
    f1[i] = __builtin_shufflevector(l1[i], h1[i], 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// Workgroup barrier for LDS only: this wave's LDS accesses complete, then
// s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global->LDS copies, which the K/V pipeline keeps in flight across it; the
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Four ds_read_b128 of f32x4 at a + OFF + STRIDE*j (j = 0..3); waits for them.
template <int OFF, int STRIDE>
__device__ __forceinline__ void lds_read_f32x4x4(f32x4 (&f)[4], uint32_t a) {
  static_assert(OFF >= 0 && OFF + 3 * STRIDE < 65536, "ds offset field");
  asm volatile(
      "ds_read_b128 %0, %4 offset:%5\n\t"
      "ds_read_b128 %1, %4 offset:%6\n\t"
      "ds_read_b128 %2, %4 offset:%7\n\t"
      "ds_read_b128 %3, %4 offset:%8\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(f[0]), "=&v"(f[1]), "=&v"(f[2]), "=&v"(f[3])
      : "v"(a), "i"(OFF), "i"(OFF + STRIDE), "i"(OFF + 2 * STRIDE), "i"(OFF + 3 * STRIDE)
      : "memory");
}

// N ds_read_b32 (N = 2, 3 or 5) at per-lane byte addresses a[i]; waits for them.
template <int N>
__device__ __forceinline__ void lds_read_i32s(int (&v)[N], const uint32_t (&a)[N]) {
  if constexpr (N == 5) {
    asm volatile(
        "ds_read_b32 %0, %5\n\t"
        "ds_read_b32 %1, %6\n\t"
        "ds_read_b32 %2, %7\n\t"
        "ds_read_b32 %3, %8\n\t"
        "ds_read_b32 %4, %9\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4])
        : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4])
        : "memory");
  } else if constexpr (N == 3) {
    asm volatile(
        "ds_read_b32 %0, %3\n\t"
        "ds_read_b32 %1, %4\n\t"
        "ds_read_b32 %2, %5\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2])
        : "v"(a[0]), "v"(a[1]), "v"(a[2])
        : "memory");
  } else {
    static_assert(N == 2, "2, 3 or 5 reads");
    asm volatile(
        "ds_read_b32 %0, %2\n\t"
        "ds_read_b32 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1])
        : "v"(a[0]), "v"(a[1])
        : "memory");
  }
}

}  // namespace sva
