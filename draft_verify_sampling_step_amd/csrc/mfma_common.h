// mfma_common.h -- device helpers shared by the matrix-core bias kernels: operand types,
// the Philox4x32-10 stream, the base-2 Gumbel offset, LDS DMA and explicit wait counts.
#pragma once

#include <type_traits>

#include "dspark_dev.h"

namespace dspark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

constexpr int kR = 256;                    // Markov rank handled by this path
constexpr int kKS = kR / 16;               // MFMA k-steps
constexpr int kPairBytes = 1024 + 32;      // two W2t rows (chunk-interleaved) + pad
constexpr int kTileBytes = 16 * kPairBytes;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -3.0e38f;        // finite "minus infinity" of the running max

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// a ^ b ^ c in one VALU op (gfx950 three-input bit operation, truth table 0x96)
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// The same with a wave-uniform third operand read straight from a scalar register (one
// scalar operand per VALU instruction is allowed), which saves a copy into a VGPR.
__device__ __forceinline__ uint32_t xor3s(uint32_t a, uint32_t b, uint32_t k) {
  uint32_t r;
  asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x96" : "=v"(r) : "v"(a), "v"(b), "s"(k));
  return r;
}

// Philox4x32-10 [SALMON] for counters (c0, k, b, s) whose last three words are fixed per
// lane: the R1 * c2 half of the first round is computed once (PhiloxLane) and the word
// fed to each call is c0 alone.
struct PhiloxLane {
  uint32_t n0;     // round-1 output word 0: hi(R1 * b) ^ k ^ key0
  uint32_t n1;     // round-1 output word 1: lo(R1 * b)
  uint32_t x3k1;   // s ^ key1, the other operand of round-1 word 2
  uint32_t key0, key1;
};

__device__ __forceinline__ PhiloxLane philox_lane(uint32_t k, uint32_t b, uint32_t s,
                                                  uint32_t key0, uint32_t key1) {
  const uint64_t p1 = (uint64_t)0xCD9E8D57u * b;
  PhiloxLane p;
  p.n0 = (uint32_t)(p1 >> 32) ^ k ^ key0;
  p.n1 = (uint32_t)p1;
  p.x3k1 = s ^ key1;
  p.key0 = key0;
  p.key1 = key1;
  return p;
}

__device__ __forceinline__ U4 philox_call(uint32_t c0, const PhiloxLane& pl) {
  const uint64_t q0 = (uint64_t)0xD2511F53u * c0;
  uint32_t x0 = pl.n0, x1 = pl.n1, x2 = (uint32_t)(q0 >> 32) ^ pl.x3k1, x3 = (uint32_t)q0;
  uint32_t k0 = pl.key0, k1 = pl.key1;
#pragma unroll
  for (int round = 1; round < 10; ++round) {
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
    const uint64_t p0 = (uint64_t)0xD2511F53u * x0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2;
    const uint32_t n0 = xor3((uint32_t)(p1 >> 32), x1, k0);
    const uint32_t n2 = xor3((uint32_t)(p0 >> 32), x3, k1);
    x1 = (uint32_t)p1;
    x3 = (uint32_t)p0;
    x0 = n0;
    x2 = n2;
  }
  return U4{x0, x1, x2, x3};
}

// N calls of one lane at counters c0[0..N-1], computed round by round in lockstep so that
// the multiplies of the calls are independent instructions (a wave has few peers on its
// SIMD to hide the latency of one call's dependent chain).
template <int N>
__device__ __forceinline__ void philox_calls(const uint32_t (&c0)[N], const PhiloxLane& pl,
                                             uint32_t (&w)[N][4]) {
  uint32_t x0[N], x1[N], x2[N], x3[N];
#pragma unroll
  for (int g = 0; g < N; ++g) {
    const uint64_t q0 = (uint64_t)0xD2511F53u * c0[g];
    x0[g] = pl.n0;
    x1[g] = pl.n1;
    x2[g] = (uint32_t)(q0 >> 32) ^ pl.x3k1;
    x3[g] = (uint32_t)q0;
  }
  uint32_t k0 = pl.key0, k1 = pl.key1;
#pragma unroll
  for (int round = 1; round < 10; ++round) {
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
#pragma unroll
    for (int g = 0; g < N; ++g) {
      const uint64_t p0 = (uint64_t)0xD2511F53u * x0[g];
      const uint64_t p1 = (uint64_t)0xCD9E8D57u * x2[g];
      const uint32_t n0 = xor3s((uint32_t)(p1 >> 32), x1[g], k0);
      const uint32_t n2 = xor3s((uint32_t)(p0 >> 32), x3[g], k1);
      x1[g] = (uint32_t)p1;
      x3[g] = (uint32_t)p0;
      x0[g] = n0;
      x2[g] = n2;
    }
  }
#pragma unroll
  for (int g = 0; g < N; ++g) {
    w[g][0] = x0[g];
    w[g][1] = x1[g];
    w[g][2] = x2[g];
    w[g][3] = x3[g];
  }
}

// Base-2 Gumbel score offset: -log2(-log2 u) (the common constant -log2(ln 2) is dropped,
// it shifts every candidate of a race equally).  u = (2 (w >> 9) + 1) 2^-24 is formed as
// the float 1.m with mantissa w >> 9 (one alignbit) minus (1 - 2^-24), which is exact.
__device__ __forceinline__ float neg_lglg(uint32_t w) {
  const float one_m = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u));
  return -lg2(-lg2(one_m - 0x1.fffffep-1f));
}

// The W2t ring is filled by LDS DMA issued from inline assembly, and everything that orders
// it is inline assembly too, so the compiler's own wait-count bookkeeping never sees the
// DMA: it still counts the ordinary logit loads exactly, and since the DMA only adds to
// the hardware count, the waits it derives stay sufficient.
//
// One global_load_lds_dwordx4: 16 bytes per lane from gbase + voff (saddr form) into LDS
// at lds + 16 * lane.  M0 carries the LDS address and is restored afterwards.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(voff), "s"(gbase)
      : "memory");
}

// The same with a per-lane 64-bit source address.
__device__ __forceinline__ void dma16v(const void* src, uint32_t lds) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(src)
      : "memory");
}

// wait until at most N vector-memory operations of this wave are outstanding (loads,
// including the DMA, complete in issue order)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"i"(N) : "memory");
}

// Workgroup barrier without the release fence of __syncthreads() (which would drain every
// outstanding load).  Each wave waits for its own DMA before it and has consumed its own
// LDS reads of the previous step; the memory clobber keeps LDS accesses on their side.
__device__ __forceinline__ void barrier_no_fence() { asm volatile("s_barrier" ::: "memory"); }

// f(step + I, integral_constant<I>, integral_constant<BASE>) for I = I0 .. N-1; BASE >= 0
// says that step == BASE at compile time, BASE < 0 that it is known at run time only
template <int I, int N, int BASE, typename F>
__device__ __forceinline__ void unroll_steps(int step, F& f) {
  if constexpr (I < N) {
    f(step + I, std::integral_constant<int, I>{}, std::integral_constant<int, BASE>{});
    unroll_steps<I + 1, N, BASE>(step, f);
  }
}

// the first TRIPS trips of UD steps, with their step numbers known at compile time
template <int T, int TRIPS, int UD, typename F>
__device__ __forceinline__ void peel_trips(F& f) {
  if constexpr (T < TRIPS) {
    unroll_steps<0, UD, T * UD>(T * UD, f);
    peel_trips<T + 1, TRIPS, UD>(f);
  }
}

}  // namespace dspark
