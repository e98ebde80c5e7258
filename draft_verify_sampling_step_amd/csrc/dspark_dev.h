// dspark_dev.h -- device helpers shared by the gfx950 kernels of the DSpark round.
//
// Counter-based randomness (Philox4x32-10, Salmon et al. SC'11), bf16 loads, the
// order-preserving (score, index) packing used for cross-workgroup argmax with a 64-bit
// atomic max, and wave/workgroup reductions for wave64.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int kWave = 64;

// ------------------------------------------------------------------------------------
// Philox4x32-10: ten rounds of two 32x32->64 multiplies; key bumped between rounds.
// ------------------------------------------------------------------------------------
struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                       uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = 0; round < 10; ++round) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return U4{c0, c1, c2, c3};
}

// The four uniforms of vocab indices 4q..4q+3 at (seed, b, k, s):
// u = (2 * (W >> 9) + 1) * 2^-24, computed exactly in fp32.
__device__ __forceinline__ float word_to_uniform(uint32_t w) {
  return fmaf((float)(w >> 9), 0x1p-23f, 0x1p-24f);
}

// Gumbel noise G = -ln(-ln u) from hardware log2 (accurate to ~1.2e-7 relative over the
// whole lattice of u, including u -> 1):  -ln u = -ln2 * log2 u,  G = -ln2 * log2(-ln u).
__device__ __forceinline__ float gumbel_from_uniform(float u) {
  const float e = -0.69314718055994531f * __builtin_amdgcn_logf(u);
  return -0.69314718055994531f * __builtin_amdgcn_logf(e);
}

// exp(x) through the hardware exp2.
__device__ __forceinline__ float fast_exp(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}
__device__ __forceinline__ float fast_log(float x) {
  return 0.69314718055994531f * __builtin_amdgcn_logf(x);
}

// A token id used as an index, clamped into [0, V): ids outside the vocabulary (caller
// error, or a position whose logits were all -inf/NaN so that no candidate won) never
// address memory outside the tables.
__device__ __forceinline__ int clamp_tok(int x, int V) {
  return x < 0 ? 0 : (x >= V ? V - 1 : x);
}

// ------------------------------------------------------------------------------------
// bf16 / fp32 element access
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float get(const float* p, size_t i) { return p[i]; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float get(const uint16_t* p, size_t i) {
    return bf16_to_f32(p[i]);
  }
};

// ------------------------------------------------------------------------------------
// (score, index) packing: larger packed value = larger score, then smaller index.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ unsigned long long pack_score(float s, uint32_t idx) {
  uint32_t b = __float_as_uint(s);
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((unsigned long long)b << 32) | (unsigned long long)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t packed_index(unsigned long long p) {
  return 0xFFFFFFFFu - (uint32_t)(p & 0xFFFFFFFFull);
}
__device__ __forceinline__ float packed_score(unsigned long long p) {
  uint32_t b = (uint32_t)(p >> 32);
  b = (b & 0x80000000u) ? (b & 0x7FFFFFFFu) : ~b;
  return __uint_as_float(b);
}
__device__ __forceinline__ void atomic_max_u64(unsigned long long* p, unsigned long long v) {
  __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------------
// Cross-workgroup hand-off without hot spots: workgroup w of a launch posts its packed
// winners with atomic maxima into sub-slot w % kSubSlots (so at most n / kSubSlots
// workgroups share an address), then counts itself in on a two-level counter; exactly one
// workgroup, the last to arrive, gets true and may read the merged sub-slots.  Each wave
// waits for its own atomics before the workgroup barrier that precedes the count, and all
// of these are device-scope atomics, performed at the device's coherence point in that
// order.  `c` is a block of kArriveInts zeroed counters (9 counters 128 bytes apart).
// ------------------------------------------------------------------------------------
constexpr int kSubSlots = 8;
constexpr int kArriveInts = 9 * 32;

__device__ __forceinline__ bool arrive_last(int32_t* c, int w, int n) {
  const int sub = w % kSubSlots;
  const int in_sub = n / kSubSlots + (sub < n % kSubSlots ? 1 : 0);
  const int nsub = n < kSubSlots ? n : kSubSlots;
  if (__hip_atomic_fetch_add(c + 32 * sub, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
      in_sub - 1)
    return false;
  return __hip_atomic_fetch_add(c + 32 * kSubSlots, 1, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT) == nsub - 1;
}

__device__ __forceinline__ unsigned long long atomic_load_u64(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ------------------------------------------------------------------------------------
// online softmax state (running max m, running sum l of exp(z - m))
// ------------------------------------------------------------------------------------
struct ML { float m, l; };

__device__ __forceinline__ ML ml_merge(ML a, ML b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return ML{-INFINITY, 0.f};
  return ML{m, a.l * fast_exp(a.m - m) + b.l * fast_exp(b.m - m)};
}

// Candidate of an argmax race: score, index, and the logit at that index.
struct Cand { float s; uint32_t i; float z; };

__device__ __forceinline__ bool cand_better(const Cand& a, const Cand& b) {
  return a.s > b.s || (a.s == b.s && a.i < b.i);
}

// ------------------------------------------------------------------------------------
// wave64 reductions
// ------------------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ ML wave_ml(ML a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    ML b{__shfl_xor(a.m, o, kWave), __shfl_xor(a.l, o, kWave)};
    a = ml_merge(a, b);
  }
  return a;
}
__device__ __forceinline__ Cand wave_cand(Cand a) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Cand b{__shfl_xor(a.s, o, kWave), (uint32_t)__shfl_xor((int)a.i, o, kWave),
           __shfl_xor(a.z, o, kWave)};
    if (cand_better(b, a)) a = b;
  }
  return a;
}

}  // namespace dspark
