// rowbias.h -- Markov-bias rows for one request at a time (the GEMV form of
// bias(v) = sum_i W1[prev][i] * W2t[v][i]), used by the row kernels.
//
// A workgroup of 256 threads computes one tile of 256 vocab rows: eight lanes share a
// W2t row (each lane reads a contiguous r/8 slice with 16-byte loads, then the eight
// partial sums are combined with xor-shuffles), 32 rows per pass, 8 passes per tile.  For
// bf16 weights of rank 256 the loads of four passes are in flight together.
#pragma once

#include "dspark_dev.h"

namespace dspark {

template <typename WT>
__device__ __forceinline__ float dot_chunk(const WT* w, const float* a, int len);

template <>
__device__ __forceinline__ float dot_chunk<uint16_t>(const uint16_t* w, const float* a,
                                                     int len) {
  float acc = 0.f;
  if ((len & 7) == 0) {
    for (int i = 0; i < len; i += 8) {
      const uint4 q = *reinterpret_cast<const uint4*>(w + i);
      const uint32_t e[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc = fmaf(a[i + 2 * j], __uint_as_float(e[j] << 16), acc);
        acc = fmaf(a[i + 2 * j + 1], __uint_as_float(e[j] & 0xFFFF0000u), acc);
      }
    }
  } else {
    for (int i = 0; i < len; ++i) acc = fmaf(a[i], bf16_to_f32(w[i]), acc);
  }
  return acc;
}

template <>
__device__ __forceinline__ float dot_chunk<float>(const float* w, const float* a, int len) {
  float acc = 0.f;
  if ((len & 3) == 0) {
    for (int i = 0; i < len; i += 4) {
      const float4 q = *reinterpret_cast<const float4*>(w + i);
      acc = fmaf(a[i], q.x, acc);
      acc = fmaf(a[i + 1], q.y, acc);
      acc = fmaf(a[i + 2], q.z, acc);
      acc = fmaf(a[i + 3], q.w, acc);
    }
  } else {
    for (int i = 0; i < len; ++i) acc = fmaf(a[i], w[i], acc);
  }
  return acc;
}

// Load the Markov embedding row W1[prev] into LDS as fp32 (all threads participate).
template <typename WT>
__device__ __forceinline__ void load_w1_row(const WT* W1, int prev, int r, float* w1s) {
  for (int i = threadIdx.x; i < r; i += blockDim.x)
    w1s[i] = Elem<WT>::get(W1, (size_t)prev * r + i);
}

// bias_s[t] = W1[prev] . W2t[tile0 + t] for t < 256 (0 for rows at or past v_end).
// Requires blockDim.x == 256; the caller synchronises before reading bias_s.
template <typename WT>
__device__ __forceinline__ void row_bias_tile(const WT* W2t, const float* w1s, float* bias_s,
                                              int r, int tile0, int v_end) {
  const int tid = threadIdx.x, sub = tid & 7, rowi = tid >> 3;
  const int len = r >> 3, i0 = sub * len;
  if constexpr (sizeof(WT) == 2) {
    if (r == 256) {
      // bf16, rank 256: each lane's slice is 32 elements (four 16-byte loads).  Four passes'
      // loads are issued before any is used; rows at or past v_end load row v_end - 1 and
      // report 0.
      for (int pass0 = 0; pass0 < 8; pass0 += 4) {
        uint4 q[4][4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int v = min(tile0 + (pass0 + p) * 32 + rowi, v_end - 1);
          const uint4* src = reinterpret_cast<const uint4*>(W2t + (size_t)v * 256 + i0);
#pragma unroll
          for (int c = 0; c < 4; ++c) q[p][c] = src[c];
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint32_t e[4] = {q[p][c].x, q[p][c].y, q[p][c].z, q[p][c].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              acc = fmaf(w1s[i0 + 8 * c + 2 * j], __uint_as_float(e[j] << 16), acc);
              acc = fmaf(w1s[i0 + 8 * c + 2 * j + 1], __uint_as_float(e[j] & 0xFFFF0000u), acc);
            }
          }
          acc += __shfl_xor(acc, 1, kWave);
          acc += __shfl_xor(acc, 2, kWave);
          acc += __shfl_xor(acc, 4, kWave);
          const int t = (pass0 + p) * 32 + rowi;
          if (sub == 0) bias_s[t] = tile0 + t < v_end ? acc : 0.f;
        }
      }
      return;
    }
  }
  for (int pass = 0; pass < 8; ++pass) {
    const int t = pass * 32 + rowi;
    const int v = tile0 + t;
    float acc = 0.f;
    if (v < v_end) acc = dot_chunk<WT>(W2t + (size_t)v * r + i0, w1s + i0, len);
    acc += __shfl_xor(acc, 1, kWave);
    acc += __shfl_xor(acc, 2, kWave);
    acc += __shfl_xor(acc, 4, kWave);
    if (sub == 0) bias_s[t] = acc;
  }
}

// Workgroup (256 threads) reductions through LDS scratch of >= 4 entries per value.
__device__ __forceinline__ ML block_ml(ML a, float* sm, float* sl) {
  a = wave_ml(a);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) { sm[w] = a.m; sl[w] = a.l; }
  __syncthreads();
  ML r{sm[0], sl[0]};
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = ml_merge(r, ML{sm[i], sl[i]});
  __syncthreads();
  return r;
}
__device__ __forceinline__ Cand block_cand(Cand a, float* ss, uint32_t* si, float* sz) {
  a = wave_cand(a);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) { ss[w] = a.s; si[w] = a.i; sz[w] = a.z; }
  __syncthreads();
  Cand r{ss[0], si[0], sz[0]};
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) {
    Cand b{ss[i], si[i], sz[i]};
    if (cand_better(b, r)) r = b;
  }
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* sv) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) sv[w] = v;
  __syncthreads();
  float r = sv[0];
  for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r += sv[i];
  __syncthreads();
  return r;
}

}  // namespace dspark
