// verify.hip -- rejection-sampling verification [XTL §1; AIMSG concept 2; CSDN roundtable:
// accept with probability min(1, p_t/p_d)], lossless: the emitted tokens follow the
// target distribution.
//
//  1. k_verify_rows    one streaming pass over the target rows 1..ell_b+1 of every request
//                      (a flattened ragged set; workgroups of unused rows exit at once):
//                      split-vocabulary (max, sum-exp) partials of T/temperature, and on
//                      row ell_b+1 the Gumbel race of the bonus token (atomic max).
//  2. k_verify_decide  per request: lse of each row, p_t(x_k), the ordered accept tests
//                      u * p_d(x_k) < p_t(x_k); n_b; the accepted prefix; the bonus token
//                      when nothing was rejected, else the residual row j = n_b + 1.
//  3. residual         for rejected requests, the draft row j is recomputed (Markov bias
//                      for x_{j-1} plus U_j) and the residual max(0, p_t - p_d) is sampled
//                      by a Gumbel race on ln rho (bf16 MFMA path for many requests, GEMV
//                      rows otherwise); a p_t race on the same noise covers the case where
//                      rounding leaves no positive residual.
//  4. k_verify_final   writes the residual/fallback token after the accepted prefix.
#include "dspark_dev.h"
#include "dspark_host.h"
#include "mfma_bias.h"
#include "mfma_common.h"
#include "rowbias.h"

namespace dspark {

// 16-byte loads per thread and item of the target-row pass (an item is 4 * 256 * this many
// entries of one row)
constexpr int kVerifyQuads = 8;

// Flattened ragged row list: rows (b, k) with k <= ell_b + 1, in request order.  One
// workgroup; writes the list, its length and the number of (row, slice) work items, and
// clears the bonus-race words.
__global__ __launch_bounds__(256) void k_verify_plan(const int32_t* __restrict__ ell, int B,
                                                     int G, int nslices,
                                                     int32_t* __restrict__ rows,
                                                     int32_t* __restrict__ counts,
                                                     unsigned long long* __restrict__ bonus) {
  __shared__ int32_t scan[256];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  for (int b = tid; b < B; b += 256) bonus[b] = 0ull;
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int b0 = 0; b0 < B; b0 += 256) {
    const int b = b0 + tid;
    int n = 0;
    if (b < B) {
      const int L = ell[b];
      n = (L < 0 ? 0 : (L > G ? G : L)) + 1;
    }
    scan[tid] = n;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {
      const int add = tid >= o ? scan[tid - o] : 0;
      __syncthreads();
      scan[tid] += add;
      __syncthreads();
    }
    const int start = carry + scan[tid] - n;
    for (int i = 0; i < n; ++i) rows[start + i] = b * (G + 1) + i;   // row id b*(G+1) + (k-1)
    __syncthreads();
    if (tid == 255) carry += scan[255];
    __syncthreads();
  }
  if (tid == 0) {
    counts[0] = carry;
    counts[1] = carry * nslices;
  }
}

// Grid-stride over (row, slice) items.  Rows 1..ell_b: split-vocabulary (max, sum-exp)
// partials of T/temperature (base 2).  Row ell_b + 1 needs no normaliser (only its bonus
// token is drawn from it): the Gumbel race over it, merged by a 64-bit atomic max.
__global__ __launch_bounds__(256, 8) void k_verify_rows(
    const float* __restrict__ T, const int32_t* __restrict__ ell,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ counts, int G, int V,
    int slice_len, int nslices, float invT, uint32_t key0, uint32_t key1,
    float2* __restrict__ part, unsigned long long* __restrict__ bonus) {
  __shared__ float red[16];
  const int nitems = counts[1];
  const float s2 = invT * 1.4426950408889634f;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
    const int row = rows[item / nslices], s = item % nslices;
    const int b = row / (G + 1), k = row % (G + 1) + 1;
    const int Lb = ell[b];
    const bool is_bonus = (k == (Lb < 0 ? 0 : (Lb > G ? G : Lb)) + 1);
    const int v_begin = s * slice_len, v_end = min(V, v_begin + slice_len);
    const float* trow = T + (size_t)row * V;
    if ((V & 3) == 0 && slice_len == 4 * 256 * kVerifyQuads) {
      // every thread's eight 16-byte loads are issued before any is consumed; entries past
      // the slice read as -inf
      constexpr int kQ = kVerifyQuads;
      f32x4_t q[kQ];
#pragma unroll
      for (int i = 0; i < kQ; ++i) {
        const int v = v_begin + 4 * (threadIdx.x + 256 * i);
        q[i] = v < v_end ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(trow + v))
                         : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
      if (!is_bonus) {
        // max first (a finite floor when every entry is padding), then one exponential per
        // entry
        float mq = -INFINITY;
#pragma unroll
        for (int i = 0; i < kQ; ++i)
          mq = fmaxf(mq, fmaxf(fmaxf(q[i][0], q[i][1]), fmaxf(q[i][2], q[i][3])));
        float m = fmaxf(mq * s2, -3.0e38f);
        float lp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kQ; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) lp[j] += ex2(fmaf(q[i][j], s2, -m));
        float l = (lp[0] + lp[1]) + (lp[2] + lp[3]);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          const float om = __shfl_xor(m, o, kWave), ol = __shfl_xor(l, o, kWave);
          const float mn = fmaxf(m, om);
          l = l * ex2(m - mn) + ol * ex2(om - mn);
          m = mn;
        }
        if (lane == 0) { red[wv] = m; red[4 + wv] = l; }
        __syncthreads();
        if (threadIdx.x == 0) {
          float mm = red[0], ll = red[4];
          for (int i = 1; i < 4; ++i) {
            const float mn = fmaxf(mm, red[i]);
            ll = ll * ex2(mm - mn) + red[4 + i] * ex2(red[i] - mn);
            mm = mn;
          }
          part[(size_t)row * nslices + s] = make_float2(mm, ll);
        }
        __syncthreads();
      } else {
        // four consecutive entries share one Philox call (words 0..3); the calls of a
        // batch run in lockstep
        const PhiloxLane pl = philox_lane((uint32_t)k, (uint32_t)b, 2u, key0, key1);
        Cand best{-INFINITY, 0xFFFFFFFFu, 0.f};
#pragma unroll
        for (int i0 = 0; i0 < kQ; i0 += 4) {
          uint32_t c0[4], w[4][4];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            c0[i] = (uint32_t)((v_begin + 4 * (threadIdx.x + 256 * (i0 + i))) >> 2);
          philox_calls<4>(c0, pl, w);
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float sc = fmaf(q[i0 + i][j], s2, neg_lglg(w[i][j]));
              if (sc > best.s) best = Cand{sc, 4 * c0[i] + (uint32_t)j, 0.f};
            }
        }
        best = block_cand(best, red + 8, reinterpret_cast<uint32_t*>(red + 12), red + 4);
        if (threadIdx.x == 0 && best.i != 0xFFFFFFFFu)
          atomic_max_u64(&bonus[b], pack_score(best.s, best.i));
      }
      continue;
    }
    // any other vocabulary size: one entry per thread and step, online state
    float m = -3.0e38f, l = 0.f;
    Cand best{-INFINITY, 0xFFFFFFFFu, 0.f};
    for (int v = v_begin + threadIdx.x; v < v_end; v += 256) {
      const float z = trow[v] * s2;
      if (is_bonus) {
        const U4 w = philox10((uint32_t)v >> 2, (uint32_t)k, (uint32_t)b, 2u, key0, key1);
        const uint32_t word = (v & 3) == 0 ? w.x : (v & 3) == 1 ? w.y : (v & 3) == 2 ? w.z : w.w;
        const float sc = z - __builtin_amdgcn_logf(-__builtin_amdgcn_logf(word_to_uniform(word)));
        if (sc > best.s) best = Cand{sc, (uint32_t)v, 0.f};
      } else {
        const float mn = fmaxf(m, z);
        l = l * ex2(m - mn) + ex2(z - mn);
        m = mn;
      }
    }
    if (!is_bonus) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float om = __shfl_xor(m, o, kWave), ol = __shfl_xor(l, o, kWave);
        const float mn = fmaxf(m, om);
        l = l * ex2(m - mn) + ol * ex2(om - mn);
        m = mn;
      }
      if (lane == 0) { red[wv] = m; red[4 + wv] = l; }
      __syncthreads();
      if (threadIdx.x == 0) {
        float mm = red[0], ll = red[4];
        for (int i = 1; i < 4; ++i) {
          const float mn = fmaxf(mm, red[i]);
          ll = ll * ex2(mm - mn) + red[4 + i] * ex2(red[i] - mn);
          mm = mn;
        }
        part[(size_t)row * nslices + s] = make_float2(mm, ll);
      }
      __syncthreads();
    } else {
      best = block_cand(best, red + 8, reinterpret_cast<uint32_t*>(red + 12), red + 4);
      if (threadIdx.x == 0 && best.i != 0xFFFFFFFFu)
        atomic_max_u64(&bonus[b], pack_score(best.s, best.i));
    }
  }
}

// One wave per request, one lane per draft row k = lane + 1 (gamma <= 64): all rows of a
// request are decided at once.  Lane k merges the base-2 slice partials of target row k in
// slice order into its lse, then takes p_t(x_k) and the accept test u * p_d(x_k) < p_t(x_k).
// The accepted prefix ends at the first rejected row, found by a ballot.
__global__ __launch_bounds__(256) void k_verify_decide(
    const float* __restrict__ T, const int32_t* __restrict__ tokens,
    const float* __restrict__ logp, const int32_t* __restrict__ ell,
    const float2* __restrict__ part, const unsigned long long* __restrict__ bonus, int B, int G,
    int V, int nslices, float invT, uint32_t key0, uint32_t key1,
    int32_t* __restrict__ n_accept, int32_t* __restrict__ out_tokens,
    float* __restrict__ pt_tok, int32_t* __restrict__ jrow, float* __restrict__ lse_t_row) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= B) return;
  const int Lb = ell[b];
  const int L = Lb < 0 ? 0 : (Lb > G ? G : Lb);   // ell outside [0, gamma] is clamped
  const int k = lane + 1;
  const bool live = k <= L;
  float lt = 0.f, pt = __builtin_nanf("");
  bool rejected = false;
  if (live) {
    const size_t row = (size_t)b * (G + 1) + (k - 1);
    const int x = clamp_tok(tokens[(size_t)b * G + (k - 1)], V);
    const float tx = T[row * V + x];
    const float lp = logp[(size_t)b * G + (k - 1)];
    const float2* p = part + row * nslices;
    float m = -3.0e38f, l = 0.f;
#pragma unroll 4
    for (int s = 0; s < nslices; ++s) {
      const float2 q = p[s];
      const float mn = fmaxf(m, q.x);
      l = l * __builtin_amdgcn_exp2f(m - mn) + q.y * __builtin_amdgcn_exp2f(q.x - mn);
      m = mn;
    }
    lt = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
    pt = fast_exp(tx * invT - lt);
    const U4 w = philox10(0u, (uint32_t)k, (uint32_t)b, 1u, key0, key1);
    rejected = !(word_to_uniform(w.x) * fast_exp(lp) < pt);
  }
  if (pt_tok && k <= G) pt_tok[(size_t)b * G + (k - 1)] = pt;
  const unsigned long long rej = __ballot(rejected);   // bit k-1: row k rejected
  const int n = rej ? __builtin_ctzll(rej) : L;          // leading accepts
  const int j = rej ? n + 1 : 0;                         // residual row, 0 = none
  const float lj = __shfl(lt, j > 0 ? j - 1 : 0, kWave);
  int32_t* out = out_tokens + (size_t)b * (G + 1);
  for (int i = lane; i <= G; i += kWave) out[i] = i < n ? tokens[(size_t)b * G + i] : -1;
  if (lane == 0) {
    if (j == 0) out[n] = (int32_t)packed_index(bonus[b]);
    n_accept[b] = n;
    jrow[b] = j;
    lse_t_row[b] = j > 0 ? lj : 0.f;
  }
}

// Row residual: grid (slices, B), 256 threads.
template <typename WT>
__global__ __launch_bounds__(256) void k_verify_resid_row(
    const float* __restrict__ U, const WT* __restrict__ W1, const WT* __restrict__ W2t,
    const float* __restrict__ T, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ lse_d,
    const int32_t* __restrict__ jrow, const float* __restrict__ lse_t_row, int B, int G, int V,
    int r, int slice_len, float invT, uint32_t key0, uint32_t key1,
    float4* __restrict__ res_part) {
  extern __shared__ float smem[];
  float* w1s = smem;
  float* bias_s = smem + r;
  float* red = bias_s + 256;
  const int s = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int j = jrow[b];
  if (j == 0) return;
  const int prev = clamp_tok((j == 1) ? anchor[b] : tokens[(size_t)b * G + (j - 2)], V);
  const int v_begin = s * slice_len, v_end = min(V, v_begin + slice_len);
  load_w1_row<WT>(W1, prev, r, w1s);
  __syncthreads();
  const float ld = lse_d[(size_t)b * G + (j - 1)], lt = lse_t_row[b];
  const float* urow = U + ((size_t)b * G + (j - 1)) * V;
  const float* trow = T + ((size_t)b * (G + 1) + (j - 1)) * V;
  Cand b1{-INFINITY, 0xFFFFFFFFu, 0.f}, b2{-INFINITY, 0xFFFFFFFFu, 0.f};
  for (int tile0 = v_begin; tile0 < v_end; tile0 += kRowTile) {
    row_bias_tile<WT>(W2t, w1s, bias_s, r, tile0, v_end);
    __syncthreads();
    const int v = tile0 + tid;
    if (v < v_end) {
      const float zd = (urow[v] + bias_s[tid]) * invT;
      const float zt = trow[v] * invT;
      const float rho = fast_exp(zt - lt) - fast_exp(zd - ld);
      const U4 w = philox10((uint32_t)v >> 2, (uint32_t)j, (uint32_t)b, 2u, key0, key1);
      const uint32_t word = (v & 3) == 0 ? w.x : (v & 3) == 1 ? w.y : (v & 3) == 2 ? w.z : w.w;
      const float gn = gumbel_from_uniform(word_to_uniform(word));
      if (rho > 0.f) {
        const float sc = fast_log(rho) + gn;
        if (sc > b1.s) b1 = Cand{sc, (uint32_t)v, 0.f};
      }
      const float sc2 = zt + gn;
      if (sc2 > b2.s) b2 = Cand{sc2, (uint32_t)v, 0.f};
    }
    __syncthreads();
  }
  b1 = block_cand(b1, red, reinterpret_cast<uint32_t*>(red + 4), red + 8);
  b2 = block_cand(b2, red, reinterpret_cast<uint32_t*>(red + 4), red + 8);
  if (tid == 0)
    res_part[(size_t)s * B + b] =
        make_float4(b1.s, __uint_as_float(b1.i), b2.s, __uint_as_float(b2.i));
}

// Thin residual pass, for at most kThinMax requests with a residual row (the usual case:
// few rejections per round) and bf16 weights of rank kR.  Grid: the nslices slices of the
// residual partials; 256 threads.  Every workgroup first lists the requests with a residual
// row in request order and leaves at once unless there are 1..kThinMax of them (the matrix-
// core pass takes more, and leaves at once in this case).  Each wave then takes four
// vocabulary rows per step, 16 lanes per row: lane part p holds elements 16 p .. 16 p + 15
// of W2t[v] and of every listed request's W1[x_{j-1}], the dot products are summed over the
// 16 lanes, and lane p < n runs the residual and fallback races of request p on row v with
// the same arithmetic as the row kernel above.
constexpr int kThinMax = 2;

// Sum over each 16-lane row of the wave by DPP moves (quad swaps 1,0,3,2 and 2,3,0,1, then
// the half-row and row mirrors): each step adds a commutative pair, so all 16 lanes end
// with the same total.
__device__ __forceinline__ float dpp_row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

__global__ __launch_bounds__(256) void k_verify_resid_thin(
    const float* __restrict__ U, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W2t, const float* __restrict__ T,
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ tokens,
    const float* __restrict__ lse_d, const int32_t* __restrict__ jrow,
    const float* __restrict__ lse_t_row, int B, int G, int V, float invT, uint32_t key0,
    uint32_t key1, int nslices, float4* __restrict__ res_part) {
  __shared__ int s_list[kThinMax];
  __shared__ int s_cnt;
  __shared__ float4 s_cand[16][kThinMax];   // [wave * 4 + row quad][request]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (wave == 0) {
    int cnt = 0;
    for (int c0 = 0; c0 < B; c0 += kWave) {
      const int bb = c0 + lane;
      const bool act = bb < B && jrow[bb] > 0;
      const unsigned long long bal = __ballot(act);
      const int at = cnt + __popcll(bal & ((1ull << lane) - 1ull));
      if (act && at < kThinMax) s_list[at] = bb;
      cnt += __popcll(bal);
    }
    if (lane == 0) s_cnt = cnt;
  }
  __syncthreads();
  const int n = s_cnt;
  if (n == 0 || n > kThinMax) return;

  const int part = lane & 15, quad = lane >> 4;
  float w1[kThinMax][16];
  const float* urow = U;
  const float* trow = T;
  float ld = 0.f, lt = 0.f;
  int myb = 0, myj = 1;
#pragma unroll
  for (int i = 0; i < kThinMax; ++i) {
    int b = 0, j = 1;
    if (i < n) { b = s_list[i]; j = jrow[b]; }
    const int prev = clamp_tok((j == 1) ? anchor[b] : tokens[(size_t)b * G + (j - 2)], V);
    const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(W1 + (size_t)prev * kR + 16 * part);
    const u32x4_t q0 = wp[0], q1 = wp[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w1[i][2 * e] = __uint_as_float(q0[e] << 16);
      w1[i][2 * e + 1] = __uint_as_float(q0[e] & 0xFFFF0000u);
      w1[i][8 + 2 * e] = __uint_as_float(q1[e] << 16);
      w1[i][8 + 2 * e + 1] = __uint_as_float(q1[e] & 0xFFFF0000u);
    }
    if (i == part && i < n) {
      myb = b;
      myj = j;
      urow = U + ((size_t)b * G + (j - 1)) * V;
      trow = T + ((size_t)b * (G + 1) + (j - 1)) * V;
      ld = lse_d[(size_t)b * G + (j - 1)];
      lt = lse_t_row[b];
    }
  }
  const int len = (V + nslices - 1) / nslices;
  const int vb = blockIdx.x * len, ve = min(V, vb + len);
  Cand c1{-INFINITY, 0xFFFFFFFFu, 0.f}, c2{-INFINITY, 0xFFFFFFFFu, 0.f};
  // four row groups per iteration (rows v0 + 16 u + quad), every load issued first; rows
  // past the slice load row v0 and are not raced
  for (int v0 = vb + 4 * wave; v0 < ve; v0 += 64) {
    u32x4_t xq[4][2];
    float uq[4], tq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vu = v0 + 16 * u + quad;
      const int vv = vu < ve ? vu : v0;
      const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(W2t + (size_t)vv * kR + 16 * part);
      xq[u][0] = xp[0];
      xq[u][1] = xp[1];
      uq[u] = urow[vv];
      tq[u] = trow[vv];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + 16 * u + quad;
      float xf[16];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xf[2 * e] = __uint_as_float(xq[u][0][e] << 16);
        xf[2 * e + 1] = __uint_as_float(xq[u][0][e] & 0xFFFF0000u);
        xf[8 + 2 * e] = __uint_as_float(xq[u][1][e] << 16);
        xf[8 + 2 * e + 1] = __uint_as_float(xq[u][1][e] & 0xFFFF0000u);
      }
      float d[kThinMax];
#pragma unroll
      for (int i = 0; i < kThinMax; ++i) {
        d[i] = 0.f;
        if (i < n) {   // uniform
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc = fmaf(xf[e], w1[i][e], acc);
          d[i] = dpp_row_sum16(acc);
        }
      }
      if (v < ve && part < n) {
        float bias = d[0];
#pragma unroll
        for (int i = 1; i < kThinMax; ++i) bias = part == i ? d[i] : bias;
        const float zd = (uq[u] + bias) * invT;
        const float zt = tq[u] * invT;
        const float rho = fast_exp(zt - lt) - fast_exp(zd - ld);
        const U4 w = philox10((uint32_t)v >> 2, (uint32_t)myj, (uint32_t)myb, 2u, key0, key1);
        const uint32_t word =
            (v & 3) == 0 ? w.x : (v & 3) == 1 ? w.y : (v & 3) == 2 ? w.z : w.w;
        const float gn = gumbel_from_uniform(word_to_uniform(word));
        if (rho > 0.f) {
          const float sc = fast_log(rho) + gn;
          if (sc > c1.s) c1 = Cand{sc, (uint32_t)v, 0.f};
        }
        const float sc2 = zt + gn;
        if (sc2 > c2.s) c2 = Cand{sc2, (uint32_t)v, 0.f};
      }
    }
  }
  // merge the candidates of request p over the 16 (wave, row quad) lanes, ties to the lower
  // index
  if (part < n)
    s_cand[wave * 4 + quad][part] =
        make_float4(c1.s, __uint_as_float(c1.i), c2.s, __uint_as_float(c2.i));
  __syncthreads();
  if (tid < n) {
    float s1 = -INFINITY, s2 = -INFINITY;
    uint32_t i1 = 0xFFFFFFFFu, i2 = 0xFFFFFFFFu;
    for (int g = 0; g < 16; ++g) {
      const float4 p = s_cand[g][tid];
      const uint32_t pi1 = __float_as_uint(p.y), pi2 = __float_as_uint(p.w);
      if (p.x > s1 || (p.x == s1 && pi1 < i1)) { s1 = p.x; i1 = pi1; }
      if (p.z > s2 || (p.z == s2 && pi2 < i2)) { s2 = p.z; i2 = pi2; }
    }
    res_part[(size_t)blockIdx.x * B + s_list[tid]] =
        make_float4(s1, __uint_as_float(i1), s2, __uint_as_float(i2));
  }
}

// One wave per request with a residual row: reduce the residual (and fallback p_t) races
// over the slice partials in a fixed order; write the token after the accepted prefix.
__global__ __launch_bounds__(256) void k_verify_final(const int32_t* __restrict__ jrow,
                                                      const int32_t* __restrict__ n_accept,
                                                      const float4* __restrict__ res_part,
                                                      int nslices, int B, int G,
                                                      int32_t* __restrict__ out_tokens) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (b >= B || jrow[b] == 0) return;
  float s1 = -INFINITY, s2 = -INFINITY;
  uint32_t i1 = 0xFFFFFFFFu, i2 = 0xFFFFFFFFu;
  for (int s = lane; s < nslices; s += kWave) {
    const float4 p = res_part[(size_t)s * B + b];
    const uint32_t pi1 = __float_as_uint(p.y), pi2 = __float_as_uint(p.w);
    if (p.x > s1 || (p.x == s1 && pi1 < i1)) { s1 = p.x; i1 = pi1; }
    if (p.z > s2 || (p.z == s2 && pi2 < i2)) { s2 = p.z; i2 = pi2; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float os1 = __shfl_xor(s1, o, kWave), os2 = __shfl_xor(s2, o, kWave);
    const uint32_t oi1 = (uint32_t)__shfl_xor((int)i1, o, kWave);
    const uint32_t oi2 = (uint32_t)__shfl_xor((int)i2, o, kWave);
    if (os1 > s1 || (os1 == s1 && oi1 < i1)) { s1 = os1; i1 = oi1; }
    if (os2 > s2 || (os2 == s2 && oi2 < i2)) { s2 = os2; i2 = oi2; }
  }
  if (lane == 0) {
    // no positive residual anywhere (rounding): fall back to the p_t race
    const uint32_t y = i1 != 0xFFFFFFFFu ? i1 : i2;
    out_tokens[(size_t)b * (G + 1) + n_accept[b]] = (int32_t)y;
  }
}

}  // namespace dspark

using namespace dspark;

namespace {

struct VerifyWs {
  float2* part;
  int32_t* rows;
  int32_t* counts;
  unsigned long long* bonus;
  float4* res_part;
  int32_t* jrow;
  float* lse_t_row;
  size_t bytes;
};

VerifyWs verify_ws(const dspark_dims* d, int nslices, int nres_slices, void* base) {
  Carve c(base);
  VerifyWs w;
  w.part = c.take<float2>((size_t)d->batch * (d->gamma + 1) * nslices);
  w.rows = c.take<int32_t>((size_t)d->batch * (d->gamma + 1));
  w.counts = c.take<int32_t>(2);
  w.bonus = c.take<unsigned long long>((size_t)d->batch);
  w.res_part = c.take<float4>((size_t)nres_slices * d->batch);
  w.jrow = c.take<int32_t>(d->batch);
  w.lse_t_row = c.take<float>(d->batch);
  w.bytes = align_up(c.off, 256);
  return w;
}

int resid_slices(const dspark_dims* d, bool mfma) {
  return mfma ? mfma_grid(d->vocab, d->batch, kModeResid) : row_slices(d->vocab, d->batch).count;
}

}  // namespace

// Target rows are streamed in slices of kVerifySlice entries per workgroup item.
constexpr int kVerifySlice = 4 * 256 * kVerifyQuads;

size_t dspark_verify_workspace(const dspark_dims* d) {
  const int ns = (d->vocab + kVerifySlice - 1) / kVerifySlice;
  const int nr = std::max(resid_slices(d, true), resid_slices(d, false));
  return verify_ws(d, ns, nr, nullptr).bytes;
}

extern "C" dspark_status dspark_verify(const dspark_dims* dm, const float* U, const void* W1,
                                       const void* W2t, int wdt, const int32_t* anchor,
                                       const int32_t* tokens, const float* logp,
                                       const float* lse, const float* T, const int32_t* ell,
                                       float temperature, uint64_t seed, int32_t* n_accept,
                                       int32_t* out_tokens, float* pt_tok, void* ws,
                                       size_t ws_bytes, void* stream) {
  if (!dm || !U || !W1 || !W2t || !anchor || !tokens || !logp || !lse || !T || !ell ||
      !n_accept || !out_tokens)
    return DSPARK_E_NULL;
  if (!dims_ok(dm)) return DSPARK_E_SHAPE;
  if (!dtype_ok(wdt)) return DSPARK_E_DTYPE;
  if (!temp_ok(temperature)) return DSPARK_E_VALUE;
  if (!ws || ws_bytes < dspark_verify_workspace(dm)) return DSPARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int B = dm->batch, G = dm->gamma, V = dm->vocab, r = dm->rank;
  const int nsl = (V + kVerifySlice - 1) / kVerifySlice;
  const bool mfma = mfma_bias_supported(B, r, wdt);
  const int nres = resid_slices(dm, mfma);
  VerifyWs w = verify_ws(dm, nsl, nres, ws);
  const float invT = 1.0f / temperature;
  const uint32_t key0 = (uint32_t)seed, key1 = (uint32_t)(seed >> 32);
  if (mfma && mfma_prepare() != DSPARK_OK) return DSPARK_E_HIP;

  hipLaunchKernelGGL(k_verify_plan, dim3(1), dim3(256), 0, st, ell, B, G, nsl, w.rows,
                     w.counts, w.bonus);
  const long long max_items = (long long)B * (G + 1) * nsl;
  const int grid = (int)std::min<long long>(max_items, 2048);
  hipLaunchKernelGGL(k_verify_rows, dim3(grid), dim3(256), 0, st, T, ell, w.rows, w.counts, G,
                     V, kVerifySlice, nsl, invT, key0, key1, w.part, w.bonus);
  hipLaunchKernelGGL(k_verify_decide, dim3((B + 3) / 4), dim3(256), 0, st, T, tokens, logp, ell,
                     w.part, w.bonus, B, G, V, nsl, invT, key0, key1, n_accept, out_tokens,
                     pt_tok, w.jrow, w.lse_t_row);
  if (mfma) {
    MfmaBiasArgs a{};
    a.mode = kModeResid;
    a.U = U; a.W1 = (const uint16_t*)W1; a.W2t = (const uint16_t*)W2t;
    a.anchor = anchor; a.tokens = tokens; a.T = T; a.lse_d = lse; a.lse_t_row = w.lse_t_row;
    a.jrow = w.jrow; a.rpart = w.res_part;
    a.B = B; a.G = G; a.V = V; a.r = r; a.k = 0; a.invT = invT; a.key0 = key0; a.key1 = key1;
    a.ncols = B; a.col0 = 0;
    // up to kThinMax residual rows take the thin pass; the matrix-core pass leaves at once
    // then (and the thin one when there are more)
    const bool thin = B <= 256;
    a.thin_max = thin ? kThinMax : 0;
    if (thin)
      hipLaunchKernelGGL(k_verify_resid_thin, dim3(nres), dim3(256), 0, st, U,
                         (const uint16_t*)W1, (const uint16_t*)W2t, T, anchor, tokens, lse,
                         w.jrow, w.lse_t_row, B, G, V, invT, key0, key1, nres, w.res_part);
    if (launch_mfma_bias(a, nres, st) != DSPARK_OK) return DSPARK_E_HIP;
  } else {
    const RowSlices rr = row_slices(V, B);
    const size_t sh = sizeof(float) * (r + 256 + 16);
    if (wdt == DSPARK_BF16)
      hipLaunchKernelGGL(k_verify_resid_row<uint16_t>, dim3(rr.count, B), dim3(256), sh, st, U,
                         (const uint16_t*)W1, (const uint16_t*)W2t, T, anchor, tokens, lse,
                         w.jrow, w.lse_t_row, B, G, V, r, rr.len, invT, key0, key1, w.res_part);
    else
      hipLaunchKernelGGL(k_verify_resid_row<float>, dim3(rr.count, B), dim3(256), sh, st, U,
                         (const float*)W1, (const float*)W2t, T, anchor, tokens, lse, w.jrow,
                         w.lse_t_row, B, G, V, r, rr.len, invT, key0, key1, w.res_part);
  }
  hipLaunchKernelGGL(k_verify_final, dim3((B + 3) / 4), dim3(256), 0, st, w.jrow, n_accept,
                     w.res_part, nres, B, G, out_tokens);
  return launch_status();
}
