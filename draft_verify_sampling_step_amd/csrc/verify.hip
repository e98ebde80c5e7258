// verify.hip -- rejection-sampling verification [XTL §1; AIMSG concept 2; CSDN roundtable:
// accept with probability min(1, p_t/p_d)], lossless: the emitted tokens follow the
// target distribution.  Three launches:
//
//  1. k_verify_rows    one streaming pass over the target rows 1..ell_b+1 of every request
//                      (a flattened ragged set that every workgroup maps for itself from
//                      ell): split-vocabulary (max, sum-exp) partials of T/temperature,
//                      and on row ell_b+1 the Gumbel race of the bonus token, one packed
//                      (score, index) slot per slice.
//  2. k_verify_decide  per request: lse of each row, p_t(x_k), the ordered accept tests
//                      u * p_d(x_k) < p_t(x_k); n_b; the accepted prefix; the bonus token
//                      when nothing was rejected, else the residual row j = n_b + 1; it
//                      also zeroes the residual pass's winners and arrival counters.
//  3. residual         for rejected requests, the draft row j is recomputed (Markov bias
//                      for x_{j-1} plus U_j) and the residual max(0, p_t - p_d) is sampled
//                      by a Gumbel race on ln rho (bf16 matrix cores for many rejections,
//                      a 16-lanes-per-row path for one or two, GEMV rows for other
//                      weights); a p_t race on the same noise covers the case where
//                      rounding leaves no positive residual.  Winners are posted as packed
//                      atomic maxima; the last workgroup to arrive writes the tokens.
// For more than kVerifyScanMax requests a plan kernel builds the ragged row list first.
#include "dspark_dev.h"
#include "dspark_host.h"
#include "mfma_bias.h"
#include "mfma_common.h"
#include "rowbias.h"

namespace dspark {

// 16-byte loads per thread and item of the target-row pass (an item is 4 * 256 * this many
// entries of one row)
constexpr int kVerifyQuads = 8;

// Requests up to which every workgroup of k_verify_rows maps the ragged row set itself
// (a prefix sum of ell_b + 1 in LDS, 4 bytes per request); beyond, a plan kernel lists it.
constexpr int kVerifyScanMax = 8192;

// Flattened ragged row list: rows (b, k) with k <= ell_b + 1, in request order.  One
// workgroup; writes the list, its length and the number of (row, slice) work items.
__global__ __launch_bounds__(256) void k_verify_plan(const int32_t* __restrict__ ell, int B,
                                                     int G, int nslices,
                                                     int32_t* __restrict__ rows,
                                                     int32_t* __restrict__ counts) {
  __shared__ int32_t scan[256];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
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

__device__ __forceinline__ int clamp_ell(int L, int G) { return L < 0 ? 0 : (L > G ? G : L); }

// Workgroup (256 threads) merge of per-thread base-2 (max, sum) states in a fixed order;
// thread 0 writes it to *out.  Uses red[0..8).
__device__ __forceinline__ void rows_put_ml(float m, float l, float* red, float2* out) {
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
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
    *out = make_float2(mm, ll);
  }
  __syncthreads();
}

// An item of the target-row pass: (request b, row id, slice s).
struct RowItem { int b, row, s; };

// Each workgroup takes a contiguous range of (row, slice) items, i.e. consecutive slices of
// consecutive rows.  Rows 1..ell_b: split-vocabulary (max, sum-exp) partials of
// T/temperature (base 2).  Row ell_b + 1 needs no normaliser (only its bonus token is
// drawn from it): the Gumbel race over it, one packed (score, index) word per slice.
// Without a plan (rows == NULL) every workgroup first forms pre[b] = sum over requests
// before b of (ell + 1) in LDS (dynamic, B + 1 ints) and maps an item by binary search.
// (Contiguous ranges measured faster than a grid-stride order, whose last round leaves
// most workgroups idle; a second register buffer that loads the next item during the
// current one halves the occupancy and was slower at the scheduled budget.)
__global__ __launch_bounds__(256, 8) void k_verify_rows(
    const float* __restrict__ T, const int32_t* __restrict__ ell,
    const int32_t* __restrict__ rows, const int32_t* __restrict__ counts, int B, int G, int V,
    int slice_len, int nslices, float invT, uint32_t key0, uint32_t key1,
    float2* __restrict__ part, unsigned long long* __restrict__ bonus_part) {
  extern __shared__ int32_t pre[];
  __shared__ float red[16];
  __shared__ int32_t wsum[4];
  const float s2 = invT * 1.4426950408889634f;
  const int tid = threadIdx.x, wv = tid >> 6, lane = tid & 63;
  int nitems;
  if (rows == nullptr) {
    const int per = (B + 255) / 256;
    const int b0 = min(B, tid * per), b1 = min(B, b0 + per);
    int local = 0;
    for (int b = b0; b < b1; ++b) local += clamp_ell(ell[b], G) + 1;
    int incl = local;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += t;
    }
    if (lane == 63) wsum[wv] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wv; ++w) run += wsum[w];
    for (int b = b0; b < b1; ++b) {
      pre[b] = run;
      run += clamp_ell(ell[b], G) + 1;
    }
    if (tid == 0) pre[B] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    __syncthreads();
    nitems = pre[B] * nslices;
  } else {
    nitems = counts[1];
  }
  const int per = nitems / (int)gridDim.x, rem = nitems % (int)gridDim.x;
  const int it0 = (int)blockIdx.x * per + min((int)blockIdx.x, rem);
  const int it1 = it0 + per + ((int)blockIdx.x < rem ? 1 : 0);
  auto locate = [&](int item) {
    const int rpos = item / nslices;
    RowItem r;
    r.s = item % nslices;
    if (rows == nullptr) {
      int lo = 0, hi = B - 1;   // the b with pre[b] <= rpos < pre[b + 1] (pre increases)
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= rpos) lo = mid;
        else hi = mid - 1;
      }
      r.b = lo;
      r.row = lo * (G + 1) + (rpos - pre[lo]);
    } else {
      r.row = rows[rpos];
      r.b = r.row / (G + 1);
    }
    return r;
  };

  if ((V & 3) == 0 && slice_len == 4 * 256 * kVerifyQuads) {
    constexpr int kQ = kVerifyQuads;
    // every thread's eight 16-byte loads of an item; entries past the slice read as -inf
    auto issue = [&](const RowItem& r, f32x4_t (&q)[kQ]) {
      const int v_begin = r.s * slice_len, v_end = min(V, v_begin + slice_len);
      const float* trow = T + (size_t)r.row * V;
#pragma unroll
      for (int i = 0; i < kQ; ++i) {
        const int v = v_begin + 4 * (tid + 256 * i);
        q[i] = v < v_end ? __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(trow + v))
                         : f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
    };
    auto consume = [&](const RowItem& r, const f32x4_t (&q)[kQ]) {
      const int k = r.row % (G + 1) + 1;
      const bool is_bonus = (k == clamp_ell(ell[r.b], G) + 1);
      const int v_begin = r.s * slice_len;
      if (!is_bonus) {
        // max first (a finite floor when every entry is padding), then one exponential
        // per entry
        float mq = -INFINITY;
#pragma unroll
        for (int i = 0; i < kQ; ++i)
          mq = fmaxf(mq, fmaxf(fmaxf(q[i][0], q[i][1]), fmaxf(q[i][2], q[i][3])));
        const float m = fmaxf(mq * s2, -3.0e38f);
        float lp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kQ; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) lp[j] += ex2(fmaf(q[i][j], s2, -m));
        rows_put_ml(m, (lp[0] + lp[1]) + (lp[2] + lp[3]), red,
                    part + (size_t)r.row * nslices + r.s);
      } else {
        // four consecutive entries share one Philox call (words 0..3); the calls of a
        // batch run in lockstep
        const PhiloxLane pl = philox_lane((uint32_t)k, (uint32_t)r.b, 2u, key0, key1);
        Cand best{-INFINITY, 0xFFFFFFFFu, 0.f};
#pragma unroll
        for (int i0 = 0; i0 < kQ; i0 += 2) {
          uint32_t c0[2], w[2][4];
#pragma unroll
          for (int i = 0; i < 2; ++i)
            c0[i] = (uint32_t)((v_begin + 4 * (tid + 256 * (i0 + i))) >> 2);
          philox_calls<2>(c0, pl, w);
#pragma unroll
          for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float sc = fmaf(q[i0 + i][j], s2, neg_lglg(w[i][j]));
              if (sc > best.s) best = Cand{sc, 4 * c0[i] + (uint32_t)j, 0.f};
            }
        }
        best = block_cand(best, red + 8, reinterpret_cast<uint32_t*>(red + 12), red + 4);
        if (tid == 0)
          bonus_part[(size_t)r.b * nslices + r.s] =
              best.i != 0xFFFFFFFFu ? pack_score(best.s, best.i) : 0ull;
      }
    };
    f32x4_t q[kQ];
    for (int item = it0; item < it1; ++item) {
      const RowItem r = locate(item);
      issue(r, q);
      consume(r, q);
    }
    return;
  }

  // any other vocabulary size: the normaliser one entry per thread and step (online
  // state); the bonus race four consecutive entries per thread and step, which share one
  // Philox call (slices start at multiples of 4)
  for (int item = it0; item < it1; ++item) {
    const RowItem r = locate(item);
    const int k = r.row % (G + 1) + 1;
    const bool is_bonus = (k == clamp_ell(ell[r.b], G) + 1);
    const int v_begin = r.s * slice_len, v_end = min(V, v_begin + slice_len);
    const float* trow = T + (size_t)r.row * V;
    if (is_bonus) {
      const PhiloxLane pl = philox_lane((uint32_t)k, (uint32_t)r.b, 2u, key0, key1);
      Cand best{-INFINITY, 0xFFFFFFFFu, 0.f};
      for (int v0 = v_begin + 4 * tid; v0 < v_end; v0 += 4 * 256) {
        const U4 w = philox_call((uint32_t)v0 >> 2, pl);
        const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
        const int n = min(4, v_end - v0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (i >= n) break;
          const float sc = fmaf(trow[v0 + i], s2, neg_lglg(wd[i]));
          if (sc > best.s) best = Cand{sc, (uint32_t)(v0 + i), 0.f};
        }
      }
      best = block_cand(best, red + 8, reinterpret_cast<uint32_t*>(red + 12), red + 4);
      if (tid == 0)
        bonus_part[(size_t)r.b * nslices + r.s] =
            best.i != 0xFFFFFFFFu ? pack_score(best.s, best.i) : 0ull;
    } else {
      float m = -3.0e38f, l = 0.f;
      for (int v = v_begin + tid; v < v_end; v += 256) {
        const float z = trow[v] * s2;
        const float mn = fmaxf(m, z);
        l = l * ex2(m - mn) + ex2(z - mn);
        m = mn;
      }
      rows_put_ml(m, l, red, part + (size_t)r.row * nslices + r.s);
    }
  }
}

// One wave per request, one lane per draft row k = lane + 1 (gamma <= 64): all rows of a
// request are decided at once.  Lane k merges the base-2 slice partials of target row k in
// slice order into its lse, then takes p_t(x_k) and the accept test u * p_d(x_k) < p_t(x_k).
// The accepted prefix ends at the first rejected row, found by a ballot.  The bonus token
// is the best of row ell_b + 1's slice winners.  The residual pass's packed winners and
// arrival counters (res_best [B][2], res_cnt [ncnt]) start from zero here.
__global__ __launch_bounds__(256) void k_verify_decide(
    const float* __restrict__ T, const int32_t* __restrict__ tokens,
    const float* __restrict__ logp, const int32_t* __restrict__ ell,
    const float2* __restrict__ part, const unsigned long long* __restrict__ bonus_part, int B,
    int G, int V, int nslices, float invT, uint32_t key0, uint32_t key1,
    int32_t* __restrict__ n_accept, int32_t* __restrict__ out_tokens,
    float* __restrict__ pt_tok, int32_t* __restrict__ jrow, float* __restrict__ lse_t_row,
    unsigned long long* __restrict__ res_best, int32_t* __restrict__ res_cnt, int ncnt) {
  const int b = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < ncnt; i += gridDim.x * blockDim.x)
    res_cnt[i] = 0;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < 2 * kSubSlots * B;
       i += gridDim.x * blockDim.x)
    res_best[i] = 0ull;
  if (b >= B) return;
  const int Lb = ell[b];
  const int L = Lb < 0 ? 0 : (Lb > G ? G : Lb);   // ell outside [0, gamma] is clamped
  const int k = lane + 1;
  const bool live = k <= L;
  float lt = 0.f, pt = __builtin_nanf("");
  bool rejected = false;
  // every draft row of the block is evaluated without waiting for ell (its loads do not
  // depend on it); rows past ell are then discarded
  if (k <= G) {
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
    rejected = live && !(word_to_uniform(w.x) * fast_exp(lp) < pt);
    if (!live) {
      lt = 0.f;
      pt = __builtin_nanf("");
    }
  }
  if (pt_tok && k <= G) pt_tok[(size_t)b * G + (k - 1)] = pt;
  const unsigned long long rej = __ballot(rejected);   // bit k-1: row k rejected
  const int n = rej ? __builtin_ctzll(rej) : L;          // leading accepts
  const int j = rej ? n + 1 : 0;                         // residual row, 0 = none
  const float lj = __shfl(lt, j > 0 ? j - 1 : 0, kWave);
  int32_t* out = out_tokens + (size_t)b * (G + 1);
  for (int i = lane; i <= G; i += kWave) out[i] = i < n ? tokens[(size_t)b * G + i] : -1;
  unsigned long long bw = 0ull;   // the bonus winner: the largest packed slice winner
  for (int s = lane; s < nslices; s += kWave) {
    const unsigned long long q = bonus_part[(size_t)b * nslices + s];
    bw = q > bw ? q : bw;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long q =
        ((unsigned long long)(uint32_t)__shfl_xor((int)(uint32_t)(bw >> 32), o, kWave) << 32) |
        (uint32_t)__shfl_xor((int)(uint32_t)bw, o, kWave);
    bw = q > bw ? q : bw;
  }
  if (lane == 0) {
    if (j == 0) out[n] = (int32_t)packed_index(bw);
    n_accept[b] = n;
    jrow[b] = j;
    lse_t_row[b] = j > 0 ? lj : 0.f;
  }
}

// Row residual: grid (slices, B), 256 threads.  As in the row draft, a step covers four
// tiles and thread t owns the rows tile0 + 4t .. + 3, drawn from one Philox call.
template <typename WT>
__global__ __launch_bounds__(256) void k_verify_resid_row(
    const float* __restrict__ U, const WT* __restrict__ W1, const WT* __restrict__ W2t,
    const float* __restrict__ T, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ lse_d,
    const int32_t* __restrict__ jrow, const float* __restrict__ lse_t_row, int B, int G, int V,
    int r, int slice_len, float invT, uint32_t key0, uint32_t key1,
    unsigned long long* __restrict__ res_best, int32_t* __restrict__ res_cnt,
    const int32_t* __restrict__ n_accept, int32_t* __restrict__ out_tokens) {
  extern __shared__ float smem[];
  float* w1s = smem;
  float* bias_s = smem + r;             // [4 kRowTile]
  float* red = bias_s + 4 * kRowTile;   // [16]
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
  const PhiloxLane pl = philox_lane((uint32_t)j, (uint32_t)b, 2u, key0, key1);
  Cand b1{-INFINITY, 0xFFFFFFFFu, 0.f}, b2{-INFINITY, 0xFFFFFFFFu, 0.f};
  for (int tile0 = v_begin; tile0 < v_end; tile0 += 4 * kRowTile) {
#pragma unroll 1
    for (int i = 0; i < 4; ++i)   // workgroup-uniform bound
      if (tile0 + i * kRowTile < v_end)
        row_bias_tile<WT>(W2t, w1s, bias_s + i * kRowTile, r, tile0 + i * kRowTile, v_end);
    __syncthreads();
    const int v0 = tile0 + 4 * tid;
    if (v0 < v_end) {
      const U4 w = philox_call((uint32_t)v0 >> 2, pl);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
      const int n = min(4, v_end - v0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= n) break;
        const int v = v0 + i;
        const float zd = (urow[v] + bias_s[4 * tid + i]) * invT;
        const float zt = trow[v] * invT;
        const float rho = fast_exp(zt - lt) - fast_exp(zd - ld);
        const float gn = gumbel_from_uniform(word_to_uniform(wd[i]));
        if (rho > 0.f) {
          const float sc = fast_log(rho) + gn;
          if (sc > b1.s) b1 = Cand{sc, (uint32_t)v, 0.f};
        }
        const float sc2 = zt + gn;
        if (sc2 > b2.s) b2 = Cand{sc2, (uint32_t)v, 0.f};
      }
    }
    __syncthreads();
  }
  b1 = block_cand(b1, red, reinterpret_cast<uint32_t*>(red + 4), red + 8);
  b2 = block_cand(b2, red, reinterpret_cast<uint32_t*>(red + 4), red + 8);
  if (tid == 0) {
    unsigned long long* slot = res_best + ((size_t)(s % kSubSlots) * B + b) * 2;
    if (b1.i != 0xFFFFFFFFu) atomic_max_u64(&slot[0], pack_score(b1.s, b1.i));
    if (b2.i != 0xFFFFFFFFu) atomic_max_u64(&slot[1], pack_score(b2.s, b2.i));
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    // the last of the request's slices to arrive writes its token after the prefix (the
    // residual winner, or the p_t fallback when no residual was positive)
    if (arrive_last(res_cnt + (size_t)b * kArriveInts, s, gridDim.x)) {
      unsigned long long r1 = 0ull, r2 = 0ull;
      for (int q = 0; q < kSubSlots; ++q) {
        const unsigned long long* sl = res_best + ((size_t)q * B + b) * 2;
        const unsigned long long x1 = atomic_load_u64(&sl[0]), x2 = atomic_load_u64(&sl[1]);
        r1 = x1 > r1 ? x1 : r1;
        r2 = x2 > r2 ? x2 : r2;
      }
      out_tokens[(size_t)b * (G + 1) + n_accept[b]] = (int32_t)packed_index(r1 ? r1 : r2);
    }
  }
}

}  // namespace dspark

using namespace dspark;

namespace {

struct VerifyWs {
  float2* part;                  // [B (G+1)][nslices] base-2 (max, sum) of target rows
  int32_t* rows;                 // [B (G+1)] ragged row list (plan path only)
  int32_t* counts;               // [2] its length and item count (plan path only)
  unsigned long long* bonus;     // [B][nslices] packed winners of the bonus race per slice
  unsigned long long* res_best;  // [kSubSlots][B][2] packed residual / fallback winners
  int32_t* res_cnt;              // [B][kArriveInts] arrival counters (per request or launch)
  int32_t* jrow;
  float* lse_t_row;
  size_t bytes;
};

VerifyWs verify_ws(const dspark_dims* d, int nslices, void* base) {
  Carve c(base);
  VerifyWs w;
  const size_t B = d->batch;
  w.part = c.take<float2>(B * (d->gamma + 1) * nslices);
  w.rows = c.take<int32_t>(B * (d->gamma + 1));
  w.counts = c.take<int32_t>(2);
  w.bonus = c.take<unsigned long long>(B * nslices);
  w.res_best = c.take<unsigned long long>(2 * kSubSlots * B);
  w.res_cnt = c.take<int32_t>(B * kArriveInts);
  w.jrow = c.take<int32_t>(B);
  w.lse_t_row = c.take<float>(B);
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
  return verify_ws(d, ns, nullptr).bytes;
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
  VerifyWs w = verify_ws(dm, nsl, ws);
  const float invT = 1.0f / temperature;
  const uint32_t key0 = (uint32_t)seed, key1 = (uint32_t)(seed >> 32);
  if (mfma && mfma_prepare() != DSPARK_OK) return DSPARK_E_HIP;

  // 1. target rows (with the ragged row list formed in every workgroup, or listed by the
  //    plan kernel for very large batches)
  const bool plan = B > kVerifyScanMax;
  if (plan)
    hipLaunchKernelGGL(k_verify_plan, dim3(1), dim3(256), 0, st, ell, B, G, nsl, w.rows,
                       w.counts);
  // contiguous item ranges, eight workgroups per compute unit
  const long long max_items = (long long)B * (G + 1) * nsl;
  const int grid = (int)std::min<long long>(max_items, 2048);
  const size_t sh_rows = plan ? 0 : sizeof(int32_t) * ((size_t)B + 1);
  hipLaunchKernelGGL(k_verify_rows, dim3(grid), dim3(256), sh_rows, st, T, ell,
                     plan ? w.rows : nullptr, plan ? w.counts : nullptr, B, G, V, kVerifySlice,
                     nsl, invT, key0, key1, w.part, w.bonus);
  // 2. decisions (and the residual pass's winners and counters reset)
  hipLaunchKernelGGL(k_verify_decide, dim3((B + 3) / 4), dim3(256), 0, st, T, tokens, logp, ell,
                     w.part, w.bonus, B, G, V, nsl, invT, key0, key1, n_accept, out_tokens,
                     pt_tok, w.jrow, w.lse_t_row, w.res_best, w.res_cnt, B * kArriveInts);
  // 3. the residual draws; the last workgroup to finish writes the tokens
  if (mfma) {
    MfmaBiasArgs a{};
    a.mode = kModeResid;
    a.U = U; a.W1 = (const uint16_t*)W1; a.W2t = (const uint16_t*)W2t;
    a.anchor = anchor; a.tokens = tokens; a.T = T; a.lse_d = lse; a.lse_t_row = w.lse_t_row;
    a.jrow = w.jrow; a.res_best = w.res_best; a.res_arrive = w.res_cnt;
    a.n_accept = n_accept; a.out_tokens = out_tokens;
    a.B = B; a.G = G; a.V = V; a.r = r; a.k = 0; a.invT = invT; a.key0 = key0; a.key1 = key1;
    a.ncols = B; a.col0 = 0;
    // one or two residual rows take the thin path inside the same kernel (one launch
    // covers every column up to 256 requests)
    a.thin_max = B <= mfma_column_group(kModeResid) ? kResidThinMax : 0;
    if (launch_mfma_bias(a, nres, st) != DSPARK_OK) return DSPARK_E_HIP;
  } else {
    const RowSlices rr = row_slices(V, B);
    const size_t sh = sizeof(float) * (r + 4 * kRowTile + 16);
    if (wdt == DSPARK_BF16)
      hipLaunchKernelGGL(k_verify_resid_row<uint16_t>, dim3(rr.count, B), dim3(256), sh, st, U,
                         (const uint16_t*)W1, (const uint16_t*)W2t, T, anchor, tokens, lse,
                         w.jrow, w.lse_t_row, B, G, V, r, rr.len, invT, key0, key1, w.res_best,
                         w.res_cnt, n_accept, out_tokens);
    else
      hipLaunchKernelGGL(k_verify_resid_row<float>, dim3(rr.count, B), dim3(256), sh, st, U,
                         (const float*)W1, (const float*)W2t, T, anchor, tokens, lse, w.jrow,
                         w.lse_t_row, B, G, V, r, rr.len, invT, key0, key1, w.res_best,
                         w.res_cnt, n_accept, out_tokens);
  }
  return launch_status();
}
