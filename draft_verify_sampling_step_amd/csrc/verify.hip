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
#include "rowbias.h"

namespace dspark {

__global__ void k_vfill_u64(unsigned long long* p, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0ull;
}

// grid (slices, B, gamma+1), 256 threads
__global__ __launch_bounds__(256) void k_verify_rows(
    const float* __restrict__ T, const int32_t* __restrict__ ell, int B, int G, int V,
    int slice_len, int nslices, float invT, uint32_t key0, uint32_t key1,
    float2* __restrict__ part, unsigned long long* __restrict__ bonus) {
  __shared__ float red[16];
  const int s = blockIdx.x, b = blockIdx.y, kk = blockIdx.z, k = kk + 1;
  const int L = ell[b];
  if (k > L + 1) return;
  const bool is_bonus = (k == L + 1);
  const int v_begin = s * slice_len, v_end = min(V, v_begin + slice_len);
  const float* row = T + ((size_t)b * (G + 1) + kk) * V;
  ML st{-INFINITY, 0.f};
  Cand best{-INFINITY, 0xFFFFFFFFu, 0.f};
  for (int v = v_begin + threadIdx.x; v < v_end; v += 256) {
    const float z = __builtin_nontemporal_load(row + v) * invT;
    if (z > st.m) {
      st.l = st.l * fast_exp(st.m - z) + 1.f;
      st.m = z;
    } else {
      st.l += fast_exp(z - st.m);
    }
    if (is_bonus) {
      const U4 w = philox10((uint32_t)v >> 2, (uint32_t)k, (uint32_t)b, 2u, key0, key1);
      const uint32_t word = (v & 3) == 0 ? w.x : (v & 3) == 1 ? w.y : (v & 3) == 2 ? w.z : w.w;
      const float sc = z + gumbel_from_uniform(word_to_uniform(word));
      if (sc > best.s) best = Cand{sc, (uint32_t)v, z};
    }
  }
  st = block_ml(st, red, red + 4);
  if (is_bonus) best = block_cand(best, red + 8, reinterpret_cast<uint32_t*>(red + 12), red + 4);
  if (threadIdx.x == 0) {
    part[((size_t)b * (G + 1) + kk) * nslices + s] = make_float2(st.m, st.l);
    if (is_bonus) atomic_max_u64(&bonus[b], pack_score(best.s, best.i));
  }
}

__device__ __forceinline__ float row_lse(const float2* p, int n) {
  ML st{-INFINITY, 0.f};
  for (int s = 0; s < n; ++s) st = ml_merge(st, ML{p[s].x, p[s].y});
  return st.m + fast_log(st.l);
}

// one thread per request
__global__ __launch_bounds__(256) void k_verify_decide(
    const float* __restrict__ T, const int32_t* __restrict__ tokens,
    const float* __restrict__ logp, const int32_t* __restrict__ ell,
    const float2* __restrict__ part, const unsigned long long* __restrict__ bonus, int B, int G,
    int V, int nslices, float invT, uint32_t key0, uint32_t key1,
    int32_t* __restrict__ n_accept, int32_t* __restrict__ out_tokens,
    float* __restrict__ pt_tok, int32_t* __restrict__ jrow, float* __restrict__ lse_t_row) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const int L = ell[b];
  int n = 0, j = 0;
  float lj = 0.f;
  for (int k = 1; k <= G; ++k) {
    if (k > L) {
      if (pt_tok) pt_tok[(size_t)b * G + (k - 1)] = __builtin_nanf("");
      continue;
    }
    const float lt = row_lse(part + ((size_t)b * (G + 1) + (k - 1)) * nslices, nslices);
    const int x = tokens[(size_t)b * G + (k - 1)];
    const float pt = fast_exp(T[((size_t)b * (G + 1) + (k - 1)) * V + x] * invT - lt);
    if (pt_tok) pt_tok[(size_t)b * G + (k - 1)] = pt;
    if (j == 0) {
      const U4 w = philox10(0u, (uint32_t)k, (uint32_t)b, 1u, key0, key1);
      const float u = word_to_uniform(w.x);
      const float pd = fast_exp(logp[(size_t)b * G + (k - 1)]);
      if (u * pd < pt) {
        ++n;
      } else {
        j = k;
        lj = lt;
      }
    }
  }
  int32_t* out = out_tokens + (size_t)b * (G + 1);
  for (int i = 0; i <= G; ++i) out[i] = i < n ? tokens[(size_t)b * G + i] : -1;
  if (j == 0) out[n] = (int32_t)packed_index(bonus[b]);
  n_accept[b] = n;
  jrow[b] = j;
  lse_t_row[b] = lj;
}

// Row residual: grid (slices, B), 256 threads.
template <typename WT>
__global__ __launch_bounds__(256) void k_verify_resid_row(
    const float* __restrict__ U, const WT* __restrict__ W1, const WT* __restrict__ W2t,
    const float* __restrict__ T, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ lse_d,
    const int32_t* __restrict__ jrow, const float* __restrict__ lse_t_row, int B, int G, int V,
    int r, int slice_len, float invT, uint32_t key0, uint32_t key1,
    unsigned long long* __restrict__ res, unsigned long long* __restrict__ fb) {
  extern __shared__ float smem[];
  float* w1s = smem;
  float* bias_s = smem + r;
  float* red = bias_s + 256;
  const int s = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int j = jrow[b];
  if (j == 0) return;
  const int prev = (j == 1) ? anchor[b] : tokens[(size_t)b * G + (j - 2)];
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
  if (tid == 0) {
    if (b1.i != 0xFFFFFFFFu) atomic_max_u64(&res[b], pack_score(b1.s, b1.i));
    if (b2.i != 0xFFFFFFFFu) atomic_max_u64(&fb[b], pack_score(b2.s, b2.i));
  }
}

__global__ __launch_bounds__(256) void k_verify_final(const int32_t* __restrict__ jrow,
                                                      const int32_t* __restrict__ n_accept,
                                                      const unsigned long long* __restrict__ res,
                                                      const unsigned long long* __restrict__ fb,
                                                      int B, int G,
                                                      int32_t* __restrict__ out_tokens) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B || jrow[b] == 0) return;
  const unsigned long long w = res[b] != 0ull ? res[b] : fb[b];
  out_tokens[(size_t)b * (G + 1) + n_accept[b]] = (int32_t)packed_index(w);
}

}  // namespace dspark

using namespace dspark;

namespace {

struct VerifyWs {
  float2* part;
  unsigned long long* bonus;
  unsigned long long* res;
  unsigned long long* fb;
  int32_t* jrow;
  float* lse_t_row;
  size_t bytes;
};

VerifyWs verify_ws(const dspark_dims* d, int nslices, void* base) {
  Carve c(base);
  VerifyWs w;
  w.part = c.take<float2>((size_t)d->batch * (d->gamma + 1) * nslices);
  w.bonus = c.take<unsigned long long>((size_t)3 * d->batch);
  w.res = w.bonus ? w.bonus + d->batch : nullptr;
  w.fb = w.bonus ? w.bonus + 2 * d->batch : nullptr;
  w.jrow = c.take<int32_t>(d->batch);
  w.lse_t_row = c.take<float>(d->batch);
  w.bytes = align_up(c.off, 256);
  return w;
}

}  // namespace

size_t dspark_verify_workspace(const dspark_dims* d) {
  const RowSlices rs = stream_slices(d->vocab, (long long)d->batch * (d->gamma + 1));
  return verify_ws(d, rs.count, nullptr).bytes;
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
  const RowSlices rs = stream_slices(V, (long long)B * (G + 1));
  VerifyWs w = verify_ws(dm, rs.count, ws);
  const float invT = 1.0f / temperature;
  const uint32_t key0 = (uint32_t)seed, key1 = (uint32_t)(seed >> 32);

  hipLaunchKernelGGL(k_vfill_u64, dim3((3 * B + 255) / 256), dim3(256), 0, st, w.bonus,
                     (size_t)3 * B);
  hipLaunchKernelGGL(k_verify_rows, dim3(rs.count, B, G + 1), dim3(256), 0, st, T, ell, B, G, V,
                     rs.len, rs.count, invT, key0, key1, w.part, w.bonus);
  hipLaunchKernelGGL(k_verify_decide, dim3((B + 255) / 256), dim3(256), 0, st, T, tokens, logp,
                     ell, w.part, w.bonus, B, G, V, rs.count, invT, key0, key1, n_accept,
                     out_tokens, pt_tok, w.jrow, w.lse_t_row);
  if (mfma_bias_supported(B, r, wdt)) {
    MfmaBiasArgs a{};
    a.mode = kModeResid;
    a.U = U; a.W1 = (const uint16_t*)W1; a.W2t = (const uint16_t*)W2t;
    a.anchor = anchor; a.tokens = tokens; a.T = T; a.lse_d = lse; a.lse_t_row = w.lse_t_row;
    a.jrow = w.jrow; a.res_best = w.res; a.fb_best = w.fb;
    a.B = B; a.G = G; a.V = V; a.r = r; a.k = 0; a.invT = invT; a.key0 = key0; a.key1 = key1;
    a.ncols = B; a.col0 = 0;
    if (launch_mfma_bias(a, mfma_grid(V, B), st) != DSPARK_OK) return DSPARK_E_HIP;
  } else {
    const RowSlices rr = row_slices(V, B);
    const size_t sh = sizeof(float) * (r + 256 + 16);
    if (wdt == DSPARK_BF16)
      hipLaunchKernelGGL(k_verify_resid_row<uint16_t>, dim3(rr.count, B), dim3(256), sh, st, U,
                         (const uint16_t*)W1, (const uint16_t*)W2t, T, anchor, tokens, lse,
                         w.jrow, w.lse_t_row, B, G, V, r, rr.len, invT, key0, key1, w.res,
                         w.fb);
    else
      hipLaunchKernelGGL(k_verify_resid_row<float>, dim3(rr.count, B), dim3(256), sh, st, U,
                         (const float*)W1, (const float*)W2t, T, anchor, tokens, lse, w.jrow,
                         w.lse_t_row, B, G, V, r, rr.len, invT, key0, key1, w.res, w.fb);
  }
  hipLaunchKernelGGL(k_verify_final, dim3((B + 255) / 256), dim3(256), 0, st, w.jrow, n_accept,
                     w.res, w.fb, B, G, out_tokens);
  return launch_status();
}
