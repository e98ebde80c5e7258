// tv.hip -- analytic accept rate [CSDN Eq. 8; XTL §5]:
//   alpha_{b,k} = 1 - |p_d,k - p_t,k|_1 / 2 = sum_v min(p_d,k(v), p_t,k(v)).
//
//  1. k_tv_rows   split-vocabulary (max, sum-exp) partials of T/temperature, rows 1..gamma
//  2. k_tv_lse    lse_t of each row (partials merged in slice order)
//  3. sum of min  the draft row is recomputed for every (b, k) column at once -- all
//                 conditioning tokens are known, so one pass over W2t serves up to 256
//                 columns (bf16 MFMA path) -- with p_d = exp(z - lse_d) using the draft's
//                 lse and p_t = exp(T/temperature - lse_t); partial sums per slice
//  4. k_tv_final  alpha = partial sums added in a fixed order
#include "dspark_dev.h"
#include "dspark_host.h"
#include "mfma_bias.h"
#include "rowbias.h"

namespace dspark {

// grid (slices, B, gamma)
__global__ __launch_bounds__(256) void k_tv_rows(const float* __restrict__ T, int G, int V,
                                                 int slice_len, int nslices, float invT,
                                                 float2* __restrict__ part) {
  __shared__ float red[16];
  const int s = blockIdx.x, b = blockIdx.y, kk = blockIdx.z;
  const int v_begin = s * slice_len, v_end = min(V, v_begin + slice_len);
  const float* row = T + ((size_t)b * (G + 1) + kk) * V;
  ML st{-INFINITY, 0.f};
  if ((V & 3) == 0 && (slice_len & 3) == 0) {
    // chunks of 8192 entries: each thread's eight 16-byte loads are issued before any is
    // used, then the chunk's max and one exponential per entry (entries past the slice
    // read as -inf; a finite floor keeps an all-padding thread at l = 0)
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    for (int c0 = v_begin; c0 < v_end; c0 += 8 * 1024) {
      f32x4 q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int v = c0 + 4 * (threadIdx.x + 256 * i);
        q[i] = v < v_end ? __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + v))
                         : f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      }
      float mq = -INFINITY;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        mq = fmaxf(mq, fmaxf(fmaxf(q[i][0], q[i][1]), fmaxf(q[i][2], q[i][3])));
      const float m = fmaxf(mq * invT, -3.0e38f);
      float l = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) l += fast_exp(fmaf(q[i][j], invT, -m));
      st = ml_merge(st, ML{m, l});
    }
  } else {
    for (int v = v_begin + threadIdx.x; v < v_end; v += 256) {
      const float z = row[v] * invT;
      if (z > st.m) {
        st.l = st.l * fast_exp(st.m - z) + 1.f;
        st.m = z;
      } else {
        st.l += fast_exp(z - st.m);
      }
    }
  }
  st = block_ml(st, red, red + 4);
  if (threadIdx.x == 0) part[((size_t)b * G + kk) * nslices + s] = make_float2(st.m, st.l);
}

__global__ __launch_bounds__(256) void k_tv_lse(const float2* __restrict__ part, int n,
                                                int nslices, float* __restrict__ lse_t) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  ML st{-INFINITY, 0.f};
  for (int s = 0; s < nslices; ++s) {
    const float2 p = part[(size_t)i * nslices + s];
    st = ml_merge(st, ML{p.x, p.y});
  }
  lse_t[i] = st.m + fast_log(st.l);
}

// Row path for the sum of minima: grid (slices, B*gamma)
template <typename WT>
__global__ __launch_bounds__(256) void k_tv_row(
    const float* __restrict__ U, const WT* __restrict__ W1, const WT* __restrict__ W2t,
    const float* __restrict__ T, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ lse_d,
    const float* __restrict__ lse_t, int B, int G, int V, int r, int slice_len, float invT,
    float* __restrict__ tv_part) {
  extern __shared__ float smem[];
  float* w1s = smem;
  float* bias_s = smem + r;
  float* red = bias_s + 256;
  const int s = blockIdx.x, col = blockIdx.y, tid = threadIdx.x;
  const int b = col / G, k = col % G + 1;
  const int prev = clamp_tok((k == 1) ? anchor[b] : tokens[(size_t)b * G + (k - 2)], V);
  const int v_begin = s * slice_len, v_end = min(V, v_begin + slice_len);
  load_w1_row<WT>(W1, prev, r, w1s);
  __syncthreads();
  const float ld = lse_d[col], lt = lse_t[col];
  const float* urow = U + ((size_t)b * G + (k - 1)) * V;
  const float* trow = T + ((size_t)b * (G + 1) + (k - 1)) * V;
  float acc = 0.f;
  for (int tile0 = v_begin; tile0 < v_end; tile0 += kRowTile) {
    row_bias_tile<WT>(W2t, w1s, bias_s, r, tile0, v_end);
    __syncthreads();
    const int v = tile0 + tid;
    if (v < v_end) {
      const float pd = fast_exp((urow[v] + bias_s[tid]) * invT - ld);
      const float pt = fast_exp(trow[v] * invT - lt);
      acc += fminf(pd, pt);
    }
    __syncthreads();
  }
  acc = block_sum(acc, red);
  if (tid == 0) tv_part[(size_t)s * ((size_t)B * G) + col] = acc;
}

// alpha of each (request, position) column: its partial sums over the slices, in a fixed
// order.  Block of 256 threads = 32 columns x 8 slice phases; phase p adds the slices p,
// p + 8, ... and the eight phase sums are added in phase order.
__global__ __launch_bounds__(256) void k_tv_final(const float* __restrict__ tv_part, int n,
                                                  int nslices, float* __restrict__ alpha) {
  __shared__ float red[8][32];
  const int c = threadIdx.x & 31, p = threadIdx.x >> 5;
  const int i = blockIdx.x * 32 + c;
  float s = 0.f;
  if (i < n) {
#pragma unroll 8
    for (int q = p; q < nslices; q += 8) s += tv_part[(size_t)q * n + i];
  }
  red[p][c] = s;
  __syncthreads();
  if (p == 0 && i < n) {
    float t = red[0][c];
    for (int k = 1; k < 8; ++k) t += red[k][c];
    alpha[i] = t;
  }
}

}  // namespace dspark

using namespace dspark;

namespace {

struct TvWs {
  float2* part;
  float* lse_t;
  float* tv_part;
  size_t bytes;
};

TvWs tv_ws(const dspark_dims* d, int nrow_slices, int nsum_slices, void* base) {
  Carve c(base);
  TvWs w;
  const size_t n = (size_t)d->batch * d->gamma;
  w.part = c.take<float2>(n * nrow_slices);
  w.lse_t = c.take<float>(n);
  w.tv_part = c.take<float>(n * nsum_slices);
  w.bytes = align_up(c.off, 256);
  return w;
}

int tv_sum_slices(const dspark_dims* d, bool mfma) {
  const long long n = (long long)d->batch * d->gamma;
  return mfma ? mfma_grid(d->vocab, (int)std::min<long long>(n, mfma_column_group(kModeTV)),
                         kModeTV)
              : row_slices(d->vocab, n).count;
}

}  // namespace

size_t dspark_tv_workspace(const dspark_dims* d) {
  const RowSlices rs = stream_slices(d->vocab, (long long)d->batch * d->gamma);
  const int ns = std::max(tv_sum_slices(d, true), tv_sum_slices(d, false));
  return tv_ws(d, rs.count, ns, nullptr).bytes;
}

extern "C" dspark_status dspark_accept_rate_tv(const dspark_dims* dm, const float* U,
                                               const void* W1, const void* W2t, int wdt,
                                               const int32_t* anchor, const int32_t* tokens,
                                               const float* lse, const float* T,
                                               float temperature, float* alpha, void* ws,
                                               size_t ws_bytes, void* stream) {
  if (!dm || !U || !W1 || !W2t || !anchor || !tokens || !lse || !T || !alpha)
    return DSPARK_E_NULL;
  if (!dims_ok(dm)) return DSPARK_E_SHAPE;
  if ((long long)dm->batch * dm->gamma > 65535) return DSPARK_E_SHAPE;
  if (!dtype_ok(wdt)) return DSPARK_E_DTYPE;
  if (!temp_ok(temperature)) return DSPARK_E_VALUE;
  if (!ws || ws_bytes < dspark_tv_workspace(dm)) return DSPARK_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int B = dm->batch, G = dm->gamma, V = dm->vocab, r = dm->rank, n = B * G;
  const bool mfma = mfma_bias_supported(n, r, wdt);
  const RowSlices rs = stream_slices(V, n);
  const int nsum = tv_sum_slices(dm, mfma);
  TvWs w = tv_ws(dm, rs.count, nsum, ws);
  const float invT = 1.0f / temperature;
  if (mfma && mfma_prepare() != DSPARK_OK) return DSPARK_E_HIP;

  hipLaunchKernelGGL(k_tv_rows, dim3(rs.count, B, G), dim3(256), 0, st, T, G, V, rs.len,
                     rs.count, invT, w.part);
  hipLaunchKernelGGL(k_tv_lse, dim3((n + 255) / 256), dim3(256), 0, st, w.part, n, rs.count,
                     w.lse_t);
  if (mfma) {
    MfmaBiasArgs a{};
    a.mode = kModeTV;
    a.U = U; a.W1 = (const uint16_t*)W1; a.W2t = (const uint16_t*)W2t;
    a.anchor = anchor; a.tokens = tokens; a.T = T; a.lse_d = lse; a.lse_t = w.lse_t;
    a.tv_part = w.tv_part;
    a.B = B; a.G = G; a.V = V; a.r = r; a.k = 0; a.invT = invT;
    a.ncols = n; a.col0 = 0;
    if (launch_mfma_bias(a, nsum, st) != DSPARK_OK) return DSPARK_E_HIP;
  } else {
    const RowSlices rr = row_slices(V, n);
    const size_t sh = sizeof(float) * (r + 256 + 16);
    if (wdt == DSPARK_BF16)
      hipLaunchKernelGGL(k_tv_row<uint16_t>, dim3(rr.count, n), dim3(256), sh, st, U,
                         (const uint16_t*)W1, (const uint16_t*)W2t, T, anchor, tokens, lse,
                         w.lse_t, B, G, V, r, rr.len, invT, w.tv_part);
    else
      hipLaunchKernelGGL(k_tv_row<float>, dim3(rr.count, n), dim3(256), sh, st, U,
                         (const float*)W1, (const float*)W2t, T, anchor, tokens, lse, w.lse_t,
                         B, G, V, r, rr.len, invT, w.tv_part);
  }
  hipLaunchKernelGGL(k_tv_final, dim3((n + 31) / 32), dim3(256), 0, st, w.tv_part, n, nsum,
                     alpha);
  return launch_status();
}
