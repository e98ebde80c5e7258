// sts.hip -- sequential temperature scaling of the confidence head [XTL §5: the scheduler
// needs confidence values that match acceptance rates, so the product of confidences is
// calibrated on held-out data from left to right; AIMSG, on STS: per position a 1-D grid
// search over the temperature, minimising the expected calibration error (ECE) of the
// cumulative product against the empirical prefix acceptance].
//
// For k = 1..gamma (one position at a time, all on the device):
//   1. k_sts_bins    grid (temperature, sample chunk): p_s = q_s * sigmoid(logit_{s,k} / t)
//                    in fp64 with q_s = prod_{i<k} sigmoid(logit_{s,i} / t_i); per bin
//                    (equal width on [0, 1]) the sum of p, the number of accepted labels
//                    and the count, as integers (p in units of 2^-40) so that the sums are
//                    order-free: LDS atomics per workgroup, then one global atomic per bin.
//   2. k_sts_select  one workgroup: ECE(t) = sum_bins |sum p - sum y| / n for every grid
//                    value, the smallest (the first on exact ties) becomes t_k; clears the
//                    accumulators for the next position.
//   3. k_sts_update  q_s *= sigmoid(logit_{s,k} / t_k), in the same fp64 order as the
//                    definition.
#include "dspark_dev.h"
#include "dspark_host.h"

namespace dspark {

constexpr double kStsFix = 1099511627776.0;   // 2^40: fixed-point unit of the p sums
constexpr int kStsMaxBins = 256;
constexpr int kStsChunk = 4096;                // samples per workgroup of k_sts_bins

__global__ __launch_bounds__(256) void k_sts_init(double* __restrict__ q, int n,
                                                  unsigned long long* __restrict__ acc,
                                                  size_t nacc) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t s = i; s < (size_t)n; s += stride) q[s] = 1.0;
  for (size_t s = i; s < nacc; s += stride) acc[s] = 0ull;
}

// acc [n_t][n_bins][3]: (sum of p in 2^-40 units, accepted labels, count)
__global__ __launch_bounds__(256) void k_sts_bins(int n, int G, int k,
                                                  const float* __restrict__ logit,
                                                  const int32_t* __restrict__ n_accept,
                                                  const double* __restrict__ q,
                                                  const double* __restrict__ temps,
                                                  int n_bins,
                                                  unsigned long long* __restrict__ acc) {
  __shared__ unsigned long long bins[kStsMaxBins * 3];
  const int ti = blockIdx.x;
  for (int i = threadIdx.x; i < n_bins * 3; i += blockDim.x) bins[i] = 0ull;
  __syncthreads();
  const double t = temps[ti];
  const int s0 = blockIdx.y * kStsChunk, s1 = min(n, s0 + kStsChunk);
  for (int s = s0 + threadIdx.x; s < s1; s += blockDim.x) {
    const double c = 1.0 / (1.0 + exp(-(double)logit[(size_t)s * G + (k - 1)] / t));
    const double p = q[s] * c;
    int m = (int)floor(p * n_bins);
    m = m < 0 ? 0 : (m >= n_bins ? n_bins - 1 : m);
    atomicAdd(&bins[3 * m], (unsigned long long)__double2ull_rn(p * kStsFix));
    if (n_accept[s] >= k) atomicAdd(&bins[3 * m + 1], 1ull);
    atomicAdd(&bins[3 * m + 2], 1ull);
  }
  __syncthreads();
  unsigned long long* out = acc + (size_t)ti * n_bins * 3;
  for (int i = threadIdx.x; i < n_bins * 3; i += blockDim.x)
    if (bins[i]) atomicAdd(&out[i], bins[i]);
}

__global__ __launch_bounds__(256) void k_sts_select(int n, int k, int n_t, int n_bins,
                                                    const double* __restrict__ temps,
                                                    unsigned long long* __restrict__ acc,
                                                    double* __restrict__ t_out,
                                                    double* __restrict__ ece_out) {
  __shared__ double best_e[256];
  __shared__ int best_i[256];
  double be = INFINITY;
  int bi = 0x7FFFFFFF;
  for (int ti = threadIdx.x; ti < n_t; ti += blockDim.x) {
    const unsigned long long* a = acc + (size_t)ti * n_bins * 3;
    double e = 0.0;
    for (int m = 0; m < n_bins; ++m) {
      const long long d = (long long)a[3 * m] - (long long)(a[3 * m + 1] << 40);
      e += (double)(d < 0 ? -d : d);
    }
    e = e / ((double)n * kStsFix);
    if (e < be) { be = e; bi = ti; }    // ti increases: strict < keeps the first
  }
  best_e[threadIdx.x] = be;
  best_i[threadIdx.x] = bi;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < (int)blockDim.x; ++i)
      if (best_e[i] < be || (best_e[i] == be && best_i[i] < bi)) { be = best_e[i]; bi = best_i[i]; }
    t_out[k - 1] = temps[bi];
    ece_out[k - 1] = be;
  }
  __syncthreads();
  // the accumulators start from zero for the next position
  for (size_t i = threadIdx.x; i < (size_t)n_t * n_bins * 3; i += blockDim.x) acc[i] = 0ull;
}

__global__ __launch_bounds__(256) void k_sts_update(int n, int G, int k,
                                                    const float* __restrict__ logit,
                                                    const double* __restrict__ t_out,
                                                    double* __restrict__ q) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= n) return;
  const double t = t_out[k - 1];
  q[s] = q[s] * (1.0 / (1.0 + exp(-(double)logit[(size_t)s * G + (k - 1)] / t)));
}

}  // namespace dspark

using namespace dspark;

namespace {

struct StsWs {
  double* q;
  unsigned long long* acc;
  size_t bytes;
};

StsWs sts_ws(int n, int n_t, int n_bins, void* base) {
  Carve c(base);
  StsWs w;
  w.q = c.take<double>((size_t)n);
  w.acc = c.take<unsigned long long>((size_t)n_t * n_bins * 3);
  w.bytes = align_up(c.off, 256);
  return w;
}

bool sts_shape_ok(int n, int G, int n_t, int n_bins) {
  return n >= 1 && n <= kMaxStsSamples && G >= 1 && G <= 64 && n_t >= 1 && n_t <= 65535 &&
         n_bins >= 1 && n_bins <= kStsMaxBins;
}

}  // namespace

extern "C" size_t dspark_sts_workspace_bytes(int32_t n, int32_t n_t, int32_t n_bins) {
  if (n < 1 || n_t < 1 || n_bins < 1) return 0;
  return sts_ws(n, n_t, n_bins, nullptr).bytes;
}

extern "C" dspark_status dspark_sts_calibrate(int32_t n, int32_t G, const float* logit,
                                              const int32_t* n_accept, const double* temps,
                                              int32_t n_t, int32_t n_bins, double* t_out,
                                              double* ece_out, void* ws, size_t ws_bytes,
                                              void* stream) {
  if (!logit || !n_accept || !temps || !t_out || !ece_out) return DSPARK_E_NULL;
  if (!sts_shape_ok(n, G, n_t, n_bins)) return DSPARK_E_SHAPE;
  const StsWs need = sts_ws(n, n_t, n_bins, nullptr);
  if (!ws || ws_bytes < need.bytes) return DSPARK_E_WORKSPACE;
  const StsWs w = sts_ws(n, n_t, n_bins, ws);
  hipStream_t st = (hipStream_t)stream;
  const size_t nacc = (size_t)n_t * n_bins * 3;
  const size_t span = std::max((size_t)n, nacc);
  hipLaunchKernelGGL(k_sts_init, dim3((unsigned)std::min<size_t>(1024, (span + 255) / 256)),
                     dim3(256), 0, st, w.q, n, w.acc, nacc);
  const dim3 grid_bins((unsigned)n_t, (unsigned)((n + kStsChunk - 1) / kStsChunk));
  for (int k = 1; k <= G; ++k) {
    hipLaunchKernelGGL(k_sts_bins, grid_bins, dim3(256), 0, st, n, G, k, logit, n_accept, w.q,
                       temps, n_bins, w.acc);
    hipLaunchKernelGGL(k_sts_select, dim3(1), dim3(256), 0, st, n, k, n_t, n_bins, temps,
                       w.acc, t_out, ece_out);
    hipLaunchKernelGGL(k_sts_update, dim3((n + 255) / 256), dim3(256), 0, st, n, G, k, logit,
                       t_out, w.q);
  }
  return launch_status();
}
