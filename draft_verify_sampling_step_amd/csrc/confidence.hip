// confidence.hip -- confidence head [CSDN Eq. 7; XTL §5]:
//   c_k = sigmoid(w . [h_k ; W1[x_{k-1}]]),  x_0 = anchor, no bias term;
// calibrated form (sequential temperature scaling, [XTL §5]): c_k = sigmoid(logit_k / t_k).
// One wave per (request, position): a wave-reduced dot product of length d + r with
// coalesced 16-byte loads where the element type allows.
#include "dspark_dev.h"
#include "dspark_host.h"

namespace dspark {

// Sum of w[j] * x[j] over j < n, lanes striding 8 elements (16-byte loads for bf16 when
// both pointers are 16-byte aligned), element by element otherwise.  Each lane adds its
// terms in index order; the loads of up to eight rounds are issued before the first add.
template <typename TA, typename TB>
__device__ __forceinline__ float lane_dot(const TA* w, const TB* x, int n, int lane) {
  float acc = 0.f;
  for (int jb = lane; jb < n; jb += 8 * kWave) {
    float a[8], b[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (jb + t * kWave < n) {
        a[t] = Elem<TA>::get(w, jb + t * kWave);
        b[t] = Elem<TB>::get(x, jb + t * kWave);
      }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (jb + t * kWave >= n) break;
      acc = fmaf(a[t], b[t], acc);
    }
  }
  return acc;
}

template <>
__device__ __forceinline__ float lane_dot<uint16_t, uint16_t>(const uint16_t* w,
                                                             const uint16_t* x, int n,
                                                             int lane) {
  float acc = 0.f;
  const bool aligned = ((((uintptr_t)w) | ((uintptr_t)x)) & 15) == 0;
  int jt = 0;
  if (aligned) {
    const int nv = n & ~511;   // whole 64-lane x 8-element rounds
    for (int jb = lane * 8; jb < nv; jb += 8 * kWave * 8) {
      uint4 a[8], b[8];
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (jb + t * kWave * 8 < nv) {
          a[t] = *reinterpret_cast<const uint4*>(w + jb + t * kWave * 8);
          b[t] = *reinterpret_cast<const uint4*>(x + jb + t * kWave * 8);
        }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (jb + t * kWave * 8 >= nv) break;
        const uint32_t av[4] = {a[t].x, a[t].y, a[t].z, a[t].w};
        const uint32_t bv[4] = {b[t].x, b[t].y, b[t].z, b[t].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc = fmaf(__uint_as_float(av[q] << 16), __uint_as_float(bv[q] << 16), acc);
          acc = fmaf(__uint_as_float(av[q] & 0xFFFF0000u),
                     __uint_as_float(bv[q] & 0xFFFF0000u), acc);
        }
      }
    }
    jt = nv;
  }
  // the rest element by element
  for (int jb = jt + lane; jb < n; jb += 8 * kWave) {
    float a[8], b[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
      if (jb + t * kWave < n) {
        a[t] = bf16_to_f32(w[jb + t * kWave]);
        b[t] = bf16_to_f32(x[jb + t * kWave]);
      }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if (jb + t * kWave >= n) break;
      acc = fmaf(a[t], b[t], acc);
    }
  }
  return acc;
}

template <typename TH, typename TW1, typename TWV>
__global__ __launch_bounds__(256) void k_confidence(const TH* __restrict__ h,
                                                    const TW1* __restrict__ W1,
                                                    const TWV* __restrict__ w,
                                                    const int32_t* __restrict__ anchor,
                                                    const int32_t* __restrict__ tokens,
                                                    const double* __restrict__ temps,
                                                    float* __restrict__ c, int B, int G, int d,
                                                    int r, int V) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= B * G) return;
  const int b = wid / G, k = wid % G + 1;
  const int prev = clamp_tok((k == 1) ? anchor[b] : tokens[(size_t)b * G + (k - 2)], V);
  float acc = lane_dot<TWV, TH>(w, h + (size_t)wid * d, d, lane);
  acc += lane_dot<TWV, TW1>(w + d, W1 + (size_t)prev * r, r, lane);
  acc = wave_sum(acc);
  if (temps) acc = (float)((double)acc / temps[k - 1]);
  if (lane == 0) c[wid] = 1.0f / (1.0f + expf(-acc));
}

template <typename TH, typename TW1, typename TWV>
static void launch_conf(const dspark_dims* dm, const void* h, const void* W1, const void* w,
                        const int32_t* anchor, const int32_t* tokens, const double* temps,
                        float* c, hipStream_t st) {
  const int n = dm->batch * dm->gamma;
  hipLaunchKernelGGL((k_confidence<TH, TW1, TWV>), dim3((n + 3) / 4), dim3(256), 0, st,
                     (const TH*)h, (const TW1*)W1, (const TWV*)w, anchor, tokens, temps, c,
                     dm->batch, dm->gamma, dm->hidden, dm->rank, dm->vocab);
}

}  // namespace dspark

using namespace dspark;

namespace {

dspark_status confidence_impl(const dspark_dims* dm, const void* h, int hdt, const void* W1,
                              int wdt, const void* w, int wvdt, const int32_t* anchor,
                              const int32_t* tokens, const double* temps, float* c,
                              void* stream) {
  if (!dm || !W1 || !w || !anchor || !tokens || !c) return DSPARK_E_NULL;
  if (!dims_ok(dm)) return DSPARK_E_SHAPE;
  if (dm->hidden > 0 && !h) return DSPARK_E_NULL;
  if (!dtype_ok(hdt) || !dtype_ok(wdt) || !dtype_ok(wvdt)) return DSPARK_E_DTYPE;
  hipStream_t st = (hipStream_t)stream;
  const int code = (hdt << 2) | (wdt << 1) | wvdt;
  const double* tp = temps;
  switch (code) {
    case 0: launch_conf<float, float, float>(dm, h, W1, w, anchor, tokens, tp, c, st); break;
    case 1: launch_conf<float, float, uint16_t>(dm, h, W1, w, anchor, tokens, tp, c, st); break;
    case 2: launch_conf<float, uint16_t, float>(dm, h, W1, w, anchor, tokens, tp, c, st); break;
    case 3: launch_conf<float, uint16_t, uint16_t>(dm, h, W1, w, anchor, tokens, tp, c, st); break;
    case 4: launch_conf<uint16_t, float, float>(dm, h, W1, w, anchor, tokens, tp, c, st); break;
    case 5: launch_conf<uint16_t, float, uint16_t>(dm, h, W1, w, anchor, tokens, tp, c, st); break;
    case 6: launch_conf<uint16_t, uint16_t, float>(dm, h, W1, w, anchor, tokens, tp, c, st); break;
    default: launch_conf<uint16_t, uint16_t, uint16_t>(dm, h, W1, w, anchor, tokens, tp, c, st); break;
  }
  return launch_status();
}

}  // namespace

extern "C" dspark_status dspark_confidence(const dspark_dims* dm, const void* h, int hdt,
                                           const void* W1, int wdt, const void* w, int wvdt,
                                           const int32_t* anchor, const int32_t* tokens,
                                           float* c, void* stream) {
  return confidence_impl(dm, h, hdt, W1, wdt, w, wvdt, anchor, tokens, nullptr, c, stream);
}

extern "C" dspark_status dspark_confidence_calibrated(const dspark_dims* dm, const void* h,
                                                      int hdt, const void* W1, int wdt,
                                                      const void* w, int wvdt,
                                                      const int32_t* anchor,
                                                      const int32_t* tokens,
                                                      const double* temps, float* c,
                                                      void* stream) {
  if (!temps) return DSPARK_E_NULL;
  return confidence_impl(dm, h, hdt, W1, wdt, w, wvdt, anchor, tokens, temps, c, stream);
}
