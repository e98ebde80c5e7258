// schedule.hip -- hardware-aware prefix scheduler [XTL §6; CSDN throughput objective
// Theta = tau * SPS(B); paper Sec. 3.2.2 as quoted in the CSDN roundtable], entirely on
// the GPU in one workgroup.
//
//  1. prefix survival a_{b,j} = prod_{i<=j} c_{b,i}: one thread per request, fp64,
//     multiplied left to right (the same rounding sequence as the plain definition);
//  2. all (b, j) candidates sorted by (a descending, b ascending, j ascending) with a
//     bitonic network over keys held in registers (pairs within a wave exchange by lane
//     shuffles, pairs across waves through LDS) -- the key (a, b*gamma + j - 1) is a
//     total order;
//  3. the greedy walk: tau accumulates in fp64 in sorted order (a sequential chain, the
//     plain definition's rounding); the stop tests of 64 candidates at a time run in
//     parallel on one wave; the walk stops at the first candidate that does not raise
//     Theta.
// Since a_{b,j} is non-increasing in j (c <= 1) and ties go to the lower j, admissions
// are always prefixes of each request's block.
#include "dspark_dev.h"
#include "dspark_host.h"

namespace dspark {

__device__ __forceinline__ bool sched_before(double a1, uint32_t i1, double a2, uint32_t i2) {
  return a1 > a2 || (a1 == a2 && i1 < i2);
}

// One candidate key of the sort: (a, index), ordered by sched_before.
struct SKey {
  double a;
  uint32_t i;
};

__device__ __forceinline__ SKey shfl_xor_key(const SKey& k, int m) {
  SKey o;
  o.a = __shfl_xor(k.a, m, kWave);
  o.i = (uint32_t)__shfl_xor((int)k.i, m, kWave);
  return o;
}

// Compare-exchange of positions p (mine) and p ^ stride (the partner's key `o`) of a bitonic
// network: the lower position of a pair keeps the earlier key when the block of `size`
// sorts up, the later one when it sorts down; the higher position keeps the other.
__device__ __forceinline__ SKey bitonic_pick(const SKey& mine, const SKey& o, int p, int stride,
                                             int size) {
  const bool lower = (p & stride) == 0;
  const bool up = (p & size) == 0;
  const bool mine_first = sched_before(mine.a, mine.i, o.a, o.i);
  const bool keep_first = lower == up;
  return (mine_first == keep_first) ? mine : o;
}

// KPT keys per thread (positions KPT * tid + e) of a bitonic sort over NP = 1024 * KPT
// positions: pairs within a thread are exchanged in registers, pairs within a wave by lane
// shuffles, and only pairs across waves through LDS.
template <int KPT>
__device__ void bitonic_sort_regs(SKey (&k)[KPT], double* xa, uint32_t* xi) {
  constexpr int NP = 1024 * KPT;
  const int tid = threadIdx.x;
  for (int size = 2; size <= NP; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < KPT) {
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
          const int pe = e ^ stride;
          if (pe > e) {
            const int p = KPT * tid + e;
            const SKey lo = k[e], hi = k[pe];
            k[e] = bitonic_pick(lo, hi, p, stride, size);
            k[pe] = bitonic_pick(hi, lo, p ^ stride, stride, size);
          }
        }
      } else if (stride < KPT * kWave) {
        const int m = stride / KPT;   // partner lane offset within the wave
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
          const SKey o = shfl_xor_key(k[e], m);
          k[e] = bitonic_pick(k[e], o, KPT * tid + e, stride, size);
        }
      } else {
        __syncthreads();   // the previous exchange's readers are done
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
          xa[KPT * tid + e] = k[e].a;
          xi[KPT * tid + e] = k[e].i;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
          const int p = KPT * tid + e;
          const SKey o{xa[p ^ stride], xi[p ^ stride]};
          k[e] = bitonic_pick(k[e], o, p, stride, size);
        }
      }
    }
  }
}

template <int KPT>
__global__ __launch_bounds__(1024) void k_schedule(const float* __restrict__ c,
                                                   const double* __restrict__ sps, int B,
                                                   int G, int mode,
                                                   int32_t* __restrict__ ell,
                                                   double* __restrict__ theta,
                                                   int32_t* __restrict__ n_total) {
#pragma clang fp contract(off)
  constexpr int NP = 1024 * KPT;
  extern __shared__ __align__(16) unsigned char smem[];
  double* key_a = reinterpret_cast<double*>(smem);               // [NP]
  uint32_t* key_i = reinterpret_cast<uint32_t*>(key_a + NP);     // [NP]
  const int tid = threadIdx.x, n = B * G;
  // 1. prefix survival, one thread per request, left to right in fp64
  for (int b = tid; b < B; b += blockDim.x) {
    double a = 1.0;
    for (int j = 0; j < G; ++j) {
      a = a * (double)c[(size_t)b * G + j];
      key_a[b * G + j] = a;
      key_i[b * G + j] = (uint32_t)(b * G + j);
    }
  }
  for (int i = n + tid; i < NP; i += blockDim.x) {
    key_a[i] = -1.0;               // padding sorts after every real candidate
    key_i[i] = 0xFFFFFFFFu;
  }
  __syncthreads();
  // 2. sort into "before" order
  SKey k[KPT];
#pragma unroll
  for (int e = 0; e < KPT; ++e) k[e] = SKey{key_a[KPT * tid + e], key_i[KPT * tid + e]};
  bitonic_sort_regs<KPT>(k, key_a, key_i);
  __syncthreads();
#pragma unroll
  for (int e = 0; e < KPT; ++e) {
    key_a[KPT * tid + e] = k[e].a;
    key_i[KPT * tid + e] = k[e].i;
  }
  __syncthreads();
  // greedy walk on wave 0, 64 candidates per chunk.  tau_t follows the sequential fp64
  // chain tau_{t+1} = tau_t + a_(t) exactly (lane 0 order, broadcast per step); the best
  // Theta before candidate t is tau_t * sps[B + t] (each admission raises it to exactly
  // that product), so the stop tests of a chunk are independent and run in parallel.
  __shared__ int stop_s;
  __shared__ double tau_s;
  if (tid < 64) {
    const int lane = tid;
    double tau = (double)B;
    int stop = n;
    for (int base = 0; base < n; base += 64) {
      const int t = base + lane;
      const double at = t < n ? key_a[t] : 0.0;
      const int cnt = min(64, n - base);
      double before = 0.0, after = 0.0, cur = tau;
      for (int i = 0; i < cnt; ++i) {
        const double ai = __shfl(at, i, 64);
        before = (lane == i) ? cur : before;
        cur = cur + ai;
        after = (lane == i) ? cur : after;
      }
      bool halt = false;
      if (mode == DSPARK_SCHED_GREEDY && t < n) {
        const double th_next = after * sps[B + t + 1];
        const double th_best = before * sps[B + t];
        halt = th_next <= th_best;
      }
      const unsigned long long hm = __ballot(halt);
      if (hm) {
        const int first = __ffsll((long long)hm) - 1;
        stop = base + first;
        tau = __shfl(before, first, 64);
        break;
      }
      tau = cur;   // every lane ran the same chain: cur is the chunk's final tau
    }
    if (lane == 0) {
      stop_s = stop;
      tau_s = tau;
    }
  }
  __syncthreads();
  const int stop = stop_s;
  for (int b = tid; b < B; b += blockDim.x) ell[b] = 0;
  __syncthreads();
  // admitted candidates form a prefix of each request's block: ell_b = the largest j
  for (int t = tid; t < stop; t += blockDim.x) {
    const uint32_t i = key_i[t];
    atomicMax(&ell[i / G], (int)(i % G) + 1);
  }
  if (tid == 0) {
    const int N = B + stop;
    theta[0] = tau_s * sps[N];
    n_total[0] = N;
  }
}

}  // namespace dspark

using namespace dspark;

extern "C" dspark_status dspark_schedule(int32_t B, int32_t G, const float* c, const double* sps,
                                         int mode, int32_t* ell, double* theta,
                                         int32_t* n_total, void* ws, size_t ws_bytes,
                                         void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!c || !sps || !ell || !theta || !n_total) return DSPARK_E_NULL;
  if (B < 1 || G < 1 || G > 64 || (long long)B * G > kMaxSchedCandidates) return DSPARK_E_SHAPE;
  if (mode != DSPARK_SCHED_GREEDY && mode != DSPARK_SCHED_FULL) return DSPARK_E_VALUE;
  const int kpt = B * G <= 1024 ? 1 : (B * G <= 2048 ? 2 : 4);
  const size_t sh = (size_t)1024 * kpt * (sizeof(double) + sizeof(uint32_t));
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_schedule<4>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)((size_t)4096 * 12)) != hipSuccess)
      return DSPARK_E_HIP;
    attr_set = true;
  }
  hipStream_t st = (hipStream_t)stream;
  if (kpt == 1)
    hipLaunchKernelGGL(k_schedule<1>, dim3(1), dim3(1024), sh, st, c, sps, B, G, mode, ell,
                       theta, n_total);
  else if (kpt == 2)
    hipLaunchKernelGGL(k_schedule<2>, dim3(1), dim3(1024), sh, st, c, sps, B, G, mode, ell,
                       theta, n_total);
  else
    hipLaunchKernelGGL(k_schedule<4>, dim3(1), dim3(1024), sh, st, c, sps, B, G, mode, ell,
                       theta, n_total);
  return launch_status();
}
