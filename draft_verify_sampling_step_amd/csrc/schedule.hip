// schedule.hip -- hardware-aware prefix scheduler [XTL §6; CSDN throughput objective
// Theta = tau * SPS(B); paper Sec. 3.2.2 as quoted in the CSDN roundtable], entirely on
// the GPU in one workgroup.
//
//  1. prefix survival a_{b,j} = prod_{i<=j} c_{b,i}: one thread per request, fp64,
//     multiplied left to right (the same rounding sequence as the plain definition);
//  2. all (b, j) candidates put in order by (a descending, b ascending, j ascending) --
//     the key (a, b*gamma + j - 1) is a total order.  Each request's run of gamma is in
//     order already (its prefix products never increase when every c <= 1; a run that is
//     not is sorted by insertion), so adjacent runs are merged level by level in LDS,
//     every output slot locating its source with a merge-path binary search.  The merged
//     blocks hold consecutive requests, so every index of the left block is below every
//     index of the right one: a tie of a goes to the left, and the merge compares the a
//     values alone (kept apart from the indices, 8 bytes per LDS read);
//  3. the greedy walk: tau accumulates in fp64 in sorted order (a sequential chain, the
//     plain definition's rounding); the stop tests of 64 candidates at a time run in
//     parallel on one wave; the walk stops at the first candidate that does not raise
//     Theta.
// Since a_{b,j} is non-increasing in j (c <= 1) and ties go to the lower j, admissions
// are always prefixes of each request's block.
#include "dspark_dev.h"
#include "dspark_host.h"

namespace dspark {

// LDS bytes per candidate: its a (fp64) and its index b * gamma + j - 1 (u32), each in
// two buffers (merge source and destination)
constexpr size_t kSchedBytesPer = 2 * (sizeof(double) + sizeof(uint32_t));

// Number of elements of A (length la) among the first `diag` elements of the merge of the
// sorted runs A and B, where every index in A is below every index in B (so an element of
// B goes first only when its a is strictly larger; the split is unique).
__device__ __forceinline__ int merge_split(const double* A, int la, const double* Bv, int lb,
                                           int diag) {
  int lo = diag > lb ? diag - lb : 0, hi = diag < la ? diag : la;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (Bv[diag - 1 - mid] > A[mid])
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

// mode of k_schedule beyond the two public ones: admit the first k_admit candidates
constexpr int kSchedTopK = 2;

// SPS entries B..B+kSpsWin staged in LDS for the walk (the walk usually stops early)
constexpr int kSpsWin = 512;

// In top-K mode with n_hist not NULL, k_admit is read on the device: n_hist[0] - B,
// clamped into [0, B * G] (n_hist is the N of a schedule made earlier on the stream).
__global__ __launch_bounds__(1024) void k_schedule(const float* __restrict__ c,
                                                   const double* __restrict__ sps, int B,
                                                   int G, int mode, int k_admit,
                                                   const int32_t* __restrict__ n_hist,
                                                   int32_t* __restrict__ ell,
                                                   double* __restrict__ theta,
                                                   int32_t* __restrict__ n_total) {
#pragma clang fp contract(off)
  extern __shared__ __align__(16) unsigned char smem[];
  const int tid = threadIdx.x, n = B * G;
  if (mode == kSchedTopK && n_hist) k_admit = min(max(n_hist[0] - B, 0), n);
  double* XA = reinterpret_cast<double*>(smem);   // a: [n], then [n] for the other buffer
  double* YA = XA + n;
  uint32_t* XI = reinterpret_cast<uint32_t*>(YA + n);   // index: [n], then [n]
  uint32_t* YI = XI + n;
  __shared__ double sps_win[kSpsWin + 1];    // sps[B + i], i <= min(n, kSpsWin)
  for (int i = tid; i <= min(n, kSpsWin); i += blockDim.x) sps_win[i] = sps[B + i];
  // 1. prefix survival, one thread per request, left to right in fp64.  With every
  // c <= 1 a request's run is already in order (a non-increasing, index increasing); a run
  // that is not (some c > 1) is put in order by insertion.
  for (int b = tid; b < B; b += blockDim.x) {
    double* ra = XA + (size_t)b * G;
    uint32_t* ri = XI + (size_t)b * G;
    double a = 1.0;
    bool sorted = true;
    for (int j = 0; j < G; ++j) {
      const double prev = a;
      a = a * (double)c[(size_t)b * G + j];
      sorted = sorted && !(a > prev);
      ra[j] = a;
      ri[j] = (uint32_t)(b * G + j);
    }
    if (!sorted) {
      // (a descending, index ascending) within the run
      for (int j = 1; j < G; ++j) {
        const double ka = ra[j];
        const uint32_t ki = ri[j];
        int q = j - 1;
        while (q >= 0 && (ka > ra[q] || (ka == ra[q] && ki < ri[q]))) {
          ra[q + 1] = ra[q];
          ri[q + 1] = ri[q];
          --q;
        }
        ra[q + 1] = ka;
        ri[q + 1] = ki;
      }
    }
  }
  __syncthreads();
  // 2. bottom-up merge of adjacent runs (length G, 2G, ...) into the full order.  A thread
  // makes two consecutive output slots: the merge-path search locates the first, the second
  // follows by one more comparison (a merged block has even length except the last, which
  // ends at n, so both slots lie in one block).
  for (int L = G; L < n; L <<= 1) {
    for (int p = 2 * tid; p < n; p += 2 * blockDim.x) {
      const int base = p / (2 * L) * (2 * L);
      const int la = min(L, n - base), lb = min(L, max(0, n - base - L));
      const double* A = XA + base;
      const double* Bv = A + la;
      const int d = p - base;
      int i = merge_split(A, la, Bv, lb, d), j = d - i;
      // the left element goes first unless the right one's a is strictly larger
      bool take_a = i < la && (j >= lb || A[i] >= Bv[j]);
      YA[p] = take_a ? A[i] : Bv[j];
      YI[p] = XI[base + (take_a ? i : la + j)];
      if (p + 1 < n) {
        i += take_a ? 1 : 0;
        j += take_a ? 0 : 1;
        take_a = i < la && (j >= lb || A[i] >= Bv[j]);
        YA[p + 1] = take_a ? A[i] : Bv[j];
        YI[p + 1] = XI[base + (take_a ? i : la + j)];
      }
    }
    __syncthreads();
    double* ta = XA;
    XA = YA;
    YA = ta;
    uint32_t* ti = XI;
    XI = YI;
    YI = ti;
  }
  // greedy walk on wave 0, 64 candidates per chunk.  tau_t follows the sequential fp64
  // chain tau_{t+1} = tau_t + a_(t) exactly: every lane runs the whole chain of the chunk
  // on a_(t) values read from LDS ahead of it (one address for all lanes), and after each
  // add all lanes store the same running value into chain[i + 1], so lane i then reads the
  // values before and after its own add.  The best Theta before candidate t is
  // tau_t * sps[B + t] (each admission raises it to exactly that product), so the stop
  // tests of a chunk are independent and run in parallel.
  __shared__ int stop_s;
  __shared__ double tau_s;
  __shared__ double chain[65];
  if (tid < 64) {
    const int lane = tid;
    double tau = (double)B;
    int stop = n;
    for (int base = 0; base < n; base += 64) {
      const int t = base + lane;
      const int cnt = min(64, n - base);
      const double* ab = XA + base;
      double cur = tau;
      chain[0] = cur;
      if (cnt == 64) {
        // a full chunk: 16 values in registers at a time, the next 16 loaded before the
        // adds of these
        double av[16], nv[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) av[i] = ab[i];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          if (blk < 3) {
#pragma unroll
            for (int i = 0; i < 16; ++i) nv[i] = ab[16 * (blk + 1) + i];
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            cur = cur + av[i];
            chain[16 * blk + i + 1] = cur;
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) av[i] = nv[i];
        }
      } else {
        for (int i = 0; i < cnt; ++i) {
          cur = cur + ab[i];
          chain[i + 1] = cur;
        }
      }
      __builtin_amdgcn_wave_barrier();
      const double before = chain[lane];
      const double after = chain[lane + 1];
      bool halt = false;
      if (mode == DSPARK_SCHED_GREEDY && t < n) {
        const double sp1 = t + 1 <= kSpsWin ? sps_win[t + 1] : sps[B + t + 1];
        const double sp0 = t <= kSpsWin ? sps_win[t] : sps[B + t];
        const double th_next = after * sp1;
        const double th_best = before * sp0;
        halt = th_next <= th_best;
      } else if (mode == kSchedTopK && t < n) {
        halt = t == k_admit;                   // the first k_admit are in, no more
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
    const uint32_t i = XI[t];
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

namespace dspark {

// the kernel's dynamic LDS may exceed the default limit: raise it once per device
dspark_status sched_prepare() {
  static LdsAttr attr;
  return attr.ensure((const void*)k_schedule,
                     (int)((size_t)kMaxSchedCandidates * kSchedBytesPer));
}

dspark_status schedule_topk_from_history(int B, int G, const float* c, const double* sps,
                                         const int32_t* n_hist, int32_t* ell, double* theta,
                                         int32_t* n_total, hipStream_t st) {
  if (!c || !sps || !n_hist || !ell || !theta || !n_total) return DSPARK_E_NULL;
  if (B < 1 || G < 1 || G > 64 || (long long)B * G > kMaxSchedCandidates) return DSPARK_E_SHAPE;
  if (sched_prepare() != DSPARK_OK) return DSPARK_E_HIP;
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(1024), (size_t)B * G * kSchedBytesPer, st, c,
                     sps, B, G, kSchedTopK, 0, n_hist, ell, theta, n_total);
  return launch_status();
}

}  // namespace dspark

extern "C" dspark_status dspark_schedule(int32_t B, int32_t G, const float* c, const double* sps,
                                         int mode, int32_t* ell, double* theta,
                                         int32_t* n_total, void* ws, size_t ws_bytes,
                                         void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!c || !sps || !ell || !theta || !n_total) return DSPARK_E_NULL;
  if (B < 1 || G < 1 || G > 64 || (long long)B * G > kMaxSchedCandidates) return DSPARK_E_SHAPE;
  if (mode != DSPARK_SCHED_GREEDY && mode != DSPARK_SCHED_FULL) return DSPARK_E_VALUE;
  const size_t sh = (size_t)B * G * kSchedBytesPer;
  if (sched_prepare() != DSPARK_OK) return DSPARK_E_HIP;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(1024), sh, st, c, sps, B, G, mode, 0, nullptr,
                     ell, theta, n_total);
  return launch_status();
}

extern "C" dspark_status dspark_schedule_topk(int32_t B, int32_t G, const float* c,
                                              const double* sps, int32_t k_admit, int32_t* ell,
                                              double* theta, int32_t* n_total, void* ws,
                                              size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (!c || !sps || !ell || !theta || !n_total) return DSPARK_E_NULL;
  if (B < 1 || G < 1 || G > 64 || (long long)B * G > kMaxSchedCandidates) return DSPARK_E_SHAPE;
  if (k_admit < 0) return DSPARK_E_VALUE;
  const int k = (long long)k_admit > (long long)B * G ? B * G : k_admit;
  const size_t sh = (size_t)B * G * kSchedBytesPer;
  if (sched_prepare() != DSPARK_OK) return DSPARK_E_HIP;
  hipLaunchKernelGGL(k_schedule, dim3(1), dim3(1024), sh, (hipStream_t)stream, c, sps, B, G,
                     kSchedTopK, k, nullptr, ell, theta, n_total);
  return launch_status();
}
