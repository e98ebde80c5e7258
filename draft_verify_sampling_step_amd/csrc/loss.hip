// loss.hip -- distribution-matching training loss of the draft and confidence heads, forward
// and backward [XTL §9: cross-entropy on the true next token, an L1 (total-variation) term
// between the draft and target distributions, binary cross-entropy training the confidence
// head on the soft accept rate 1 - |p_d - p_t|_1 / 2, position weights exp(-(k-1)/gamma);
// XTL §5: the soft label is built from the two softmaxes; XTL §8: weights 0.1, 0.9, 1.0 in
// the open configuration].
//
// Per row (b, k) of V logits:
//   p_d = softmax(zd), p_t = softmax(zt), y = label
//   ce = -log p_d(y), l1 = sum |p_d - p_t|, a = 1 - l1/2 (held fixed), c = sigmoid(l),
//   bce = log(1 + e^l) - a l
//   loss = sum_rows w_k (alpha_ce ce + alpha_l1 l1 + alpha_conf bce) / W,
//   W = B sum_k w_k, w_k = exp(-(k-1)/gamma)
//   dloss/dzd_j = w_k/W (alpha_ce (p_d(j) - [j = y]) + alpha_l1 p_d(j) (s_j - S)),
//   s_j = sign(p_d(j) - p_t(j)), S = sum_v s_v p_d(v);  dloss/dl = w_k/W alpha_conf (c - a)
//
// The softmax normalisers, l1 and S are sums over the whole row, and the gradient needs all
// of them, so a row is three dependent sweeps.  Rows of 150k fp32 logits do not fit one
// compute unit, and re-reading them twice from HBM would more than double the traffic.
// Instead one cooperative launch keeps every logit in registers from its single read to the
// gradient write:
//   * a row's vocabulary is cut into C chunks of at most 4096 entries; a "stream" of C
//     workgroups (chunk c of rows p, p + P, p + 2P, ...) works through its rows together,
//     P streams at once, every workgroup resident (cooperative launch);
//   * each workgroup has four compute waves (16 entries of each row per lane, in registers)
//     and one control wave; while a row is processed the next row's chunk streams into LDS
//     by direct global-to-LDS loads, which the compiler's wait counting does not see, so
//     nothing in the row's three sweeps waits for them;
//   * the control wave alone talks to the other workgroups of its stream: it publishes the
//     workgroup's partials with device-scope stores, counts arrivals on a per-row counter,
//     polls it, and combines the C partials in fp64.  Keeping all polling and atomics on
//     that wave means the compute waves never wait on a counter load, so their prefetch
//     stays in flight; they meet the control wave at plain (fence-free) barriers.
//   * every wait is bounded: a poll that runs past its limit raises a fault word, the
//     stream stops, and the loss is written as NaN.
// HBM traffic: 8 bytes read and 4 written per logit (the gradient), plus 32 bytes of
// partials per chunk and row.
#include "dspark_dev.h"
#include "dspark_host.h"
#include "mfma_common.h"

namespace dspark {

constexpr int kLossComputeWaves = 4;
constexpr int kLossThreads = (kLossComputeWaves + 1) * kWave;   // + the control wave
constexpr int kLossPer = 16;                                     // entries per lane per row
constexpr int kLossChunk = kLossComputeWaves * kWave * kLossPer;  // 4096 entries
constexpr int kLossMaxVocab = 1 << 22;

struct LossArgs {
  const float* zd;
  const float* zt;
  const int32_t* labels;
  const float* conf;
  float* grad;          // [R][V] or null
  float* grad_conf;     // [R] or null
  float* terms;         // [R][3] or null
  double* rowloss;      // [R] weighted row contributions
  double* part1;        // [R][C][4] (max_d, sum_d, max_t, sum_t)
  double* part2;        // [R][C][2] (l1, S)
  uint32_t* cnt;        // [R][2] arrivals per row and exchange
  uint32_t* fault;
  int R, G, V, C, L, P;
  double a_ce, a_l1, a_conf, inv_W;
  uint32_t spin_limit;
};

__device__ __forceinline__ void raw_barrier() {
  // LDS writes complete, then a barrier without the release fence of __syncthreads()
  // (that fence would wait for the register prefetch as well)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ double ld_dev(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Control wave: publish this workgroup's partials (n doubles, held by lanes 0..n-1), arrive
// on the row's counter, wait for all C arrivals.  Lane 0 does the stores, the releasing
// increment and the polling; the whole wave then takes the acquire.  Returns false when the
// wait gave up.
__device__ __forceinline__ bool exchange(const LossArgs& a, double* slot, int n, double v,
                                         uint32_t* counter, int lane) {
  double vals[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vals[i] = __shfl(v, i, kWave);
  bool ok = true;
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i < n) st_dev(slot + i, vals[i]);
    __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t polls = 0;
    while (__hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
           (uint32_t)a.C) {
      if (++polls > a.spin_limit ||
          __hip_atomic_load(a.fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
        __hip_atomic_store(a.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return __shfl(ok ? 1 : 0, 0, kWave) != 0;
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, kWave));
  return v;
}

typedef float f4v __attribute__((ext_vector_type(4)));

// Entry e of a lane's slice: chunk-relative offset 4*lane' + 1024*(e/4) + e%4, lane' the
// lane index over the four compute waves.  Quad e/4 of the four compute waves is one
// contiguous 4 KiB piece of the chunk, 1 KiB per wave.
__device__ __forceinline__ int slice_off(int ct, int e) { return 4 * ct + 1024 * (e >> 2) + (e & 3); }

// Start the direct global-to-LDS loads of row r's chunk (draft logits at stage, target
// logits at stage + 16 KiB), each lane's quads landing where that same lane reads them back.
// A lane past the chunk's end loads its last quad (len is a positive multiple of 4); the
// entries it does not own are masked where they are used.
__device__ __forceinline__ void dma_row(const LossArgs& a, int r, int c, int ct, int wave,
                                        uint32_t stage) {
  const int c0 = c * a.L;
  const int len = min(a.L, a.V - c0);
  const size_t base = (size_t)r * a.V + c0;
  const float* pd = a.zd + base;
  const float* pt = a.zt + base;
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // earlier reads of the stage are done
#pragma unroll
  for (int q = 0; q < kLossPer / 4; ++q) {
    const int o = 4 * ct + 1024 * q;
    const uint32_t voff = 4u * (uint32_t)(o < len ? o : len - 4);
    // wave-uniform LDS address (M0)
    const uint32_t dst = __builtin_amdgcn_readfirstlane(stage + 4u * (uint32_t)(1024 * q + 256 * wave));
    dma16(pd, voff, dst);
    dma16(pt, voff, dst + 4u * kLossChunk);
  }
}

// the lane's entries of the staged chunk into registers
__device__ __forceinline__ void read_stage(const float* stage, int ct, float* d, float* t) {
#pragma unroll
  for (int q = 0; q < kLossPer / 4; ++q) {
    const f4v vd = *reinterpret_cast<const f4v*>(stage + 4 * ct + 1024 * q);
    const f4v vt = *reinterpret_cast<const f4v*>(stage + kLossChunk + 4 * ct + 1024 * q);
    d[4 * q] = vd.x; d[4 * q + 1] = vd.y; d[4 * q + 2] = vd.z; d[4 * q + 3] = vd.w;
    t[4 * q] = vt.x; t[4 * q + 1] = vt.y; t[4 * q + 2] = vt.z; t[4 * q + 3] = vt.w;
  }
}

// the lane's entries of row r straight from global memory (rows whose logits are not
// 16-byte aligned)
__device__ __forceinline__ void load_direct(const LossArgs& a, int r, int c, int ct, float* d,
                                            float* t) {
  const int c0 = c * a.L;
  const int len = min(a.L, a.V - c0);
  const size_t base = (size_t)r * a.V + c0;
#pragma unroll
  for (int e = 0; e < kLossPer; ++e) {
    const int o = slice_off(ct, e);
    const uint32_t oc = (uint32_t)(o < len ? o : len - 1);
    d[e] = a.zd[base + oc];
    t[e] = a.zt[base + oc];
  }
}

template <bool VEC>
__device__ __forceinline__ void store_grad(const LossArgs& a, int r, int c, int ct,
                                           const float* g) {
  const int c0 = c * a.L;
  const int len = min(a.L, a.V - c0);
  float* out = a.grad + (size_t)r * a.V + c0;
  if constexpr (VEC) {
#pragma unroll
    for (int q = 0; q < kLossPer / 4; ++q) {
      const int o = 4 * ct + 1024 * q;
      if (o < len)
        __builtin_nontemporal_store(f4v{g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]},
                                    reinterpret_cast<f4v*>(out + o));
    }
  } else {
#pragma unroll
    for (int e = 0; e < kLossPer; ++e) {
      const int o = slice_off(ct, e);
      if (o < len) out[o] = g[e];
    }
  }
}

// Entry e of the lane's slice lies inside the chunk (bit e of the lane's mask).
__device__ __forceinline__ bool live(uint32_t mask, int e) { return (mask >> e) & 1u; }

// (max, sum of exp(x - max)) of one lane's live entries; none live, or all -inf, gives
// (-inf, 0)
__device__ __forceinline__ ML lane_ml(const float* x, uint32_t mask) {
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < kLossPer; ++e) m = fmaxf(m, live(mask, e) ? x[e] : -INFINITY);
  if (m == -INFINITY) return ML{-INFINITY, 0.f};
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < kLossPer; ++e) s += live(mask, e) ? fast_exp(x[e] - m) : 0.f;
  return ML{m, s};
}

struct LossShared {
  float w1[kLossComputeWaves][4];   // per compute wave: (m_d, s_d, m_t, s_t)
  float w2[kLossComputeWaves][2];   // per compute wave: (l1, S)
  float r1[4];                      // row: (max_d, log sum_d, max_t, log sum_t)
  float r2[3];                      // row: (S, w alpha_ce, w alpha_l1)
  int y;                            // row: the label, clamped into the vocabulary
  double lse_d;                     // row: log-sum-exp of the draft logits (fp64)
  int stop;
};

// One row of the stream; the compute waves hold its slice in d, t.  Returns false when the
// stream must stop.
template <bool VEC>
__device__ __forceinline__ bool loss_row(const LossArgs& a, LossShared& sh, int r, int c,
                                         uint32_t mask, const float* d, const float* t) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const bool control = wave == kLossComputeWaves;
  const int ct = tid;   // lane index over the compute waves (control: unused)

  // ---- sweep 1: per-chunk softmax normalisers
  if (!control) {
    const ML md = wave_ml(lane_ml(d, mask));
    const ML mt = wave_ml(lane_ml(t, mask));
    if (lane == 0) {
      sh.w1[wave][0] = md.m; sh.w1[wave][1] = md.l;
      sh.w1[wave][2] = mt.m; sh.w1[wave][3] = mt.l;
    }
  }
  raw_barrier();
  if (control) {
    // combine the four waves (fp64), publish, wait, combine the C chunks (fp64)
    double v = 0.0;
    if (lane < 4) {
      const int off = (lane & 2);   // 0: draft, 2: target
      double m = -INFINITY;
      for (int w = 0; w < kLossComputeWaves; ++w) m = fmax(m, (double)sh.w1[w][off]);
      if (lane & 1) {
        double s = 0.0;
        if (m != -INFINITY)
          for (int w = 0; w < kLossComputeWaves; ++w)
            s += (double)sh.w1[w][off + 1] * (double)fast_exp(sh.w1[w][off] - (float)m);
        v = s;
      } else {
        v = m;
      }
    }
    double* slot = a.part1 + ((size_t)r * a.C + c) * 4;
    const bool ok = exchange(a, slot, 4, v, a.cnt + 2 * (size_t)r, lane);
    if (ok) {
      double m_d = -INFINITY, m_t = -INFINITY;
      for (int cc = lane; cc < a.C; cc += kWave) {
        const double* p = a.part1 + ((size_t)r * a.C + cc) * 4;
        m_d = fmax(m_d, ld_dev(p));
        m_t = fmax(m_t, ld_dev(p + 2));
      }
      m_d = wave_max_d(m_d);
      m_t = wave_max_d(m_t);
      double s_d = 0.0, s_t = 0.0;
      for (int cc = lane; cc < a.C; cc += kWave) {
        const double* p = a.part1 + ((size_t)r * a.C + cc) * 4;
        const double pm_d = ld_dev(p), ps_d = ld_dev(p + 1);
        const double pm_t = ld_dev(p + 2), ps_t = ld_dev(p + 3);
        if (ps_d > 0.0) s_d += ps_d * (double)fast_exp((float)(pm_d - m_d));
        if (ps_t > 0.0) s_t += ps_t * (double)fast_exp((float)(pm_t - m_t));
      }
      s_d = wave_sum_d(s_d);
      s_t = wave_sum_d(s_t);
      if (lane == 0) {
        const float ls_d = fast_log((float)s_d), ls_t = fast_log((float)s_t);
        sh.r1[0] = (float)m_d; sh.r1[1] = ls_d;
        sh.r1[2] = (float)m_t; sh.r1[3] = ls_t;
        sh.lse_d = m_d + (double)ls_d;
        sh.stop = 0;
      }
    } else if (lane == 0) {
      sh.stop = 1;
    }
  }
  raw_barrier();
  if (sh.stop) return false;

  // ---- sweep 2: l1 and S partials
  const float Md = sh.r1[0], Ld = sh.r1[1], Mt = sh.r1[2], Lt = sh.r1[3];
  if (!control) {
    float l1 = 0.f, S = 0.f;
#pragma unroll
    for (int e = 0; e < kLossPer; ++e) {
      const float pd = fast_exp((d[e] - Md) - Ld);
      const float pt = fast_exp((t[e] - Mt) - Lt);
      const float df = live(mask, e) ? pd - pt : 0.f;
      l1 += fabsf(df);
      S += df > 0.f ? pd : (df < 0.f ? -pd : 0.f);
    }
    l1 = wave_sum(l1);
    S = wave_sum(S);
    if (lane == 0) { sh.w2[wave][0] = l1; sh.w2[wave][1] = S; }
  }
  raw_barrier();
  if (control) {
    double v = 0.0;
    if (lane < 2)
      for (int w = 0; w < kLossComputeWaves; ++w) v += (double)sh.w2[w][lane];
    double* slot = a.part2 + ((size_t)r * a.C + c) * 2;
    const bool ok = exchange(a, slot, 2, v, a.cnt + 2 * (size_t)r + 1, lane);
    if (ok) {
      double l1 = 0.0, S = 0.0;
      for (int cc = lane; cc < a.C; cc += kWave) {
        const double* p = a.part2 + ((size_t)r * a.C + cc) * 2;
        l1 += ld_dev(p);
        S += ld_dev(p + 1);
      }
      l1 = wave_sum_d(l1);
      S = wave_sum_d(S);
      const int k = r % a.G;
      const double wk = (double)fast_exp(-(float)k / (float)a.G) * a.inv_W;
      if (lane == 0) {
        sh.r2[0] = (float)S;
        sh.r2[1] = (float)(wk * a.a_ce);
        sh.r2[2] = (float)(wk * a.a_l1);
        sh.y = clamp_tok(a.labels[r], a.V);
        sh.stop = 0;
      }
      if (c == 0 && lane == 0) {
        // the row's scalar terms (chunk 0's control wave)
        const int y = clamp_tok(a.labels[r], a.V);
        const double ce = sh.lse_d - (double)a.zd[(size_t)r * a.V + y];
        const double at = 1.0 - 0.5 * l1;
        // log(1 + e^l) and sigmoid(l) in fp32 through e = exp(-|l|) in (0, 1]
        const float lf = a.conf[r];
        const float e = fast_exp(-fabsf(lf));
        const double l = (double)lf;
        const double softplus = (double)fmaxf(lf, 0.f) + (double)log1pf(e);
        const double bce = softplus - at * l;
        const double cs = lf >= 0.f ? 1.0 / (1.0 + (double)e) : (double)e / (1.0 + (double)e);
        a.rowloss[r] = wk * (a.a_ce * ce + a.a_l1 * l1 + a.a_conf * bce);
        if (a.terms) {
          a.terms[3 * (size_t)r] = (float)ce;
          a.terms[3 * (size_t)r + 1] = (float)l1;
          a.terms[3 * (size_t)r + 2] = (float)bce;
        }
        if (a.grad_conf) a.grad_conf[r] = (float)(wk * a.a_conf * (cs - at));
      }
    } else if (lane == 0) {
      sh.stop = 1;
    }
  }
  raw_barrier();
  if (sh.stop) return false;

  // ---- sweep 3: the gradient of the draft logits
  if (!control && a.grad) {
    const float S = sh.r2[0], fa = sh.r2[1], fb = sh.r2[2];
    const int y = sh.y - c * a.L;   // chunk-relative label
    float g[kLossPer];
#pragma unroll
    for (int e = 0; e < kLossPer; ++e) {
      const float pd = fast_exp((d[e] - Md) - Ld);
      const float pt = fast_exp((t[e] - Mt) - Lt);
      const float df = pd - pt;
      const float s = df > 0.f ? 1.f : (df < 0.f ? -1.f : 0.f);
      const float oh = slice_off(ct, e) == y ? 1.f : 0.f;
      g[e] = fa * (pd - oh) + fb * pd * (s - S);
    }
    store_grad<VEC>(a, r, c, ct, g);
  }
  return true;
}

template <bool VEC>
__global__ __launch_bounds__(kLossThreads) void k_draft_loss(LossArgs a) {
  __shared__ LossShared sh;
  __shared__ __align__(16) float stage[VEC ? 2 * kLossChunk : 1];   // the next row's chunk
  const int p = blockIdx.x / a.C, c = blockIdx.x % a.C;
  if (p >= a.P) return;
  const int tid = threadIdx.x, wave = tid / kWave;
  const bool compute = wave < kLossComputeWaves;
  const uint32_t stage_lds = (uint32_t)(uintptr_t)(lds_ptr_t)stage;
  // which of the lane's entries lie inside its chunk (the same for every row)
  const int len = min(a.L, a.V - c * a.L);
  uint32_t mask = 0;
#pragma unroll
  for (int e = 0; e < kLossPer; ++e) mask |= (slice_off(tid, e) < len ? 1u : 0u) << e;
  float d[kLossPer], t[kLossPer];
  if constexpr (VEC) {
    if (compute) dma_row(a, p, c, tid, wave, stage_lds);
  }
  for (int r = p; r < a.R; r += a.P) {
    if (compute) {
      if constexpr (VEC) {
        wait_vm<0>();                    // this lane's share of row r has landed
        read_stage(stage, tid, d, t);
        if (r + a.P < a.R) dma_row(a, r + a.P, c, tid, wave, stage_lds);
      } else {
        load_direct(a, r, c, tid, d, t);
      }
    }
    if (!loss_row<VEC>(a, sh, r, c, mask, d, t)) break;
  }
  if constexpr (VEC) wait_vm<0>();   // nothing in flight into LDS when the workgroup ends
}

__global__ __launch_bounds__(256) void k_loss_init(uint32_t* __restrict__ cnt, size_t n,
                                                   uint32_t* __restrict__ fault) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  for (size_t j = i; j < n; j += (size_t)gridDim.x * blockDim.x) cnt[j] = 0u;
  if (i == 0) *fault = 0u;
}

// loss = sum of the row contributions in a fixed order (deterministic), NaN after a fault
__global__ __launch_bounds__(256) void k_loss_sum(const double* __restrict__ rowloss, int R,
                                                  const uint32_t* __restrict__ fault,
                                                  double* __restrict__ loss) {
  __shared__ double part[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < R; i += 256) s += rowloss[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = *fault ? NAN : part[0];
}

}  // namespace dspark

using namespace dspark;

namespace {

struct LossWs {
  double* part1;
  double* part2;
  double* rowloss;
  uint32_t* cnt;
  uint32_t* fault;
  size_t bytes;
};

int loss_chunks(int V) { return (V + kLossChunk - 1) / kLossChunk; }

LossWs loss_ws(int R, int V, void* base) {
  const int C = loss_chunks(V);
  Carve c(base);
  LossWs w;
  w.part1 = c.take<double>((size_t)R * C * 4);
  w.part2 = c.take<double>((size_t)R * C * 2);
  w.rowloss = c.take<double>((size_t)R);
  w.cnt = c.take<uint32_t>((size_t)R * 2);
  w.fault = c.take<uint32_t>(1);
  w.bytes = align_up(c.off, 256);
  return w;
}

bool loss_shape_ok(int B, int G, int V) {
  return B >= 1 && G >= 1 && G <= 64 && (long long)B * G <= (1 << 24) && V >= 1 &&
         V <= kLossMaxVocab;
}

// resident workgroups of the loss kernel on the current device (0 when cooperative launch
// is unavailable)
template <bool VEC>
int loss_capacity() {
  static int cap = -1;
  if (cap < 0) {
    int dev = 0, coop = 0, ncu = 0, per_cu = 0;
    cap = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_draft_loss<VEC>,
                                                     kLossThreads, 0) == hipSuccess && coop)
      cap = per_cu * ncu;
  }
  return cap;
}

}  // namespace

extern "C" size_t dspark_loss_workspace_bytes(int32_t B, int32_t G, int32_t V) {
  if (!loss_shape_ok(B, G, V)) return 0;
  return loss_ws(B * G, V, nullptr).bytes;
}

extern "C" dspark_status dspark_draft_loss(int32_t B, int32_t G, int32_t V, const float* zd,
                                           const float* zt, const int32_t* labels,
                                           const float* conf_logit, double alpha_ce,
                                           double alpha_l1, double alpha_conf, double* loss,
                                           float* terms, float* grad_zd, float* grad_conf,
                                           void* ws, size_t ws_bytes, void* stream) {
  if (!zd || !zt || !labels || !conf_logit || !loss) return DSPARK_E_NULL;
  if (!loss_shape_ok(B, G, V)) return DSPARK_E_SHAPE;
  if (!std::isfinite(alpha_ce) || !std::isfinite(alpha_l1) || !std::isfinite(alpha_conf))
    return DSPARK_E_VALUE;
  const int R = B * G;
  const LossWs need = loss_ws(R, V, nullptr);
  if (!ws || ws_bytes < need.bytes) return DSPARK_E_WORKSPACE;
  const LossWs w = loss_ws(R, V, ws);
  const bool vec = V % 4 == 0 && ((uintptr_t)zd % 16 == 0) && ((uintptr_t)zt % 16 == 0) &&
                   (!grad_zd || (uintptr_t)grad_zd % 16 == 0);
  const int cap = vec ? loss_capacity<true>() : loss_capacity<false>();
  LossArgs a;
  a.zd = zd; a.zt = zt; a.labels = labels; a.conf = conf_logit;
  a.grad = grad_zd; a.grad_conf = grad_conf; a.terms = terms;
  a.rowloss = w.rowloss; a.part1 = w.part1; a.part2 = w.part2; a.cnt = w.cnt; a.fault = w.fault;
  a.R = R; a.G = G; a.V = V;
  a.C = loss_chunks(V);
  a.L = (V + 4 * a.C - 1) / (4 * a.C) * 4;
  if (cap < a.C) return DSPARK_E_HIP;   // no cooperative launch, or a row does not fit
  a.P = std::min(R, cap / a.C);
  double wsum = 0.0;
  for (int k = 0; k < G; ++k) wsum += std::exp(-(double)k / G);
  a.inv_W = 1.0 / ((double)B * wsum);
  a.a_ce = alpha_ce; a.a_l1 = alpha_l1; a.a_conf = alpha_conf;
  a.spin_limit = 1u << 22;
  hipStream_t st = (hipStream_t)stream;
  const size_t ncnt = (size_t)R * 2;
  hipLaunchKernelGGL(k_loss_init, dim3((unsigned)std::min<size_t>(256, (ncnt + 255) / 256)),
                     dim3(256), 0, st, w.cnt, ncnt, w.fault);
  if (launch_status() != DSPARK_OK) return DSPARK_E_HIP;
  void* args[] = {&a};
  const void* fn = vec ? (const void*)k_draft_loss<true> : (const void*)k_draft_loss<false>;
  if (hipLaunchCooperativeKernel(fn, dim3((unsigned)(a.P * a.C)), dim3(kLossThreads), args, 0,
                                 st) != hipSuccess) {
    (void)hipGetLastError();
    return DSPARK_E_HIP;
  }
  hipLaunchKernelGGL(k_loss_sum, dim3(1), dim3(256), 0, st, w.rowloss, R, w.fault, loss);
  return launch_status();
}
