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
// Instead one cooperative launch keeps every logit on chip from its single read to the
// gradient write:
//   * a row's vocabulary is cut into C chunks of at most 8192 entries; a "stream" of C
//     workgroups (chunk c of each of its rows) works through its rows together, P streams
//     at once, every workgroup resident (cooperative launch).  Stream p starts with rows p
//     and p + P; every further row is claimed from a row counter one exchange ahead, so
//     the streams that run faster (their workgroups placed first on their compute units)
//     take more rows;
//   * a workgroup is eight waves (two per SIMD, so two workgroups pack evenly on a compute
//     unit), 16 entries of the current row per lane in registers; the next row's chunk
//     streams into LDS by direct global-to-LDS loads, which the compiler's wait counting
//     does not see, so nothing waits for them before they are needed;
//   * the stream meets once per row: one exchange carries the current row's L1 and S
//     partials together with the next row's (max, sum) partials, which the waves compute
//     from the LDS copy; wave 0 publishes each as one 64-bit word (a written-mark and the
//     fp32 value) with a device-scope atomic store, then polls the C workgroups' words
//     directly -- the data arrive with the poll -- and combines them in fp64.  No counter,
//     no store-completion wait and no cache-wide fence is involved;
//   * every wait is bounded: a poll that runs past its limit raises a fault word, the
//     stream stops, and the loss is written as NaN.
// HBM traffic: 8 bytes read and 4 written per logit (the gradient), plus 56 bytes of
// published words per chunk and row (cleared before the launch).
#include <atomic>

#include "dspark_dev.h"
#include "dspark_host.h"
#include "mfma_common.h"

namespace dspark {

constexpr int kLossWaves = 8;                             // every wave holds entries
constexpr int kLossThreads = kLossWaves * kWave;          // two waves per SIMD
constexpr int kLossWavesPerSimd = 4;                      // occupancy target (<= 128 VGPRs)
constexpr int kLossPer = 16;                              // entries per lane per row
constexpr int kLossChunk = kLossThreads * kLossPer;       // 8192 entries
constexpr int kQuad = 4 * kLossThreads;                   // chunk offset between a lane's quads
constexpr int kLossMaxVocab = 1 << 22;
// Polls between two looks at the fault word (every poller reading one shared word each
// time would make it a hot spot).
constexpr uint32_t kFaultCheckPolls = 64;
// A published partial is the 64-bit word kSlotValid | (fp32 bits): the words are cleared to
// zero before the launch, so one atomic store both carries a value and announces it, and a
// reader needs no separate arrival counter.
constexpr unsigned long long kSlotValid = 1ull << 32;

struct LossArgs {
  const float* zd;
  const float* zt;
  const int32_t* labels;
  const float* conf;
  float* grad;          // [R][V] or null
  float* grad_conf;     // [R] or null
  float* terms;         // [R][3] or null
  double* rowloss;      // [R] weighted row contributions (device-scope atomic stores)
  double* loss;         // [1] out: their sum, taken by the last workgroup to finish
  unsigned long long* part1;   // [R][C][4] published (max_d, sum_d, max_t, sum_t)
  unsigned long long* part2;   // [R][C][3] published (l1, S, chunk 0 only: the row after
                               // the next one of the stream, claimed; R when none)
  unsigned int* row_ctr;       // rows claimed beyond the first 2P (cleared before launch)
  unsigned int* done_ctr;      // workgroups finished (cleared before launch)
  uint32_t* fault;
  int R, G, V, C, L, P;
  double a_ce, a_l1, a_conf, inv_W;
  uint32_t spin_limit;
  uint32_t unreachable;   // testing: no published word is ever taken as published
};

__device__ __forceinline__ void raw_barrier() {
  // LDS writes complete, then a barrier without the release fence of __syncthreads()
  // (that fence would wait for the LDS prefetch as well)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wave 0: publish this workgroup's partials -- lanes 0..na-1 hold the values of slot_a,
// lanes na..na+nb-1 those of slot_b.  Each lane's word is a device-scope atomic store that
// needs no ordering against any other (see kSlotValid), so nothing waits for it.
// Lane raw_lane (if any) publishes raw_bits as the word's value instead of a float.
__device__ __forceinline__ void publish(unsigned long long* slot_a, int na,
                                        unsigned long long* slot_b, int nb, double v, int lane,
                                        int raw_lane = -1, uint32_t raw_bits = 0u) {
  unsigned long long* w = lane < na ? slot_a + lane : (lane < na + nb ? slot_b + (lane - na) : nullptr);
  const uint32_t bits = lane == raw_lane ? raw_bits : __float_as_uint((float)v);
  if (w)
    __hip_atomic_store(w, kSlotValid | (unsigned long long)bits, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Poll the NA words at pa and the NB words at pb (device-scope atomic loads, which bypass
// the non-coherent caches) until every one is published -- of pa's words only the first
// na_need must be, the others are read as they are; their values into qa, qb.  Returns
// false when the wait gave up: its poll limit ran out (the fault word is raised) or another
// workgroup raised the fault word.
template <int NA, int NB>
__device__ __forceinline__ bool await_words(const LossArgs& a, const unsigned long long* pa,
                                            const unsigned long long* pb, float* qa,
                                            float* qb, int na_need = NA) {
  uint32_t polls = 0;
  for (;;) {
    unsigned long long wa[NA], wb[NB > 0 ? NB : 1];
#pragma unroll
    for (int i = 0; i < NA; ++i)
      wa[i] = __hip_atomic_load(pa + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      wb[i] = __hip_atomic_load(pb + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool all = true;
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      all = all && (i >= na_need || (wa[i] >> 32) != 0ull);
      qa[i] = __uint_as_float((uint32_t)wa[i]);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      all = all && (wb[i] >> 32) != 0ull;
      qb[i] = __uint_as_float((uint32_t)wb[i]);
    }
    if (all && a.unreachable == 0u) return true;
    ++polls;
    if (polls > a.spin_limit ||
        (polls % kFaultCheckPolls == 0 &&
         __hip_atomic_load(a.fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
      __hip_atomic_store(a.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(2);
  }
}

// online (max, sum) merge of one published partial pair into (m, s), in fp64
__device__ __forceinline__ void ml_add(double& m, double& s, float pm, float ps) {
  if (ps > 0.f) {
    const double mm = fmax(m, (double)pm);
    s = s * (double)fast_exp((float)(m - mm)) + (double)ps * (double)fast_exp((float)((double)pm - mm));
    m = mm;
  }
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

// Entry e of a lane's slice: chunk-relative offset 4*lane' + kQuad*(e/4) + e%4, lane' the
// lane index in the workgroup.  Quad e/4 of all the waves is one contiguous piece of the
// chunk, 1 KiB per wave.  The LDS stage mirrors the chunk: draft logits at float 0,
// target logits at float kLossChunk, each entry where its owner lane reads it back.
__device__ __forceinline__ int slice_off(int ct, int e) { return 4 * ct + kQuad * (e >> 2) + (e & 3); }

// Start staging row r's chunk into LDS.  16-byte rows: direct global-to-LDS loads, which the
// compiler's wait counting does not see (nothing waits for them until wait_stage).  A lane
// past the chunk's end loads its last quad (len is a positive multiple of 4) or entry; the
// entries it does not own are masked where they are used.  Other rows: plain loads written
// to the stage.
// A lane's loop-invariant offsets are recomputed from its index at each use (the asm hides
// the index from the optimiser) rather than held in registers across the row loop.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <bool VEC>
__device__ __forceinline__ void stage_row(const LossArgs& a, int r, int c, int ct_,
                                          uint32_t stage_lds, float* stage) {
  const int ct = fresh(ct_);
  const int c0 = c * a.L;
  const int len = min(a.L, a.V - c0);
  const size_t base = (size_t)r * a.V + c0;
  const float* pd = a.zd + base;   // uniform chunk bases: the loads take a scalar base
  const float* pt = a.zt + base;   // and a 32-bit lane offset
  if constexpr (VEC) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // earlier reads of the stage are done
#pragma unroll
    for (int q = 0; q < kLossPer / 4; ++q) {
      const int o = 4 * ct + kQuad * q;
      const uint32_t voff = 4u * (uint32_t)(o < len ? o : len - 4);
      // wave-uniform LDS address (M0), formed in scalar registers
      const uint32_t wv = __builtin_amdgcn_readfirstlane((uint32_t)ct >> 6);
      const uint32_t dst = stage_lds + 4u * ((uint32_t)kQuad * q + 256u * wv);
      dma16(pd, voff, dst);
      dma16(pt, voff, dst + 4u * kLossChunk);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kLossPer; ++e) {
      const int o = slice_off(ct, e);
      const uint32_t oc = (uint32_t)(o < len ? o : len - 1);
      const float vd = pd[oc], vt = pt[oc];
      stage[o] = vd;
      stage[kLossChunk + o] = vt;
    }
  }
}

// this lane's staged entries are in LDS
template <bool VEC>
__device__ __forceinline__ void wait_stage() {
  if constexpr (VEC) wait_vm<0>();
}

// the lane's entries of the staged chunk into registers
__device__ __forceinline__ void read_stage(const float* stage, int ct, float* d, float* t) {
#pragma unroll
  for (int q = 0; q < kLossPer / 4; ++q) {
    const f4v vd = *reinterpret_cast<const f4v*>(stage + 4 * ct + kQuad * q);
    const f4v vt = *reinterpret_cast<const f4v*>(stage + kLossChunk + 4 * ct + kQuad * q);
    d[4 * q] = vd.x; d[4 * q + 1] = vd.y; d[4 * q + 2] = vd.z; d[4 * q + 3] = vd.w;
    t[4 * q] = vt.x; t[4 * q + 1] = vt.y; t[4 * q + 2] = vt.z; t[4 * q + 3] = vt.w;
  }
}

template <bool VEC>
__device__ __forceinline__ void store_grad(const LossArgs& a, int r, int c, int ct_,
                                           const float* g) {
  const int ct = fresh(ct_);
  const int c0 = c * a.L;
  const int len = min(a.L, a.V - c0);
  float* out = a.grad + (size_t)r * a.V + c0;
  if constexpr (VEC) {
#pragma unroll
    for (int q = 0; q < kLossPer / 4; ++q) {
      const int o = 4 * ct + kQuad * q;
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

// Per-lane (max, sum of exp(x - max)) of both logit sets of the staged chunk, reading LDS
// twice rather than holding a second row in registers; none live or all -inf: (-inf, 0).
__device__ __forceinline__ void stage_ml(const float* stage, int ct, uint32_t mask, ML& md,
                                         ML& mt) {
  float xd = -INFINITY, xt = -INFINITY;
#pragma unroll
  for (int q = 0; q < kLossPer / 4; ++q) {
    const f4v vd = *reinterpret_cast<const f4v*>(stage + 4 * ct + kQuad * q);
    const f4v vt = *reinterpret_cast<const f4v*>(stage + kLossChunk + 4 * ct + kQuad * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool on = live(mask, 4 * q + i);
      xd = fmaxf(xd, on ? vd[i] : -INFINITY);
      xt = fmaxf(xt, on ? vt[i] : -INFINITY);
    }
  }
  const float bd = xd == -INFINITY ? 0.f : xd, bt = xt == -INFINITY ? 0.f : xt;
  float sd = 0.f, st = 0.f;
#pragma unroll
  for (int q = 0; q < kLossPer / 4; ++q) {
    const f4v vd = *reinterpret_cast<const f4v*>(stage + 4 * ct + kQuad * q);
    const f4v vt = *reinterpret_cast<const f4v*>(stage + kLossChunk + 4 * ct + kQuad * q);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool on = live(mask, 4 * q + i);
      sd += on ? fast_exp(vd[i] - bd) : 0.f;
      st += on ? fast_exp(vt[i] - bt) : 0.f;
    }
  }
  md = ML{xd, sd};
  mt = ML{xt, st};
}

struct LossShared {
  float w1[kLossWaves][4];   // per wave: (m_d, s_d, m_t, s_t) of the staged row
  float w2[kLossWaves][2];   // per wave: (l1, S) of the current row
  float r1[4];               // staged row: (max_d, log sum_d, max_t, log sum_t)
  float r2[3];               // current row: (S, w alpha_ce, w alpha_l1)
  int y;                     // current row: the label, clamped into the vocabulary
  int stop;
  int rn2;                   // the stream's row after the next one (R: none)
  double lse;                // wave 0's: lse of the current row's draft logits (kept in LDS
                             // rather than across the sweeps in registers)
};

// wave 0: the four waves' (max, sum) pairs of one logit set combined in fp64 (lanes 0..3
// of the caller give (m_d, s_d, m_t, s_t); others 0)
__device__ __forceinline__ double combine_waves1(const LossShared& sh, int lane) {
  double v = 0.0;
  if (lane < 4) {
    const int off = lane & 2;   // 0: draft, 2: target
    double m = -INFINITY;
    for (int w = 0; w < kLossWaves; ++w) m = fmax(m, (double)sh.w1[w][off]);
    if (lane & 1) {
      if (m != -INFINITY)
        for (int w = 0; w < kLossWaves; ++w)
          v += (double)sh.w1[w][off + 1] * (double)fast_exp(sh.w1[w][off] - (float)m);
    } else {
      v = m;
    }
  }
  return v;
}

// Values the kernel only reads, loaded through the scalar unit (uniform addresses): they
// land in scalar registers and their waits never involve the vector-memory counter.
__device__ __forceinline__ int32_t ld_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)(uintptr_t)p;
}
__device__ __forceinline__ float ld_uniform(const float* p) {
  return *(const __attribute__((address_space(4))) float*)(uintptr_t)p;
}

// Row scalars that do not depend on the exchange, fetched before it.
struct RowScalars {
  int y;        // label, clamped into the vocabulary
  float zy;     // draft logit at the label
  float lf;     // confidence logit
};

__device__ __forceinline__ RowScalars row_scalars(const LossArgs& a, int r) {
  RowScalars rs;
  rs.y = clamp_tok(ld_uniform(a.labels + r), a.V);
  rs.zy = ld_uniform(a.zd + (size_t)r * a.V + rs.y);
  rs.lf = ld_uniform(a.conf + r);
  return rs;
}

// wave 0, after the prologue's exchange: row r's normalisers from its C chunk partials
// -> sh.r1 (lane 0 writes); returns lse of the draft logits in fp64
__device__ __forceinline__ double combine_part1(const LossArgs& a, LossShared& sh, int r,
                                                int lane, bool& ok) {
  // per lane: online (max, sum) over its chunks, each polled until published
  double m_d = -INFINITY, s_d = 0.0, m_t = -INFINITY, s_t = 0.0;
  bool mine = true;
  for (int cc = lane; cc < a.C && mine; cc += kWave) {
    float q[4];
    mine = await_words<4, 0>(a, a.part1 + ((size_t)r * a.C + cc) * 4, nullptr, q, nullptr);
    ml_add(m_d, s_d, q[0], q[1]);
    ml_add(m_t, s_t, q[2], q[3]);
  }
  ok = __ballot(!mine) == 0ull;
  const double M_d = wave_max_d(m_d), M_t = wave_max_d(m_t);
  s_d = s_d > 0.0 ? s_d * (double)fast_exp((float)(m_d - M_d)) : 0.0;
  s_t = s_t > 0.0 ? s_t * (double)fast_exp((float)(m_t - M_t)) : 0.0;
  s_d = wave_sum_d(s_d);
  s_t = wave_sum_d(s_t);
  const float ls_d = fast_log((float)s_d), ls_t = fast_log((float)s_t);
  if (lane == 0) {
    sh.r1[0] = (float)M_d; sh.r1[1] = ls_d;
    sh.r1[2] = (float)M_t; sh.r1[3] = ls_t;
  }
  return M_d + (double)ls_d;
}

// wave 0, after a loop exchange: row r's l1 and S and (has_next) row rn's normalisers from
// the C chunk partials, all loaded in one round trip; the row's scalar outputs (chunk 0's
// workgroup) and the gradient coefficients -> sh.r2, sh.y; rn's normalisers -> sh.r1.
// sh.lse: read as row r's lse, then replaced by row rn's.
__device__ __forceinline__ void combine_step(const LossArgs& a, LossShared& sh, int r, int rn,
                                             bool has_next, int c,
                                             const RowScalars& rs, int lane, bool& ok) {
  double l1 = 0.0, S = 0.0, m_d = -INFINITY, s_d = 0.0, m_t = -INFINITY, s_t = 0.0;
  bool mine = true;
  for (int cc = lane; cc < a.C && mine; cc += kWave) {
    const unsigned long long* p2 = a.part2 + ((size_t)r * a.C + cc) * 3;
    const unsigned long long* p1 = a.part1 + ((size_t)rn * a.C + cc) * 4;
    // chunk 0 also carries the claimed row (a third word; the other chunks leave theirs
    // unpublished)
    float q2[3], q1[4];
    const int need = cc == 0 ? 3 : 2;
    mine = has_next ? await_words<3, 4>(a, p2, p1, q2, q1, need)
                    : await_words<3, 0>(a, p2, nullptr, q2, nullptr, need);
    if (has_next) {
      ml_add(m_d, s_d, q1[0], q1[1]);
      ml_add(m_t, s_t, q1[2], q1[3]);
    }
    l1 += (double)q2[0];
    S += (double)q2[1];
    if (cc == 0) sh.rn2 = (int)__float_as_uint(q2[2]);
  }
  ok = __ballot(!mine) == 0ull;
  if (!ok) return;
  l1 = wave_sum_d(l1);
  S = wave_sum_d(S);
  if (lane == 0) {
    const int k = r % a.G;
    const double wk = (double)fast_exp(-(float)k / (float)a.G) * a.inv_W;
    sh.r2[0] = (float)S;
    sh.r2[1] = (float)(wk * a.a_ce);
    sh.r2[2] = (float)(wk * a.a_l1);
    sh.y = rs.y;
    if (c == 0) {
      const double ce = sh.lse - (double)rs.zy;
      const double at = 1.0 - 0.5 * l1;
      // log(1 + e^l) and sigmoid(l) in fp32 through e = exp(-|l|) in (0, 1]
      const float lf = rs.lf;
      const float e = fast_exp(-fabsf(lf));
      const double l = (double)lf;
      const double softplus = (double)fmaxf(lf, 0.f) + (double)log1pf(e);
      const double bce = softplus - at * l;
      const double cs = lf >= 0.f ? 1.0 / (1.0 + (double)e) : (double)e / (1.0 + (double)e);
      // read by the last workgroup to finish, at the device's coherence point
      __hip_atomic_store(a.rowloss + r, wk * (a.a_ce * ce + a.a_l1 * l1 + a.a_conf * bce),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (a.terms) {
        a.terms[3 * (size_t)r] = (float)ce;
        a.terms[3 * (size_t)r + 1] = (float)l1;
        a.terms[3 * (size_t)r + 2] = (float)bce;
      }
      if (a.grad_conf) a.grad_conf[r] = (float)(wk * a.a_conf * (cs - at));
    }
  }
  if (has_next) {
    const double M_d = wave_max_d(m_d), M_t = wave_max_d(m_t);
    s_d = s_d > 0.0 ? s_d * (double)fast_exp((float)(m_d - M_d)) : 0.0;
    s_t = s_t > 0.0 ? s_t * (double)fast_exp((float)(m_t - M_t)) : 0.0;
    s_d = wave_sum_d(s_d);
    s_t = wave_sum_d(s_t);
    const float ls_d = fast_log((float)s_d), ls_t = fast_log((float)s_t);
    if (lane == 0) {
      sh.r1[0] = (float)M_d; sh.r1[1] = ls_d;
      sh.r1[2] = (float)M_t; sh.r1[3] = ls_t;
    }
    if (lane == 0) sh.lse = M_d + (double)ls_d;
  }
}

// A stream of C workgroups (chunk c of rows p, p + P, ...).  Per row r, with the next row
// rn = r + P already staged in LDS:
//   1. every wave: l1 and S partials of r (its registers); (max, sum) partials of rn (the
//      stage);
//   2. wave 0: one exchange carries both -- the stream meets once per row;
//   3. every wave: the gradient of r; rn moves from the stage to the registers and the row
//      after it starts streaming into the stage.
template <bool VEC>
__global__ __launch_bounds__(kLossThreads, kLossWavesPerSimd) void k_draft_loss(LossArgs a) {
  __shared__ LossShared sh;
  __shared__ __align__(16) float stage[2 * kLossChunk];
  const int p = blockIdx.x / a.C, c = blockIdx.x % a.C;
  if (p >= a.P) return;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const bool lead = wave == 0;
  const uint32_t stage_lds = (uint32_t)(uintptr_t)(lds_ptr_t)stage;
  // which of the lane's entries lie inside its chunk (the same for every row)
  const int len = min(a.L, a.V - c * a.L);
  uint32_t mask = 0;
#pragma unroll
  for (int e = 0; e < kLossPer; ++e) mask |= (slice_off(tid, e) < len ? 1u : 0u) << e;
  float d[kLossPer], t[kLossPer];

  // prologue: row p's normalisers
  stage_row<VEC>(a, p, c, tid, stage_lds, stage);
  wait_stage<VEC>();
  {
    ML md, mt;
    stage_ml(stage, tid, mask, md, mt);
    md = wave_ml(md);
    mt = wave_ml(mt);
    if (lane == 0) {
      sh.w1[wave][0] = md.m; sh.w1[wave][1] = md.l;
      sh.w1[wave][2] = mt.m; sh.w1[wave][3] = mt.l;
    }
  }
  read_stage(stage, tid, d, t);
  if (p + a.P < a.R) stage_row<VEC>(a, p + a.P, c, tid, stage_lds, stage);
  raw_barrier();
  if (lead) {
    const double v = combine_waves1(sh, lane);
    publish(a.part1 + ((size_t)p * a.C + c) * 4, 4, nullptr, 0, v, lane);
    bool ok = true;
    const double lse0 = combine_part1(a, sh, p, lane, ok);
    if (lane == 0) sh.lse = lse0;
    if (lane == 0) sh.stop = ok ? 0 : 1;
  }
  raw_barrier();

  // The stream's first two rows are p and p + P; each later one is claimed from the row
  // counter by lane 2 of chunk 0's lead wave an exchange before that exchange publishes it
  // (so the claim's round trip is long over when its value is used): `pending` is the row
  // after the next one.
  auto claim = [&]() -> uint32_t {   // (R < 2^24 rows: no overflow)
    return __hip_atomic_fetch_add(a.row_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  int r = p, rn = p + a.P;
  uint32_t pending = 0u;   // a claim: the row 2P + pending
  if (c == 0 && lead && lane == 2 && rn < a.R) pending = claim();
  while (r < a.R && !sh.stop) {
    const bool has_next = rn < a.R;
    // 1. partials
    const float Md = sh.r1[0], Ld = sh.r1[1], Mt = sh.r1[2], Lt = sh.r1[3];
    {
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
    const RowScalars rs = row_scalars(a, r);   // scalar loads, in flight during the sweeps
    if (has_next) {
      wait_stage<VEC>();
      ML md, mt;
      stage_ml(stage, tid, mask, md, mt);
      md = wave_ml(md);
      mt = wave_ml(mt);
      if (lane == 0) {
        sh.w1[wave][0] = md.m; sh.w1[wave][1] = md.l;
        sh.w1[wave][2] = mt.m; sh.w1[wave][3] = mt.l;
      }
    }
    raw_barrier();
    // 2. the stream's exchange
    if (lead) {
      const int na = c == 0 ? 3 : 2;   // chunk 0: l1, S and the claimed row
      double v = has_next ? combine_waves1(sh, lane - na < 0 ? 63 : lane - na) : 0.0;
      if (lane < 2)
        for (int w = 0; w < kLossWaves; ++w) v += (double)sh.w2[w][lane];
      publish(a.part2 + ((size_t)r * a.C + c) * 3, na,
              a.part1 + ((size_t)(has_next ? rn : r) * a.C + c) * 4, has_next ? 4 : 0, v, lane,
              c == 0 ? 2 : -1,
              has_next ? min(2u * (uint32_t)a.P + pending, (uint32_t)a.R) : (uint32_t)a.R);
      bool ok = true;
      combine_step(a, sh, r, rn, has_next, c, rs, lane, ok);
      if (lane == 0) sh.stop = ok ? 0 : 1;
    }
    raw_barrier();
    if (sh.stop) break;
    // 3. the gradient of row r; the next row into registers, the one after it into LDS
    if (a.grad) {
      const float S = sh.r2[0], fa = sh.r2[1], fb = sh.r2[2];
      const int y = sh.y - c * a.L;   // chunk-relative label
      float g[kLossPer];
#pragma unroll
      for (int e = 0; e < kLossPer; ++e) {
        const float pd = fast_exp((d[e] - Md) - Ld);
        const float pt = fast_exp((t[e] - Mt) - Lt);
        const float df = pd - pt;
        const float sg = df > 0.f ? 1.f : (df < 0.f ? -1.f : 0.f);
        const float oh = slice_off(tid, e) == y ? 1.f : 0.f;
        g[e] = fa * (pd - oh) + fb * pd * (sg - S);
      }
      store_grad<VEC>(a, r, c, tid, g);
    }
    const int rn2 = sh.rn2;
    if (c == 0 && lead && lane == 2 && rn2 < a.R) pending = claim();   // for the next exchange
    if (has_next) {
      read_stage(stage, tid, d, t);
      if (rn2 < a.R) stage_row<VEC>(a, rn2, c, tid, stage_lds, stage);
    }
    r = rn;
    rn = rn2;
  }
  // nothing in flight into LDS when the workgroup ends; this workgroup's row outputs have
  // reached the coherence point before it counts itself in
  wait_vm<0>();
  raw_barrier();
  if (tid == 0)
    sh.stop = __hip_atomic_fetch_add(a.done_ctr, 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(a.P * a.C) - 1u;
  raw_barrier();
  if (!sh.stop) return;
  // the last one: the loss as a fixed-order sum (256 strided partial sums, then a tree),
  // NaN after a fault
  __shared__ double psum[256];
  if (tid < 256) {
    double v = 0.0;
    for (int i = tid; i < a.R; i += 256)
      v += __hip_atomic_load(a.rowloss + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    psum[tid] = v;
  }
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) psum[tid] += psum[tid + o];
    __syncthreads();
  }
  if (tid == 0)
    a.loss[0] = __hip_atomic_load(a.fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u
                    ? (double)NAN
                    : psum[0];
}

// clears the published words (part1, part2 and the two counters, n words from `words`) and
// the fault word
__global__ __launch_bounds__(256) void k_loss_init(unsigned long long* __restrict__ words,
                                                   size_t n, uint32_t* __restrict__ fault) {
  const size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  for (size_t j = i; j < n; j += (size_t)gridDim.x * blockDim.x) words[j] = 0ull;
  if (i == 0) *fault = 0u;
}

}  // namespace dspark

using namespace dspark;

namespace {

struct LossWs {
  unsigned long long* part1;   // published words: part1, part2 and the two counters, one block
  unsigned long long* part2;
  unsigned int* row_ctr;
  unsigned int* done_ctr;
  size_t nwords;
  double* rowloss;
  uint32_t* fault;
  size_t bytes;
};

int loss_chunks(int V) { return (V + kLossChunk - 1) / kLossChunk; }

LossWs loss_ws(int R, int V, void* base) {
  const int C = loss_chunks(V);
  Carve c(base);
  LossWs w;
  w.nwords = (size_t)R * C * 7 + 2;
  w.part1 = c.take<unsigned long long>(w.nwords);
  w.part2 = w.part1 ? w.part1 + (size_t)R * C * 4 : nullptr;
  w.row_ctr = w.part1 ? reinterpret_cast<unsigned int*>(w.part1 + (size_t)R * C * 7) : nullptr;
  w.done_ctr = w.part1 ? reinterpret_cast<unsigned int*>(w.part1 + (size_t)R * C * 7 + 1) : nullptr;
  w.rowloss = c.take<double>((size_t)R);
  w.fault = c.take<uint32_t>(1);
  w.bytes = align_up(c.off, 256);
  return w;
}

bool loss_shape_ok(int B, int G, int V) {
  return B >= 1 && G >= 1 && G <= 64 && (long long)B * G <= (1 << 24) && V >= 1 &&
         V <= kLossMaxVocab;
}

// Resident workgroups of the loss kernel on the current device (0 when cooperative launch
// is unavailable), looked up once per device.
constexpr int kMaxDevices = 64;

// Each entry is the capacity + 1 once known (0 = not looked up yet); a racing second lookup
// computes and stores the same value.
template <bool VEC>
int loss_capacity() {
  static std::atomic<int> cap1[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 0;
  const int known = cap1[dev].load(std::memory_order_acquire);
  if (known > 0) return known - 1;
  int coop = 0, ncu = 0, per_cu = 0, cap = 0;
  if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)k_draft_loss<VEC>,
                                                   kLossThreads, 0) == hipSuccess && coop)
    cap = per_cu * ncu;
  cap1[dev].store(cap + 1, std::memory_order_release);
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
  a.rowloss = w.rowloss; a.part1 = w.part1; a.part2 = w.part2; a.fault = w.fault;
  a.row_ctr = w.row_ctr;
  a.done_ctr = w.done_ctr;
  a.loss = loss;
  a.R = R; a.G = G; a.V = V;
  a.C = loss_chunks(V);
  a.L = (V + 4 * a.C - 1) / (4 * a.C) * 4;
  if (cap < a.C) return DSPARK_E_HIP;   // no cooperative launch, or a row does not fit
  a.P = std::min(R, cap / a.C);
  double wsum = 0.0;
  for (int k = 0; k < G; ++k) wsum += std::exp(-(double)k / G);
  a.inv_W = 1.0 / ((double)B * wsum);
  a.a_ce = alpha_ce; a.a_l1 = alpha_l1; a.a_conf = alpha_conf;
  const WaitPolicy wp = wait_policy();
  a.spin_limit = wp.limit;
  a.unreachable = wp.unreachable;
  hipStream_t st = (hipStream_t)stream;
  hipLaunchKernelGGL(k_loss_init,
                     dim3((unsigned)std::min<size_t>(2048, (w.nwords + 255) / 256)), dim3(256),
                     0, st, w.part1, w.nwords, w.fault);
  if (launch_status() != DSPARK_OK) return DSPARK_E_HIP;
  void* args[] = {&a};
  const void* fn = vec ? (const void*)k_draft_loss<true> : (const void*)k_draft_loss<false>;
  if (hipLaunchCooperativeKernel(fn, dim3((unsigned)(a.P * a.C)), dim3(kLossThreads), args, 0,
                                 st) != hipSuccess) {
    (void)hipGetLastError();
    return DSPARK_E_HIP;
  }
  return DSPARK_OK;
}
