// mfma16.hip -- the draft-position kernel on 16-column waves (v_mfma_f32_16x16x32_bf16).
//
// It computes exactly what the draft mode of mfma_bias.hip computes (bias = W1[prev] W2,
// z = (U + bias)/T, online base-2 (max, sum) and the Gumbel-max race; [XTL §4], [CSDN
// Eq. 4]), with a layout chosen for occupancy: the per-element epilogue (a Philox call per
// four rows, two logarithms, an exponential) dominates the instruction count, so what
// limits the kernel is how well the SIMDs hide its latencies, i.e. how many waves each SIMD
// holds.  A wave owns 16 columns here, so its gathered W1 operand takes 32 VGPRs per lane
// (64 for 32-column waves) and four waves fit on every SIMD.
//
// Per step the workgroup consumes one 32-row W2t tile from the same LDS ring as the other
// kernel (DMA, chunk-interleaved row pairs, SA stages).  Each wave runs two 16 x 16 output
// blocks (rows 0-15 and 16-31 of the tile) over it, eight k-steps of 32 each.  Output
// lane l of a block holds column l%16 and the four consecutive rows 4(l/16) + i, i < 4:
// one aligned 16-byte logit load and one Philox4x32 call per block.  The base logits are
// loaded in that layout and seed the accumulator, so the MFMA result is U + bias itself.
//
// Workgroup shapes: 8 waves (128 columns, two workgroups per CU) for 65..128 columns,
// 16 waves (256 columns, one per CU) beyond, and 4 waves (64 columns, two per CU, so two
// waves per SIMD) up to 64 columns: there a half-idle 8-wave workgroup would spend its
// idle waves' MFMA and epilogue work on dummy columns, which measured 10-20% slower.  The
// TV mode takes the 4- and 8-wave shapes (up to 128 columns per launch).
#include "mfma_bias.h"
#include "mfma_common.h"

namespace dspark {

constexpr int kKS32 = kR / 32;   // k-steps of 32

template <int NW, bool TV = false>
struct Shape16 {
  static constexpr int NT = 64 * NW;
  static constexpr int NC = 16 * NW;          // columns
  static constexpr int SA = 4;                // W2t ring stages
  static constexpr int UD = 3;                // logit register buffers
  static constexpr int WG_PER_CU = NW == 4 ? 2 : 16 / NW;   // LDS: at most two rings
  static constexpr int NA = 16 / NW;          // DMA instructions per wave per step
  static constexpr int NU = TV ? 4 : 2;       // logit (and target) loads per wave per step
  // The stage of step s is waited for at step s.  A stage issued inside the loop (at step
  // s-SA+1) is followed by at least the loads of the SA-2 steps after that one (each step
  // issues NA + NU), so once at most that many are outstanding it has landed.
  static constexpr int kWaitSS = (SA - 2) * (NA + NU);
  static constexpr bool kW1Staged = (size_t)(NC / 2) * kPairBytes <= (size_t)SA * kTileBytes;
  // Before the loop the stages of steps 0..SA-2 and the logit slices of steps 0..UD-2 are
  // issued in the order they are needed (stage p, then slice p); loads issued after the
  // stage of such an early step p, up to its wait: the rest of that sequence and the loads
  // of steps 0..p-1.
  static constexpr int PRE = SA - 1 > UD - 1 ? SA - 1 : UD - 1;
  static constexpr int early_after(int p) {
    int n = p < UD - 1 ? NU : 0;
    for (int q = p + 1; q < PRE; ++q) n += (q < SA - 1 ? NA : 0) + (q < UD - 1 ? NU : 0);
    return n + p * (NA + NU);
  }
  static constexpr int kPeelTrips = (SA - 1 + UD - 1) / UD;
  static constexpr int wait_early(int p) {
    return early_after(p) < kWaitSS ? early_after(p) : kWaitSS;
  }
  static constexpr size_t kOffMeta = (size_t)SA * kTileBytes;
  // column metadata: logit row offset, column, conditioning token; TV adds the target row
  // offset and the two base-2 normalisers
  static constexpr size_t kLds = kOffMeta + (size_t)NC * (8 + 4 + 4) + (TV ? (size_t)NC * 16 : 0);
  static_assert(NW == 4 || NW == 8 || NW == 16, "whole DMA instructions per wave");
  static_assert(kLds * WG_PER_CU <= 160 * 1024, "LDS budget");
  static_assert(kWaitSS < 64, "vmcnt range");
};

// TV = true: the same stream computes the TV accept rate [CSDN Eq. 8] of up to 128 (request,
// position) columns instead of a draft position: p_d = 2^(z log2 e - lse_d), p_t from the
// target slices loaded beside the logit slices, and the per-lane sum of min(p_d, p_t).
template <int NW, bool TV = false>
__global__ __launch_bounds__(64 * NW, (NW == 4 ? 2 : 4)) void k_draft16(const MfmaBiasArgs a) {
  using S = Shape16<NW, TV>;
  constexpr int NC = S::NC, SA = S::SA, UD = S::UD;
  extern __shared__ __align__(16) unsigned char smem[];
  long long* col_urow = reinterpret_cast<long long*>(smem + S::kOffMeta);   // [NC]
  int* col_b = reinterpret_cast<int*>(col_urow + NC);
  int* col_prev = col_b + NC;
  long long* col_trow = reinterpret_cast<long long*>(col_prev + NC);   // TV: [NC]
  float* col_ld = reinterpret_cast<float*>(col_trow + NC);             // TV: [NC] base 2
  float* col_lt = col_ld + NC;                                        // TV: [NC] base 2
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q = lane >> 4, n16 = lane & 15;
  const int G = a.G, V = a.V;
  const float s2 = a.invT * kLog2e;   // logit -> base-2 scale

  // ---- this workgroup's contiguous range of 32-row vocab tiles, one per step
  const int ntiles = (V + 31) >> 5;
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int per = ntiles / nwg, rem = ntiles % nwg;
  const int t0 = wg * per + min(wg, rem);
  const int t1 = t0 + per + (wg < rem ? 1 : 0);
  const int nsteps = t1 - t0;

  // ---- W2t ring: DMA of step `step` into stage step % SA.  Lane l of instruction j moves
  // chunk l>>1 (16 bytes) of stage row 2j + (l&1); rows past V repeat row V-1.  A step past
  // the last one issues the same instructions on one cached line (its stage is never read),
  // which keeps the per-step load count constant.
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
  auto issue_dma = [&](int step) {
    const int row0 = (t0 + step) * 32;
    const uint32_t stage = ring_lds + (uint32_t)((step % SA) * kTileBytes);
    const bool dummy = step >= nsteps;
    const uint16_t* gbase = dummy ? a.W2t : a.W2t + (size_t)row0 * kR;
#pragma unroll
    for (int i = 0; i < S::NA; ++i) {
      const int j = wave + NW * i;
      const int row = dummy ? 0 : min(row0 + 2 * j + (lane & 1), V - 1) - row0;
      const uint32_t voff = dummy ? 0u : (uint32_t)(row * kR * 2 + (lane >> 1) * 16);
      dma16(gbase, voff, stage + (uint32_t)(j * kPairBytes));
    }
  };
  // ---- column metadata: request, conditioning token, base-logit row offset
  for (int c = tid; c < NC; c += S::NT) {
    int b = -1, prev = 0;
    if constexpr (TV) {
      // column = (request, position): b = gc / G, k = gc % G + 1
      long long urow = -1, trow = -1;
      float ld = 0.f, lt = 0.f;
      if (c < a.ncols) {
        const int gc = a.col0 + c, rb = gc / G, k = gc % G + 1;
        b = gc;
        prev = (k == 1) ? a.anchor[rb] : a.tokens[(size_t)rb * G + (k - 2)];
        urow = ((long long)rb * G + (k - 1)) * V;
        trow = ((long long)rb * (G + 1) + (k - 1)) * V;
        ld = a.lse_d[(size_t)rb * G + (k - 1)] * kLog2e;
        lt = a.lse_t[(size_t)rb * G + (k - 1)] * kLog2e;
      }
      col_b[c] = b;
      col_prev[c] = clamp_tok(prev, V);
      col_urow[c] = urow;
      col_trow[c] = trow;
      col_ld[c] = ld;
      col_lt[c] = lt;
    } else {
      if (c < a.ncols) {
        b = a.col0 + c;
        prev = (a.k == 1) ? a.anchor[b]
                          : (a.forced ? a.forced[(size_t)b * G + (a.k - 2)]
                                      : (int)packed_index(a.best_prev[b]));
      }
      col_b[c] = b;
      col_prev[c] = clamp_tok(prev, V);
      col_urow[c] = b >= 0 ? ((long long)b * G + (a.k - 1)) * V : -1;
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // ---- this lane's column; its gathered W1 row is the MFMA B operand: lane l holds
  // elements 32 kk + 8 (l/16) .. +7 of column l%16's row (idle columns gather row 0 and are
  // never reported)
  const int col = wave * 16 + n16;
  const int cb = col_b[col];
  const long long curow = col_urow[col];
  const long long ctrow = TV ? col_trow[col] : -1;   // TV: target row, base-2 normalisers
  const float cld = TV ? col_ld[col] : 0.f, clt = TV ? col_lt[col] : 0.f;
  u32x4_t Bop[kKS32];
  if constexpr (S::kW1Staged) {
    // whole 512-byte rows by DMA, two rows per instruction in the pair layout, then the
    // fragments from LDS: row `col`, chunk 4 kk + q
#pragma unroll
    for (int i = 0; i < NC / 2 / NW; ++i) {
      const int j = wave + NW * i;
      const uint16_t* src = a.W1 + (size_t)col_prev[2 * j + (lane & 1)] * kR + (lane >> 1) * 8;
      dma16v(src, ring_lds + (uint32_t)(j * kPairBytes));
    }
    wait_vm<0>();
    barrier_no_fence();
    const unsigned char* Bl = smem + (col >> 1) * kPairBytes + (2 * q + (col & 1)) * 16;
#pragma unroll
    for (int kk = 0; kk < kKS32; ++kk)
      Bop[kk] = *reinterpret_cast<const u32x4_t*>(Bl + kk * 128);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // ring free again
  } else {
    const uint16_t* wrow = a.W1 + (size_t)col_prev[col] * kR + 8 * q;
#pragma unroll
    for (int kk = 0; kk < kKS32; ++kk)
      Bop[kk] = *reinterpret_cast<const u32x4_t*>(wrow + kk * 32);
  }

  // ---- base logits of one step in the output layout: block rb, rows 16 rb + 4q + i
  f32x4_t Ub[UD][2];
  f32x4_t Tb[TV ? UD : 1][2];                  // TV: the target slices, same layout
  auto load_logits = [&](int step, f32x4_t (&u)[2], f32x4_t (&tt)[2]) {
    const int t = t0 + step;
    const bool live = cb >= 0 && t < t1;       // else one valid dummy address per load
    const int vb = t * 32 + 4 * q;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int v = min(vb + 16 * rb, V - 4);
      const float* pu = live ? a.U + curow + v : a.U;
      u[rb] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pu));
      if constexpr (TV) {
        const float* pt = live ? a.T + ctrow + v : a.T;
        tt[rb] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pt));
      }
    }
    if (__builtin_expect((t + 1) * 32 > V, 0)) {
      // the vocabulary's last tile: a whole run lies past V (V % 4 == 0); its logits
      // become -inf, which removes it from the max, the sum and the race
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
        if (vb + 16 * rb >= V) u[rb] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    }
  };

  const PhiloxLane pl = philox_lane((uint32_t)a.k, (uint32_t)(cb < 0 ? 0 : cb), 0u, a.key0,
                                    a.key1);

  // the first stages and logit slices, in the order they are needed
#pragma unroll
  for (int p = 0; p < S::PRE; ++p) {
    if (p < SA - 1) issue_dma(p);
    if (p < UD - 1) load_logits(p, Ub[p], Tb[TV ? p : 0]);
  }

  // per-lane running state of the lane's column
  float st_m = kNegBig, st_l = 0.f, st_s = -INFINITY;
  uint32_t st_v = 0xFFFFFFFFu;
  float st_tv = 0.f;                           // TV: running sum of min(p_d, p_t)

  // lane's A-fragment base within a stage: row n16 of block rb, chunk 4 kk + q
  const int a_lane = (n16 >> 1) * kPairBytes + (2 * q + (n16 & 1)) * 16;

  auto step_body = [&](int step, auto bufc, auto basec) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int BASE = decltype(basec)::value;   // >= 0: step == BASE + BUF
    constexpr int NXT = (BUF + UD - 1) % UD;
    // stage `step` complete for this wave, then for all; stage step-1 free for reuse
    if constexpr (BASE >= 0 && BASE + BUF < SA - 1) {
      wait_vm<S::wait_early(BASE + BUF)>();
    } else {
      wait_vm<S::kWaitSS>();
    }
    barrier_no_fence();
    issue_dma(step + SA - 1);
    load_logits(step + UD - 1, Ub[NXT], Tb[TV ? NXT : 0]);

    const int t = t0 + step;
    if (t >= t1) return;                       // wave-uniform (also every step >= nsteps);
                                               // idle lanes (cb < 0) compute on dummies and
                                               // are never reported
    const unsigned char* At = smem + (size_t)(step % SA) * kTileBytes + a_lane;
    // two accumulation chains (row blocks 0 and 1), seeded with the base logits
    f32x4_t acc[2] = {Ub[BUF][0], Ub[BUF][1]};
    constexpr int kAhead = 4;                  // A fragments read ahead of their MFMA
    u32x4_t av[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i)
      av[i] = *reinterpret_cast<const u32x4_t*>(At + (i & 1) * 8 * kPairBytes + (i >> 1) * 128);
#pragma unroll
    for (int i = 0; i < 2 * kKS32; ++i) {      // i = 2 kk + rb
      const int rb = i & 1, kk = i >> 1;
      acc[rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av[i % kAhead]),
                                                        as_bf16x8(Bop[kk]), acc[rb], 0, 0, 0);
      const int nx = i + kAhead;
      if (nx < 2 * kKS32)
        av[i % kAhead] = *reinterpret_cast<const u32x4_t*>(At + (nx & 1) * 8 * kPairBytes +
                                                           (nx >> 1) * 128);
    }
    // element e = 4 rb + i of the lane is vocab row t*32 + 16 rb + 4q + i (rows past V
    // carry -inf logits); e increases with the row
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = acc[e >> 2][e & 3];
    if constexpr (TV) {
      // p_d = 2^(z s2 - lse_d), p_t = 2^(t s2 - lse_t) (rows past V: p_d = 0)
      float mn[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        mn[e] = fminf(ex2(fmaf(y[e], s2, -cld)), ex2(fmaf(Tb[BUF][0][e], s2, -clt))) +
                fminf(ex2(fmaf(y[e + 4], s2, -cld)), ex2(fmaf(Tb[BUF][1][e], s2, -clt)));
      st_tv += (mn[0] + mn[1]) + (mn[2] + mn[3]);
      return;
    }
    float mx = fmaxf(y[0], y[1]);
#pragma unroll
    for (int e = 2; e < 8; ++e) mx = fmaxf(mx, y[e]);
    const float mnew = fmaxf(st_m, mx * s2);
    float lp[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      lp[e] = ex2(fmaf(y[e], s2, -mnew)) + ex2(fmaf(y[e + 4], s2, -mnew));
    st_l = st_l * ex2(st_m - mnew) + ((lp[0] + lp[1]) + (lp[2] + lp[3]));
    st_m = mnew;
    uint32_t c0[2], wd[2][4];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) c0[rb] = (uint32_t)(t * 8 + 4 * rb + q);
    philox_calls<2>(c0, pl, wd);
    float sc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) sc[e] = fmaf(y[e], s2, neg_lglg(wd[e >> 2][e & 3]));
    // tree arg-max: the later (higher-row) side of a pair wins only when strictly greater,
    // so ties keep the lowest row, as does the running best
    float bs[4];
    int bi[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bool hi2 = sc[2 * e + 1] > sc[2 * e];
      bs[e] = hi2 ? sc[2 * e + 1] : sc[2 * e];
      bi[e] = hi2 ? 2 * e + 1 : 2 * e;
    }
#pragma unroll
    for (int n = 2; n >= 1; n >>= 1)
#pragma unroll
      for (int e = 0; e < n; ++e) {
        const bool hi2 = bs[2 * e + 1] > bs[2 * e];
        bs[e] = hi2 ? bs[2 * e + 1] : bs[2 * e];
        bi[e] = hi2 ? bi[2 * e + 1] : bi[2 * e];
      }
    const bool lead = bs[0] > st_s;
    st_s = lead ? bs[0] : st_s;
    st_v = lead ? (uint32_t)(t * 32 + 16 * (bi[0] >> 2) + 4 * q + (bi[0] & 3)) : st_v;
  };

  // UD unconditional bodies per trip (steps past the last compute nothing but still issue
  // their dummy loads), so that every body sees the same load history; the first trips are
  // peeled, so the compiler's bookkeeping enters the loop in its steady state (every early
  // step, whose stage was issued before the loop, falls in a peeled trip)
  peel_trips<0, S::kPeelTrips, UD>(step_body);
  for (int step = S::kPeelTrips * UD; step < nsteps; step += UD)
    unroll_steps<0, UD, -1>(step, step_body);
  __builtin_amdgcn_s_waitcnt(0);   // dummy DMAs of the last steps have landed

  if constexpr (TV) {
    float sum = st_tv;
    sum += __shfl_xor(sum, 16, kWave);
    sum += __shfl_xor(sum, 32, kWave);
    if (q == 0 && cb >= 0) a.tv_part[(size_t)wg * ((size_t)a.B * a.G) + cb] = sum;
    return;
  }
  // ---- merge the four row quads of each column (lanes n16 + 16 q), in a fixed order
  float m = st_m, l = st_l, sc = st_s;
  uint32_t v = st_v;
#pragma unroll
  for (int o = 16; o <= 32; o <<= 1) {
    const float om = __shfl_xor(m, o, kWave);
    const float ol = __shfl_xor(l, o, kWave);
    const float os = __shfl_xor(sc, o, kWave);
    const uint32_t ov = (uint32_t)__shfl_xor((int)v, o, kWave);
    const float mm = fmaxf(m, om);
    l = l * ex2(m - mm) + ol * ex2(om - mm);
    m = mm;
    if (os > sc || (os == sc && ov < v)) { sc = os; v = ov; }
  }
  if (q == 0 && cb >= 0) {
    a.part[(size_t)wg * a.B + cb] = make_float2(m, l);
    if (v != 0xFFFFFFFFu) atomic_max_u64(&a.best_cur[cb], pack_score(sc, v));
  }
}

template <int NW, bool TV = false>
static dspark_status attr16() {
  static LdsAttr attr;
  return attr.ensure((const void*)k_draft16<NW, TV>, (int)Shape16<NW, TV>::kLds);
}

template <int NW, bool TV = false>
static dspark_status launch16(const MfmaBiasArgs& a, int nwg, hipStream_t st) {
  using S = Shape16<NW, TV>;
  if (attr16<NW, TV>() != DSPARK_OK) return DSPARK_E_HIP;
  hipLaunchKernelGGL((k_draft16<NW, TV>), dim3(nwg), dim3(S::NT), S::kLds, st, a);
  return launch_status();
}

dspark_status draft16_prepare() {
  if (attr16<4>() != DSPARK_OK || attr16<8>() != DSPARK_OK || attr16<16>() != DSPARK_OK ||
      attr16<4, true>() != DSPARK_OK || attr16<8, true>() != DSPARK_OK)
    return DSPARK_E_HIP;
  return DSPARK_OK;
}

bool draft16_supported(const MfmaBiasArgs& a) {
  if (a.mode == kModeTV) return a.ncols > 32 && a.ncols <= 128 && (a.V & 3) == 0;
  return a.mode == kModeDraft && a.ncols > 32 && a.ncols <= 256 && (a.V & 3) == 0;
}

dspark_status launch_draft16(const MfmaBiasArgs& a, int nwg, hipStream_t st) {
  if (a.mode == kModeTV)
    return a.ncols <= 64 ? launch16<4, true>(a, nwg, st) : launch16<8, true>(a, nwg, st);
  if (a.ncols <= 64) return launch16<4>(a, nwg, st);
  return a.ncols <= 128 ? launch16<8>(a, nwg, st) : launch16<16>(a, nwg, st);
}

}  // namespace dspark
