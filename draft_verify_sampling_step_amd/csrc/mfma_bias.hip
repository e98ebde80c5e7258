// mfma_bias.hip -- batched Markov bias on bf16 MFMA with fused epilogues (see mfma_bias.h).
//
// Memory pipeline of one workgroup (NW waves; each wave owns one 32-column block of one
// 32-row vocab tile per step):
//   * W2t tiles go HBM -> LDS by DMA (global_load_lds_dwordx4), into a ring of SA stages,
//     SA-1 steps ahead.  A DMA instruction moves two W2t rows (1 KB); in LDS the two rows
//     are interleaved by 16-byte chunk and each pair is padded to 1056 bytes, so that the
//     MFMA A-fragment read of a lane is base + 64*kk (no per-step address arithmetic) and
//     16 consecutive lanes hit 16 distinct bank groups.
//   * the base (and target) logit slices are loaded straight into registers in the MFMA
//     output layout, UD-1 steps ahead; every wave issues the same number of loads each
//     step (idle lanes read a valid dummy address), so the outstanding-load count that
//     proves a ring stage has landed is a compile-time constant.
//   * one barrier per step: after it, stage s is complete for every wave and every wave
//     is done with stage s-1, which the same step refills.
#include "mfma_bias.h"
#include "mfma_common.h"

namespace dspark {

template <int NCB, int MODE>
struct Shape {
  static constexpr int NCW = NCB;                        // column blocks = waves per tile
  static constexpr int TSPLIT = NCB >= 4 ? 1 : 4 / NCB;  // tiles per step
  static constexpr int NW = NCW * TSPLIT;                // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int NC = NCB * 32;                    // columns
  static constexpr bool HAS_T = MODE != kModeDraft;
  static constexpr int SA = NCB == 4 ? 4 : (NCB == 8 ? 6 : 2);   // W2t ring stages
  static constexpr int UD = HAS_T ? 2 : 3;                       // logit register buffers
  static constexpr int WG_PER_CU = (NCB == 4 || NCB == 2) ? 2 : 1;
  static constexpr int kStage = TSPLIT * kTileBytes;
  static constexpr int NA = TSPLIT * 16 / NW;            // DMA instructions per wave per step
  static constexpr int NU = HAS_T ? 8 : 4;               // logit loads per wave per step
  // The stage of step s is waited for at step s.  A stage issued inside the loop (at step
  // s-SA+1) is followed by the loads of the SA-2 steps after that one (every step issues
  // NA + NU), so once at most that many are outstanding it has landed.
  static constexpr int kWaitSS = (SA - 2) * (NA + NU);
  // The gathered W1 rows of the columns are staged in the ring (same pair layout) before
  // the ring is used, when they fit.
  static constexpr bool kW1Staged = (size_t)(NC / 2) * kPairBytes <= (size_t)SA * kStage;
  // Before the loop the stages of steps 0..SA-2 and the logit slices of steps 0..UD-2 are
  // issued in the order they are needed: stage p, then slice p, for p = 0, 1, ...  The
  // loads after the stage of such an early step p, up to its wait: the rest of that
  // sequence and the loads of steps 0..p-1.
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
  static constexpr size_t kOffMeta = (size_t)SA * kStage;
  static constexpr size_t kMetaBytes = (size_t)NC * (8 + 8 + 4 + 4 + 4 + 4 + 4);
  static constexpr size_t kRed = (size_t)TSPLIT * NC * 4 * 4;
  static constexpr size_t kLds = kOffMeta + kMetaBytes;
  static_assert(TSPLIT * 16 % NW == 0, "DMA split");
  static_assert(kRed + 16 <= kOffMeta, "reduction scratch (and a flag) reuses the ring");
  static_assert(kLds * WG_PER_CU <= 160 * 1024, "LDS budget");
  static_assert(kWaitSS < 64, "vmcnt range");
};

// ---- residual mode helpers --------------------------------------------------------
// Thin path: with at most kThinMax requests to resample (the usual case) the matrix-core
// machinery would still stream W2t through 32-column blocks; instead every wave takes four
// vocabulary rows per step, 16 lanes per row: lane part p holds elements 16 p .. 16 p + 15
// of W2t[v] and of every listed request's W1[x_{j-1}], the dot products are summed over
// the 16 lanes by DPP moves, and lane p < n runs request p's residual and fallback races
// on row v.
constexpr int kThinMax = kResidThinMax;

// Sum over each 16-lane row of the wave by DPP moves (quad swaps 1,0,3,2 and 2,3,0,1, then
// the half-row and row mirrors): each step adds a commutative pair, so all 16 lanes end
// with the same total.
__device__ __forceinline__ float dpp_row_sum16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  return x;
}

// The thin path over this workgroup's slice of the vocabulary for the n <= kThinMax listed
// columns clist[0..n) of the launch; scratch holds 4 * NW * kThinMax float4.  Each request's
// best (score, index) of both races goes to its packed winner words.
template <int NW>
__device__ __forceinline__ void resid_thin(const MfmaBiasArgs& a, const int* clist, int n,
                                           float4* scratch) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int part = lane & 15, quad = lane >> 4;
  const int G = a.G, V = a.V;
  float w1[kThinMax][16];
  const float* urow = a.U;
  const float* trow = a.T;
  float ld = 0.f, lt = 0.f;
  int myb = 0, myj = 1;
#pragma unroll
  for (int i = 0; i < kThinMax; ++i) {
    int b = 0, j = 1;
    if (i < n) { b = a.col0 + clist[i]; j = a.jrow[b]; }
    const int prev = clamp_tok((j == 1) ? a.anchor[b] : a.tokens[(size_t)b * G + (j - 2)], V);
    const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(a.W1 + (size_t)prev * kR + 16 * part);
    const u32x4_t q0 = wp[0], q1 = wp[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w1[i][2 * e] = __uint_as_float(q0[e] << 16);
      w1[i][2 * e + 1] = __uint_as_float(q0[e] & 0xFFFF0000u);
      w1[i][8 + 2 * e] = __uint_as_float(q1[e] << 16);
      w1[i][8 + 2 * e + 1] = __uint_as_float(q1[e] & 0xFFFF0000u);
    }
    if (i == part && i < n) {
      myb = b;
      myj = j;
      urow = a.U + ((size_t)b * G + (j - 1)) * V;
      trow = a.T + ((size_t)b * (G + 1) + (j - 1)) * V;
      ld = a.lse_d[(size_t)b * G + (j - 1)] * kLog2e;
      lt = a.lse_t_row[b] * kLog2e;
    }
  }
  const float s2 = a.invT * kLog2e;
  const PhiloxLane pl = philox_lane((uint32_t)myj, (uint32_t)myb, 2u, a.key0, a.key1);
  const int len = (V + (int)gridDim.x - 1) / (int)gridDim.x;
  const int vb = blockIdx.x * len, ve = min(V, vb + len);
  Cand c1{-INFINITY, 0xFFFFFFFFu, 0.f}, c2{-INFINITY, 0xFFFFFFFFu, 0.f};
  // four row groups per iteration (rows v0 + 4 NW u + quad), every load issued first; rows
  // past the slice load row v0 and are not raced
  for (int v0 = vb + 4 * wave; v0 < ve; v0 += 16 * NW) {
    u32x4_t xq[4][2];
    float uq[4], tq[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int vu = v0 + 4 * NW * u + quad;
      const int vv = vu < ve ? vu : v0;
      const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(a.W2t + (size_t)vv * kR + 16 * part);
      xq[u][0] = xp[0];
      xq[u][1] = xp[1];
      uq[u] = urow[vv];
      tq[u] = trow[vv];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int v = v0 + 4 * NW * u + quad;
      float xf[16];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xf[2 * e] = __uint_as_float(xq[u][0][e] << 16);
        xf[2 * e + 1] = __uint_as_float(xq[u][0][e] & 0xFFFF0000u);
        xf[8 + 2 * e] = __uint_as_float(xq[u][1][e] << 16);
        xf[8 + 2 * e + 1] = __uint_as_float(xq[u][1][e] & 0xFFFF0000u);
      }
      float d[kThinMax];
#pragma unroll
      for (int i = 0; i < kThinMax; ++i) {
        d[i] = 0.f;
        if (i < n) {   // uniform
          float acc = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) acc = fmaf(xf[e], w1[i][e], acc);
          d[i] = dpp_row_sum16(acc);
        }
      }
      if (v < ve && part < n) {
        float bias = d[0];
#pragma unroll
        for (int i = 1; i < kThinMax; ++i) bias = part == i ? d[i] : bias;
        // base 2, as in the matrix-core epilogue: the same races, the same scores
        const float zd2 = (uq[u] + bias) * s2;
        const float zt2 = tq[u] * s2;
        const float rho = ex2(zt2 - lt) - ex2(zd2 - ld);
        const U4 w = philox_call((uint32_t)v >> 2, pl);
        const uint32_t word =
            (v & 3) == 0 ? w.x : (v & 3) == 1 ? w.y : (v & 3) == 2 ? w.z : w.w;
        const float gn = neg_lglg(word);
        if (rho > 0.f) {
          const float sc = lg2(rho) + gn;
          if (sc > c1.s) c1 = Cand{sc, (uint32_t)v, 0.f};
        }
        const float sc2 = zt2 + gn;
        if (sc2 > c2.s) c2 = Cand{sc2, (uint32_t)v, 0.f};
      }
    }
  }
  // merge the candidates of request p over the 4 NW (wave, row quad) lanes, ties to the
  // lower index
  float4 (*s_cand)[kThinMax] = reinterpret_cast<float4 (*)[kThinMax]>(scratch);
  if (part < n)
    s_cand[wave * 4 + quad][part] =
        make_float4(c1.s, __uint_as_float(c1.i), c2.s, __uint_as_float(c2.i));
  __syncthreads();
  if (tid < n) {
    float s1 = -INFINITY, ss2 = -INFINITY;
    uint32_t i1 = 0xFFFFFFFFu, i2 = 0xFFFFFFFFu;
    for (int g = 0; g < 4 * NW; ++g) {
      const float4 p = s_cand[g][tid];
      const uint32_t pi1 = __float_as_uint(p.y), pi2 = __float_as_uint(p.w);
      if (p.x > s1 || (p.x == s1 && pi1 < i1)) { s1 = p.x; i1 = pi1; }
      if (p.z > ss2 || (p.z == ss2 && pi2 < i2)) { ss2 = p.z; i2 = pi2; }
    }
    const int b = a.col0 + clist[tid];
    unsigned long long* slot = a.res_best + ((size_t)(blockIdx.x % kSubSlots) * a.B + b) * 2;
    if (i1 != 0xFFFFFFFFu) atomic_max_u64(&slot[0], pack_score(s1, i1));
    if (i2 != 0xFFFFFFFFu) atomic_max_u64(&slot[1], pack_score(ss2, i2));
  }
}

// After every thread of the workgroup has posted its winners: count the workgroup in; the
// last of the launch to arrive writes, for every request of the launch with a residual
// row, the residual winner (the p_t fallback when no residual was positive) after the
// accepted prefix.  No workgroup waits for another.
__device__ __forceinline__ void resid_finish(const MfmaBiasArgs& a, int* s_flag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's atomics have completed
  __syncthreads();
  if (threadIdx.x == 0) *s_flag = arrive_last(a.res_arrive, blockIdx.x, gridDim.x);
  __syncthreads();
  if (!*s_flag) return;
  for (int c = threadIdx.x; c < a.ncols; c += blockDim.x) {
    const int b = a.col0 + c;
    if (a.jrow[b] == 0) continue;
    unsigned long long r1 = 0ull, r2 = 0ull;
#pragma unroll
    for (int q = 0; q < kSubSlots; ++q) {
      const unsigned long long* slot = a.res_best + ((size_t)q * a.B + b) * 2;
      const unsigned long long x1 = atomic_load_u64(&slot[0]), x2 = atomic_load_u64(&slot[1]);
      r1 = x1 > r1 ? x1 : r1;
      r2 = x2 > r2 ? x2 : r2;
    }
    const uint32_t y = packed_index(r1 != 0ull ? r1 : r2);
    a.out_tokens[(size_t)b * (a.G + 1) + a.n_accept[b]] = (int32_t)y;
  }
}

template <int NCB> constexpr int kThreads = Shape<NCB, kModeDraft>::NT;
template <int NCB> constexpr int kWgPerCu = Shape<NCB, kModeDraft>::WG_PER_CU;

// VEC4: V % 4 == 0, so every 4-row run of a logit row is one aligned 16-byte load
template <int NCB, int MODE, bool VEC4>
__global__ __launch_bounds__(kThreads<NCB>, kWgPerCu<NCB>) void
k_mfma_bias(const MfmaBiasArgs a) {
  using S = Shape<NCB, MODE>;
  constexpr int NCW = S::NCW, TSPLIT = S::TSPLIT, NC = S::NC, SA = S::SA, UD = S::UD;
  constexpr int NT = S::NT, NW = S::NW;
  extern __shared__ __align__(16) unsigned char smem[];
  long long* col_urow = reinterpret_cast<long long*>(smem + S::kOffMeta);   // [NC]
  long long* col_trow = col_urow + NC;
  int* col_b = reinterpret_cast<int*>(col_trow + NC);
  int* col_k = col_b + NC;
  int* col_prev = col_k + NC;
  float* col_ld = reinterpret_cast<float*>(col_prev + NC);
  float* col_lt = col_ld + NC;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, n32 = lane & 31;
  const int cb0 = wave % NCW, toff = wave / NCW;
  const int G = a.G, V = a.V;
  const float s2 = a.invT * kLog2e;   // logit -> base-2 scale

  // ---- this workgroup's contiguous range of 32-row vocab tiles, TSPLIT per step
  const int ntiles = (V + 31) >> 5;
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int per = ntiles / nwg, rem = ntiles % nwg;
  const int t0 = wg * per + min(wg, rem);
  const int t1 = t0 + per + (wg < rem ? 1 : 0);
  const int nsteps = (t1 - t0 + TSPLIT - 1) / TSPLIT;

  // ---- W2t ring: DMA of step `step` into stage step % SA.  Lane l of instruction j moves
  // chunk l>>1 (16 bytes) of stage row 2j + (l&1); rows past V repeat row V-1.  A step past
  // the last one issues the same instructions on one cached line (its stage is never read
  // again), which keeps the per-step load count constant.
  const uint32_t ring_lds = (uint32_t)(uintptr_t)(lds_ptr_t)smem;
  auto issue_dma = [&](int step) {
    const int row0 = (t0 + step * TSPLIT) * 32;
    const uint32_t stage = ring_lds + (uint32_t)((step % SA) * S::kStage);
    const bool dummy = step >= nsteps;
    const uint16_t* gbase = dummy ? a.W2t : a.W2t + (size_t)row0 * kR;
#pragma unroll
    for (int i = 0; i < S::NA; ++i) {
      const int j = wave + NW * i;
      const int row = min(row0 + 2 * j + (lane & 1), V - 1) - row0;   // >= 0: row0 < V
      const uint32_t voff = dummy ? 0u : (uint32_t)(row * kR * 2 + (lane >> 1) * 16);
      dma16(gbase, voff, stage + (uint32_t)(j * kPairBytes));
    }
  };
  // ---- residual mode: the requests with a residual row (usually few) are compacted, in
  // order, to the front of the columns, so that waves whose column block has none skip the
  // epilogue (they still issue their share of the loads and meet every barrier)
  int n_live = NC;
  if constexpr (MODE == kModeResid) {
    int* clist = reinterpret_cast<int*>(smem);   // [NC] list, [NC] count, [NC+1..] per wave
    const bool act = tid < a.ncols && a.jrow[a.col0 + tid] > 0;   // NC <= NT
    const unsigned long long bal = __ballot(act);
    const int below = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) clist[NC + 1 + wave] = __popcll(bal);
    __syncthreads();
    int off = 0;
    for (int w = 0; w < wave; ++w) off += clist[NC + 1 + w];
    if (act) clist[off + below] = tid;
    if (tid == NT - 1) clist[NC] = off + __popcll(bal);
    __syncthreads();
    n_live = clist[NC];
    if (n_live == 0) return;   // nothing to resample (uniform exit, no load issued yet)
    if (n_live <= a.thin_max) {
      resid_thin<NW>(a, clist, n_live, reinterpret_cast<float4*>(smem + 4096));
      resid_finish(a, clist + NC + 1 + NW);
      return;
    }
  }
  // ---- column metadata: request, position, conditioning token, logit row offsets, lse
  for (int c = tid; c < NC; c += NT) {
    int b = -1, k = 0, prev = 0;
    float ld = 0.f, lt = 0.f;
    if (c < a.ncols) {
      const int gc = a.col0 + c;
      if (MODE == kModeDraft) {
        b = gc;
        k = a.k;
        prev = (k == 1) ? a.anchor[b]
                        : (a.forced ? a.forced[(size_t)b * G + (k - 2)]
                                    : (int)packed_index(a.best_prev[b]));
      } else if (MODE == kModeResid) {
        const int gr = c < n_live ? a.col0 + reinterpret_cast<const int*>(smem)[c] : gc;
        const int j = c < n_live ? a.jrow[gr] : 0;
        if (j > 0) {
          b = gr;
          k = j;
          prev = (j == 1) ? a.anchor[b] : a.tokens[(size_t)b * G + (j - 2)];
          ld = a.lse_d[(size_t)b * G + (j - 1)] * kLog2e;
          lt = a.lse_t_row[b] * kLog2e;
        }
      } else {
        b = gc / G;
        k = gc % G + 1;
        prev = (k == 1) ? a.anchor[b] : a.tokens[(size_t)b * G + (k - 2)];
        ld = a.lse_d[(size_t)b * G + (k - 1)] * kLog2e;
        lt = a.lse_t[(size_t)b * G + (k - 1)] * kLog2e;
      }
    }
    col_b[c] = b;
    col_k[c] = k;
    col_prev[c] = clamp_tok(prev, V);
    col_ld[c] = ld;
    col_lt[c] = lt;
    col_urow[c] = b >= 0 ? ((long long)b * G + (k - 1)) * V : -1;
    col_trow[c] = b >= 0 ? ((long long)b * (G + 1) + (k - 1)) * V : -1;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // ---- this lane's column; its gathered W1 row is the MFMA B operand (idle lanes gather
  // row 0 and are never reported)
  const int col = cb0 * 32 + n32;
  const int cb = col_b[col], ck = col_k[col];
  const bool wave_live = MODE != kModeResid || cb0 * 32 < n_live;
  const float cld = col_ld[col], clt = col_lt[col];
  const long long curow = col_urow[col], ctrow = col_trow[col];
  // ---- logit slices in the MFMA output layout: lane rows 8g + 4h + j of the tile
  f32x4_t Ub[UD][4], Tb[S::HAS_T ? UD : 1][4];
  auto load_logits = [&](int step, f32x4_t (&u)[4], f32x4_t (&tt)[4]) {
    const int t = t0 + step * TSPLIT + toff;
    const bool live = cb >= 0 && t < t1;       // else one valid dummy address per load
    if (VEC4) {
      const int vb = t * 32 + 4 * h;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int v = min(vb + 8 * g, V - 4);
        const float* pu = live ? a.U + curow + v : a.U;
        u[g] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pu));
        if (S::HAS_T) {
          const float* pt = live ? a.T + ctrow + v : a.T;
          tt[g] = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(pt));
        }
      }
      if (__builtin_expect((t + 1) * 32 > V, 0)) {
        // the vocabulary's last tile: a whole run lies past V (V % 4 == 0); its logits
        // become -inf, which removes it from the max, the sums and every race
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (vb + 8 * g >= V) {
            u[g] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
            if (S::HAS_T) tt[g] = f32x4_t{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
          }
      }
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int v = t * 32 + 8 * g + 4 * h + j;
          const int vc = min(v, V - 1);
          u[g][j] = v >= V ? -INFINITY : (live ? a.U[curow + vc] : 0.f);
          if (S::HAS_T) tt[g][j] = v >= V ? -INFINITY : (live ? a.T[ctrow + vc] : 0.f);
        }
    }
  };
  u32x4_t Bop[kKS];
  if constexpr (S::kW1Staged) {
    // whole 512-byte rows by DMA (full cache lines, unlike 32-byte pieces of 32 rows per
    // instruction), two rows per instruction in the pair layout, then the fragments from
    // LDS: B row n32, chunk 2kk + h
#pragma unroll
    for (int i = 0; i < NC / 2 / NW; ++i) {
      const int j = wave + NW * i;
      const uint16_t* src = a.W1 + (size_t)col_prev[2 * j + (lane & 1)] * kR + (lane >> 1) * 8;
      dma16v(src, ring_lds + (uint32_t)(j * kPairBytes));
    }
    wait_vm<0>();
    barrier_no_fence();
    const unsigned char* Bl = smem + (col >> 1) * kPairBytes + (2 * h + (col & 1)) * 16;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) Bop[kk] = *reinterpret_cast<const u32x4_t*>(Bl + kk * 64);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // ring free again
  } else {
    const uint16_t* wrow = a.W1 + (size_t)col_prev[col] * kR + 8 * h;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) Bop[kk] = *reinterpret_cast<const u32x4_t*>(wrow + kk * 16);
  }

  const PhiloxLane pl = philox_lane((uint32_t)ck, (uint32_t)(cb < 0 ? 0 : cb),
                                    MODE == kModeResid ? 2u : 0u, a.key0, a.key1);

  // the first stages and logit slices, in the order they are needed
#pragma unroll
  for (int p = 0; p < S::PRE; ++p) {
    if (p < SA - 1) issue_dma(p);
    if (p < UD - 1) load_logits(p, Ub[p], Tb[S::HAS_T ? p : 0]);
  }

  // per-lane running state of the lane's column
  float st_m = kNegBig, st_l = 0.f, st_s = -INFINITY, st_s2 = -INFINITY;
  uint32_t st_v = 0xFFFFFFFFu, st_v2 = 0xFFFFFFFFu;

  // lane's A-fragment base within a stage: row n32 of tile toff, chunk 2kk + h
  const int a_lane = toff * kTileBytes + (n32 >> 1) * kPairBytes + (2 * h + (n32 & 1)) * 16;

  auto step_body = [&](int step, auto bufc, auto basec) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr int BASE = decltype(basec)::value;   // >= 0: step == BASE + BUF
    constexpr int NXT = (BUF + UD - 1) % UD;
    // stage `step` complete for this wave, then for all; stage step-1 free for reuse
    if constexpr (!VEC4) {
      wait_vm<0>();
    } else if constexpr (BASE >= 0 && BASE + BUF < SA - 1) {
      wait_vm<S::wait_early(BASE + BUF)>();
    } else {
      wait_vm<S::kWaitSS>();
    }
    barrier_no_fence();
    issue_dma(step + SA - 1);
    load_logits(step + UD - 1, Ub[NXT], Tb[S::HAS_T ? NXT : 0]);

    const int t = t0 + step * TSPLIT + toff;
    if (t >= t1 || !wave_live) return;        // wave-uniform (also every step >= nsteps);
                                               // idle lanes (cb < 0) compute on zeros and
                                               // are never reported
    const unsigned char* At = smem + (size_t)(step % SA) * S::kStage + a_lane;
    f32x16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                    0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // A fragments are read kAhead k-steps ahead of their MFMA
    constexpr int kAhead = 4;
    u32x4_t av[kAhead];
#pragma unroll
    for (int kk = 0; kk < kAhead; ++kk) av[kk] = *reinterpret_cast<const u32x4_t*>(At + kk * 64);
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av[kk % kAhead]),
                                                    as_bf16x8(Bop[kk]), acc, 0, 0, 0);
      if (kk + kAhead < kKS)
        av[kk % kAhead] = *reinterpret_cast<const u32x4_t*>(At + (kk + kAhead) * 64);
    }
    const int vrow = t * 32 + 4 * h;           // first row of this lane's runs
    // element i = 4g + j of the lane is vocab row vrow + 8g + j (rows past V carry -inf
    // logits); i increases with the row, so a strict '>' keeps the lowest row on ties
    auto row_of = [&](int i) { return (uint32_t)(vrow + 8 * (i >> 2) + (i & 3)); };
    float y[16];                               // unscaled draft logit U + bias
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int j = 0; j < 4; ++j) y[4 * g + j] = Ub[BUF][g][j] + acc[4 * g + j];
    if (MODE == kModeDraft) {
      float mx = y[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) mx = fmaxf(mx, y[i]);
      const float mnew = fmaxf(st_m, mx * s2);
      // four independent partial sums of the step's terms
      float lp[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        lp[q] = ex2(fmaf(y[q], s2, -mnew));
#pragma unroll
        for (int i = q + 4; i < 16; i += 4) lp[q] += ex2(fmaf(y[i], s2, -mnew));
      }
      st_l = st_l * ex2(st_m - mnew) + ((lp[0] + lp[1]) + (lp[2] + lp[3]));
      st_m = mnew;
      uint32_t c0[4], wd[4][4];
#pragma unroll
      for (int g = 0; g < 4; ++g) c0[g] = (uint32_t)(t * 8 + 2 * g + h);
      philox_calls<4>(c0, pl, wd);
      float sc[16];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[4 * g + j] = fmaf(y[4 * g + j], s2, neg_lglg(wd[g][j]));
      // tree arg-max over the step's elements: the later (higher-row) side of a pair wins
      // only when strictly greater, so ties keep the lowest row, as does the running best
      float bs8[8];
      int bi8[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool hi2 = sc[2 * i + 1] > sc[2 * i];
        bs8[i] = hi2 ? sc[2 * i + 1] : sc[2 * i];
        bi8[i] = hi2 ? 2 * i + 1 : 2 * i;
      }
#pragma unroll
      for (int n = 4; n >= 1; n >>= 1)
#pragma unroll
        for (int i = 0; i < n; ++i) {
          const bool hi2 = bs8[2 * i + 1] > bs8[2 * i];
          bs8[i] = hi2 ? bs8[2 * i + 1] : bs8[2 * i];
          bi8[i] = hi2 ? bi8[2 * i + 1] : bi8[2 * i];
        }
      const bool lead = bs8[0] > st_s;
      st_s = lead ? bs8[0] : st_s;
      st_v = lead ? row_of(bi8[0]) : st_v;
    } else {
      float zt[16];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) zt[4 * g + j] = Tb[S::HAS_T ? BUF : 0][g][j] * s2;
      if (MODE == kModeResid) {
        float bs = st_s, bs2 = st_s2;
        int bi = -1, bi2 = -1;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const U4 w = philox_call((uint32_t)(t * 8 + 2 * g + h), pl);
          const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 4 * g + j;
            const float gn = neg_lglg(wd[j]);
            const float rho = ex2(zt[i] - clt) - ex2(fmaf(y[i], s2, -cld));
            const float sc = rho > 0.f ? lg2(rho) + gn : -INFINITY;
            const bool better = sc > bs;
            bs = better ? sc : bs;
            bi = better ? i : bi;
            const float sc2 = zt[i] + gn;
            const bool better2 = sc2 > bs2;
            bs2 = better2 ? sc2 : bs2;
            bi2 = better2 ? i : bi2;
          }
        }
        st_s = bs;
        st_v = bi >= 0 ? row_of(bi) : st_v;
        st_s2 = bs2;
        st_v2 = bi2 >= 0 ? row_of(bi2) : st_v2;
      } else {
        float sum = st_l;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          sum += fminf(ex2(fmaf(y[i], s2, -cld)), ex2(zt[i] - clt));
        st_l = sum;
      }
    }
  };

  // step 0 waits for everything anyway; draining here (with a wait the compiler sees) lets
  // the loop start with no prologue load pending in its bookkeeping
  // UD unconditional bodies per trip (steps past the last compute nothing but still issue
  // their dummy loads), so that every body sees the same load history; the first trips are
  // peeled, so the compiler's bookkeeping enters the loop in its steady state
  // (every early step, whose stage was issued before the loop, falls in a peeled trip)
  peel_trips<0, S::kPeelTrips, UD>(step_body);
  for (int step = S::kPeelTrips * UD; step < nsteps; step += UD)
    unroll_steps<0, UD, -1>(step, step_body);
  __builtin_amdgcn_s_waitcnt(0);   // dummy DMAs of the last steps have landed
  __syncthreads();                 // every wave is done with the ring; reuse it below

  // ---- merge the two lane halves holding the same column, then the TSPLIT waves that
  // covered disjoint tiles of it, in a fixed order: deterministic
  float* red = reinterpret_cast<float*>(smem);   // [TSPLIT][NC][4] over the ring
  {
    float m = st_m, l = st_l, sc = st_s, sc2 = st_s2;
    uint32_t v = st_v, v2 = st_v2;
    const float om = __shfl_xor(m, 32, kWave);
    const float ol = __shfl_xor(l, 32, kWave);
    const float os = __shfl_xor(sc, 32, kWave);
    const uint32_t ov = (uint32_t)__shfl_xor((int)v, 32, kWave);
    const float os2 = __shfl_xor(sc2, 32, kWave);
    const uint32_t ov2 = (uint32_t)__shfl_xor((int)v2, 32, kWave);
    if (MODE == kModeDraft) {
      const float mm = fmaxf(m, om);
      l = l * ex2(m - mm) + ol * ex2(om - mm);
      m = mm;
    } else {
      l = l + ol;
    }
    if (os > sc || (os == sc && ov < v)) { sc = os; v = ov; }
    if (os2 > sc2 || (os2 == sc2 && ov2 < v2)) { sc2 = os2; v2 = ov2; }
    if (h == 0) {
      float* e = red + ((size_t)toff * NC + col) * 4;
      if (MODE == kModeDraft) {
        e[0] = m; e[1] = l; e[2] = sc; e[3] = __uint_as_float(v);
      } else if (MODE == kModeResid) {
        e[0] = sc; e[1] = __uint_as_float(v); e[2] = sc2; e[3] = __uint_as_float(v2);
      } else {
        e[0] = l;
      }
    }
  }
  __syncthreads();
  for (int c = tid; c < a.ncols; c += NT) {
    const int b = col_b[c];
    if (b < 0) continue;
    if (MODE == kModeDraft) {
      float m = kNegBig, l = 0.f, sc = -INFINITY;
      uint32_t v = 0xFFFFFFFFu;
      for (int w = 0; w < TSPLIT; ++w) {
        const float* e = red + ((size_t)w * NC + c) * 4;
        const float mm = fmaxf(m, e[0]);
        l = l * ex2(m - mm) + e[1] * ex2(e[0] - mm);
        m = mm;
        const uint32_t ev = __float_as_uint(e[3]);
        if (e[2] > sc || (e[2] == sc && ev < v)) { sc = e[2]; v = ev; }
      }
      a.part[(size_t)wg * a.B + b] = make_float2(m, l);
      if (v != 0xFFFFFFFFu) atomic_max_u64(&a.best_cur[b], pack_score(sc, v));
    } else if (MODE == kModeResid) {
      float sc = -INFINITY, sc2 = -INFINITY;
      uint32_t v = 0xFFFFFFFFu, v2 = 0xFFFFFFFFu;
      for (int w = 0; w < TSPLIT; ++w) {
        const float* e = red + ((size_t)w * NC + c) * 4;
        const uint32_t ev = __float_as_uint(e[1]), ev2 = __float_as_uint(e[3]);
        if (e[0] > sc || (e[0] == sc && ev < v)) { sc = e[0]; v = ev; }
        if (e[2] > sc2 || (e[2] == sc2 && ev2 < v2)) { sc2 = e[2]; v2 = ev2; }
      }
      unsigned long long* slot = a.res_best + ((size_t)(wg % kSubSlots) * a.B + b) * 2;
      if (v != 0xFFFFFFFFu) atomic_max_u64(&slot[0], pack_score(sc, v));
      if (v2 != 0xFFFFFFFFu) atomic_max_u64(&slot[1], pack_score(sc2, v2));
    } else {
      float sum = 0.f;
      for (int w = 0; w < TSPLIT; ++w) sum += red[((size_t)w * NC + c) * 4];
      a.tv_part[(size_t)wg * ((size_t)a.B * a.G) + (a.col0 + c)] = sum;
    }
  }
  if constexpr (MODE == kModeResid) resid_finish(a, reinterpret_cast<int*>(red) + TSPLIT * NC * 4);
}

template <int NCB, int MODE, bool VEC4>
static dspark_status attr_v() {
  static LdsAttr attr;
  return attr.ensure((const void*)k_mfma_bias<NCB, MODE, VEC4>, (int)Shape<NCB, MODE>::kLds);
}

template <int NCB, int MODE, bool VEC4>
static dspark_status launch_v(const MfmaBiasArgs& a, int nwg, hipStream_t st) {
  using S = Shape<NCB, MODE>;
  if (attr_v<NCB, MODE, VEC4>() != DSPARK_OK) return DSPARK_E_HIP;
  hipLaunchKernelGGL((k_mfma_bias<NCB, MODE, VEC4>), dim3(nwg), dim3(S::NT), S::kLds, st, a);
  return launch_status();
}

template <int MODE>
static dspark_status attr_mode() {
  const dspark_status r[] = {attr_v<1, MODE, true>(), attr_v<1, MODE, false>(),
                             attr_v<2, MODE, true>(), attr_v<2, MODE, false>(),
                             attr_v<4, MODE, true>(), attr_v<4, MODE, false>(),
                             attr_v<8, MODE, true>(), attr_v<8, MODE, false>()};
  for (dspark_status x : r)
    if (x != DSPARK_OK) return x;
  return DSPARK_OK;
}

template <int NCB, int MODE>
static dspark_status launch_t(const MfmaBiasArgs& a, int nwg, hipStream_t st) {
  return (a.V & 3) == 0 ? launch_v<NCB, MODE, true>(a, nwg, st)
                        : launch_v<NCB, MODE, false>(a, nwg, st);
}

template <int MODE>
static dspark_status launch_mode(const MfmaBiasArgs& a, int nwg, hipStream_t st) {
  const int ncb = (a.ncols + 31) / 32;
  if (ncb <= 1) return launch_t<1, MODE>(a, nwg, st);
  if (ncb <= 2) return launch_t<2, MODE>(a, nwg, st);
  if (ncb <= 4) return launch_t<4, MODE>(a, nwg, st);
  return launch_t<8, MODE>(a, nwg, st);
}

int mfma_grid(int V, int ncols, int mode) {
  // one resident wave of workgroups: per-CU occupancy of each variant (registers, LDS)
  (void)mode;
  const int ntiles = (V + 31) / 32;
  const int ncb = (std::min(ncols, 256) + 31) / 32;
  const int per_cu = (ncb == 2 || (ncb > 2 && ncb <= 4)) ? 2 : 1;
  return std::max(1, std::min(ntiles, per_cu * 256));
}

dspark_status mfma_prepare() {
  if (attr_mode<kModeDraft>() != DSPARK_OK || attr_mode<kModeResid>() != DSPARK_OK ||
      attr_mode<kModeTV>() != DSPARK_OK || draft16_prepare() != DSPARK_OK)
    return DSPARK_E_HIP;
  return DSPARK_OK;
}

dspark_status launch_mfma_bias(const MfmaBiasArgs& args, int nwg, hipStream_t st) {
  // columns beyond one group run as further launches over the same vocabulary tiles
  const int group = mfma_column_group(args.mode);
  for (int c0 = 0; c0 < args.ncols; c0 += group) {
    MfmaBiasArgs a = args;
    a.col0 = args.col0 + c0;
    a.ncols = std::min(group, args.ncols - c0);
    if (a.mode == kModeResid) a.res_arrive = args.res_arrive + (c0 / group) * kArriveInts;
    dspark_status s = DSPARK_OK;
    if (a.mode == kModeDraft)
      s = draft16_supported(a) ? launch_draft16(a, nwg, st) : launch_mode<kModeDraft>(a, nwg, st);
    else if (a.mode == kModeResid) s = launch_mode<kModeResid>(a, nwg, st);
    else s = draft16_supported(a) ? launch_draft16(a, nwg, st) : launch_mode<kModeTV>(a, nwg, st);
    if (s != DSPARK_OK) return s;
  }
  return DSPARK_OK;
}

}  // namespace dspark
