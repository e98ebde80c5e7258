// mfma_bias.hip -- batched Markov bias on bf16 MFMA with fused epilogues (see mfma_bias.h).
#include "mfma_bias.h"

namespace dspark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kR = 256;               // Markov rank handled by this path
constexpr int kKS = kR / 16;          // MFMA k-steps
constexpr int kRowStride = kR + 8;    // bf16 per LDS row of the gathered W1 (16-byte pad)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -3.0e38f;   // finite "minus infinity" of the running max

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// Base-2 Gumbel score offset: -log2(-log2 u) (the common constant -log2(ln 2) is dropped,
// it shifts every candidate of a race equally).
__device__ __forceinline__ float neg_lglg(uint32_t w) {
  return -lg2(-lg2(word_to_uniform(w)));
}

template <int NCB, int MODE>
struct Shape {
  static constexpr int CBW = NCB >= 4 ? NCB / 4 : 1;     // column blocks per wave
  static constexpr int NCW = NCB >= 4 ? 4 : NCB;         // distinct column sets
  static constexpr int TSPLIT = 4 / NCW;                 // tiles per step
  static constexpr int NC = NCB * 32;                    // columns
  static constexpr bool HAS_T = MODE != kModeDraft;
  static constexpr int kUStride = 36;                    // floats per staged logit row
  static constexpr int kARows = TSPLIT * 32;             // staged W2t rows per step
  static constexpr int kURows = TSPLIT * NC;             // staged logit rows per step
  static constexpr int kAChunks = kARows * (kR / 8);     // 16-byte chunks
  static constexpr int kUChunks = kURows * 8;
  static constexpr int kAPer = kAChunks / 256;
  static constexpr int kUPer = kUChunks / 256;
  // LDS byte offsets
  static constexpr size_t kOffA = 0;
  static constexpr size_t kOffU = kOffA + (size_t)kARows * kRowStride * 2;
  static constexpr size_t kOffT = kOffU + (size_t)kURows * kUStride * 4;
  static constexpr size_t kOffMeta = kOffT + (HAS_T ? (size_t)kURows * kUStride * 4 : 0);
  static constexpr size_t kMetaBytes = (size_t)NC * (8 + 8 + 4 + 4 + 4 + 4 + 4);
  static constexpr size_t kRed = (size_t)TSPLIT * NC * 4 * 4;
  static constexpr size_t kLds = kOffMeta + kMetaBytes;
  static_assert(kAChunks % 256 == 0 && kUChunks % 256 == 0, "chunk split");
  static_assert(kRed <= kOffMeta, "reduction scratch reuses the staging area");
};

template <int NCB, int MODE>
__global__ __launch_bounds__(256, (NCB > 4 ? 1 : 2)) void
k_mfma_bias(const MfmaBiasArgs a) {
  using S = Shape<NCB, MODE>;
  constexpr int CBW = S::CBW, NCW = S::NCW, TSPLIT = S::TSPLIT, NC = S::NC;
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* sA = reinterpret_cast<uint16_t*>(smem + S::kOffA);     // [kARows][kRowStride]
  float* sU = reinterpret_cast<float*>(smem + S::kOffU);           // [kURows][kUStride]
  float* sT = reinterpret_cast<float*>(smem + S::kOffT);
  long long* col_urow = reinterpret_cast<long long*>(smem + S::kOffMeta);   // [NC]
  long long* col_trow = col_urow + NC;
  int* col_b = reinterpret_cast<int*>(col_trow + NC);
  int* col_k = col_b + NC;
  int* col_prev = col_k + NC;
  float* col_ld = reinterpret_cast<float*>(col_prev + NC);
  float* col_lt = col_ld + NC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, n32 = lane & 31;
  const int cb0 = wave % NCW, toff = wave / NCW;
  const int G = a.G, V = a.V;
  const float s2 = a.invT * kLog2e;   // logit -> base-2 scale
  const bool vec4 = (V & 3) == 0;

  // ---- column metadata: request, position, conditioning token, logit row offsets, lse
  for (int c = tid; c < NC; c += 256) {
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
        const int j = a.jrow[gc];
        if (j > 0) {
          b = gc;
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
  __syncthreads();

  // ---- this workgroup's contiguous range of 32-row vocab tiles, TSPLIT per step
  const int ntiles = (V + 31) >> 5;
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int per = ntiles / nwg, rem = ntiles % nwg;
  const int t0 = wg * per + min(wg, rem);
  const int t1 = t0 + per + (wg < rem ? 1 : 0);
  const int nsteps = (t1 - t0 + TSPLIT - 1) / TSPLIT;

  // ---- staging: coalesced global loads of a step's tiles into registers, then LDS
  u32x4_t RA[S::kAPer];
  f32x4_t RU[S::kUPer], RT[S::HAS_T ? S::kUPer : 1];
  auto stage_load = [&](int step) {
#pragma unroll
    for (int i = 0; i < S::kAPer; ++i) {
      const int chunk = tid + 256 * i;
      const int row = chunk / (kR / 8), col = chunk % (kR / 8);
      const int v = min((t0 + step * TSPLIT) * 32 + row, V - 1);   // tile-major rows
      RA[i] = *reinterpret_cast<const u32x4_t*>(a.W2t + (size_t)v * kR + col * 8);
    }
#pragma unroll
    for (int i = 0; i < S::kUPer; ++i) {
      const int chunk = tid + 256 * i;
      const int ur = chunk >> 3, p = chunk & 7;
      const int tl = ur / NC, c = ur % NC;
      const int v = (t0 + step * TSPLIT + tl) * 32 + 4 * p;
      const long long uo = col_urow[c];
      f32x4_t qu = {0.f, 0.f, 0.f, 0.f}, qt = {0.f, 0.f, 0.f, 0.f};
      if (uo >= 0) {
        if (vec4) {
          if (v < V) {
            qu = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(a.U + uo + v));
            if (S::HAS_T)
              qt = __builtin_nontemporal_load(
                  reinterpret_cast<const f32x4_t*>(a.T + col_trow[c] + v));
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (v + j < V) {
              qu[j] = a.U[uo + v + j];
              if (S::HAS_T) qt[j] = a.T[col_trow[c] + v + j];
            }
        }
      }
      RU[i] = qu;
      if (S::HAS_T) RT[i] = qt;
    }
  };
  auto stage_store = [&]() {
#pragma unroll
    for (int i = 0; i < S::kAPer; ++i) {
      const int chunk = tid + 256 * i;
      const int row = chunk / (kR / 8), col = chunk % (kR / 8);
      *reinterpret_cast<u32x4_t*>(sA + row * kRowStride + col * 8) = RA[i];
    }
#pragma unroll
    for (int i = 0; i < S::kUPer; ++i) {
      const int chunk = tid + 256 * i;
      const int ur = chunk >> 3, p = chunk & 7;
      *reinterpret_cast<f32x4_t*>(sU + ur * S::kUStride + 4 * p) = RU[i];
      if (S::HAS_T) *reinterpret_cast<f32x4_t*>(sT + ur * S::kUStride + 4 * p) = RT[i];
    }
  };

  if (nsteps > 0) stage_load(0);   // first tiles in flight before the dependent gathers

  // ---- this lane's column in each owned block; gathered W1 row = MFMA B operand
  int cbb[CBW], cbk[CBW];
  float cbld[CBW], cblt[CBW];
  uint4 Bop[CBW][kKS];
#pragma unroll
  for (int q = 0; q < CBW; ++q) {
    const int c = (cb0 + 4 * q) * 32 + n32;
    cbb[q] = col_b[c];
    cbk[q] = col_k[c];
    cbld[q] = col_ld[c];
    cblt[q] = col_lt[c];
    const uint16_t* wrow = a.W1 + (size_t)col_prev[c] * kR + 8 * h;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk)
      Bop[q][kk] = cbb[q] >= 0 ? *reinterpret_cast<const uint4*>(wrow + kk * 16)
                               : make_uint4(0u, 0u, 0u, 0u);
  }

  // per-lane running state of the lane's column in each owned block
  float st_m[CBW], st_l[CBW], st_s[CBW], st_s2[CBW];
  uint32_t st_v[CBW], st_v2[CBW];
#pragma unroll
  for (int q = 0; q < CBW; ++q) {
    st_m[q] = kNegBig;
    st_l[q] = 0.f;
    st_s[q] = -INFINITY;
    st_s2[q] = -INFINITY;
    st_v[q] = 0xFFFFFFFFu;
    st_v2[q] = 0xFFFFFFFFu;
  }

  if (nsteps > 0) stage_store();
  __syncthreads();
  for (int step = 0; step < nsteps; ++step) {
    const bool more = step + 1 < nsteps;
    if (more) stage_load(step + 1);            // in flight while this step computes
    const int t = t0 + step * TSPLIT + toff;
    const bool active = t < t1;                // wave-uniform
    const bool full = (t + 1) * 32 <= V;       // every row of this tile is a vocab entry
    const int vrow = t * 32 + 4 * h;           // first row of this lane's runs
    const uint16_t* At = sA + (toff * 32 + n32) * kRowStride + 8 * h;
#pragma unroll
    for (int q = 0; q < CBW; ++q) {
      const int b = cbb[q];
      if (!active) continue;
      f32x16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                      0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) {
        const uint4 av = *reinterpret_cast<const uint4*>(At + kk * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(av), as_bf16x8(Bop[q][kk]), acc,
                                                      0, 0, 0);
      }
      if (b < 0) continue;
      const int k = cbk[q];
      const int ur = toff * NC + (cb0 + 4 * q) * 32 + n32;   // staged logit row
      f32x4_t uq[4];
#pragma unroll
      for (int g = 0; g < 4; ++g)
        uq[g] = *reinterpret_cast<const f32x4_t*>(sU + ur * S::kUStride + 8 * g + 4 * h);
      // base-2 logits of the 16 rows; rows past V become -inf
      float z[16];
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) z[4 * g + j] = (uq[g][j] + acc[4 * g + j]) * s2;
      if (!full) {   // wave-uniform: only the last tile of the vocabulary is partial
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (vrow + 8 * g + j >= V) z[4 * g + j] = -INFINITY;
      }
      if (MODE == kModeDraft) {
        float mx = z[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, z[i]);
        const float mnew = fmaxf(st_m[q], mx);
        float l = st_l[q] * ex2(st_m[q] - mnew);
#pragma unroll
        for (int i = 0; i < 16; ++i) l += ex2(z[i] - mnew);
        st_m[q] = mnew;
        st_l[q] = l;
        float bs = st_s[q];
        uint32_t bvx = st_v[q];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const U4 w = philox10((uint32_t)(t * 8 + 2 * g + h), (uint32_t)k, (uint32_t)b, 0u,
                                a.key0, a.key1);
          const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float sc = z[4 * g + j] + neg_lglg(wd[j]);
            const bool better = sc > bs;
            bs = better ? sc : bs;
            bvx = better ? (uint32_t)(vrow + 8 * g + j) : bvx;
          }
        }
        st_s[q] = bs;
        st_v[q] = bvx;
      } else {
        const float ld = cbld[q], lt = cblt[q];
        f32x4_t tq[4];
#pragma unroll
        for (int g = 0; g < 4; ++g)
          tq[g] = *reinterpret_cast<const f32x4_t*>(sT + ur * S::kUStride + 8 * g + 4 * h);
        float zt[16];
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int j = 0; j < 4; ++j) zt[4 * g + j] = tq[g][j] * s2;
        if (!full) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (vrow + 8 * g + j >= V) zt[4 * g + j] = -INFINITY;
        }
        if (MODE == kModeResid) {
          float bs = st_s[q], bs2 = st_s2[q];
          uint32_t bvx = st_v[q], bvx2 = st_v2[q];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const U4 w = philox10((uint32_t)(t * 8 + 2 * g + h), (uint32_t)k, (uint32_t)b, 2u,
                                  a.key0, a.key1);
            const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = 4 * g + j;
              const float gn = neg_lglg(wd[j]);
              const float rho = ex2(zt[i] - lt) - ex2(z[i] - ld);
              const float sc = rho > 0.f ? lg2(rho) + gn : -INFINITY;
              const bool better = sc > bs;
              bs = better ? sc : bs;
              bvx = better ? (uint32_t)(vrow + 8 * g + j) : bvx;
              const float sc2 = zt[i] + gn;
              const bool better2 = sc2 > bs2;
              bs2 = better2 ? sc2 : bs2;
              bvx2 = better2 ? (uint32_t)(vrow + 8 * g + j) : bvx2;
            }
          }
          st_s[q] = bs;
          st_v[q] = bvx;
          st_s2[q] = bs2;
          st_v2[q] = bvx2;
        } else {
          float sum = st_l[q];
#pragma unroll
          for (int i = 0; i < 16; ++i) sum += fminf(ex2(z[i] - ld), ex2(zt[i] - lt));
          st_l[q] = sum;
        }
      }
    }
    __syncthreads();                // every wave is done reading this step's tiles
    if (more) {
      stage_store();
      __syncthreads();
    }
  }

  // ---- merge the two lane halves holding the same column, then the TSPLIT waves that
  // covered disjoint tiles of it, in a fixed order: deterministic
  float* red = reinterpret_cast<float*>(smem);   // [TSPLIT][NC][4] over the staging area
#pragma unroll
  for (int q = 0; q < CBW; ++q) {
    const int cb = cb0 + 4 * q;
    float m = st_m[q], l = st_l[q], sc = st_s[q], sc2 = st_s2[q];
    uint32_t v = st_v[q], v2 = st_v2[q];
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
      float* e = red + ((size_t)toff * NC + cb * 32 + n32) * 4;
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
  for (int c = tid; c < a.ncols; c += 256) {
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
      a.rpart[(size_t)wg * a.B + b] = make_float4(sc, __uint_as_float(v), sc2, __uint_as_float(v2));
    } else {
      float sum = 0.f;
      for (int w = 0; w < TSPLIT; ++w) sum += red[((size_t)w * NC + c) * 4];
      a.tv_part[(size_t)wg * ((size_t)a.B * a.G) + (a.col0 + c)] = sum;
    }
  }
}

template <int NCB, int MODE>
static dspark_status launch_t(const MfmaBiasArgs& a, int nwg, hipStream_t st) {
  const size_t sh = Shape<NCB, MODE>::kLds;
  static bool attr_set = false;
  if (!attr_set) {
    if (hipFuncSetAttribute((const void*)k_mfma_bias<NCB, MODE>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh) != hipSuccess)
      return DSPARK_E_HIP;
    attr_set = true;
  }
  hipLaunchKernelGGL((k_mfma_bias<NCB, MODE>), dim3(nwg), dim3(256), sh, st, a);
  return launch_status();
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
  const int ntiles = (V + 31) / 32;
  const int ncb = (std::min(ncols, 256) + 31) / 32;
  const int per_cu = (ncb > 4 || ncb == 1) ? 1 : 2;
  return std::max(1, std::min(ntiles, per_cu * 256));
}

dspark_status launch_mfma_bias(const MfmaBiasArgs& args, int nwg, hipStream_t st) {
  // columns beyond 256 run as further launches over the same vocabulary tiles
  for (int c0 = 0; c0 < args.ncols; c0 += 256) {
    MfmaBiasArgs a = args;
    a.col0 = args.col0 + c0;
    a.ncols = std::min(256, args.ncols - c0);
    dspark_status s = DSPARK_OK;
    if (a.mode == kModeDraft) s = launch_mode<kModeDraft>(a, nwg, st);
    else if (a.mode == kModeResid) s = launch_mode<kModeResid>(a, nwg, st);
    else s = launch_mode<kModeTV>(a, nwg, st);
    if (s != DSPARK_OK) return s;
  }
  return DSPARK_OK;
}

}  // namespace dspark
