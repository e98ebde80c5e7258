// mfma_bias.hip -- batched Markov bias on bf16 MFMA with fused epilogues (see mfma_bias.h).
#include "mfma_bias.h"

namespace dspark {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kR = 256;               // Markov rank handled by this path
constexpr int kKS = kR / 16;          // MFMA k-steps
constexpr int kRowStride = kR + 8;    // bf16 per LDS row of the gathered W1 (16-byte pad)
constexpr int kMetaBytes = 5 * 256 * 4;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int NCB, int MODE>
__global__ __launch_bounds__(256, (NCB > 4 ? 1 : 2)) void k_mfma_bias(const MfmaBiasArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  int* col_b = reinterpret_cast<int*>(smem);
  int* col_k = col_b + 256;
  int* col_prev = col_k + 256;
  float* col_ld = reinterpret_cast<float*>(col_prev + 256);
  float* col_lt = col_ld + 256;
  uint16_t* w1g = reinterpret_cast<uint16_t*>(smem + kMetaBytes);
  constexpr int NC = NCB * 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int G = a.G, V = a.V;
  const float invT = a.invT;

  // ---- column metadata: request, position, conditioning token, lse values
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
          ld = a.lse_d[(size_t)b * G + (j - 1)];
          lt = a.lse_t_row[b];
        }
      } else {
        b = gc / G;
        k = gc % G + 1;
        prev = (k == 1) ? a.anchor[b] : a.tokens[(size_t)b * G + (k - 2)];
        ld = a.lse_d[(size_t)b * G + (k - 1)];
        lt = a.lse_t[(size_t)b * G + (k - 1)];
      }
    }
    col_b[c] = b;
    col_k[c] = k;
    col_prev[c] = prev;
    col_ld[c] = ld;
    col_lt[c] = lt;
  }
  __syncthreads();
  // ---- gather W1[prev_c] rows into LDS (the MFMA B operand), zero for unused columns
  for (int q = tid; q < NC * (kR / 8); q += 256) {
    const int c = q / (kR / 8), ch = q % (kR / 8);
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (col_b[c] >= 0)
      v = *reinterpret_cast<const uint4*>(a.W1 + (size_t)col_prev[c] * kR + ch * 8);
    *reinterpret_cast<uint4*>(w1g + c * kRowStride + ch * 8) = v;
  }
  __syncthreads();

  // ---- this workgroup's contiguous range of 32-row vocab tiles.  Waves split the
  // column blocks (NCB >= 4: wave w owns blocks w, w+4, ...) or, with fewer blocks, the
  // tiles (every TSPLIT-th tile); all waves of a column set read the same W2t tiles, so
  // HBM sees each tile once and the repeats are L1/L2 hits.
  constexpr int CBW = NCB >= 4 ? NCB / 4 : 1;        // column blocks per wave
  constexpr int NCW = NCB >= 4 ? 4 : NCB;            // distinct column sets over waves
  constexpr int TSPLIT = 4 / NCW;                    // tile interleave
  const int ntiles = (V + 31) >> 5;
  const int nwg = gridDim.x, wg = blockIdx.x;
  const int per = ntiles / nwg, rem = ntiles % nwg;
  const int t0 = wg * per + min(wg, rem);
  const int t1 = t0 + per + (wg < rem ? 1 : 0);
  const int h = lane >> 5, n32 = lane & 31;
  const int cb0 = wave % NCW, toff = wave / NCW;
  const bool vec4 = (V & 3) == 0;

  // per-lane running state for the lane's column in each owned column block
  float s_m[CBW], s_l[CBW], s_s[CBW], s_z[CBW], s_s2[CBW];
  uint32_t s_i[CBW], s_i2[CBW];
#pragma unroll
  for (int q = 0; q < CBW; ++q) {
    s_m[q] = -INFINITY;
    s_l[q] = 0.f;
    s_s[q] = -INFINITY;
    s_z[q] = 0.f;
    s_s2[q] = -INFINITY;
    s_i[q] = 0xFFFFFFFFu;
    s_i2[q] = 0xFFFFFFFFu;
  }

  uint4 A[kKS], An[kKS];
  int t = t0 + toff;
  if (t < t1) {
    const int v = min(t * 32 + n32, V - 1);
    const uint16_t* row = a.W2t + (size_t)v * kR + 8 * h;
#pragma unroll
    for (int kk = 0; kk < kKS; ++kk) A[kk] = *reinterpret_cast<const uint4*>(row + kk * 16);
  }
  for (; t < t1; t += TSPLIT) {
    const bool more = t + TSPLIT < t1;
    if (more) {
      const int v = min((t + TSPLIT) * 32 + n32, V - 1);
      const uint16_t* row = a.W2t + (size_t)v * kR + 8 * h;
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) An[kk] = *reinterpret_cast<const uint4*>(row + kk * 16);
    }
#pragma unroll
    for (int q = 0; q < CBW; ++q) {
      const int cb = cb0 + 4 * q;
      f32x16_t acc = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f,
                      0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      const uint16_t* bp = w1g + (cb * 32 + n32) * kRowStride + 8 * h;
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) {
        const uint4 bv = *reinterpret_cast<const uint4*>(bp + kk * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(A[kk]), as_bf16x8(bv), acc, 0,
                                                      0, 0);
      }
      const int c = cb * 32 + n32;
      const int b = col_b[c];
      if (b < 0) continue;
      const int k = col_k[c];
      const float* urow = a.U + ((size_t)b * G + (k - 1)) * V;
      const float* trow = (MODE == kModeDraft) ? nullptr : a.T + ((size_t)b * (G + 1) + (k - 1)) * V;
      const float ld = col_ld[c], lt = col_lt[c];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int v0 = t * 32 + 8 * g + 4 * h;
        if (v0 >= V) continue;
        float u[4], tt[4];
        if (vec4) {
          const f32x4_t qv = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(urow + v0));
          u[0] = qv[0]; u[1] = qv[1]; u[2] = qv[2]; u[3] = qv[3];
          if (MODE != kModeDraft) {
            const f32x4_t p = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(trow + v0));
            tt[0] = p[0]; tt[1] = p[1]; tt[2] = p[2]; tt[3] = p[3];
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            u[j] = (v0 + j < V) ? urow[v0 + j] : 0.f;
            if (MODE != kModeDraft) tt[j] = (v0 + j < V) ? trow[v0 + j] : 0.f;
          }
        }
        const int nvalid = min(4, V - v0);
        if (MODE == kModeDraft) {
          const U4 w = philox10((uint32_t)v0 >> 2, (uint32_t)k, (uint32_t)b, 0u, a.key0, a.key1);
          const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
          float z[4];
          float gm = -INFINITY;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            z[j] = (u[j] + acc[4 * g + j]) * invT;
            if (j < nvalid) gm = fmaxf(gm, z[j]);
          }
          if (gm > s_m[q]) {
            s_l[q] *= fast_exp(s_m[q] - gm);
            s_m[q] = gm;
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j < nvalid) {
              s_l[q] += fast_exp(z[j] - s_m[q]);
              const float sc = z[j] + gumbel_from_uniform(word_to_uniform(wd[j]));
              if (sc > s_s[q]) {
                s_s[q] = sc;
                s_i[q] = (uint32_t)(v0 + j);
                s_z[q] = z[j];
              }
            }
          }
        } else if (MODE == kModeResid) {
          const U4 w = philox10((uint32_t)v0 >> 2, (uint32_t)k, (uint32_t)b, 2u, a.key0, a.key1);
          const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j < nvalid) {
              const float zd = (u[j] + acc[4 * g + j]) * invT;
              const float zt = tt[j] * invT;
              const float rho = fast_exp(zt - lt) - fast_exp(zd - ld);
              const float gn = gumbel_from_uniform(word_to_uniform(wd[j]));
              if (rho > 0.f) {
                const float sc = fast_log(rho) + gn;
                if (sc > s_s[q]) { s_s[q] = sc; s_i[q] = (uint32_t)(v0 + j); }
              }
              const float sc2 = zt + gn;
              if (sc2 > s_s2[q]) { s_s2[q] = sc2; s_i2[q] = (uint32_t)(v0 + j); }
            }
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j < nvalid) {
              const float pd = fast_exp((u[j] + acc[4 * g + j]) * invT - ld);
              const float pt = fast_exp(tt[j] * invT - lt);
              s_l[q] += fminf(pd, pt);
            }
          }
        }
      }
    }
    if (more) {
#pragma unroll
      for (int kk = 0; kk < kKS; ++kk) A[kk] = An[kk];
    }
  }

  // ---- merge the two lane halves holding the same column, then the TSPLIT waves that
  // covered disjoint tiles of it (fixed order: deterministic)
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem + kMetaBytes);   // [TSPLIT][NC][5]
#pragma unroll
  for (int q = 0; q < CBW; ++q) {
    const int cb = cb0 + 4 * q;
    const float om = __shfl_xor(s_m[q], 32, kWave);
    const float ol = __shfl_xor(s_l[q], 32, kWave);
    const float os = __shfl_xor(s_s[q], 32, kWave);
    const float oz = __shfl_xor(s_z[q], 32, kWave);
    const uint32_t oi = (uint32_t)__shfl_xor((int)s_i[q], 32, kWave);
    const float os2 = __shfl_xor(s_s2[q], 32, kWave);
    const uint32_t oi2 = (uint32_t)__shfl_xor((int)s_i2[q], 32, kWave);
    float m = s_m[q], l = s_l[q], sc = s_s[q], z = s_z[q], sc2 = s_s2[q];
    uint32_t i = s_i[q], i2 = s_i2[q];
    if (MODE == kModeDraft) {
      const ML mm = ml_merge(ML{m, l}, ML{om, ol});
      m = mm.m;
      l = mm.l;
    } else {
      l = l + ol;
    }
    if (os > sc || (os == sc && oi < i)) { sc = os; i = oi; z = oz; }
    if (os2 > sc2 || (os2 == sc2 && oi2 < i2)) { sc2 = os2; i2 = oi2; }
    if (h == 0) {
      float* e = red + ((size_t)toff * NC + cb * 32 + n32) * 5;
      if (MODE == kModeDraft) {
        e[0] = m; e[1] = l; e[2] = sc; e[3] = z; e[4] = __uint_as_float(i);
      } else if (MODE == kModeResid) {
        e[0] = sc; e[1] = __uint_as_float(i); e[2] = sc2; e[3] = __uint_as_float(i2);
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
      ML st{-INFINITY, 0.f};
      Cand best{-INFINITY, 0xFFFFFFFFu, 0.f};
      for (int w = 0; w < TSPLIT; ++w) {
        const float* e = red + ((size_t)w * NC + c) * 5;
        st = ml_merge(st, ML{e[0], e[1]});
        const Cand o{e[2], __float_as_uint(e[4]), e[3]};
        if (cand_better(o, best)) best = o;
      }
      a.part[(size_t)wg * a.B + b] = make_float4(st.m, st.l, best.z, __uint_as_float(best.i));
      atomic_max_u64(&a.best_cur[b], pack_score(best.s, best.i));
    } else if (MODE == kModeResid) {
      Cand b1{-INFINITY, 0xFFFFFFFFu, 0.f}, b2{-INFINITY, 0xFFFFFFFFu, 0.f};
      for (int w = 0; w < TSPLIT; ++w) {
        const float* e = red + ((size_t)w * NC + c) * 5;
        const Cand o1{e[0], __float_as_uint(e[1]), 0.f}, o2{e[2], __float_as_uint(e[3]), 0.f};
        if (cand_better(o1, b1)) b1 = o1;
        if (cand_better(o2, b2)) b2 = o2;
      }
      if (b1.i != 0xFFFFFFFFu) atomic_max_u64(&a.res_best[b], pack_score(b1.s, b1.i));
      if (b2.i != 0xFFFFFFFFu) atomic_max_u64(&a.fb_best[b], pack_score(b2.s, b2.i));
    } else {
      float sum = 0.f;
      for (int w = 0; w < TSPLIT; ++w) sum += red[((size_t)w * NC + c) * 5];
      a.tv_part[(size_t)wg * ((size_t)a.B * a.G) + (a.col0 + c)] = sum;
    }
  }
}

template <int NCB>
static size_t lds_bytes() {
  const size_t w1g = (size_t)NCB * 32 * kRowStride * 2;
  const size_t red = (size_t)4 * NCB * 32 * 5 * 4;
  return kMetaBytes + (w1g > red ? w1g : red);
}

template <int NCB, int MODE>
static dspark_status launch_t(const MfmaBiasArgs& a, int nwg, hipStream_t st) {
  const size_t sh = lds_bytes<NCB>();
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

int mfma_grid(int V, int ncols) {
  const int ntiles = (V + 31) / 32;
  const int ncb = (std::min(ncols, 256) + 31) / 32;
  const int resident = (ncb > 4 ? 1 : 2) * 256;
  return std::max(1, std::min(ntiles, resident));
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
