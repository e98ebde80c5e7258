// gemv.hip -- the draft position kernel for one request with bf16 weights of rank 256, where
// the resident draft does not apply: the Markov bias W1[x_{k-1}] . W2t[v] is a
// matrix-vector product [CSDN Eq. 4; XTL §4], and one position streams all of W2t
// (V x 512 bytes).  (The kernel takes a grid row per request and so streams W2t once per
// request; from two requests on the matrix-core kernels, which stream it once for all, are
// used instead.)  The kernel is a plain HBM stream, laid out so that nothing waits on the
// serial chain of the draft:
//   - a workgroup owns a contiguous range of the vocabulary, kGvRows rows per chunk, and
//     the grid is at most 768 workgroups (three per CU at the kernel's register count), so
//     for one request every workgroup is resident from the start (no second round of
//     workgroups, no tail of short-lived ones);
//   - each thread issues the W2t loads of its whole chunk (16 bytes x 4 per row pass, 8
//     lanes per row) and its base-logit quad before it reads the conditioning token, so
//     the dependent chain x_{k-1} (a 64-bit atomic word of the previous position) ->
//     W1[x_{k-1}] overlaps the stream instead of preceding it;
//   - the epilogue runs one Philox4x32-10 call per four consecutive vocabulary rows (the
//     four uniforms of the call are exactly those rows' draws), base-2 logits, an online
//     (max, sum) and a Gumbel-max race, then the same per-workgroup partial slot and
//     packed atomic winner as the other draft kernels.
#include "dspark_dev.h"
#include "dspark_host.h"
#include "gemv.h"
#include "mfma_common.h"

namespace dspark {

namespace {

constexpr int kGvThreads = 256;
constexpr int kGvPasses = 7;                       // 32 rows per pass (8 lanes per row)
constexpr int kGvRows = kGvPasses * 32;            // rows per chunk
// 168 VGPRs: three workgroups of four waves per CU, 768 on the chip, all resident
constexpr int kGvMaxWorkgroups = 768;

__device__ __forceinline__ int gv_prev(const int32_t* anchor, const int32_t* forced,
                                       const unsigned long long* best_prev, int b, int G,
                                       int k, int V) {
  if (k == 1) return clamp_tok(anchor[b], V);
  if (forced) return clamp_tok(forced[(size_t)b * G + (k - 2)], V);
  return clamp_tok((int)packed_index(best_prev[b]), V);
}

// grid (nwg, B); workgroup s covers rows [s * span, min(V, (s + 1) * span)) of request b,
// span a multiple of kGvRows
__global__ __launch_bounds__(kGvThreads, 3) void k_draft_gemv(
    const float* __restrict__ U, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ W2t, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ forced, const unsigned long long* __restrict__ best_prev,
    unsigned long long* __restrict__ best_cur, float2* __restrict__ part, int B, int G, int V,
    int k, float invT, uint32_t key0, uint32_t key1, int span) {
  __shared__ float bias_s[kGvRows];
  __shared__ float red[16];
  const int b = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
  const int sub = tid & 7, rowi = tid >> 3;
  const int v_lo = s * span, v_hi = min(V, v_lo + span);
  const float* Urow = U + ((size_t)b * G + (k - 1)) * V;
  const float s2 = invT * kLog2e;
  const PhiloxLane pl = philox_lane((uint32_t)k, (uint32_t)b, 0u, key0, key1);
  float m = kNegBig, l = 0.f, best_s = -INFINITY;
  uint32_t best_v = 0xFFFFFFFFu;
  bool have_w1 = false;
  uint32_t wp[16];   // this lane's 32 W1 entries as bf16 pairs (widened where used)
  for (int v0 = v_lo; v0 < v_hi; v0 += kGvRows) {
    // 1. the first pass of this chunk's W2t slices and its base-logit quad, 2. the
    //    conditioning token and this lane's 32 entries of its W1 row (first chunk only),
    //    3. the other passes: loads complete in issue order, so the dots of pass p wait
    //    for pass p (and W1) only, while the later passes are still streaming
    uint4 q[kGvPasses][4];
    auto load_pass = [&](int p) {
      const int v = min(v0 + p * 32 + rowi, V - 1);
      const uint4* src = reinterpret_cast<const uint4*>(W2t + (size_t)v * kR + sub * 32);
#pragma unroll
      for (int c = 0; c < 4; ++c) q[p][c] = src[c];
    };
    load_pass(0);
    const int vq = v0 + 4 * tid;                   // this thread's quad (tid < kGvRows / 4)
    const bool has_quad = tid < kGvRows / 4 && vq < v_hi;
    float4 uq = make_float4(0.f, 0.f, 0.f, 0.f);
    if (has_quad) uq = *reinterpret_cast<const float4*>(Urow + vq);
    if (!have_w1) {
      const int prev = gv_prev(anchor, forced, best_prev, b, G, k, V);
      const uint4* w1src = reinterpret_cast<const uint4*>(W1 + (size_t)prev * kR + sub * 32);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint4 e = w1src[c];
        wp[4 * c] = e.x;
        wp[4 * c + 1] = e.y;
        wp[4 * c + 2] = e.z;
        wp[4 * c + 3] = e.w;
      }
      have_w1 = true;
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 1; p < kGvPasses; ++p) load_pass(p);
    __builtin_amdgcn_sched_barrier(0);
    // 3. the bias of every row of the chunk (8 lanes per row, xor-combined)
#pragma unroll
    for (int p = 0; p < kGvPasses; ++p) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t e[4] = {q[p][c].x, q[p][c].y, q[p][c].z, q[p][c].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t w = wp[4 * c + j];
          acc = fmaf(__uint_as_float(w << 16), __uint_as_float(e[j] << 16), acc);
          acc = fmaf(__uint_as_float(w & 0xFFFF0000u), __uint_as_float(e[j] & 0xFFFF0000u),
                     acc);
        }
      }
      acc += __shfl_xor(acc, 1, kWave);
      acc += __shfl_xor(acc, 2, kWave);
      acc += __shfl_xor(acc, 4, kWave);
      if (sub == 0) bias_s[p * 32 + rowi] = acc;
    }
    __syncthreads();
    // 4. epilogue on the quad: base-2 logits, online (max, sum), Gumbel race
    if (has_quad) {
      const U4 w = philox_call((uint32_t)vq >> 2, pl);
      const float4 bq = *reinterpret_cast<const float4*>(bias_s + 4 * tid);
      const float z[4] = {(uq.x + bq.x) * s2, (uq.y + bq.y) * s2, (uq.z + bq.z) * s2,
                          (uq.w + bq.w) * s2};
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
      float qm = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      const float mn = fmaxf(m, qm);
      float add = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (vq + i >= v_hi) break;
        add += ex2(z[i] - mn);
        const float sc = z[i] + neg_lglg(wd[i]);
        if (sc > best_s) { best_s = sc; best_v = (uint32_t)(vq + i); }
      }
      l = l * ex2(m - mn) + add;
      m = mn;
    }
    __syncthreads();
  }
  // workgroup merge of (max, sum) in a fixed order, then of the candidates
  const int wv = tid >> 6, lane = tid & 63;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, kWave), ol = __shfl_xor(l, o, kWave);
    const float mn = fmaxf(m, om);
    l = l * ex2(m - mn) + ol * ex2(om - mn);
    m = mn;
    const float os = __shfl_xor(best_s, o, kWave);
    const uint32_t ov = (uint32_t)__shfl_xor((int)best_v, o, kWave);
    if (os > best_s || (os == best_s && ov < best_v)) { best_s = os; best_v = ov; }
  }
  if (lane == 0) {
    red[wv] = m;
    red[4 + wv] = l;
    red[8 + wv] = best_s;
    red[12 + wv] = __uint_as_float(best_v);
  }
  __syncthreads();
  if (tid == 0) {
    m = red[0];
    l = red[4];
    best_s = red[8];
    best_v = __float_as_uint(red[12]);
    for (int i = 1; i < 4; ++i) {
      const float mn = fmaxf(m, red[i]);
      l = l * ex2(m - mn) + red[4 + i] * ex2(red[i] - mn);
      m = mn;
      const uint32_t ov = __float_as_uint(red[12 + i]);
      if (red[8 + i] > best_s || (red[8 + i] == best_s && ov < best_v)) {
        best_s = red[8 + i];
        best_v = ov;
      }
    }
    part[(size_t)s * B + b] = make_float2(m, l);
    if (best_v != 0xFFFFFFFFu) atomic_max_u64(&best_cur[b], pack_score(best_s, best_v));
  }
}

}  // namespace

bool draft_gemv_supported(int B, int V, int r, int wdt) {
  return wdt == DSPARK_BF16 && r == kR && B < 32 && (V & 3) == 0;
}

GemvPlan draft_gemv_plan(int V) {
  const int chunks = (V + kGvRows - 1) / kGvRows;
  const int per = (chunks + kGvMaxWorkgroups - 1) / kGvMaxWorkgroups;   // chunks per workgroup
  GemvPlan p;
  p.span = per * kGvRows;
  p.nwg = (V + p.span - 1) / p.span;
  return p;
}

void launch_draft_gemv(const GemvPlan& p, const float* U, const uint16_t* W1,
                       const uint16_t* W2t, const int32_t* anchor, const int32_t* forced,
                       const unsigned long long* best_prev, unsigned long long* best_cur,
                       float2* part, int B, int G, int V, int k, float invT, uint32_t key0,
                       uint32_t key1, hipStream_t st) {
  hipLaunchKernelGGL(k_draft_gemv, dim3(p.nwg, B), dim3(kGvThreads), 0, st, U, W1, W2t, anchor,
                     forced, best_prev, best_cur, part, B, G, V, k, invT, key0, key1, p.span);
}

}  // namespace dspark
