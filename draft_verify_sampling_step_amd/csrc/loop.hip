// loop.hip -- a closed loop of DSpark rounds on one stream, with a synthetic Markov target
// standing in for the target model.  Per round t (no host synchronisation in between):
//   draft      gamma Markov-head positions from anchor_t            [CSDN Eq. 4; XTL §3-4]
//   confidence c_k = sigmoid(w . [h_k ; W1[x_{k-1}]])               [CSDN Eq. 7; XTL §5]
//   schedule   greedy prefix scheduler (or full block)              [XTL §6]
//              or its production form: top-K admission over the round's own confidences
//              with K = N - B of the greedy schedule made two rounds earlier, the greedy
//              schedule itself in rounds 0 and 1                     [XTL §7]
//   target     stand-in logits of positions 1..gamma+1 given the drafted block
//   verify     rejection sampling, residual or bonus token          [XTL §1; AIMSG 2]
//   anchor_{t+1} = the last token the round emitted (the corrected or bonus token),
// with the round's random numbers keyed by seed + t.  The accepted length per request and
// round, n + 1 tokens, is what the latency model per token, (T_draft + T_verify) / tau,
// divides by [CSDN Eq. 1].
//
// The stand-in target is a Markov chain over tokens: the logits of position j + 1 are the
// draft's base logits of position min(j + 1, gamma) plus sigma sqrt(3) (2 u - 1), with
// u = u(target_seed, prev, 0, 3, v) from the library's random-number definition keyed by
// the previous token prev -- a zero-mean transition term of variance sigma^2 that the
// draft does not model, so acceptance falls below one as sigma grows.
#include "dspark_dev.h"
#include "dspark_host.h"

size_t dspark_draft_workspace(const dspark_dims* d);
size_t dspark_verify_workspace(const dspark_dims* d);

namespace dspark {

constexpr int kTargetChunk = 256 * 4;   // vocab entries per workgroup of k_markov_target

// one workgroup per (row b*(G+1)+j, chunk of 1024 vocab entries); a thread writes 4
// consecutive entries from one Philox call (16-byte accesses when rows are 16-byte aligned)
template <bool VEC>
__global__ __launch_bounds__(256) void k_markov_target(const float* __restrict__ U,
                                                       const int32_t* __restrict__ anchor,
                                                       const int32_t* __restrict__ tokens,
                                                       int G, int V, int nchunk, float scale,
                                                       uint32_t key0, uint32_t key1,
                                                       float* __restrict__ T) {
  const int row = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
  const int b = row / (G + 1), j = row % (G + 1);
  const int prev = clamp_tok(j == 0 ? anchor[b] : tokens[(size_t)b * G + j - 1], V);
  const float* base = U + ((size_t)b * G + min(j, G - 1)) * V;
  float* out = T + (size_t)row * V;
  const int q = chunk * 256 + threadIdx.x;   // quad index: entries 4q..4q+3
  const int v0 = 4 * q;
  if (v0 >= V) return;
  const U4 w = philox10((uint32_t)q, 0u, (uint32_t)prev, 3u, key0, key1);
  // 2u - 1 is exact in fp32 (u is an odd multiple of 2^-24)
  const float n0 = scale * (2.f * word_to_uniform(w.x) - 1.f);
  const float n1 = scale * (2.f * word_to_uniform(w.y) - 1.f);
  const float n2 = scale * (2.f * word_to_uniform(w.z) - 1.f);
  const float n3 = scale * (2.f * word_to_uniform(w.w) - 1.f);
  if constexpr (VEC) {   // V % 4 == 0: the quad lies inside the row
    const float4 bv = *reinterpret_cast<const float4*>(base + v0);
    *reinterpret_cast<float4*>(out + v0) = make_float4(bv.x + n0, bv.y + n1, bv.z + n2, bv.w + n3);
  } else {
    const float nz[4] = {n0, n1, n2, n3};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (v0 + i < V) out[v0 + i] = base[v0 + i] + nz[i];
  }
}

// anchor of the next round: the token at index n_accept of the emitted block
__global__ __launch_bounds__(256) void k_next_anchor(const int32_t* __restrict__ n_accept,
                                                     const int32_t* __restrict__ out_tokens,
                                                     int B, int G, int32_t* __restrict__ next,
                                                     int32_t* __restrict__ log) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  int n = n_accept[b];
  n = n < 0 ? 0 : (n > G ? G : n);
  const int32_t y = out_tokens[(size_t)b * (G + 1) + n];
  next[b] = y;
  if (log) log[b] = y;
}

__global__ __launch_bounds__(256) void k_copy_i32(const int32_t* __restrict__ src, int n,
                                                  int32_t* __restrict__ dst) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

}  // namespace dspark

using namespace dspark;

namespace {

struct LoopWs {
  float* T;
  float* logp;
  float* lse;
  int32_t* anc;
  double* theta;
  int32_t* ell_g;     // delayed top-K: the round's greedy schedule (its N is kept)
  double* theta_g;
  int32_t* n_greedy;  // N of the greedy schedules of the last three rounds (ring)
  void* op;
  size_t op_bytes;
  size_t bytes;
};

LoopWs loop_ws(const dspark_dims* d, void* base) {
  const size_t B = d->batch, G = d->gamma, V = d->vocab;
  Carve c(base);
  LoopWs w;
  w.T = c.take<float>(B * (G + 1) * V);
  w.logp = c.take<float>(B * G);
  w.lse = c.take<float>(B * G);
  w.anc = c.take<int32_t>(B);
  w.theta = c.take<double>(1);
  w.ell_g = c.take<int32_t>(B);
  w.theta_g = c.take<double>(1);
  w.n_greedy = c.take<int32_t>(3);
  w.op_bytes = std::max(dspark_draft_workspace(d), dspark_verify_workspace(d));
  w.op = c.take<unsigned char>(w.op_bytes);
  w.bytes = align_up(c.off, 256);
  return w;
}

}  // namespace

namespace {
void launch_markov_target(const float* U, const int32_t* anchor, const int32_t* tokens, int B,
                          int G, int V, float scale, uint32_t tk0, uint32_t tk1, float* T,
                          hipStream_t st) {
  const int nchunk = (V + kTargetChunk - 1) / kTargetChunk;
  const size_t BG1 = (size_t)B * (G + 1);
  const bool vec = V % 4 == 0 && (uintptr_t)U % 16 == 0 && (uintptr_t)T % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(k_markov_target<true>, dim3((unsigned)(BG1 * nchunk)), dim3(256), 0, st,
                       U, anchor, tokens, G, V, nchunk, scale, tk0, tk1, T);
  else
    hipLaunchKernelGGL(k_markov_target<false>, dim3((unsigned)(BG1 * nchunk)), dim3(256), 0,
                       st, U, anchor, tokens, G, V, nchunk, scale, tk0, tk1, T);
}
}  // namespace

extern "C" dspark_status dspark_markov_target(const dspark_dims* dims, const float* U,
                                              const int32_t* anchor, const int32_t* tokens,
                                              float target_sigma, uint64_t target_seed,
                                              float* T, void* stream) {
  if (!dims || !U || !anchor || !tokens || !T) return DSPARK_E_NULL;
  if (!dims_ok(dims)) return DSPARK_E_SHAPE;
  if ((size_t)dims->batch * (dims->gamma + 1) * ((dims->vocab + kTargetChunk - 1) / kTargetChunk) >
      0x7FFFFFFFull)
    return DSPARK_E_SHAPE;
  if (!std::isfinite(target_sigma) || target_sigma < 0.f) return DSPARK_E_VALUE;
  launch_markov_target(U, anchor, tokens, dims->batch, dims->gamma, dims->vocab,
                       (float)((double)target_sigma * std::sqrt(3.0)), (uint32_t)target_seed,
                       (uint32_t)(target_seed >> 32), T, (hipStream_t)stream);
  return launch_status();
}

extern "C" size_t dspark_loop_workspace_bytes(const dspark_dims* dims) {
  if (!dims_ok(dims)) return 0;
  return loop_ws(dims, nullptr).bytes;
}

extern "C" dspark_status dspark_closed_loop(
    const dspark_dims* dims, const float* U, const void* W1, const void* W2t, int wdt,
    const void* h, int hdt, const void* w, int wvdt, const int32_t* anchor, const double* sps,
    int sched_mode, float temperature, uint64_t seed, float target_sigma, uint64_t target_seed,
    int32_t rounds, int32_t* anchors, int32_t* tokens, float* c, int32_t* ell, double* theta,
    int32_t* n_total, int32_t* n_accept, int32_t* out_tokens, float* pt_tok, void* ws,
    size_t ws_bytes, void* stream) {
  if (!dims || !U || !W1 || !W2t || !h || !w || !anchor || !sps || !tokens || !c || !ell ||
      !n_total || !n_accept || !out_tokens)
    return DSPARK_E_NULL;
  if (!dims_ok(dims) || rounds < 1 || rounds > 65536) return DSPARK_E_SHAPE;
  if ((long long)dims->batch * dims->gamma > kMaxSchedCandidates) return DSPARK_E_SHAPE;
  if (!dtype_ok(wdt) || !dtype_ok(hdt) || !dtype_ok(wvdt)) return DSPARK_E_DTYPE;
  if (!temp_ok(temperature) || !std::isfinite(target_sigma) || target_sigma < 0.f ||
      (sched_mode != DSPARK_SCHED_GREEDY && sched_mode != DSPARK_SCHED_FULL &&
       sched_mode != DSPARK_SCHED_TOPK_DELAYED))
    return DSPARK_E_VALUE;
  const LoopWs need = loop_ws(dims, nullptr);
  if (!ws || ws_bytes < need.bytes) return DSPARK_E_WORKSPACE;
  const LoopWs lw = loop_ws(dims, ws);
  // every kernel attribute the rounds need, before the first launch
  if (mfma_prepare() != DSPARK_OK || sched_prepare() != DSPARK_OK) return DSPARK_E_HIP;
  hipStream_t st = (hipStream_t)stream;
  const int B = dims->batch, G = dims->gamma, V = dims->vocab;
  const size_t BG = (size_t)B * G, BG1 = (size_t)B * (G + 1);
  if (BG1 * ((V + kTargetChunk - 1) / kTargetChunk) > 0x7FFFFFFFull) return DSPARK_E_SHAPE;
  const float scale = (float)((double)target_sigma * std::sqrt(3.0));
  const uint32_t tk0 = (uint32_t)target_seed, tk1 = (uint32_t)(target_seed >> 32);
  const unsigned bgrid = (unsigned)((B + 255) / 256);
  if (anchors) {
    hipLaunchKernelGGL(k_copy_i32, dim3(bgrid), dim3(256), 0, st, anchor, B, anchors);
    if (launch_status() != DSPARK_OK) return DSPARK_E_HIP;
  }
  for (int t = 0; t < rounds; ++t) {
    const int32_t* anc_t = t == 0 ? anchor : lw.anc;
    const uint64_t seed_t = seed + (uint64_t)t;
    int32_t* tok_t = tokens + (size_t)t * BG;
    float* c_t = c + (size_t)t * BG;
    int32_t* ell_t = ell + (size_t)t * B;
    int32_t* n_t = n_accept + (size_t)t * B;
    int32_t* out_t = out_tokens + (size_t)t * BG1;
    dspark_status s = dspark_draft_markov(dims, U, W1, W2t, wdt, anc_t, nullptr, temperature,
                                          seed_t, tok_t, lw.logp, lw.lse, lw.op, lw.op_bytes,
                                          stream);
    if (s != DSPARK_OK) return s;
    s = dspark_confidence(dims, h, hdt, W1, wdt, w, wvdt, anc_t, tok_t, c_t, stream);
    if (s != DSPARK_OK) return s;
    double* theta_t = theta ? theta + t : lw.theta;
    if (sched_mode == DSPARK_SCHED_TOPK_DELAYED) {
      // the greedy schedule of this round, kept for round t + 2; the admission takes K from
      // round t - 2's (from this round's own in rounds 0 and 1, which reproduces it)
      s = dspark_schedule(B, G, c_t, sps, DSPARK_SCHED_GREEDY, lw.ell_g, lw.theta_g,
                          lw.n_greedy + t % 3, nullptr, 0, stream);
      if (s != DSPARK_OK) return s;
      s = schedule_topk_from_history(B, G, c_t, sps, lw.n_greedy + (t >= 2 ? t - 2 : t) % 3,
                                     ell_t, theta_t, n_total + t, st);
    } else {
      s = dspark_schedule(B, G, c_t, sps, sched_mode, ell_t, theta_t, n_total + t, nullptr, 0,
                          stream);
    }
    if (s != DSPARK_OK) return s;
    launch_markov_target(U, anc_t, tok_t, B, G, V, scale, tk0, tk1, lw.T, st);
    if (launch_status() != DSPARK_OK) return DSPARK_E_HIP;
    s = dspark_verify(dims, U, W1, W2t, wdt, anc_t, tok_t, lw.logp, lw.lse, lw.T, ell_t,
                      temperature, seed_t, n_t, out_t, pt_tok ? pt_tok + (size_t)t * BG : nullptr,
                      lw.op, lw.op_bytes, stream);
    if (s != DSPARK_OK) return s;
    hipLaunchKernelGGL(k_next_anchor, dim3(bgrid), dim3(256), 0, st, n_t, out_t, B, G, lw.anc,
                       anchors && t + 1 < rounds ? anchors + (size_t)(t + 1) * B : nullptr);
    if (launch_status() != DSPARK_OK) return DSPARK_E_HIP;
  }
  return DSPARK_OK;
}
