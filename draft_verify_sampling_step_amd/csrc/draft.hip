// draft.hip -- Markov-head draft step [CSDN Eq. 4; XTL §3-4]: gamma sequential positions,
// each a rank-r bias added to the backbone logits, a full-vocabulary softmax and a
// Gumbel-max draw.
//
// One launch per position; the launch boundary carries the device-wide dependency
// x_{k-1} -> bias of position k (on MI355X an in-kernel grid barrier, with the next
// position's independent loads prefetched across it, measured no faster).  Each workgroup
// covers a vocabulary slice for every request and reports
//   - its best Gumbel candidate as a packed (score, index) word through a 64-bit atomic
//     max per request (order-free, so the winner is deterministic), and
//   - its base-2 softmax state (max, sum) to a fixed slot.
// The next position decodes x_{k-1} from the atomic word.  After the last position one
// merge kernel reduces the slots in slice order into lse and log p_d(x_k) (the winner's
// logit is recomputed from U, W1 and W2t).
#include <mutex>

#include "dspark_dev.h"
#include "dspark_host.h"
#include "gemv.h"
#include "mfma_bias.h"
#include "mfma_common.h"
#include "resident.h"
#include "rowbias.h"

namespace dspark {

__global__ void k_fill_u64(unsigned long long* p, size_t n, unsigned long long v) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

// Token that position k conditions on: the anchor, the forced prefix, or the winner of
// position k-1 decoded from its packed atomic word.
__device__ __forceinline__ int draft_prev(const int32_t* anchor, const int32_t* forced,
                                          const unsigned long long* best_prev, int b, int G,
                                          int k, int V) {
  if (k == 1) return clamp_tok(anchor[b], V);
  if (forced) return clamp_tok(forced[(size_t)b * G + (k - 2)], V);
  return clamp_tok((int)packed_index(best_prev[b]), V);
}

// Row path: grid (slices, B), 256 threads.  A step covers four tiles (kRowTile rows each,
// biases in LDS); thread t then owns the four consecutive rows tile0 + 4t .. + 3, whose
// uniforms are the four words of one Philox call.  Base-2 logits z2 = z log2 e; the
// partial is (max z2, sum 2^(z2 - max)).
template <typename WT>
__global__ __launch_bounds__(256) void k_draft_row(
    const float* __restrict__ U, const WT* __restrict__ W1, const WT* __restrict__ W2t,
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ forced,
    const unsigned long long* __restrict__ best_prev, unsigned long long* __restrict__ best_cur,
    float2* __restrict__ part, int B, int G, int V, int r, int k, float invT, uint32_t key0,
    uint32_t key1, int slice_len) {
  extern __shared__ float smem[];
  float* w1s = smem;            // [r]
  float* bias_s = smem + r;     // [4 kRowTile]
  float* red = bias_s + 4 * kRowTile;   // [16]
  const int b = blockIdx.y, s = blockIdx.x, tid = threadIdx.x;
  const int v_begin = s * slice_len;   // a multiple of kRowTile
  const int v_end = min(V, v_begin + slice_len);
  const int prev = draft_prev(anchor, forced, best_prev, b, G, k, V);
  const float s2 = invT * 1.4426950408889634f;
  const PhiloxLane pl = philox_lane((uint32_t)k, (uint32_t)b, 0u, key0, key1);
  load_w1_row<WT>(W1, prev, r, w1s);
  __syncthreads();
  const float* Urow = U + ((size_t)b * G + (k - 1)) * V;
  float m = -3.0e38f, l = 0.f;
  Cand best{-INFINITY, 0xFFFFFFFFu, 0.f};
  for (int tile0 = v_begin; tile0 < v_end; tile0 += 4 * kRowTile) {
#pragma unroll 1
    for (int i = 0; i < 4; ++i)   // workgroup-uniform bound
      if (tile0 + i * kRowTile < v_end)
        row_bias_tile<WT>(W2t, w1s, bias_s + i * kRowTile, r, tile0 + i * kRowTile, v_end);
    __syncthreads();
    const int v0 = tile0 + 4 * tid;
    if (v0 < v_end) {
      const U4 w = philox_call((uint32_t)v0 >> 2, pl);
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
      const int n = min(4, v_end - v0);
      float z[4];
      float qm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[i] = i < n ? (Urow[v0 + i] + bias_s[4 * tid + i]) * s2 : -INFINITY;
        qm = fmaxf(qm, z[i]);
      }
      const float mn = fmaxf(m, qm);
      float add = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= n) break;
        add += __builtin_amdgcn_exp2f(z[i] - mn);
        const float score = z[i] + neg_lglg(wd[i]);
        if (score > best.s) best = Cand{score, (uint32_t)(v0 + i), 0.f};
      }
      l = l * __builtin_amdgcn_exp2f(m - mn) + add;
      m = mn;
    }
    __syncthreads();
  }
  // workgroup merge of the base-2 state, then of the candidates
  {
    const int wv = tid >> 6, lane = tid & 63;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float om = __shfl_xor(m, o, kWave), ol = __shfl_xor(l, o, kWave);
      const float mn = fmaxf(m, om);
      l = l * __builtin_amdgcn_exp2f(m - mn) + ol * __builtin_amdgcn_exp2f(om - mn);
      m = mn;
    }
    if (lane == 0) { red[wv] = m; red[4 + wv] = l; }
    __syncthreads();
    m = red[0];
    l = red[4];
    for (int i = 1; i < 4; ++i) {
      const float mn = fmaxf(m, red[i]);
      l = l * __builtin_amdgcn_exp2f(m - mn) + red[4 + i] * __builtin_amdgcn_exp2f(red[i] - mn);
      m = mn;
    }
    __syncthreads();
  }
  best = block_cand(best, red + 8, reinterpret_cast<uint32_t*>(red + 12), red + 4);
  if (tid == 0) {
    part[(size_t)s * B + b] = make_float2(m, l);
    if (best.i != 0xFFFFFFFFu) atomic_max_u64(&best_cur[b], pack_score(best.s, best.i));
  }
}

// Final merge: one workgroup of four waves per (position, 8 consecutive requests).  Lane
// (i, p) = (l % 8, l / 8) of wave w takes request b0 + i and merges, in order, the base-2
// states of the slots 8 w + p + 32 j, j = 0, 1, ...; one load instruction thus reads eight
// slots of 64 contiguous bytes each (the slots are [slots][B]).  The 32 phases are combined
// by a fixed butterfly over the lanes and then over the waves, in wave order.  The winner's
// logit z_x = (U[x] + W1[prev] . W2t[x]) / T is recomputed with the rank split the same way.
template <typename WT>
__global__ __launch_bounds__(256) void k_draft_final(
    const float2* __restrict__ part, const unsigned long long* __restrict__ best,
    const float* __restrict__ U, const WT* __restrict__ W1, const WT* __restrict__ W2t,
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ forced, int B, int G, int V,
    int r, float invT, int nslices, const uint32_t* __restrict__ fault,
    int32_t* __restrict__ tokens, float* __restrict__ logp, float* __restrict__ lse) {
  __shared__ float red[4][8][3];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int noct = (B + 7) / 8;
  const int kk = blockIdx.x / noct, i8 = lane & 7, ph = 8 * wv + (lane >> 3);
  const int b = (blockIdx.x % noct) * 8 + i8;
  const bool live = b < B;
  const int bb = live ? b : B - 1;   // lanes past B work on a valid request, report nothing
  const float2* pp = part + (size_t)kk * nslices * B + bb;
  float m = -3.0e38f, l = 0.f;
#pragma unroll 4
  for (int s = ph; s < nslices; s += 32) {
    const float2 q = pp[(size_t)s * B];
    const float mn = fmaxf(m, q.x);
    l = l * __builtin_amdgcn_exp2f(m - mn) + q.y * __builtin_amdgcn_exp2f(q.x - mn);
    m = mn;
  }
  const uint32_t idx = packed_index(best[(size_t)kk * B + bb]);
  const bool won = idx < (uint32_t)V;   // false only if no candidate had a finite score
  const int x = won ? (int)idx : 0;
  const int prev = draft_prev(anchor, forced, kk > 0 ? best + (size_t)(kk - 1) * B : nullptr,
                              bb, G, kk + 1, V);
  const float ux = U[((size_t)bb * G + kk) * V + x];   // issued with the dot's loads
  float dot = 0.f;
  for (int i = ph; i < r; i += 32)
    dot = fmaf(Elem<WT>::get(W1, (size_t)prev * r + i), Elem<WT>::get(W2t, (size_t)x * r + i),
               dot);
#pragma unroll
  for (int o = 8; o < 64; o <<= 1) {
    const float om = __shfl_xor(m, o, kWave), ol = __shfl_xor(l, o, kWave);
    const float mn = fmaxf(m, om);
    l = l * __builtin_amdgcn_exp2f(m - mn) + ol * __builtin_amdgcn_exp2f(om - mn);
    m = mn;
    dot += __shfl_xor(dot, o, kWave);
  }
  if (lane < 8) {
    red[wv][i8][0] = m;
    red[wv][i8][1] = l;
    red[wv][i8][2] = dot;
  }
  __syncthreads();
  if (wv != 0 || lane >= 8 || !live) return;
  for (int w = 1; w < 4; ++w) {
    const float om = red[w][i8][0], ol = red[w][i8][1];
    const float mn = fmaxf(m, om);
    l = l * __builtin_amdgcn_exp2f(m - mn) + ol * __builtin_amdgcn_exp2f(om - mn);
    m = mn;
    dot += red[w][i8][2];
  }
  const float lz = (m + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
  const float zx = (ux + dot) * invT;
  const size_t o = (size_t)b * G + kk;
  // a draft kernel that gave up a bounded wait has left the slots incomplete
  const bool failed =
      fault && __hip_atomic_load(fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
  tokens[o] = won && !failed ? (int32_t)idx : -1;
  lse[o] = failed ? __builtin_nanf("") : lz;
  logp[o] = won && !failed ? zx - lz : __builtin_nanf("");
}

}  // namespace dspark

using namespace dspark;

namespace {

struct DraftPlan {
  bool mfma;
  bool resident;   // all positions in one launch, W2t on chip (resident.hip)
  bool gemv;       // the streaming kernel for few requests (gemv.hip)
  int nslices;     // partial slots per (position, request)
  int slice_len;   // row path only
  GemvPlan gp;
  ResidentPlan rp;
};

DraftPlan draft_plan(const dspark_dims* d, int wdt) {
  DraftPlan p{};
  // up to 16 requests: W2t resident across the positions; one request beyond the resident
  // kernel's vocabulary: the streaming kernel; else the matrix-core kernels, which stream
  // W2t once per position for all requests (the streaming kernel streams it per request)
  p.rp = resident_plan(d->batch, d->vocab, d->rank, wdt);
  p.resident = p.rp.ok;
  p.gemv = !p.resident && d->batch == 1 &&
           draft_gemv_supported(d->batch, d->vocab, d->rank, wdt);
  p.mfma = !p.resident && !p.gemv && mfma_bias_supported(d->batch, d->rank, wdt);
  if (p.mfma) {
    p.nslices = mfma_grid(d->vocab, d->batch, kModeDraft);
    p.slice_len = 0;
  } else if (p.resident) {
    p.nslices = p.rp.nwg;
    p.slice_len = 0;
  } else if (p.gemv) {
    p.gp = draft_gemv_plan(d->vocab);
    p.nslices = p.gp.nwg;
    p.slice_len = p.gp.span;
  } else {
    RowSlices s = row_slices(d->vocab, d->batch);
    p.nslices = s.count;
    p.slice_len = s.len;
  }
  return p;
}

// Scratch of a draft call: the packed winners [G][B], then the resident kernel's arrival
// counters [G][kArriveInts], winner slots [G][B][nres] and fault word, all cleared by one
// fill (in that order, contiguous, `nclear` 64-bit words; the counters and slots only when
// the resident kernel runs, nres > 0), then the softmax partials [G][nslices][B].
struct DraftWs {
  unsigned long long* best;
  int32_t* cnt;
  unsigned long long* slot;
  uint32_t* fault;
  float2* part;
  size_t nclear;
  size_t bytes;
};

DraftWs draft_ws(const dspark_dims* d, int nslices, int nres, void* base) {
  DraftWs w;
  Carve c(base);
  const size_t G = (size_t)d->gamma, B = (size_t)d->batch;
  static_assert(kArriveInts % 2 == 0, "counters pack into 64-bit words");
  const size_t ncnt = nres > 0 ? G * kArriveInts : 0;
  const size_t nslot = G * B * (size_t)nres;
  w.nclear = G * B + ncnt / 2 + nslot + 1;
  w.best = c.take<unsigned long long>(w.nclear);
  w.cnt = w.best ? reinterpret_cast<int32_t*>(w.best + G * B) : nullptr;
  w.slot = w.cnt ? reinterpret_cast<unsigned long long*>(w.cnt + ncnt) : nullptr;
  w.fault = w.slot ? reinterpret_cast<uint32_t*>(w.slot + nslot) : nullptr;
  w.part = c.take<float2>(G * nslices * B);
  w.bytes = align_up(c.off, 256);
  return w;
}

}  // namespace

size_t dspark_draft_workspace(const dspark_dims* d) {
  int ns = std::max(row_slices(d->vocab, d->batch).count, mfma_workgroups(d->vocab));
  const int nres =
      d->batch <= kResMaxBatch ? std::min((d->vocab + 15) / 16, kResMaxWorkgroups) : 0;
  return draft_ws(d, std::max(ns, nres), nres, nullptr).bytes;
}

namespace {

// The draft with its scratch (packed winners and softmax partials) at `ws`, which holds at
// least draft_ws(dm, plan.nslices) bytes; arguments already validated.
dspark_status draft_run(const dspark_dims* dm, const DraftPlan& plan, const float* U,
                        const void* W1, const void* W2t, int wdt, const int32_t* anchor,
                        const int32_t* forced, float temperature, uint64_t seed,
                        int32_t* tokens, float* logp, float* lse, void* ws, hipStream_t st) {
  const int B = dm->batch, G = dm->gamma, V = dm->vocab, r = dm->rank;
  const DraftWs w = draft_ws(dm, plan.nslices, plan.resident ? plan.nslices : 0, ws);
  unsigned long long* best = w.best;
  float2* part = w.part;
  const float invT = 1.0f / temperature;
  const uint32_t key0 = (uint32_t)seed, key1 = (uint32_t)(seed >> 32);
  if (plan.mfma && mfma_prepare() != DSPARK_OK) return DSPARK_E_HIP;
  if (plan.resident && resident_prepare() != DSPARK_OK) return DSPARK_E_HIP;

  // the winners (zero is below every packed candidate), arrival counters and fault word
  // start at zero on every call
  hipLaunchKernelGGL(k_fill_u64, dim3((unsigned)std::min<size_t>(1024, (w.nclear + 255) / 256)),
                     dim3(256), 0, st, best, w.nclear, 0ull);
  if (plan.resident) {
    prof_begin(st);
    const dspark_status ls =
        launch_draft_resident(plan.rp, U, (const uint16_t*)W1, (const uint16_t*)W2t, anchor,
                              forced, best, part, w.cnt, w.slot, w.fault, B, G, V, invT, key0,
                              key1, st);
    prof_end(st, ls == DSPARK_OK ? G : -1, 1);
    if (ls != DSPARK_OK) return DSPARK_E_HIP;
  }
  // one timing span over the G position launches (they run back to back on `st`)
  if (!plan.resident) prof_begin(st);
  for (int k = 1; k <= G && !plan.resident; ++k) {
    const unsigned long long* bprev = k > 1 ? best + (size_t)(k - 2) * B : nullptr;
    unsigned long long* bcur = best + (size_t)(k - 1) * B;
    float2* pk = part + (size_t)(k - 1) * plan.nslices * B;
    if (plan.mfma) {
      MfmaBiasArgs a{};
      a.mode = kModeDraft;
      a.U = U; a.W1 = (const uint16_t*)W1; a.W2t = (const uint16_t*)W2t;
      a.anchor = anchor; a.forced = forced; a.best_prev = bprev; a.best_cur = bcur;
      a.part = pk;
      a.B = B; a.G = G; a.V = V; a.r = r; a.k = k; a.invT = invT; a.key0 = key0; a.key1 = key1;
      a.ncols = B;
      const dspark_status ls = launch_mfma_bias(a, plan.nslices, st);
      if (ls != DSPARK_OK) {
        prof_end(st, -1, 0);
        return DSPARK_E_HIP;
      }
    } else if (plan.gemv) {
      launch_draft_gemv(plan.gp, U, (const uint16_t*)W1, (const uint16_t*)W2t, anchor, forced,
                        bprev, bcur, pk, B, G, V, k, invT, key0, key1, st);
    } else {
      const size_t sh = sizeof(float) * (r + 4 * kRowTile + 16);
      dim3 grid(plan.nslices, B);
      if (wdt == DSPARK_BF16)
        hipLaunchKernelGGL(k_draft_row<uint16_t>, grid, dim3(256), sh, st, U,
                           (const uint16_t*)W1, (const uint16_t*)W2t, anchor, forced, bprev,
                           bcur, pk, B, G, V, r, k, invT, key0, key1, plan.slice_len);
      else
        hipLaunchKernelGGL(k_draft_row<float>, grid, dim3(256), sh, st, U, (const float*)W1,
                           (const float*)W2t, anchor, forced, bprev, bcur, pk, B, G, V, r, k,
                           invT, key0, key1, plan.slice_len);
    }
  }
  if (!plan.resident) prof_end(st, G, G);
  const int fblocks = G * ((B + 7) / 8);   // one workgroup per (position, 8 requests)
  if (wdt == DSPARK_BF16)
    hipLaunchKernelGGL(k_draft_final<uint16_t>, dim3(fblocks), dim3(256), 0, st, part,
                       best, U, (const uint16_t*)W1, (const uint16_t*)W2t, anchor, forced, B, G,
                       V, r, invT, plan.nslices, plan.resident ? w.fault : nullptr, tokens,
                       logp, lse);
  else
    hipLaunchKernelGGL(k_draft_final<float>, dim3(fblocks), dim3(256), 0, st, part, best,
                       U, (const float*)W1, (const float*)W2t, anchor, forced, B, G, V, r, invT,
                       plan.nslices, nullptr, tokens, logp, lse);
  return launch_status();
}

dspark_status draft_validate(const dspark_dims* dm, const float* U, const void* W1,
                             const void* W2t, int wdt, const int32_t* anchor, int32_t* tokens,
                             float* logp, float* lse, float temperature) {
  if (!dm || !U || !W1 || !W2t || !anchor || !tokens || !logp || !lse) return DSPARK_E_NULL;
  if (!dims_ok(dm)) return DSPARK_E_SHAPE;
  if (!dtype_ok(wdt)) return DSPARK_E_DTYPE;
  if (!temp_ok(temperature)) return DSPARK_E_VALUE;
  return DSPARK_OK;
}

// ---- the variant that allocates nothing: its scratch is this file's device array ----
// Each device holds its own copy of `scratch` for the life of the process; the host never
// uses the name itself as an address, only the device address looked up once per device.
constexpr size_t kDraftStaticScratch = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kDraftStaticScratch];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];

dspark_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
    return DSPARK_E_HIP;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return DSPARK_E_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSPARK_OK;
}

}  // namespace

extern "C" dspark_status dspark_draft_markov(const dspark_dims* dm, const float* U,
                                             const void* W1, const void* W2t, int wdt,
                                             const int32_t* anchor, const int32_t* forced,
                                             float temperature, uint64_t seed,
                                             int32_t* tokens, float* logp, float* lse,
                                             void* ws, size_t ws_bytes, void* stream) {
  const dspark_status v =
      draft_validate(dm, U, W1, W2t, wdt, anchor, tokens, logp, lse, temperature);
  if (v != DSPARK_OK) return v;
  if (!ws || ws_bytes < dspark_draft_workspace(dm)) return DSPARK_E_WORKSPACE;
  return draft_run(dm, draft_plan(dm, wdt), U, W1, W2t, wdt, anchor, forced, temperature,
                   seed, tokens, logp, lse, ws, (hipStream_t)stream);
}

extern "C" dspark_status dspark_draft_markov_noalloc(const dspark_dims* dm, const float* U,
                                                     const void* W1, const void* W2t, int wdt,
                                                     const int32_t* anchor,
                                                     const int32_t* forced, float temperature,
                                                     uint64_t seed, int32_t* tokens,
                                                     float* logp, float* lse, void* stream) {
  const dspark_status v =
      draft_validate(dm, U, W1, W2t, wdt, anchor, tokens, logp, lse, temperature);
  if (v != DSPARK_OK) return v;
  const DraftPlan plan = draft_plan(dm, wdt);
  if (draft_ws(dm, plan.nslices, plan.resident ? plan.nslices : 0, nullptr).bytes >
      kDraftStaticScratch)
    return DSPARK_E_WORKSPACE;
  void* ws = nullptr;
  const dspark_status sc = static_scratch(&ws);
  if (sc != DSPARK_OK) return sc;
  return draft_run(dm, plan, U, W1, W2t, wdt, anchor, forced, temperature, seed, tokens, logp,
                   lse, ws, (hipStream_t)stream);
}
