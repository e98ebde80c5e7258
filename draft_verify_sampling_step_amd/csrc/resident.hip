// resident.hip -- the draft for few requests, with W2t held on chip for the whole call.
//
// The Markov bias of a position is W1[x_{k-1}] . W2t[v] for every vocabulary row v [XTL §4;
// CSDN Eq. 4], and W2t is the same matrix at every one of the gamma positions.  With few
// requests the position kernels are a stream of W2t (V x 512 bytes, 78 MB at V = 151936)
// per position; the request's own logit row is 0.6 MB.  MI355X has 512 KB of vector
// registers and 160 KB of LDS on each of its 256 compute units, so W2t fits on chip: this
// kernel reads it once per call and then, per position, only the logit rows and one W1 row
// per request.
//
// One cooperative launch runs all gamma positions:
//   - a workgroup per compute unit, four waves (one per SIMD, 512 registers each).  It owns
//     a contiguous range of 16-row vocabulary blocks.  The first 32 blocks of the range sit
//     in the waves' accumulation registers, 8 blocks (128 rows, 256 AGPRs) per wave, in the
//     MFMA A-operand layout; the rest sit in LDS in the pair layout of the other matrix-core
//     kernels;
//   - per position each lane loads the W1 row of its column's conditioning token (the B
//     operand; column = request = lane % 16, 16 B per k-step), each block is eight
//     v_mfma_f32_16x16x32_bf16 seeded with the base logits (so the result is U + bias), and
//     the epilogue is that of the position kernels: base-2 online (max, sum), one
//     Philox4x32-10 call per four consecutive rows, a Gumbel-max race, ties to the lowest
//     row;
//   - with four requests or fewer, most columns of the MFMA output are idle, so the logits
//     of the live columns go through LDS and the epilogue is spread over all 64 lanes;
//   - the workgroup writes its (max, sum) partial to slot w of the position and its packed
//     winner of each request to the request's 64-bit atomic max for the final merge.
//     Position k + 1 starts in a workgroup once every workgroup's winners of position k are
//     known to it, by one of two hand-offs (every read a device-scope load, so no cache
//     holds a stale copy, and no address is read by every thread of the chip):
//       * one or two requests: each workgroup also stores its winners to slots of its own
//         (zero = not yet written); every thread of the next position reads a share of the
//         slots until all are written, and the winners arrive with the poll;
//       * more requests: the workgroup waits for its winner atomics and counts itself in on
//         the position's two-level arrival counter; one lane polls the top count, then B
//         lanes read the winners into LDS;
//     the logits of position k + 1 are already in flight by then.  A teacher-forced draft
//     has no wait at all;
//   - every wait is bounded: a poll past its limit raises the fault word, every workgroup
//     leaves, and the final merge reports token -1 and NaN for the call.
// The final merge of the slots is the other draft paths' k_draft_final.
#include <atomic>

#include "dspark_dev.h"
#include "dspark_host.h"
#include "mfma_common.h"
#include "resident.h"

namespace dspark {

namespace {

constexpr int kResThreads = 256;                     // four waves, one per SIMD
constexpr int kResKS = kR / 32;                      // k-steps of 32
constexpr int kResRegBlocks = 8;                     // 16-row blocks per wave in AGPRs
constexpr int kResRegPerWg = 4 * kResRegBlocks;      // 32
constexpr int kResBlkBytes = 8 * kPairBytes;         // a 16-row block in LDS (8448 bytes)
constexpr int kResLdsBlocks = 8;                     // LDS blocks per workgroup at most
constexpr int kResLdsSlots = 2;                      // per wave (>= ceil(8 / 4), even)
constexpr int kResWaveBlocks = kResRegBlocks + kResLdsSlots;       // 10 blocks per wave
constexpr int kResSpreadMax = 4;                     // requests whose epilogue is spread
constexpr size_t kResOffMerge = (size_t)kResLdsBlocks * kResBlkBytes;
constexpr size_t kResMergeFloats = 2 * 4 * 16 * 4;   // [parity][wave][column][m, l, s, v]
constexpr size_t kResOffWin = kResOffMerge + kResMergeFloats * 4;   // [16] winners + flag
constexpr size_t kResOffZ = kResOffWin + 32 * 8;
// spread epilogue: [wave][column < 4][row < 16 * 10] logits of the live columns
constexpr size_t kResZFloats = (size_t)4 * kResSpreadMax * 16 * kResWaveBlocks;
constexpr size_t kResLds = kResOffZ + kResZFloats * 4;
constexpr uint32_t kResFaultCheck = 64;              // polls between looks at the fault word
static_assert(kResLds <= 160 * 1024, "LDS budget");
static_assert(kResLdsSlots * 4 >= kResLdsBlocks && kResLdsSlots % 2 == 0, "LDS slots");

struct ResArgs {
  const float* U;
  const uint16_t* W1;
  const uint16_t* W2t;
  const int32_t* anchor;
  const int32_t* forced;
  unsigned long long* best;   // [G][B]
  float2* part;               // [G][nwg][B]
  int32_t* cnt;               // [G][kArriveInts] arrival counters (more than 2 requests)
  unsigned long long* slot;   // [G][B][nwg] winners, nonzero once written (1 or 2)
  uint32_t* fault;
  int B, G, V, nwg;
  float invT;
  uint32_t key0, key1;
  uint32_t spin_limit;
  uint32_t unreachable;       // testing: no wait ever completes
};

// Both hand-offs leave the winners of position `pos` (0-based) in win[0 .. B-1] (LDS) for
// every thread of the workgroup.  False when the wait gave up (its poll limit ran out, or
// another workgroup's did); every thread takes the same decision.

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int o) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o, kWave);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, kWave);
  return ((unsigned long long)hi << 32) | lo;
}

// One or two requests: thread t serves request t / g and slots t % g + g i (g = 256 / B2,
// at most 256 / g slots each).
template <int B2>
__device__ bool res_wait_slots(const ResArgs& a, int pos, unsigned long long* win,
                               unsigned long long* red) {
  constexpr int g = kResThreads / B2;
  constexpr int NE = (kResMaxWorkgroups + g - 1) / g;
  static_assert(g >= kWave, "whole waves per request");
  const int t = threadIdx.x, c = t / g, sub = t % g;
  const bool live = c < a.B;
  const unsigned long long* sl = a.slot + ((size_t)pos * a.B + (live ? c : 0)) * a.nwg;
  unsigned long long mx = 0;
  uint32_t polls = 0;
  for (;;) {
    unsigned long long w[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      const int s = sub + g * i;
      w[i] = live && s < a.nwg
                 ? __hip_atomic_load(sl + s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                 : ~0ull;
    }
    bool missing = a.unreachable != 0u;
    mx = 0;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
      missing = missing || w[i] == 0ull;
      if (w[i] != ~0ull && w[i] > mx) mx = w[i];
    }
    if (!__syncthreads_or(missing)) break;
    ++polls;
    bool give_up = polls > a.spin_limit;
    if (polls % kResFaultCheck == 0 && t == 0)
      give_up = give_up ||
                __hip_atomic_load(a.fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u;
    if (__syncthreads_or(give_up)) {
      if (t == 0) __hip_atomic_store(a.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  // the maximum over each request's g threads: a fixed butterfly per wave, then its waves
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const unsigned long long ov = shfl_xor_u64(mx, o);
    if (ov > mx) mx = ov;
  }
  if ((t & (kWave - 1)) == 0) red[t / kWave] = mx;
  __syncthreads();
  if (t < a.B) {
    constexpr int WPR = g / kWave;   // waves per request
    unsigned long long m = red[t * WPR];
    for (int i = 1; i < WPR; ++i) m = red[t * WPR + i] > m ? red[t * WPR + i] : m;
    // a workgroup without a finite candidate posted 1 (below every candidate); the final
    // merge reports such a request from the atomic maximum
    win[t] = m;
  }
  __syncthreads();
  return true;
}

// More requests: lane 0 of wave 0 polls the top count of the position's two-level counter,
// then lanes 0 .. B-1 read the winners.
__device__ bool res_wait_count(const ResArgs& a, int pos, unsigned long long* win, int* flag) {
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int32_t* top = a.cnt + (size_t)pos * kArriveInts + 32 * kSubSlots;
    const int want = (a.nwg < kSubSlots ? a.nwg : kSubSlots) + (int)a.unreachable;
    int ok = 1;
    if (lane == 0) {
      uint32_t polls = 0;
      while (__hip_atomic_load(top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want) {
        ++polls;
        if (polls > a.spin_limit ||
            (polls % kResFaultCheck == 0 &&
             __hip_atomic_load(a.fault, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u)) {
          __hip_atomic_store(a.fault, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    ok = __shfl(ok, 0, kWave);
    if (ok && lane < a.B) win[lane] = atomic_load_u64(a.best + (size_t)pos * a.B + lane);
    if (lane == 0) *flag = ok;
  }
  __syncthreads();
  return *flag != 0;
}

// One base-2 epilogue step on four consecutive rows v0 .. v0 + 3 of one column (logits y,
// -inf past V) with their Philox words: online (max, sum) and the Gumbel-max race, ties to
// the lowest row.
struct ResState {
  float m, l, s;
  uint32_t v;
};

__device__ __forceinline__ void res_update(ResState& st, const float (&y)[4], const uint32_t (&wd)[4],
                                           int v0, float s2) {
  const float mx = fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3]));
  const float mnew = fmaxf(st.m, mx * s2);
  const float lp = (ex2(fmaf(y[0], s2, -mnew)) + ex2(fmaf(y[1], s2, -mnew))) +
                   (ex2(fmaf(y[2], s2, -mnew)) + ex2(fmaf(y[3], s2, -mnew)));
  st.l = st.l * ex2(st.m - mnew) + lp;
  st.m = mnew;
  float sc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) sc[i] = fmaf(y[i], s2, neg_lglg(wd[i]));
  // the higher row of a pair wins only when strictly greater
  const bool h01 = sc[1] > sc[0], h23 = sc[3] > sc[2];
  const float s01 = h01 ? sc[1] : sc[0], s23 = h23 ? sc[3] : sc[2];
  const int i01 = h01 ? 1 : 0, i23 = h23 ? 3 : 2;
  const bool hi = s23 > s01;
  const float bs = hi ? s23 : s01;
  if (bs > st.s) {
    st.s = bs;
    st.v = (uint32_t)(v0 + (hi ? i23 : i01));
  }
}

// merge of (max, sum) and candidate with the state of lane ^ o
__device__ __forceinline__ void res_merge_lanes(ResState& st, int o) {
  const float om = __shfl_xor(st.m, o, kWave);
  const float ol = __shfl_xor(st.l, o, kWave);
  const float os = __shfl_xor(st.s, o, kWave);
  const uint32_t ov = (uint32_t)__shfl_xor((int)st.v, o, kWave);
  const float mm = fmaxf(st.m, om);
  st.l = st.l * ex2(st.m - mm) + ol * ex2(om - mm);
  st.m = mm;
  if (os > st.s || (os == st.s && ov < st.v)) {
    st.s = os;
    st.v = ov;
  }
}

// B2: the power of two >= B (1 .. 16); SPREAD: B <= 4, epilogue over all lanes via LDS
template <int B2>
__global__ __launch_bounds__(kResThreads, 1) void k_draft_resident(const ResArgs a) {
  constexpr bool SPREAD = B2 <= kResSpreadMax;
  constexpr bool SLOTS = B2 <= 2;
  extern __shared__ __align__(16) unsigned char smem[];
  float* merge = reinterpret_cast<float*>(smem + kResOffMerge);
  unsigned long long* win = reinterpret_cast<unsigned long long*>(smem + kResOffWin);
  unsigned long long* red = win + 16;            // [4]
  int* flag = reinterpret_cast<int*>(win + 20);
  float* zbuf = reinterpret_cast<float*>(smem + kResOffZ);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, q = lane >> 4;
  const int B = a.B, G = a.G, V = a.V, wg = blockIdx.x;
  const bool live = n16 < B;
  const int col = live ? n16 : 0;   // idle columns compute on request 0 and never report
  const float s2 = a.invT * kLog2e;

  // ---- this workgroup's 16-row blocks [b0, b0 + nb): the first 32 in registers, eight per
  // wave; block b0 + 32 + j in LDS slot j, taken by wave j % 4
  const int nblk = (V + 15) >> 4;
  const int per = nblk / a.nwg, rem = nblk % a.nwg;
  const int b0 = wg * per + min(wg, rem);
  const int nb = per + (wg < rem ? 1 : 0);
  const int nreg = min(nb, kResRegPerWg);
  const int nlds = nb - nreg;
  const int cnt = max(0, min(kResRegBlocks, nreg - kResRegBlocks * wave));
  const int rblk0 = b0 + kResRegBlocks * wave;
  const int nmy = nlds > wave ? (nlds - wave + 3) / 4 : 0;
  // the wave's blocks in order: register blocks 0 .. cnt-1, then its LDS slots
  auto wave_block = [&](int jj) {
    return jj < cnt ? rblk0 + jj : b0 + kResRegPerWg + wave + 4 * (jj - cnt);
  };

  // ---- W2t into accumulation registers: A[j][kk] holds row 16 (rblk0 + j) + n16, entries
  // 32 kk + 8 q .. +7 (rows past V repeat row V - 1; their logits are -inf)
  u32x4_t A[kResRegBlocks][kResKS];
#pragma unroll
  for (int j = 0; j < kResRegBlocks; ++j) {
    if (j < cnt) {
      const int row = min(16 * (rblk0 + j) + n16, V - 1);
      const uint16_t* src = a.W2t + (size_t)row * kR + 8 * q;
#pragma unroll
      for (int kk = 0; kk < kResKS; ++kk) {
        A[j][kk] = *reinterpret_cast<const u32x4_t*>(src + 32 * kk);
        asm volatile("" : "+a"(A[j][kk]));
      }
    }
  }
  // ---- the remaining blocks into LDS: chunk c of row r at pair r/2, offset (2c + r%2) 16
  for (int j = 0; j < nlds; ++j) {
    const int row0 = 16 * (b0 + kResRegPerWg + j);
    for (int c = tid; c < 16 * 32; c += kResThreads) {
      const int r = c >> 5, ch = c & 31;
      const int row = min(row0 + r, V - 1);
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(a.W2t + (size_t)row * kR + ch * 8);
      *reinterpret_cast<u32x4_t*>(smem + (size_t)j * kResBlkBytes + (r >> 1) * kPairBytes +
                                  (2 * ch + (r & 1)) * 16) = v;
    }
  }
  __syncthreads();
  // lane's A-fragment offset within an LDS block: row n16, chunk 4 kk + q
  const int a_lane = (n16 >> 1) * kPairBytes + (2 * q + (n16 & 1)) * 16;

  // ---- base logits of a position in the output layout (column n16, rows 4q .. 4q + 3 of
  // each block); rows past V are replaced by -inf where they are used
  f32x4_t ur[kResRegBlocks], ul[kResLdsSlots];
  auto load_u = [&](int k, int blk) {
    const int v = min(16 * blk + 4 * q, V - 4);
    return __builtin_nontemporal_load(
        reinterpret_cast<const f32x4_t*>(a.U + ((size_t)col * G + (k - 1)) * V + v));
  };
  auto prefetch = [&](int k) {
#pragma unroll
    for (int j = 0; j < kResRegBlocks; ++j)
      if (j < cnt) ur[j] = load_u(k, rblk0 + j);
#pragma unroll
    for (int i = 0; i < kResLdsSlots; ++i)
      if (i < nmy) ul[i] = load_u(k, b0 + kResRegPerWg + wave + 4 * i);
  };
  prefetch(1);

  // spread epilogue: lane serves column sc_c (rows in groups of four), sc_g lanes a column
  constexpr int sc_g = kWave / (SPREAD ? B2 : 1);
  const int sc_c = SPREAD ? lane / sc_g : 0, sc_sub = lane % sc_g;
  float* zw = zbuf + (size_t)wave * kResSpreadMax * 16 * kResWaveBlocks;

  for (int k = 1; k <= G; ++k) {
    // ---- the lane's conditioning token: anchor, forced prefix, or position k-1's winner
    // (left in win[] by the poll at the end of the previous position)
    int prev;
    if (k == 1) prev = a.anchor[col];
    else if (a.forced) prev = a.forced[(size_t)col * G + (k - 2)];
    else prev = (int)packed_index(win[col]);
    prev = clamp_tok(prev, V);
    u32x4_t Bop[kResKS];
    {
      const uint16_t* w1 = a.W1 + (size_t)prev * kR + 8 * q;
#pragma unroll
      for (int kk = 0; kk < kResKS; ++kk)
        Bop[kk] = *reinterpret_cast<const u32x4_t*>(w1 + 32 * kk);
    }
    ResState st{kNegBig, 0.f, -INFINITY, 0xFFFFFFFFu};
    const PhiloxLane pl = philox_lane((uint32_t)k, (uint32_t)(SPREAD ? (sc_c < B ? sc_c : 0) : col),
                                      0u, a.key0, a.key1);

    // the logits of two blocks: in place (epilogue now) or into LDS (spread epilogue later)
    auto consume = [&](const f32x4_t& acc0, int jj0, const f32x4_t& acc1, int jj1, bool two) {
      const int v00 = 16 * wave_block(jj0) + 4 * q, v01 = 16 * wave_block(jj1) + 4 * q;
      if constexpr (SPREAD) {
        if (live) {
          float* z = zw + (size_t)n16 * 16 * kResWaveBlocks;
#pragma unroll
          for (int i = 0; i < 4; ++i) z[16 * jj0 + 4 * q + i] = v00 < V ? acc0[i] : -INFINITY;
          if (two) {
#pragma unroll
            for (int i = 0; i < 4; ++i) z[16 * jj1 + 4 * q + i] = v01 < V ? acc1[i] : -INFINITY;
          }
        }
      } else {
        uint32_t c0[2] = {(uint32_t)v00 >> 2, (uint32_t)v01 >> 2};
        uint32_t wd[2][4];
        philox_calls<2>(c0, pl, wd);
        float y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = v00 < V ? acc0[i] : -INFINITY;
        res_update(st, y, wd[0], v00, s2);
        if (two) {
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = v01 < V ? acc1[i] : -INFINITY;
          res_update(st, y, wd[1], v01, s2);
        }
      }
    };

    // ---- register blocks, four accumulation chains at a time
#pragma unroll
    for (int j = 0; j < kResRegBlocks; j += 4) {
      if (j < cnt) {
        f32x4_t acc[4] = {ur[j], ur[j + 1], ur[j + 2], ur[j + 3]};
#pragma unroll
        for (int kk = 0; kk < kResKS; ++kk)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (j + t < cnt)
              acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                  as_bf16x8(A[j + t][kk]), as_bf16x8(Bop[kk]), acc[t], 0, 0, 0);
        consume(acc[0], j, acc[1], j + 1, j + 1 < cnt);
        if (j + 2 < cnt) consume(acc[2], j + 2, acc[3], j + 3, j + 3 < cnt);
      }
    }
    // ---- LDS blocks, two at a time
#pragma unroll
    for (int i = 0; i < kResLdsSlots; i += 2) {
      if (i < nmy) {
        const bool two = i + 1 < nmy;
        const int j0 = wave + 4 * i, j1 = two ? j0 + 4 : j0;
        const unsigned char* A0 = smem + (size_t)j0 * kResBlkBytes + a_lane;
        const unsigned char* A1 = smem + (size_t)j1 * kResBlkBytes + a_lane;
        f32x4_t acc0 = ul[i], acc1 = ul[i + 1];
#pragma unroll
        for (int kk = 0; kk < kResKS; ++kk) {
          const u32x4_t f0 = *reinterpret_cast<const u32x4_t*>(A0 + kk * 128);
          const u32x4_t f1 = *reinterpret_cast<const u32x4_t*>(A1 + kk * 128);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f0), as_bf16x8(Bop[kk]),
                                                         acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(f1), as_bf16x8(Bop[kk]),
                                                         acc1, 0, 0, 0);
        }
        consume(acc0, cnt + i, acc1, cnt + i + 1, two);
      }
    }

    if constexpr (SPREAD) {
      // ---- the live columns' logits from LDS (written by this wave): lane serves rows
      // 4 qq .. 4 qq + 3 of column sc_c for qq = sc_sub, sc_sub + sc_g, ...
      const int nq = 4 * (cnt + nmy);
      if (sc_c < B) {
        const float* z = zw + (size_t)sc_c * 16 * kResWaveBlocks;
        for (int qq = sc_sub; qq < nq; qq += 2 * sc_g) {
          const bool two = qq + sc_g < nq;
          const int qa = qq, qb = two ? qq + sc_g : qq;
          const int va = 16 * wave_block(qa >> 2) + 4 * (qa & 3);
          const int vb = 16 * wave_block(qb >> 2) + 4 * (qb & 3);
          uint32_t c0[2] = {(uint32_t)va >> 2, (uint32_t)vb >> 2};
          uint32_t wd[2][4];
          philox_calls<2>(c0, pl, wd);
          const f32x4_t za = *reinterpret_cast<const f32x4_t*>(z + 4 * qa);
          float y[4] = {za[0], za[1], za[2], za[3]};
          res_update(st, y, wd[0], va, s2);
          if (two) {
            const f32x4_t zb = *reinterpret_cast<const f32x4_t*>(z + 4 * qb);
            float yb[4] = {zb[0], zb[1], zb[2], zb[3]};
            res_update(st, yb, wd[1], vb, s2);
          }
        }
      }
      // ---- merge the sc_g lanes of each column, a fixed butterfly
#pragma unroll
      for (int o = 1; o < sc_g; o <<= 1) res_merge_lanes(st, o);
    } else {
      // ---- merge the four row quads of each column (lanes n16 + 16 q)
      res_merge_lanes(st, 16);
      res_merge_lanes(st, 32);
    }
    float* mg = merge + (size_t)(k & 1) * 4 * 64;   // [wave][column][4], by position parity
    const bool writer = SPREAD ? (sc_sub == 0 && sc_c < B) : q == 0;
    const int wcol = SPREAD ? sc_c : n16;
    if (writer) {
      float* e = mg + (wave * 16 + wcol) * 4;
      e[0] = st.m;
      e[1] = st.l;
      e[2] = st.s;
      e[3] = __uint_as_float(st.v);
    }
    __syncthreads();
    // ---- the workgroup's state of each request, the waves merged in order
    if (wave == 0 && q == 0 && live) {
      float m = mg[n16 * 4], l = mg[n16 * 4 + 1], s = mg[n16 * 4 + 2];
      uint32_t v = __float_as_uint(mg[n16 * 4 + 3]);
      for (int w = 1; w < 4; ++w) {
        const float* e = mg + (w * 16 + n16) * 4;
        const float mm = fmaxf(m, e[0]);
        l = l * ex2(m - mm) + e[1] * ex2(e[0] - mm);
        m = mm;
        const uint32_t ev = __float_as_uint(e[3]);
        if (e[2] > s || (e[2] == s && ev < v)) {
          s = e[2];
          v = ev;
        }
      }
      a.part[((size_t)(k - 1) * a.nwg + wg) * B + n16] = make_float2(m, l);
      if (v != 0xFFFFFFFFu) atomic_max_u64(a.best + (size_t)(k - 1) * B + n16, pack_score(s, v));
      if (SLOTS && k < G && !a.forced)
        __hip_atomic_store(a.slot + ((size_t)(k - 1) * B + n16) * a.nwg + wg,
                           v != 0xFFFFFFFFu ? pack_score(s, v) : 1ull, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!SLOTS && wave == 0 && k < G && !a.forced) {
      // this wave's winner atomics are performed before the count (device-scope atomics,
      // at the device's coherence point in that order)
      __builtin_amdgcn_s_waitcnt(0);
      if (lane == 0) (void)arrive_last(a.cnt + (size_t)(k - 1) * kArriveInts, wg, a.nwg);
    }
    if (k < G) {
      prefetch(k + 1);
      if (!a.forced) {
        bool ok;
        if constexpr (SLOTS) ok = res_wait_slots<B2>(a, k - 1, win, red);
        else ok = res_wait_count(a, k - 1, win, flag);
        if (!ok) return;   // the call has failed; every workgroup leaves
      }
    }
  }
}

template <int B2>
LdsAttr& res_attr() {
  static LdsAttr attr;
  return attr;
}

template <int B2>
dspark_status res_prepare1() {
  return res_attr<B2>().ensure((const void*)k_draft_resident<B2>, (int)kResLds);
}

const void* res_kernel(int B) {
  return B <= 1 ? (const void*)k_draft_resident<1>
       : B <= 2 ? (const void*)k_draft_resident<2>
       : B <= 4 ? (const void*)k_draft_resident<4>
       : B <= 8 ? (const void*)k_draft_resident<8>
                : (const void*)k_draft_resident<16>;
}

// Compute units when the kernel can run one resident workgroup on each of them under a
// cooperative launch, else 0; looked up once per device.  Each entry holds the value + 1
// once known; a racing second lookup stores the same value.
constexpr int kResDevices = 64;
std::atomic<int> g_res_cap1[kResDevices];

int resident_capacity() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kResDevices) return 0;
  const int known = g_res_cap1[dev].load(std::memory_order_acquire);
  if (known > 0) return known - 1;
  int coop = 0, ncu = 0, per_cu = 0, cap = 0;
  // every variant has the same registers, LDS and workgroup shape
  if (res_prepare1<16>() == DSPARK_OK &&
      hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) == hipSuccess &&
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, res_kernel(16), kResThreads,
                                                   kResLds) == hipSuccess &&
      coop && per_cu >= 1)
    cap = std::min(ncu, kResMaxWorkgroups);
  (void)hipGetLastError();
  g_res_cap1[dev].store(cap + 1, std::memory_order_release);
  return cap;
}

}  // namespace

ResidentPlan resident_plan(int B, int V, int r, int wdt) {
  ResidentPlan p{false, 0};
  if (wdt != DSPARK_BF16 || r != kR || B < 1 || B > kResMaxBatch || (V & 3) != 0) return p;
  const int ncu = resident_capacity();
  if (ncu <= 0) return p;
  const int nblk = (V + 15) / 16;
  const int nwg = std::min(ncu, nblk);
  if ((nblk + nwg - 1) / nwg > kResRegPerWg + kResLdsBlocks) return p;
  p.ok = true;
  p.nwg = nwg;
  return p;
}

dspark_status resident_prepare() {
  if (res_prepare1<1>() != DSPARK_OK || res_prepare1<2>() != DSPARK_OK ||
      res_prepare1<4>() != DSPARK_OK || res_prepare1<8>() != DSPARK_OK ||
      res_prepare1<16>() != DSPARK_OK)
    return DSPARK_E_HIP;
  return DSPARK_OK;
}

dspark_status launch_draft_resident(const ResidentPlan& p, const float* U, const uint16_t* W1,
                                    const uint16_t* W2t, const int32_t* anchor,
                                    const int32_t* forced, unsigned long long* best,
                                    float2* part, int32_t* cnt, unsigned long long* slot,
                                    uint32_t* fault, int B, int G, int V, float invT,
                                    uint32_t key0, uint32_t key1, hipStream_t st) {
  ResArgs a;
  a.U = U; a.W1 = W1; a.W2t = W2t; a.anchor = anchor; a.forced = forced;
  a.best = best; a.part = part; a.cnt = cnt; a.slot = slot; a.fault = fault;
  a.B = B; a.G = G; a.V = V; a.nwg = p.nwg;
  a.invT = invT; a.key0 = key0; a.key1 = key1;
  const WaitPolicy wp = wait_policy();
  a.spin_limit = wp.limit;
  a.unreachable = wp.unreachable;
  void* args[] = {&a};
  if (hipLaunchCooperativeKernel(res_kernel(B), dim3((unsigned)p.nwg),
                                 dim3(kResThreads), args, (unsigned)kResLds, st) != hipSuccess) {
    (void)hipGetLastError();
    return DSPARK_E_HIP;
  }
  return DSPARK_OK;
}

}  // namespace dspark
