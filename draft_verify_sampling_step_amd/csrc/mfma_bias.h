// mfma_bias.h -- the batched Markov bias on bf16 matrix cores, fused with the per-element
// work that consumes it.
//
// For a set of columns c (a request b_c at a position k_c with conditioning token
// prev_c), the bias of every vocab row v is
//     bias[v][c] = sum_i W2t[v][i] * W1[prev_c][i]          ([XTL §4]: W1 embedding,
//                                                           W2 bias-free projection)
// i.e. the product of the streamed W2t [V][r] with the gathered W1 rows, a dense
// [V x r] x [r x ncols] contraction done with v_mfma_f32_32x32x16_bf16.  The bias never
// leaves registers: the epilogue of each 32 x 32 output tile reads the matching base
// logits (and target logits) and does one of
//   kModeDraft  z = (U + bias)/T; online (max, sum-exp); Gumbel-max race   [CSDN Eq. 4]
//   kModeResid  rho = max(0, p_t - p_d); Gumbel race on ln rho            (verification);
//               with at most thin_max rows to do, a thin path without matrix cores
//   kModeTV     sum_v min(p_d, p_t)                                      [CSDN Eq. 8]
//
// Layout (per workgroup of 4 waves): each wave keeps the gathered W1 rows of its column
// block in registers (the MFMA B operand).  Per step the workgroup stages the next
// 32-row W2t tile(s) and the matching 32-entry slices of every column's logit rows in
// LDS with coalesced 1 KB loads (one HBM read each, issued a step ahead), and the waves
// read their MFMA A fragments and epilogue operands from there.  Output lane l of a tile
// holds column l%32 and the vocab rows 8g + 4(l/32) + j (g, j < 4): four runs of four
// consecutive rows, which is exactly one Philox4x32 call per run.  The draft epilogue
// works in base 2 (z2 = z log2 e), branch-free.
#pragma once

#include "dspark_dev.h"
#include "dspark_host.h"

namespace dspark {

enum { kModeDraft = 0, kModeResid = 1, kModeTV = 2 };

struct MfmaBiasArgs {
  int mode;
  const float* U;
  const uint16_t* W1;
  const uint16_t* W2t;
  const int32_t* anchor;
  const int32_t* forced;                 // draft: teacher-forced prefix or NULL
  const int32_t* tokens;                 // resid/tv: drafted tokens [B][G]
  const unsigned long long* best_prev;   // draft: packed winners of position k-1
  unsigned long long* best_cur;          // draft: packed winners of position k (atomic max)
  float2* part;                          // draft: [slices][B] base-2 softmax state (max, sum)
  unsigned long long* res_best;          // resid: [kSubSlots][B][2] packed (score, index)
                                         //        winners of the residual race and of the
                                         //        p_t fallback race, zero before the launch
  int* res_arrive;                       // resid: kArriveInts arrival counters of this
                                         //        launch's workgroups, zero before it
  const int32_t* n_accept;               // resid: accepted prefix length per request
  int32_t* out_tokens;                   // resid: [B][G+1]; the last workgroup to finish
                                         //        writes each residual token at n_accept
  const float* T;                        // resid/tv: target logits [B][G+1][V]
  const float* lse_d;                    // resid/tv: draft lse [B][G]
  const float* lse_t_row;                // resid: lse of target row j_b [B]
  const int32_t* jrow;                   // resid: row j_b (1-based), 0 = no residual
  const float* lse_t;                    // tv: target lse [B][G]
  float* tv_part;                        // tv: [slices][B*G] partial sums of min(p_d, p_t)
  int B, G, V, r, k;
  float invT;
  uint32_t key0, key1;
  int ncols;                             // columns of this launch (<= 256)
  int col0;                              // first global column of this launch
  int thin_max;                          // resid: 1..thin_max residual rows take the
                                         //        thin path (16 lanes per row, no MFMA)
};

// Residual rows per launch that take the thin path of the residual mode.
constexpr int kResidThinMax = 2;

// The MFMA path handles bf16 weights with r = 256 (16 k-steps of 16), any column count: it
// streams W2t once per launch whatever the columns, where the row kernels stream it once
// per column (the draft of one request prefers its own kernels, see draft.hip).
inline bool mfma_bias_supported(int ncols, int r, int wdt) {
  return wdt == DSPARK_BF16 && r == 256 && ncols >= 1;
}

// Workgroups of one launch over V for `ncols` columns in `mode` (all resident at once).
int mfma_grid(int V, int ncols, int mode);

dspark_status launch_mfma_bias(const MfmaBiasArgs& a, int nwg, hipStream_t st);

// Columns per launch.  The TV pass runs 128 at a time: two workgroups then fit a CU (at 256
// only one does), which measured faster although W2t is streamed twice as often.
inline int mfma_column_group(int mode) { return mode == kModeTV ? 128 : 256; }

// Draft mode on 16-column waves (mfma16.hip): 33..256 columns, V % 4 == 0; same grid and
// partial-slot layout as the 32-column kernel.
bool draft16_supported(const MfmaBiasArgs& a);
dspark_status launch_draft16(const MfmaBiasArgs& a, int nwg, hipStream_t st);

}  // namespace dspark
