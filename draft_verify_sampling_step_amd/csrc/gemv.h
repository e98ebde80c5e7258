// gemv.h -- the draft position kernel for one request with bf16 weights of rank 256
// (gemv.hip): one workgroup per contiguous vocabulary range and request.
#pragma once

#include "dspark_host.h"

namespace dspark {

struct GemvPlan {
  int span;   // vocabulary rows per workgroup (a multiple of the kernel's chunk)
  int nwg;    // workgroups per request (at most 1024)
};

// bf16 weights, r = 256, fewer than 32 requests, V % 4 == 0 (16-byte logit quads); the
// draft plan takes it for one request only
bool draft_gemv_supported(int B, int V, int r, int wdt);
GemvPlan draft_gemv_plan(int V);

// Same partial-slot ([nwg][B] base-2 (max, sum)) and packed-winner conventions as the
// other draft kernels.
void launch_draft_gemv(const GemvPlan& p, const float* U, const uint16_t* W1,
                       const uint16_t* W2t, const int32_t* anchor, const int32_t* forced,
                       const unsigned long long* best_prev, unsigned long long* best_cur,
                       float2* part, int B, int G, int V, int k, float invT, uint32_t key0,
                       uint32_t key1, hipStream_t st);

}  // namespace dspark
