// resident.h -- the draft for few requests with W2t kept on chip across the positions of a
// call (resident.hip).
#pragma once

#include "dspark_host.h"

namespace dspark {

// Most requests the resident draft takes (one 16-column MFMA block).
constexpr int kResMaxBatch = 16;
// Upper bound of its workgroup count (one per compute unit), for workspace sizing.
constexpr int kResMaxWorkgroups = 256;

struct ResidentPlan {
  bool ok;     // the device can run it for this shape
  int nwg;     // workgroups: one per compute unit, at most one per 16-row vocabulary block
};

// bf16 weights, r = 256, 1 <= B <= 16, V % 4 == 0, and the vocabulary fits the chip's
// registers and LDS at one resident workgroup per compute unit (cooperative launch).
ResidentPlan resident_plan(int B, int V, int r, int wdt);

// Sets the kernel's LDS attribute on the current device (before any launch of a call).
dspark_status resident_prepare();

// All G positions in one cooperative launch.  best [G][B] (packed winners), cnt
// [G][kArriveInts] (arrival counters), slot [G][B][nwg] (winner slots, one or two requests)
// and *fault must be zero before it; part is [G][nwg][B].
dspark_status launch_draft_resident(const ResidentPlan& p, const float* U, const uint16_t* W1,
                                    const uint16_t* W2t, const int32_t* anchor,
                                    const int32_t* forced, unsigned long long* best,
                                    float2* part, int32_t* cnt, unsigned long long* slot,
                                    uint32_t* fault, int B, int G, int V, float invT,
                                    uint32_t key0, uint32_t key1, hipStream_t st);

}  // namespace dspark
