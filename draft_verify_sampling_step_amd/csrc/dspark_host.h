// dspark_host.h -- host-side helpers of the C ABI: validation, work partitioning and the
// workspace layout shared by the launchers and dspark_workspace_bytes().
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "dspark.h"

namespace dspark {

constexpr int kRowTile = 256;        // vocab rows per tile in the row (GEMV) kernels
constexpr int kMaxSchedCandidates = 4096;
// Calibration samples per call: the integer bin sums (p in 2^-40 units, labels shifted by
// 40 bits) then stay below 2^62.
constexpr int kMaxStsSamples = 1 << 22;

inline bool dims_ok(const dspark_dims* d) {
  return d && d->batch >= 1 && d->batch <= 65535 && d->gamma >= 1 && d->gamma <= 64 &&
         d->vocab >= 2 && d->vocab <= (1 << 28) && d->rank >= 8 && d->rank <= 1024 &&
         d->rank % 8 == 0 && d->hidden >= 0 && d->hidden <= 65536;
}
inline bool dtype_ok(int t) { return t == DSPARK_F32 || t == DSPARK_BF16; }
inline bool temp_ok(float t) { return isfinite(t) && t > 0.f; }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Row-path vocabulary slices: each workgroup of the row kernels covers `tiles` tiles of
// kRowTile entries of one row; the slice count keeps the grid near 2048 workgroups.
struct RowSlices { int len; int count; };
inline RowSlices row_slices(int V, long long rows) {
  const long long tiles = (V + kRowTile - 1) / kRowTile;
  long long per = (tiles * rows + 2047) / 2048;
  if (per < 1) per = 1;
  if (per > tiles) per = tiles;
  RowSlices s;
  s.len = (int)(per * kRowTile);
  s.count = (int)((V + s.len - 1) / s.len);
  return s;
}

// Vocabulary slices of the streaming (no-bias) row kernels over T.
inline RowSlices stream_slices(int V, long long rows) { return row_slices(V, rows); }

// MFMA path: vocab tiles of 32 rows, contiguous tile ranges per workgroup.
constexpr int kMfmaTile = 32;
inline int mfma_workgroups(int V) {
  const int tiles = (V + kMfmaTile - 1) / kMfmaTile;
  return tiles < 1024 ? tiles : 1024;
}

// Launch timing (api.hip): while enabled, prof_begin/prof_end bracket `launches`
// consecutive launches of one kernel with a pair of events on `st`; `positions` is the
// number of draft positions they covered (a negative count withdraws a begin whose launch
// was refused).
void prof_begin(hipStream_t st);
void prof_end(hipStream_t st, int positions, int launches);

// A kernel's dynamic-LDS limit raised to `bytes`, once per device (devices 0..63), safe to
// call from several host threads: the first caller on a device sets the attribute under a
// library-wide lock (api.hip), later calls read one atomic word.
struct LdsAttr {
  std::atomic<uint64_t> done{0};
  dspark_status ensure(const void* kernel, int bytes);
};

// Bounded cross-workgroup waits of the cooperative kernels (resident draft, training loss):
// the poll limit, and whether the completion a wait looks for is made unreachable (set
// only through dspark_test_wait_limit, to run the give-up path deterministically).
struct WaitPolicy {
  uint32_t limit;
  uint32_t unreachable;
};
WaitPolicy wait_policy();

// Every matrix-core kernel variant's LDS attribute set on the current device.  The entry
// points that may launch one call it after validating their arguments and before their
// first launch, so a refusal returns before anything is enqueued.
dspark_status mfma_prepare();
dspark_status draft16_prepare();
dspark_status sched_prepare();

// Top-K admission (the scheduler's production form) whose K is read on the device:
// n_hist[0] - B, n_hist being the N of a greedy schedule made earlier on the stream.
dspark_status schedule_topk_from_history(int B, int G, const float* c, const double* sps,
                                         const int32_t* n_hist, int32_t* ell, double* theta,
                                         int32_t* n_total, hipStream_t st);

inline dspark_status launch_status() {
  return hipGetLastError() == hipSuccess ? DSPARK_OK : DSPARK_E_HIP;
}

// Workspace carving: a bump allocator over the caller's buffer, 256-byte aligned.
struct Carve {
  char* base;
  size_t off = 0;
  explicit Carve(void* p) : base((char*)p) {}
  template <typename T> T* take(size_t n) {
    off = align_up(off, 256);
    T* p = (T*)(base ? base + off : nullptr);
    off += n * sizeof(T);
    return p;
  }
};

}  // namespace dspark
