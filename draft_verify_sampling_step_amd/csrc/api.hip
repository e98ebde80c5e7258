// api.hip -- library-wide entry points: workspace sizes, status names, version, the
// generator check hook dspark_rng_uniforms and the launch-timing switch.
#include <vector>

#include "dspark_dev.h"
#include "dspark_host.h"

size_t dspark_draft_workspace(const dspark_dims* d);
size_t dspark_verify_workspace(const dspark_dims* d);
size_t dspark_tv_workspace(const dspark_dims* d);

namespace dspark {

__global__ void k_rng_uniforms(uint32_t key0, uint32_t key1, uint32_t b, uint32_t k,
                               uint32_t s, uint32_t v0, int64_t n, float* __restrict__ out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t v = v0 + (uint32_t)i;
    const U4 w = philox10(v >> 2, k, b, s, key0, key1);
    const uint32_t word = (v & 3) == 0 ? w.x : (v & 3) == 1 ? w.y : (v & 3) == 2 ? w.z : w.w;
    out[i] = word_to_uniform(word);
  }
}

// Launch timing: while enabled, the draft records a HIP event pair around each of its
// per-position kernels on the caller's stream (measurement only; not thread-safe).
namespace {
bool g_prof_on = false;
int g_prof_n = 0;              // events recorded (pairs are complete when even)
long long g_prof_positions = 0;
std::vector<hipEvent_t> g_prof_ev;
}  // namespace

void prof_begin(hipStream_t st) {
  if (!g_prof_on || g_prof_n + 2 > (int)g_prof_ev.size()) return;
  (void)hipEventRecord(g_prof_ev[g_prof_n++], st);
}

void prof_end(hipStream_t st, int positions) {
  if (!g_prof_on || (g_prof_n & 1) == 0) return;
  if (positions < 0) {   // the launch was refused: drop its begin event
    --g_prof_n;
    return;
  }
  (void)hipEventRecord(g_prof_ev[g_prof_n++], st);
  g_prof_positions += positions;
}

}  // namespace dspark

using namespace dspark;

extern "C" dspark_status dspark_profile_start(int max_launches) {
  if (max_launches < 1 || max_launches > (1 << 16)) return DSPARK_E_VALUE;
  const size_t need = 2 * (size_t)max_launches;
  while (g_prof_ev.size() < need) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return DSPARK_E_HIP;
    g_prof_ev.push_back(e);
  }
  g_prof_n = 0;
  g_prof_positions = 0;
  g_prof_on = true;
  return DSPARK_OK;
}

extern "C" dspark_status dspark_profile_stop(double* mean_ms, int* launches,
                                           double* positions_per_launch) {
  if (!mean_ms || !launches || !positions_per_launch) return DSPARK_E_NULL;
  g_prof_on = false;
  const int pairs = g_prof_n / 2;
  double total = 0.0;
  for (int i = 0; i < pairs; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(g_prof_ev[2 * i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, g_prof_ev[2 * i], g_prof_ev[2 * i + 1]) != hipSuccess)
      return DSPARK_E_HIP;
    total += ms;
  }
  *launches = pairs;
  *mean_ms = pairs ? total / pairs : 0.0;
  *positions_per_launch = pairs ? (double)g_prof_positions / pairs : 0.0;
  g_prof_n = 0;
  g_prof_positions = 0;
  return DSPARK_OK;
}

extern "C" size_t dspark_workspace_bytes(int op, const dspark_dims* d) {
  switch (op) {
    case DSPARK_OP_DRAFT: return dims_ok(d) ? dspark_draft_workspace(d) : 0;
    case DSPARK_OP_CONFIDENCE: return 0;
    case DSPARK_OP_SCHEDULE: return 0;
    case DSPARK_OP_VERIFY: return dims_ok(d) ? dspark_verify_workspace(d) : 0;
    case DSPARK_OP_TV: return dims_ok(d) ? dspark_tv_workspace(d) : 0;
    default: return 0;
  }
}

extern "C" const char* dspark_status_string(int s) {
  switch (s) {
    case DSPARK_OK: return "DSPARK_OK";
    case DSPARK_E_NULL: return "DSPARK_E_NULL: a required pointer is NULL";
    case DSPARK_E_SHAPE: return "DSPARK_E_SHAPE: dimension out of the supported range";
    case DSPARK_E_DTYPE: return "DSPARK_E_DTYPE: unknown dtype code";
    case DSPARK_E_VALUE: return "DSPARK_E_VALUE: invalid temperature or scheduler mode";
    case DSPARK_E_WORKSPACE: return "DSPARK_E_WORKSPACE: workspace missing or too small";
    case DSPARK_E_HIP: return "DSPARK_E_HIP: the HIP runtime refused a launch";
    default: return "DSPARK_E_UNKNOWN";
  }
}

extern "C" int dspark_version(void) { return 100; }

extern "C" dspark_status dspark_rng_uniforms(uint64_t seed, uint32_t b, uint32_t k, uint32_t s,
                                             uint32_t v0, int64_t n, float* out,
                                             void* stream) {
  if (!out) return DSPARK_E_NULL;
  if (n < 0 || n > ((int64_t)1 << 32)) return DSPARK_E_SHAPE;
  if (n == 0) return DSPARK_OK;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(k_rng_uniforms, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (uint32_t)seed, (uint32_t)(seed >> 32), b, k, s, v0, n, out);
  return launch_status();
}
