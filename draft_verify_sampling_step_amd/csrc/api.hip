// api.hip -- library-wide entry points: workspace sizes, status names, version, and the
// generator check hook dspark_rng_uniforms.
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

}  // namespace dspark

using namespace dspark;

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
