// Uniforms from a seed: out[i] = top 24 bits of SplitMix64 output number
// counter0 + i, times 2^-24 (Steele, Lea & Flood, OOPSLA 2014).  The same
// counter form is evaluated inline by the sampling kernels when the caller
// passes no uniform array.
#include "device_common.h"

namespace specv {

__global__ __launch_bounds__(kThreads) void k_fill_uniforms(uint64_t seed, uint64_t ctr0,
                                                            int64_t n, float* __restrict__ out) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride)
    out[i] = splitmix_uniform(seed, ctr0 + (uint64_t)i);
}

hipError_t launch_fill_uniforms(uint64_t seed, uint64_t counter0, int64_t n, float* out,
                                hipStream_t s) {
  int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 65536) blocks = 65536;
  return launch_timed(kProfUniforms, &k_fill_uniforms, dim3((unsigned)blocks), dim3(kThreads), 0, s,
                      seed, counter0, n, out);
}

}  // namespace specv
