// Auxiliary-loss-free bias update (DeepSeek-V3 notes page, "V3 improvement 1";
// DeepSeek-R1 analysis page, MoE hyper-parameters paragraph): every expert's
// bias moves by gamma against its load, the count of pairs the permute routed
// to it.  One thread per expert; the load is compared with the mean T*K/E
// exactly, as load*E against T*K in 64-bit integers.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void bias_update_kernel(const int32_t *__restrict__ counts,
                                                               int E, int64_t total, float gamma,
                                                               float *__restrict__ bias) {
  const int e = blockIdx.x * kThreads + threadIdx.x;
  if (e >= E) return;
  const int64_t scaled = static_cast<int64_t>(counts[e]) * E;
  if (scaled > total)
    bias[e] = bias[e] - gamma;
  else if (scaled < total)
    bias[e] = bias[e] + gamma;
  // at the mean the bias is left untouched (not even rewritten)
}

}  // namespace

hipError_t launch_bias_update(const moe_config &cfg, int64_t T, const moe_routing &r, float gamma,
                              float *bias, hipStream_t st) {
  const int E = cfg.n_routed;
  const dim3 grid(static_cast<unsigned>((E + kThreads - 1) / kThreads)), block(kThreads);
  hipLaunchKernelGGL(bias_update_kernel, grid, block, 0, st, r.counts, E, T * cfg.top_k, gamma, bias);
  return hipGetLastError();
}

}  // namespace moe
