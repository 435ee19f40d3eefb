// Sequence-wise balance loss (DeepSeek-V3 notes page, "V3 improvement 2"; the
// paper's eqs. 17-20): for each sequence of seq_len tokens
//     L = alpha * sum_i f_i P_i,   f_i = E/(K seq_len) * (tokens choosing expert i),
//     P_i = (1/seq_len) * sum_t s_{i,t} / sum_j s_{j,t},
// with s the gate's unbiased score (sigmoid of the logit, or the softmax
// probability) and the choices read from topk_idx.
//
// One workgroup per sequence.  Counts go into an LDS histogram with integer
// atomics (order-free, so exact).  Each wavefront takes a fixed strided set of
// the sequence's tokens, normalises a token's scores with a wavefront sum (DPP
// row moves, then the four rows in order) and accumulates s' in fp64 per lane;
// the wavefronts' sums and the final dot product are added in a fixed order,
// so the result is the same on every run.
#include <math.h>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxE = 512;
constexpr int kNpl = kMaxE / 64;

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return ((lane_f32(v, 0) + lane_f32(v, 16)) + lane_f32(v, 32)) + lane_f32(v, 48);
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));
  v = fmaxf(v, dpp_f32<0x4E>(v));
  v = fmaxf(v, dpp_f32<0x141>(v));
  v = fmaxf(v, dpp_f32<0x140>(v));
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}

__global__ __launch_bounds__(kThreads) void balance_loss_kernel(const float *__restrict__ logits,
                                                                const int32_t *__restrict__ idx,
                                                                int E, int K, int seq_len, int softmax,
                                                                float alpha, float *__restrict__ loss) {
  __shared__ int s_cnt[kMaxE];
  __shared__ double s_p[kWaves][kMaxE];
  __shared__ double s_part[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * seq_len;

  for (int e = threadIdx.x; e < kMaxE; e += kThreads) s_cnt[e] = 0;
  __syncthreads();
  for (int64_t p = threadIdx.x; p < static_cast<int64_t>(seq_len) * K; p += kThreads) {
    const int e = idx[t0 * K + p];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }

  double acc[kNpl];
#pragma unroll
  for (int j = 0; j < kNpl; ++j) acc[j] = 0.0;
  const int npl = (E + 63) / 64;
  for (int t = wave; t < seq_len; t += kWaves) {
    const float *row = logits + (t0 + t) * E;
    float s[kNpl];
#pragma unroll
    for (int j = 0; j < kNpl; ++j) {
      const int e = lane + 64 * j;
      s[j] = (j < npl && e < E) ? row[e] : -INFINITY;
    }
    if (softmax) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < kNpl; ++j) m = fmaxf(m, s[j]);
      m = wave_max(m);
      float z = 0.0f;
#pragma unroll
      for (int j = 0; j < kNpl; ++j) {
        s[j] = (j < npl && lane + 64 * j < E) ? expf(s[j] - m) : 0.0f;
        z += s[j];
      }
      z = wave_sum(z);
#pragma unroll
      for (int j = 0; j < kNpl; ++j) s[j] = s[j] / z;
    } else {
#pragma unroll
      for (int j = 0; j < kNpl; ++j)
        s[j] = (j < npl && lane + 64 * j < E) ? 1.0f / (1.0f + expf(-s[j])) : 0.0f;
    }
    float tot = 0.0f;
#pragma unroll
    for (int j = 0; j < kNpl; ++j) tot += s[j];
    tot = wave_sum(tot);
#pragma unroll
    for (int j = 0; j < kNpl; ++j) acc[j] += static_cast<double>(s[j] / tot);
  }
#pragma unroll
  for (int j = 0; j < kNpl; ++j) s_p[wave][lane + 64 * j] = acc[j];
  __syncthreads();

  // P_e (wavefronts in order) times f_e, summed per lane over e = lane, lane+64, ...
  if (wave == 0) {
    double part = 0.0;
    for (int e = lane; e < E; e += 64) {
      double p = 0.0;
      for (int w = 0; w < kWaves; ++w) p += s_p[w][e];
      const double f = static_cast<double>(s_cnt[e]) * E / (static_cast<double>(K) * seq_len);
      part += f * (p / seq_len);
    }
    s_part[lane] = part;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
    for (int l = 0; l < 64; ++l) sum += s_part[l];
    loss[blockIdx.x] = static_cast<float>(static_cast<double>(alpha) * sum);
  }
}

}  // namespace

hipError_t launch_balance_loss(const moe_config &cfg, int64_t T, int seq_len, const float *logits,
                               const int32_t *topk_idx, float alpha, float *loss, hipStream_t st) {
  const int64_t nseq = T / seq_len;
  hipLaunchKernelGGL(balance_loss_kernel, dim3(static_cast<unsigned>(nseq)), dim3(kThreads), 0, st,
                     logits, topk_idx, cfg.n_routed, cfg.top_k, seq_len,
                     cfg.score_func == MOE_SCORE_SOFTMAX ? 1 : 0, alpha, loss);
  return hipGetLastError();
}

}  // namespace moe
