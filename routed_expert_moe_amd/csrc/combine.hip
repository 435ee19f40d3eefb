// Combine (DeepSeek-V3 notes page, "DeepSeekMoE" total-output equation):
//   out[t] = u[t] + z[t] + sum_k w[t,k] * y[pair_row[t*K+k]]
// grid.x is the token, grid.y splits the row; every thread owns 16-byte column chunks and sums in
// fp32 in a fixed order (u, z, then slots k = 0..K-1, which the gate emits in
// ascending expert order), rounding once.  No atomics: the result is unique.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxK = 32;
constexpr int kBatch = 8;   // y rows loaded before the first is summed

template <bool BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(int64_t T, int D, int K,
                                                           const void *__restrict__ u,
                                                           const void *__restrict__ z,
                                                           const void *__restrict__ y,
                                                           const int32_t *__restrict__ pair_row,
                                                           const float *__restrict__ w,
                                                           void *__restrict__ out, int residual) {
  __shared__ int s_row[kMaxK];
  __shared__ float s_w[kMaxK];
  const int64_t t = blockIdx.x;
  if (threadIdx.x < K) {
    s_row[threadIdx.x] = pair_row[t * K + threadIdx.x];
    s_w[threadIdx.x] = w[t * K + threadIdx.x];
  }
  __syncthreads();
  constexpr int V = BF16 ? 8 : 4;   // elements per 16-byte chunk
  const int nchunks = D / V;
  for (int c = blockIdx.y * kThreads + threadIdx.x; c < nchunks; c += kThreads * gridDim.y) {
    float acc[V];
#pragma unroll
    for (int i = 0; i < V; ++i) acc[i] = 0.0f;
    auto load = [&](const void *base, int64_t row) -> u32x4_t {
      return reinterpret_cast<const u32x4_t *>(base)[(row * D) / V + c];
    };
    auto add_row = [&](const u32x4_t v, float scale, bool fma_mode) {
      if (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xFFFF0000u);
          acc[2 * i] = fma_mode ? fmaf(scale, lo, acc[2 * i]) : acc[2 * i] + lo;
          acc[2 * i + 1] = fma_mode ? fmaf(scale, hi, acc[2 * i + 1]) : acc[2 * i + 1] + hi;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float f = __uint_as_float(v[i]);
          acc[i] = fma_mode ? fmaf(scale, f, acc[i]) : acc[i] + f;
        }
      }
    };
    // loads are issued in batches before their first use; an absent term (no
    // residual, no shared expert, a dropped slot with row -1) reads row 0 of y,
    // which always exists, and is skipped when summing
    const u32x4_t vu = residual ? load(u, t) : load(y, 0);
    const u32x4_t vz = z != nullptr ? load(z, t) : load(y, 0);
    if (residual) add_row(vu, 1.0f, false);
    if (z != nullptr) add_row(vz, 1.0f, false);
    for (int k0 = 0; k0 < K; k0 += kBatch) {
      u32x4_t v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) v[i] = load(y, max(s_row[min(k0 + i, K - 1)], 0));
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (k0 + i < K && s_row[k0 + i] >= 0) add_row(v[i], s_w[k0 + i], true);
    }
    u32x4_t o;
    if (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[i]);
    }
    reinterpret_cast<u32x4_t *>(out)[(t * D) / V + c] = o;
  }
}

}  // namespace

hipError_t launch_combine(const moe_config &cfg, int64_t T, const void *u, const void *z,
                          const void *y, const moe_routing &r, const float *w, void *out,
                          hipStream_t st) {
  // grid.x = token; grid.y spreads a row's 16-byte chunks over workgroups so a
  // short batch still occupies many CUs
  const int V = cfg.act_dtype == MOE_BF16 ? 8 : 4;
  const int nchunks = cfg.dim / V;
  const int per_token = T >= 1024 ? 1 : (nchunks + kThreads - 1) / kThreads;
  const dim3 grid(static_cast<unsigned>(T), static_cast<unsigned>(per_token)), block(kThreads);
  if (cfg.act_dtype == MOE_BF16)
    hipLaunchKernelGGL(combine_kernel<true>, grid, block, 0, st, T, cfg.dim, cfg.top_k, u, z, y,
                       r.pair_row, w, out, cfg.add_residual);
  else
    hipLaunchKernelGGL(combine_kernel<false>, grid, block, 0, st, T, cfg.dim, cfg.top_k, u, z, y,
                       r.pair_row, w, out, cfg.add_residual);
  return hipGetLastError();
}

}  // namespace moe
