// Combine (DeepSeek-V3 notes page, "DeepSeekMoE" total-output equation):
//   out[t] = u[t] + z[t] + sum_k w[t,k] * y[pair_row[t*K+k]]
// grid.x is the token, grid.y splits the row; every thread owns 16-byte column chunks, two
// at a time with all their loads issued before the first sum (the kernel is bound by the
// loads it keeps in flight), and sums each in fp32 in a fixed order (u, z, then slots
// k = 0..K-1, which the gate emits in ascending expert order), rounding once.  No
// atomics: the result is unique.  Every row this kernel reads (u, z, the pairs' y rows) is
// read once and the output is written once, so loads and stores carry the non-temporal
// hint: the V3 prefill combine took 237 us with it against 253 us without.
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
  constexpr int CH = 2;   // chunks per thread and iteration
  const int stride = kThreads * gridDim.y;
  for (int c0 = blockIdx.y * kThreads + threadIdx.x; c0 < nchunks; c0 += CH * stride) {
    int cc[CH];
    bool ok[CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      cc[q] = c0 + q * stride;
      ok[q] = cc[q] < nchunks;
      if (!ok[q]) cc[q] = c0;            // a chunk past the row loads a valid one, unused
    }
    float acc[CH][V];
#pragma unroll
    for (int q = 0; q < CH; ++q)
#pragma unroll
      for (int i = 0; i < V; ++i) acc[q][i] = 0.0f;
    auto load = [&](const void *base, int64_t row, int q) -> u32x4_t {
      return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(base) + (row * D) / V + cc[q]);
    };
    auto add_row = [&](int q, const u32x4_t v, float scale, bool fma_mode) {
      if (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xFFFF0000u);
          acc[q][2 * i] = fma_mode ? fmaf(scale, lo, acc[q][2 * i]) : acc[q][2 * i] + lo;
          acc[q][2 * i + 1] = fma_mode ? fmaf(scale, hi, acc[q][2 * i + 1]) : acc[q][2 * i + 1] + hi;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float f = __uint_as_float(v[i]);
          acc[q][i] = fma_mode ? fmaf(scale, f, acc[q][i]) : acc[q][i] + f;
        }
      }
    };
    // every load of the first batch (u, z and kBatch y rows) goes out before the first sum;
    // the sums keep their order: u, z, then slots 0..K-1
    u32x4_t vu[CH], vz[CH];
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      vu[q] = residual ? load(u, t, q) : load(y, 0, q);
      vz[q] = z != nullptr ? load(z, t, q) : load(y, 0, q);
    }
    for (int k0 = 0; k0 < K; k0 += kBatch) {
      int row[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) row[i] = s_row[min(k0 + i, K - 1)];
      u32x4_t v[CH][kBatch];
#pragma unroll
      for (int q = 0; q < CH; ++q)
#pragma unroll
        for (int i = 0; i < kBatch; ++i) v[q][i] = load(y, max(row[i], 0), q);
      if (k0 == 0) {
#pragma unroll
        for (int q = 0; q < CH; ++q) {
          if (residual) add_row(q, vu[q], 1.0f, false);
          if (z != nullptr) add_row(q, vz[q], 1.0f, false);
        }
      }
#pragma unroll
      for (int q = 0; q < CH; ++q)
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
          if (k0 + i < K && row[i] >= 0) add_row(q, v[q][i], s_w[k0 + i], true);
    }
#pragma unroll
    for (int q = 0; q < CH; ++q) {
      if (!ok[q]) continue;
      u32x4_t o;
      if (BF16) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[q][2 * i], acc[q][2 * i + 1]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __float_as_uint(acc[q][i]);
      }
      __builtin_nontemporal_store(o, reinterpret_cast<u32x4_t *>(out) + (t * D) / V + cc[q]);
    }
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
