// Elementwise and reduction kernels of the layer's backward pass: the chain
// rule of the forward steps (DeepSeek-V3 notes page: total-output equation,
// gate flow steps 1-5, MoE forward steps; SwiGLU expert FFN), in reverse:
//
//   combine   dw[p] = <dout_t, y[row(p)]>,  dy[row(p)] = w[p] dout_t   (p = t*K + k)
//   SwiGLU    h = silu(a) c,  da = dh c silu'(a),  dc = dh silu(a)  from a, c, dh
//   gate      ds at the chosen experts from dw (through route_scale and the
//             optional renormalisation), then dlogits through sigmoid or softmax
//   tokens    dx_t = dout_t (residual) + dx_shared_t + sum_k dx_pair(t, k) + dx_gate_t
//
// Every sum runs in a fixed order; the outputs are the same on every run.
#include <math.h>

#include "backward.hpp"

namespace moe {
namespace {

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// wavefront sum, the same on every lane, fixed order
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

// 128-row tiles over each expert's rows [off[e], off[e+1]): one thread per expert
// counts its tiles, an exclusive scan in LDS places them, each thread writes its own
constexpr int kTilesThreads = 512;   // >= the largest supported n_routed
__global__ __launch_bounds__(kTilesThreads) void bwd_tiles_kernel(
    const int32_t *__restrict__ expert_off, int E, int32_t *tile_row, int32_t *tile_expert,
    int32_t *tile_end, int32_t *tile_first, int32_t *n_tiles) {
  __shared__ int s_n[kTilesThreads];
  const int e = threadIdx.x;
  int a = 0, b = 0;
  if (e < E) {
    a = expert_off[e];
    b = expert_off[e + 1];
  }
  const int cnt = (b - a + 127) / 128;
  s_n[e] = cnt;
  __syncthreads();
  for (int off = 1; off < kTilesThreads; off <<= 1) {   // inclusive scan
    const int v = e >= off ? s_n[e - off] : 0;
    __syncthreads();
    s_n[e] += v;
    __syncthreads();
  }
  const int first = s_n[e] - cnt;
  for (int j = 0; j < cnt; ++j) {
    tile_row[first + j] = a + 128 * j;
    tile_expert[first + j] = e;
    tile_end[first + j] = b;
    tile_first[first + j] = first;
  }
  if (e == kTilesThreads - 1) *n_tiles = s_n[e];
}

// one workgroup (256 threads) per used row of the expert-sorted layout
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const uint16_t *__restrict__ dout, const uint16_t *__restrict__ y, const int32_t *__restrict__ sorted_pair,
    const float *__restrict__ topk_w, const int32_t *__restrict__ n_tiles, int tile_m, int K, int D,
    uint16_t *__restrict__ dy, float *__restrict__ dw) {
  __shared__ float s_part[4];
  const int row = blockIdx.x;
  if (row >= *n_tiles * tile_m) return;
  const int p = sorted_pair[row];
  const int nc = D / 8;
  u32x4_t *dyr = reinterpret_cast<u32x4_t *>(dy + static_cast<int64_t>(row) * D);
  if (p < 0) {   // padding row: zero, so the weight-gradient sums over it add nothing
    for (int c = threadIdx.x; c < nc; c += 256) dyr[c] = u32x4_t{0, 0, 0, 0};
    return;
  }
  const int t = p / K;
  const float w = topk_w[p];
  const u32x4_t *gr = reinterpret_cast<const u32x4_t *>(dout + static_cast<int64_t>(t) * D);
  const u32x4_t *yr = reinterpret_cast<const u32x4_t *>(y + static_cast<int64_t>(row) * D);
  float dot = 0.0f;
  for (int c = threadIdx.x; c < nc; c += 256) {
    const u32x4_t gv = gr[c], yv = yr[c];
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float g0 = __uint_as_float(gv[i] << 16), g1 = __uint_as_float(gv[i] & 0xFFFF0000u);
      const float y0 = __uint_as_float(yv[i] << 16), y1 = __uint_as_float(yv[i] & 0xFFFF0000u);
      dot += g0 * y0;
      dot += g1 * y1;
      o[i] = pack_bf16x2(w * g0, w * g1);
    }
    dyr[c] = o;
  }
  dot = wave_sum(dot);
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = dot;
  __syncthreads();
  if (threadIdx.x == 0) dw[p] = ((s_part[0] + s_part[1]) + s_part[2]) + s_part[3];
}

// rows [0, rows) (rows_dev: n_tiles * tile_m when given), I columns
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(
    const float *__restrict__ ab, const float *__restrict__ dh, const int32_t *__restrict__ n_tiles,
    int tile_m, int64_t rows_host, int I, const int32_t *__restrict__ row_pair,
    uint16_t *__restrict__ h, uint16_t *__restrict__ dab) {
  const int64_t rows = n_tiles ? static_cast<int64_t>(*n_tiles) * tile_m : rows_host;
  const int64_t n = rows * I;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < n;
       q += static_cast<int64_t>(gridDim.x) * 256) {
    const int64_t r = q / I;
    const int i = static_cast<int>(q - r * I);
    if (row_pair != nullptr && row_pair[r] < 0) {   // a padding row: its a and c may be unset
      h[r * I + i] = 0;
      dab[r * 2 * I + i] = 0;
      dab[r * 2 * I + I + i] = 0;
      continue;
    }
    const float a = ab[r * 2 * I + i], c = ab[r * 2 * I + I + i], d = dh[r * I + i];
    const float sa = 1.0f / (1.0f + expf(-a));
    h[r * I + i] = f32_to_bf16_bits(a * sa * c);
    dab[r * 2 * I + i] = f32_to_bf16_bits(d * c * (sa * (1.0f + a * (1.0f - sa))));
    dab[r * 2 * I + I + i] = f32_to_bf16_bits(d * a * sa);
  }
}

// x in routed-row order: xs[r] = x[token of sorted_pair[r]], zeros for a padding
// row; one workgroup per used row, 16 bytes per thread
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ x,
                                                          const int32_t *__restrict__ sorted_pair,
                                                          const int32_t *__restrict__ n_tiles, int tile_m, int K,
                                                          int D, uint16_t *__restrict__ xs) {
  const int row = blockIdx.x;
  if (row >= *n_tiles * tile_m) return;
  const int p = sorted_pair[row];
  const int nc = D / 8;
  u32x4_t *dst = reinterpret_cast<u32x4_t *>(xs + static_cast<int64_t>(row) * D);
  if (p < 0) {
    for (int c = threadIdx.x; c < nc; c += 256) dst[c] = u32x4_t{0, 0, 0, 0};
    return;
  }
  const u32x4_t *src = reinterpret_cast<const u32x4_t *>(x + static_cast<int64_t>(p / K) * D);
  for (int c = threadIdx.x; c < nc; c += 256) dst[c] = src[c];
}

// one wavefront per token
__global__ __launch_bounds__(64) void gate_bwd_kernel(
    const float *__restrict__ logits, const int32_t *__restrict__ topk_idx, const int32_t *__restrict__ pair_row,
    const float *__restrict__ dw, int E, int K, int softmax, int normalise, float route_scale,
    uint16_t *__restrict__ dl) {
  __shared__ float s_s[512];
  __shared__ float s_ds[512];
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  const float *l = logits + t * E;
  float m = -INFINITY;
  for (int e = lane; e < E; e += 64) m = fmaxf(m, l[e]);
  if (softmax) m = wave_max(m);
  float z = 0.0f;
  for (int e = lane; e < E; e += 64) {
    const float v = softmax ? expf(l[e] - m) : 1.0f / (1.0f + expf(-l[e]));
    s_s[e] = v;
    s_ds[e] = 0.0f;
    z += v;
  }
  if (softmax) {
    z = wave_sum(z);
    for (int e = lane; e < E; e += 64) s_s[e] = s_s[e] / z;
  }
  __syncthreads();
  // chosen experts, in slot order (the same loop on every lane)
  float tot = 0.0f, dot = 0.0f;
  for (int k = 0; k < K; ++k) {
    const int64_t p = t * K + k;
    const int e = topk_idx[p];
    if (pair_row[p] < 0 || e < 0 || e >= E) continue;
    const float s = s_s[e];
    tot += s;
    dot += dw[p] * route_scale * s;
  }
  __syncthreads();
  if (lane == 0) {
    for (int k = 0; k < K; ++k) {
      const int64_t p = t * K + k;
      const int e = topk_idx[p];
      if (pair_row[p] < 0 || e < 0 || e >= E) continue;
      const float dwr = dw[p] * route_scale;
      s_ds[e] = normalise ? dwr / tot - dot / (tot * tot) : dwr;
    }
  }
  __syncthreads();
  float sd = 0.0f;
  if (softmax) {
    for (int e = lane; e < E; e += 64) sd += s_ds[e] * s_s[e];
    sd = wave_sum(sd);
  }
  for (int e = lane; e < E; e += 64) {
    const float s = s_s[e], ds = s_ds[e];
    const float v = softmax ? s * (ds - sd) : ds * s * (1.0f - s);
    dl[t * E + e] = f32_to_bf16_bits(v);
  }
}

// one workgroup (256 threads) per token, 8 columns per thread step
__global__ __launch_bounds__(256) void dx_final_kernel(
    const uint16_t *__restrict__ dout, const float *__restrict__ dx_shared, const float *__restrict__ dx_pairs,
    const float *__restrict__ dx_gate, const int32_t *__restrict__ pair_row, int K, int D, int residual,
    uint16_t *__restrict__ dx) {
  const int64_t t = blockIdx.x;
  for (int c = threadIdx.x * 8; c < D; c += 256 * 8) {
    float acc[8];
    const u32x4_t g = *reinterpret_cast<const u32x4_t *>(dout + t * D + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = residual ? __uint_as_float(g[i] << 16) : 0.0f;
      acc[2 * i + 1] = residual ? __uint_as_float(g[i] & 0xFFFF0000u) : 0.0f;
    }
    if (dx_shared != nullptr) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += dx_shared[t * D + c + i];
    }
    for (int k = 0; k < K; ++k) {
      const int row = pair_row[t * K + k];
      if (row < 0) continue;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += dx_pairs[static_cast<int64_t>(row) * D + c + i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += dx_gate[t * D + c + i];
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *reinterpret_cast<u32x4_t *>(dx + t * D + c) = o;
  }
}

}  // namespace

hipError_t launch_bwd_tiles(const int32_t *expert_off, int E, int32_t *tile_row, int32_t *tile_expert,
                            int32_t *tile_end, int32_t *tile_first, int32_t *n_tiles, hipStream_t st) {
  if (E > kTilesThreads) return hipErrorInvalidValue;
  hipLaunchKernelGGL(bwd_tiles_kernel, dim3(1), dim3(kTilesThreads), 0, st, expert_off, E, tile_row, tile_expert,
                     tile_end, tile_first, n_tiles);
  return hipGetLastError();
}

hipError_t launch_combine_bwd(const void *dout, const void *y, const moe_routing &r, const float *topk_w,
                              int K, int D, void *dy, float *dw, hipStream_t st) {
  if (r.max_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(combine_bwd_kernel, dim3(static_cast<unsigned>(r.max_rows)), dim3(256), 0, st,
                     static_cast<const uint16_t *>(dout), static_cast<const uint16_t *>(y), r.sorted_pair,
                     topk_w, r.n_tiles, r.tile_m, K, D, static_cast<uint16_t *>(dy), dw);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float *ab, const float *dh, const int32_t *n_tiles, int tile_m,
                             int64_t rows_host, int I, const int32_t *row_pair, void *h, void *dab,
                             hipStream_t st) {
  const int64_t n = rows_host * I;
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, ab, dh,
                     n_tiles, tile_m, rows_host, I, row_pair, static_cast<uint16_t *>(h),
                     static_cast<uint16_t *>(dab));
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *x, const moe_routing &r, int K, int D, void *xs, hipStream_t st) {
  if (r.max_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(static_cast<unsigned>(r.max_rows)), dim3(256), 0, st,
                     static_cast<const uint16_t *>(x), r.sorted_pair, r.n_tiles, r.tile_m, K, D,
                     static_cast<uint16_t *>(xs));
  return hipGetLastError();
}

hipError_t launch_gate_bwd(const moe_config &cfg, int64_t T, const float *logits, const int32_t *topk_idx,
                           const int32_t *pair_row, const float *dw, void *dl, hipStream_t st) {
  const int sm = cfg.score_func == MOE_SCORE_SOFTMAX ? 1 : 0;
  const int norm = cfg.norm_topk >= 0 ? cfg.norm_topk : (sm ? 0 : 1);
  hipLaunchKernelGGL(gate_bwd_kernel, dim3(static_cast<unsigned>(T)), dim3(64), 0, st, logits, topk_idx,
                     pair_row, dw, cfg.n_routed, cfg.top_k, sm, norm, cfg.route_scale,
                     static_cast<uint16_t *>(dl));
  return hipGetLastError();
}

hipError_t launch_dx_final(int64_t T, int K, int D, int residual, const void *dout, const float *dx_shared,
                           const float *dx_pairs, const float *dx_gate, const int32_t *pair_row, void *dx,
                           hipStream_t st) {
  hipLaunchKernelGGL(dx_final_kernel, dim3(static_cast<unsigned>(T)), dim3(256), 0, st,
                     static_cast<const uint16_t *>(dout), dx_shared, dx_pairs, dx_gate, pair_row, K, D,
                     residual, static_cast<uint16_t *>(dx));
  return hipGetLastError();
}

}  // namespace moe
