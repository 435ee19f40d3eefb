// Sequence-wise balance loss (DeepSeek-V3 notes page, "V3 improvement 2"; the
// paper's eqs. 17-20): for each sequence of seq_len tokens
//     L = alpha * sum_i f_i P_i,   f_i = E/(K seq_len) * (tokens choosing expert i),
//     P_i = (1/seq_len) * sum_t s_{i,t} / sum_j s_{j,t},
// with s the gate's unbiased score (sigmoid of the logit, or the softmax
// probability) and the choices read from topk_idx.
//
// Two launches, so that the [T, E] logits stream through the whole chip:
//  1. one workgroup per chunk of kChunk tokens of a sequence.  Each wavefront
//     loads its kTokW tokens' rows up front (all loads in flight at once),
//     normalises each token's scores with a wavefront sum (DPP row moves, then
//     the four rows in order) and adds s' into fp64 per-lane sums, token by
//     token; the four wavefronts' sums are added in order and written as the
//     chunk's partial P (fp64) next to its choice histogram (LDS integer
//     atomics, order-free and exact);
//  2. one workgroup per sequence adds the chunks' partials in chunk order,
//     forms f_i P_i and sums over the experts in a fixed order.
// Every floating-point sum has a fixed order, so the result is the same on
// every run.
#include <math.h>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kMaxE = 512;
constexpr int kNpl = kMaxE / 64;          // experts per lane
constexpr int kThreads1 = 256;
constexpr int kWaves1 = kThreads1 / 64;
constexpr int kTokW = 16;                 // tokens per wavefront
constexpr int kChunk = kWaves1 * kTokW;   // tokens per workgroup
constexpr int kThreads2 = 512;
constexpr int kWaves2 = kThreads2 / 64;

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

// one workgroup per (sequence q, chunk c), block q * nchunk + c; chunk c covers
// tokens [c * kChunk, min(seq_len, (c + 1) * kChunk)) of the sequence
template <int NPL>
__global__ __launch_bounds__(kThreads1) void balance_partial_kernel(
    const float *__restrict__ logits, const int32_t *__restrict__ idx, int E, int K, int seq_len,
    int nchunk, int softmax, double *__restrict__ part_p, int32_t *__restrict__ part_n) {
  __shared__ int s_cnt[kMaxE];
  __shared__ double s_p[kWaves1][kMaxE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = blockIdx.x / nchunk, c = blockIdx.x - q * nchunk;
  const int tb = c * kChunk;
  const int nt = min(kChunk, seq_len - tb);
  const int64_t t0 = static_cast<int64_t>(q) * seq_len + tb;   // first token of the chunk

  for (int e = threadIdx.x; e < kMaxE; e += kThreads1) s_cnt[e] = 0;
  __syncthreads();
  for (int p = threadIdx.x; p < nt * K; p += kThreads1) {
    const int e = idx[t0 * K + p];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }

  // this wavefront's tokens: all rows in flight before the first is used
  float v[kTokW][NPL];
#pragma unroll
  for (int u = 0; u < kTokW; ++u) {
    const int t = wave * kTokW + u;
    const float *row = logits + (t0 + t) * E;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      v[u][j] = (t < nt && e < E) ? row[e] : -INFINITY;
    }
  }
  double acc[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) acc[j] = 0.0;
#pragma unroll
  for (int u = 0; u < kTokW; ++u) {
    if (wave * kTokW + u >= nt) break;   // wavefront-uniform
    float s[NPL];
    if (softmax) {
      float m = -INFINITY;
#pragma unroll
      for (int j = 0; j < NPL; ++j) m = fmaxf(m, v[u][j]);
      m = wave_max(m);
      float z = 0.0f;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        s[j] = lane + 64 * j < E ? expf(v[u][j] - m) : 0.0f;
        z += s[j];
      }
      z = wave_sum(z);
#pragma unroll
      for (int j = 0; j < NPL; ++j) s[j] = s[j] / z;
    } else {
#pragma unroll
      for (int j = 0; j < NPL; ++j) s[j] = lane + 64 * j < E ? 1.0f / (1.0f + expf(-v[u][j])) : 0.0f;
    }
    float tot = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) tot += s[j];
    tot = wave_sum(tot);
#pragma unroll
    for (int j = 0; j < NPL; ++j) acc[j] += static_cast<double>(s[j] / tot);
  }
#pragma unroll
  for (int j = 0; j < NPL; ++j) s_p[wave][lane + 64 * j] = acc[j];
  __syncthreads();

  const int64_t out = (static_cast<int64_t>(q) * nchunk + c) * E;
  for (int e = threadIdx.x; e < E; e += kThreads1) {
    double p = 0.0;
#pragma unroll
    for (int w = 0; w < kWaves1; ++w) p += s_p[w][e];
    part_p[out + e] = p;
    part_n[out + e] = s_cnt[e];
  }
}

// one workgroup per sequence
template <int NPL>
__global__ __launch_bounds__(kThreads2) void balance_final_kernel(
    const double *__restrict__ part_p, const int32_t *__restrict__ part_n, int nchunk, int E, int K,
    int seq_len, float alpha, float *__restrict__ loss) {
  __shared__ double s_p[kWaves2][kMaxE];
  __shared__ int s_n[kWaves2][kMaxE];
  __shared__ double s_part[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int q = blockIdx.x;
  const int64_t base = static_cast<int64_t>(q) * nchunk * E;

  // wavefront w adds chunks w, w + 8, ... in order, for experts lane + 64j,
  // loading kBatch chunks before adding any of them
  constexpr int kBatch = 4;
  double p[NPL];
  int n[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    p[j] = 0.0;
    n[j] = 0;
  }
  for (int c0 = wave; c0 < nchunk; c0 += kBatch * kWaves2) {
    double pv[kBatch][NPL];
    int nv[kBatch][NPL];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int c = c0 + b * kWaves2;
      const int64_t row = base + static_cast<int64_t>(c) * E;
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int e = lane + 64 * j;
        const bool in = c < nchunk && e < E;
        pv[b][j] = in ? part_p[row + e] : 0.0;
        nv[b][j] = in ? part_n[row + e] : 0;
      }
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b)
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        p[j] += pv[b][j];
        n[j] += nv[b][j];
      }
  }
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    s_p[wave][lane + 64 * j] = p[j];
    s_n[wave][lane + 64 * j] = n[j];
  }
  __syncthreads();

  // P_e (wavefronts in order) times f_e, summed per lane over e = lane, lane + 64, ...
  if (wave == 0) {
    double part = 0.0;
    for (int e = lane; e < E; e += 64) {
      double pe = 0.0;
      int ne = 0;
      for (int w = 0; w < kWaves2; ++w) {
        pe += s_p[w][e];
        ne += s_n[w][e];
      }
      const double f = static_cast<double>(ne) * E / (static_cast<double>(K) * seq_len);
      part += f * (pe / seq_len);
    }
    s_part[lane] = part;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double sum = 0.0;
    for (int l = 0; l < 64; ++l) sum += s_part[l];
    loss[q] = static_cast<float>(static_cast<double>(alpha) * sum);
  }
}

int chunks_per_seq(int seq_len) { return (seq_len + kChunk - 1) / kChunk; }

}  // namespace

size_t balance_loss_workspace_bytes(const moe_config &cfg, int64_t T, int seq_len) {
  const int64_t nseq = T / seq_len;
  const int64_t slots = nseq * chunks_per_seq(seq_len) * static_cast<int64_t>(cfg.n_routed);
  const size_t pbytes = (static_cast<size_t>(slots) * sizeof(double) + 255) / 256 * 256;
  return pbytes + static_cast<size_t>(slots) * sizeof(int32_t);
}

hipError_t launch_balance_loss(const moe_config &cfg, int64_t T, int seq_len, const float *logits,
                               const int32_t *topk_idx, float alpha, void *workspace, float *loss,
                               hipStream_t st) {
  const int64_t nseq = T / seq_len;
  const int nchunk = chunks_per_seq(seq_len);
  const int64_t slots = nseq * nchunk * static_cast<int64_t>(cfg.n_routed);
  double *part_p = static_cast<double *>(workspace);
  int32_t *part_n = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                                (static_cast<size_t>(slots) * sizeof(double) + 255) / 256 * 256);
  const int E = cfg.n_routed, K = cfg.top_k, sm = cfg.score_func == MOE_SCORE_SOFTMAX ? 1 : 0;
  const dim3 g1(static_cast<unsigned>(nseq * nchunk));
  // lanes hold experts lane + 64j for j < NPL
  if (E <= 64) hipLaunchKernelGGL(balance_partial_kernel<1>, g1, dim3(kThreads1), 0, st, logits, topk_idx, E, K, seq_len, nchunk, sm, part_p, part_n);
  else if (E <= 128) hipLaunchKernelGGL(balance_partial_kernel<2>, g1, dim3(kThreads1), 0, st, logits, topk_idx, E, K, seq_len, nchunk, sm, part_p, part_n);
  else if (E <= 256) hipLaunchKernelGGL(balance_partial_kernel<4>, g1, dim3(kThreads1), 0, st, logits, topk_idx, E, K, seq_len, nchunk, sm, part_p, part_n);
  else hipLaunchKernelGGL(balance_partial_kernel<kNpl>, g1, dim3(kThreads1), 0, st, logits, topk_idx, E, K, seq_len, nchunk, sm, part_p, part_n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 g2(static_cast<unsigned>(nseq));
  if (E <= 64) hipLaunchKernelGGL(balance_final_kernel<1>, g2, dim3(kThreads2), 0, st, part_p, part_n, nchunk, E, K, seq_len, alpha, loss);
  else if (E <= 128) hipLaunchKernelGGL(balance_final_kernel<2>, g2, dim3(kThreads2), 0, st, part_p, part_n, nchunk, E, K, seq_len, alpha, loss);
  else if (E <= 256) hipLaunchKernelGGL(balance_final_kernel<4>, g2, dim3(kThreads2), 0, st, part_p, part_n, nchunk, E, K, seq_len, alpha, loss);
  else hipLaunchKernelGGL(balance_final_kernel<kNpl>, g2, dim3(kThreads2), 0, st, part_p, part_n, nchunk, E, K, seq_len, alpha, loss);
  return hipGetLastError();
}

}  // namespace moe
