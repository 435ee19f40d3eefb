// Gate, steps 1b-5 (DeepSeek-V3 notes page, gate flow): scores from the fp32
// logits, group-limited selection, global top-k, weights from the unbiased
// scores.  One 64-lane wavefront per token; four tokens per workgroup.
//
// Selection is exact integer work on packed 64-bit keys
//     (orderable(key) << 32) | (0xFFFFFFFF - expert)
// so the maximum is unique and equal keys rank the lower expert first.  The
// top-k runs as K rounds of a wavefront max reduction.
#include <math.h>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxE = 512;

__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ranks equal to +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Wavefront reductions without LDS traffic: DPP moves combine the 16 lanes of
// each row (swap neighbours, swap pairs, mirror halves of 8, mirror 16), then
// the four row results are read as scalars and combined in row order.  Every
// lane gets the same value, and the order of operations is fixed.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return (static_cast<uint64_t>(dpp_u32<CTRL>(static_cast<uint32_t>(v >> 32))) << 32) |
         dpp_u32<CTRL>(static_cast<uint32_t>(v));
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(v)), l)));
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), l));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ float row_sum_f32(float v) {
  v += dpp_f32<kDppXor1>(v);
  v += dpp_f32<kDppXor2>(v);
  v += dpp_f32<kDppHalfMirror>(v);
  v += dpp_f32<kDppMirror>(v);
  return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, dpp_f32<kDppXor1>(v));
  v = fmaxf(v, dpp_f32<kDppXor2>(v));
  v = fmaxf(v, dpp_f32<kDppHalfMirror>(v));
  v = fmaxf(v, dpp_f32<kDppMirror>(v));
  return fmaxf(fmaxf(lane_f32(v, 0), lane_f32(v, 16)), fmaxf(lane_f32(v, 32), lane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum_f32(float v) {
  v = row_sum_f32(v);
  return ((lane_f32(v, 0) + lane_f32(v, 16)) + lane_f32(v, 32)) + lane_f32(v, 48);
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = max_u64(v, dpp_u64<kDppXor1>(v));
  v = max_u64(v, dpp_u64<kDppXor2>(v));
  v = max_u64(v, dpp_u64<kDppHalfMirror>(v));
  v = max_u64(v, dpp_u64<kDppMirror>(v));
  return max_u64(max_u64(lane_u64(v, 0), lane_u64(v, 16)), max_u64(lane_u64(v, 32), lane_u64(v, 48)));
}

template <int NPL>
__global__ __launch_bounds__(256) void gate_route_kernel(
    const float *__restrict__ logits, const float *__restrict__ bias, int64_t T, int E, int G,
    int TG, int K, int softmax, int normalise, float route_scale, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, float *__restrict__ keys_out) {
  __shared__ float s_key[kWaves][kMaxE];
  __shared__ float s_score[kWaves][kMaxE];
  __shared__ float s_w[kWaves][32];

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kWaves + wave;
  if (t >= T) return;  // uniform per wavefront; no workgroup barrier below

  const float *lrow = logits + t * E;
  // loads use clamped indices so they all issue before the first wait
  float l[NPL], s[NPL], key[NPL], b[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    const float v = lrow[min(e, E - 1)];
    l[j] = e < E ? v : -INFINITY;
    b[j] = bias != nullptr ? bias[min(e, E - 1)] : 0.0f;
  }

  // step 1: scores and ranked keys
  if (!softmax) {
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      s[j] = 1.0f / (1.0f + expf(-l[j]));
      key[j] = bias != nullptr && e < E ? s[j] + b[j] : s[j];
    }
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPL; ++j) m = fmaxf(m, l[j]);
    m = wave_max_f32(m);
    float sum = 0.0f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      s[j] = e < E ? expf(l[j] - m) : 0.0f;
      sum += s[j];
    }
    sum = wave_sum_f32(sum);
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
      const int e = lane + 64 * j;
      s[j] = s[j] / sum;
      key[j] = bias != nullptr && e < E ? s[j] + b[j] : l[j];
    }
  }
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      s_key[wave][e] = key[j];
      s_score[wave][e] = s[j];
      if (keys_out != nullptr) keys_out[t * E + e] = key[j];
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");

  // steps 2-3: group scores (top-2 sum with a bias, else max), keep topk_groups
  uint64_t keep = ~0ull;
  const int gsz = E / G;
  if (G > 1) {
    float gs = -INFINITY;
    if (lane < G) {
      float b1 = -INFINITY, b2 = -INFINITY;
      const float *gk = &s_key[wave][lane * gsz];
#pragma unroll 8
      for (int i = 0; i < gsz; ++i) {
        const float v = gk[i];
        if (v > b1) {
          b2 = b1;
          b1 = v;
        } else if (v > b2) {
          b2 = v;
        }
      }
      gs = bias != nullptr ? b1 + b2 : b1;
    }
    int rank = 0;
    for (int g = 0; g < G; ++g) {
      const float o = lane_f32(gs, g);
      rank += (o > gs) || (o == gs && g < lane);
    }
    keep = __ballot(lane < G && rank < TG);
  }

  // step 4: global top-k over the surviving experts
  uint64_t pk[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    const int e = lane + 64 * j;
    const bool on = e < E && ((keep >> (e / gsz)) & 1ull);
    pk[j] = on ? ((static_cast<uint64_t>(orderable(key[j])) << 32) | (0xFFFFFFFFu - e)) : 0ull;
  }
  int mine = 0x7FFFFFFF;
  for (int r = 0; r < K; ++r) {
    uint64_t best = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) best = pk[j] > best ? pk[j] : best;
    best = wave_max_u64(best);
    const int e = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(best));
    if (lane == r) mine = e;
#pragma unroll
    for (int j = 0; j < NPL; ++j)
      if (pk[j] == best) pk[j] = 0ull;
  }

  // ascending expert order: lane r (< K) holds the r-th pick; place it by rank
  int pos = 0;
  for (int r = 0; r < K; ++r) pos += __builtin_amdgcn_readlane(mine, r) < mine;
  // step 5: unbiased scores at the chosen experts, renormalised, scaled
  float val = lane < K ? s_score[wave][mine] : 0.0f;
  if (lane < K) s_w[wave][pos] = val;
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  float scale = route_scale;
  if (normalise) {
    float tot = 0.0f;
    for (int r = 0; r < K; ++r) tot += s_w[wave][r];  // ascending expert order
    scale = route_scale / tot;
  }
  if (lane < K) {
    topk_idx[t * K + pos] = mine;
    topk_w[t * K + pos] = val * scale;
  }
}

}  // namespace

hipError_t launch_gate_route(const moe_config &cfg, int64_t T, const float *logits,
                             const float *bias, int32_t *topk_idx, float *topk_w, float *keys,
                             hipStream_t st) {
  const int E = cfg.n_routed;
  const int softmax = cfg.score_func == MOE_SCORE_SOFTMAX;
  const int normalise = cfg.norm_topk >= 0 ? cfg.norm_topk : !softmax;
  const dim3 grid(static_cast<unsigned>((T + kWaves - 1) / kWaves));
  const dim3 block(64 * kWaves);
#define MOE_ROUTE(NPL)                                                                       \
  hipLaunchKernelGGL(gate_route_kernel<NPL>, grid, block, 0, st, logits, bias, T, E,          \
                     cfg.n_groups, cfg.topk_groups, cfg.top_k, softmax, normalise,            \
                     cfg.route_scale, topk_idx, topk_w, keys)
  if (E <= 64) MOE_ROUTE(1);
  else if (E <= 128) MOE_ROUTE(2);
  else if (E <= 256) MOE_ROUTE(4);
  else MOE_ROUTE(8);
#undef MOE_ROUTE
  return hipGetLastError();
}

}  // namespace moe

// ---------------------------------------------------------------------------
// Gate logits for small batches (T < 64, bf16): l[t][e] = x_t . W_g[e].
// A GEMM tile would leave most CUs idle here.  Each workgroup takes one expert
// row (E workgroups: at E = 256 every CU streams one row of W_g; four rows per
// workgroup kept 64 CUs busy and took 1.8 us longer per V3 decode step); its 8
// wavefronts split K eight ways and form the dot products of up to 8 tokens per
// pass in fp32 (lanes stride over their K range in 16-byte pieces), sum the 16
// lanes of each row with DPP moves, then add the rows and wavefronts in LDS in a
// fixed order.
namespace moe {
namespace {

constexpr int kGemvTokens = 8;
constexpr int kGemvExperts = 1;
constexpr int kGemvWaves = 8;

__device__ __forceinline__ void bf16x8_to_f32(const u32x4_t v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
}

__global__ __launch_bounds__(64 * kGemvWaves) void gate_logits_gemv_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg, int T, int E, int K,
    float *__restrict__ logits) {
  __shared__ float part[kGemvWaves][4][kGemvExperts * kGemvTokens];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e0 = blockIdx.x * kGemvExperts;
  const int units = K / 8;                                    // 16-byte pieces per row
  const int u0 = wave * units / kGemvWaves, u1 = (wave + 1) * units / kGemvWaves;
  for (int t0 = 0; t0 < T; t0 += kGemvTokens) {
    const int nt = min(kGemvTokens, T - t0);
    float acc[kGemvExperts][kGemvTokens];
#pragma unroll
    for (int j = 0; j < kGemvExperts; ++j)
#pragma unroll
      for (int t = 0; t < kGemvTokens; ++t) acc[j][t] = 0.0f;
    for (int u = u0 + lane; u < u1; u += 64) {
      const int k = u * 8;
      // every load is issued before the first use: rows past the last expert or
      // token are clamped to a valid row and their sums are never stored
      u32x4_t wr[kGemvExperts], xr[kGemvTokens];
#pragma unroll
      for (int j = 0; j < kGemvExperts; ++j)
        wr[j] = *reinterpret_cast<const u32x4_t *>(wg + static_cast<int64_t>(min(e0 + j, E - 1)) * K + k);
#pragma unroll
      for (int t = 0; t < kGemvTokens; ++t)
        xr[t] = *reinterpret_cast<const u32x4_t *>(x + static_cast<int64_t>(t0 + min(t, nt - 1)) * K + k);
      float w[kGemvExperts][8];
#pragma unroll
      for (int j = 0; j < kGemvExperts; ++j) bf16x8_to_f32(wr[j], w[j]);
#pragma unroll
      for (int t = 0; t < kGemvTokens; ++t) {
        float xv[8];
        bf16x8_to_f32(xr[t], xv);
#pragma unroll
        for (int j = 0; j < kGemvExperts; ++j)
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[j][t] = fmaf(w[j][i], xv[i], acc[j][t]);
      }
    }
    // per-row sums by DPP; one lane per row stores them; then each output adds
    // its 8 wavefronts x 4 rows in a fixed order
#pragma unroll
    for (int j = 0; j < kGemvExperts; ++j)
#pragma unroll
      for (int t = 0; t < kGemvTokens; ++t) {
        const float v = row_sum_f32(acc[j][t]);
        if ((lane & 15) == 0) part[wave][lane >> 4][j * kGemvTokens + t] = v;
      }
    __syncthreads();
    if (threadIdx.x < kGemvExperts * kGemvTokens) {
      const int j = threadIdx.x / kGemvTokens, t = threadIdx.x % kGemvTokens;
      float v = 0.0f;
      for (int w = 0; w < kGemvWaves; ++w)   // K order
#pragma unroll
        for (int r = 0; r < 4; ++r) v += part[w][r][threadIdx.x];
      if (t < nt && e0 + j < E) logits[static_cast<int64_t>(t0 + t) * E + e0 + j] = v;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_gate_logits_gemv(const moe_config &cfg, int64_t T, const void *x,
                                   const void *w_gate, float *logits, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((cfg.n_routed + kGemvExperts - 1) / kGemvExperts));
  const dim3 block(64 * kGemvWaves);
  hipLaunchKernelGGL(gate_logits_gemv_kernel, grid, block, 0, st, static_cast<const uint16_t *>(x),
                     static_cast<const uint16_t *>(w_gate), static_cast<int>(T), cfg.n_routed, cfg.dim,
                     logits);
  return hipGetLastError();
}

}  // namespace moe
