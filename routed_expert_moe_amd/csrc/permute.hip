// Dispatch of (token, slot) pairs into expert-sorted rows padded to tile_m.
//
// It replaces the per-expert gather of the DeepSeek-V3 notes page (MoE
// forward, step 2: for each expert, the tokens that chose it) with a counting
// sort that is stable in the pair id p = t*K + k:
//   1. count:   each workgroup takes 2048 consecutive pairs (four wavefronts
//               of 512); a wavefront ranks equal experts within 64 pairs by
//               ballot matching and keeps running per-expert counts in LDS.
//               It writes each pair's rank inside the workgroup and the
//               workgroup's histogram.
//   2. scan:    one workgroup turns the histograms into per-workgroup bases,
//               counts, padded expert offsets, tile lists and -1 padding rows.
//   3. scatter: row = expert_off[e] + base[blk][e] + rank.
// With a single count workgroup (T*K <= 2048) the three phases run in one
// launch that keeps its intermediate tables in LDS.  Every value is computed without atomics, so the result is unique.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kPermThreads = 256;
constexpr int kPermWaves = kPermThreads / 64;
constexpr int kPairsPerWave = 512;
constexpr int kPairsPerBlock = kPermWaves * kPairsPerWave;
constexpr int kMaxE = 512;

struct PermArgs {
  const int32_t *idx;
  int64_t P;
  int E;
  int TM;
  int nblk;
  int32_t *counts, *expert_off, *sorted_pair, *pair_row, *tile_expert, *tile_row, *n_tiles;
  int32_t *local_rank;  // [P]
  int32_t *hist;        // [nblk][E]
};

__device__ __forceinline__ int expert_of(const PermArgs &a, int64_t p) {
  if (p >= a.P) return -1;
  const int e = a.idx[p];
  return (e >= 0 && e < a.E) ? e : -1;  // out-of-range entries are dropped
}

// phase 1 for workgroup `blk`; s_cnt holds kPermWaves x E counters
__device__ void count_block(const PermArgs &a, int blk, int (*s_cnt)[kMaxE]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kPermWaves * kMaxE; i += kPermThreads) (&s_cnt[0][0])[i] = 0;
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
  const int64_t base = static_cast<int64_t>(blk) * kPairsPerBlock + wave * kPairsPerWave;
  for (int c = 0; c < kPairsPerWave / 64; ++c) {
    const int64_t p = base + c * 64 + lane;
    const int e = expert_of(a, p);
    uint64_t todo = __ballot(e >= 0);
    int rank = 0, same = 0;
    while (todo) {
      const int leader = __ffsll(static_cast<long long>(todo)) - 1;
      const int el = __builtin_amdgcn_readlane(e, leader);   // leader is wavefront-uniform
      const uint64_t m = __ballot(e == el);
      if (e == el) {
        rank = __popcll(m & below);
        same = __popcll(m);
      }
      todo &= ~m;
    }
    int r = 0;
    if (e >= 0) r = s_cnt[wave][e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && rank == same - 1) s_cnt[wave][e] += same;
    __builtin_amdgcn_wave_barrier();
    if (p < a.P) a.local_rank[p] = r;
  }
  __syncthreads();
  // exclusive prefix over the wavefronts, histogram of the workgroup
  for (int e = threadIdx.x; e < a.E; e += kPermThreads) {
    int run = 0;
    for (int w = 0; w < kPermWaves; ++w) {
      const int v = s_cnt[w][e];
      s_cnt[w][e] = run;
      run += v;
    }
    a.hist[static_cast<int64_t>(blk) * a.E + e] = run;
  }
  __syncthreads();
  for (int c = 0; c < kPairsPerWave / 64; ++c) {
    const int64_t p = base + c * 64 + lane;
    const int e = expert_of(a, p);
    if (e >= 0) a.local_rank[p] += s_cnt[wave][e];
  }
}

// phase 2, one workgroup of kPermThreads
__device__ void scan_all(const PermArgs &a, int *s_pad) {
  for (int e = threadIdx.x; e < a.E; e += kPermThreads) {
    int run = 0;
    for (int b = 0; b < a.nblk; ++b) {
      int32_t *h = a.hist + static_cast<int64_t>(b) * a.E + e;
      const int v = *h;
      *h = run;
      run += v;
    }
    a.counts[e] = run;
    s_pad[e] = (run + a.TM - 1) / a.TM * a.TM;
  }
  for (int e = a.E + threadIdx.x; e < kMaxE; e += kPermThreads) s_pad[e] = 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over kMaxE entries, two per thread
  for (int off = 1; off < kMaxE; off <<= 1) {
    int v0 = 0, v1 = 0;
    const int i0 = threadIdx.x, i1 = threadIdx.x + kPermThreads;
    if (i0 >= off) v0 = s_pad[i0 - off];
    if (i1 >= off) v1 = s_pad[i1 - off];
    __syncthreads();
    s_pad[i0] += v0;
    s_pad[i1] += v1;
    __syncthreads();
  }
  for (int e = threadIdx.x; e < a.E; e += kPermThreads) {
    const int end = s_pad[e];
    const int cnt = a.counts[e];
    const int padded = (cnt + a.TM - 1) / a.TM * a.TM;
    const int off = end - padded;
    a.expert_off[e] = off;
    for (int j = 0; j < padded / a.TM; ++j) {
      a.tile_expert[off / a.TM + j] = e;
      a.tile_row[off / a.TM + j] = off + j * a.TM;
    }
    for (int r = off + cnt; r < end; ++r) a.sorted_pair[r] = -1;
  }
  if (threadIdx.x == 0) {
    a.expert_off[a.E] = s_pad[a.E - 1];
    *a.n_tiles = s_pad[a.E - 1] / a.TM;
  }
}

// phase 3 for pairs [p0, min(p1, P))
__device__ void scatter_range(const PermArgs &a, int64_t p0, int64_t p1, int stride) {
  if (p1 > a.P) p1 = a.P;
  for (int64_t p = p0; p < p1; p += stride) {
    const int e = expert_of(a, p);
    if (e < 0) {
      a.pair_row[p] = -1;
      continue;
    }
    const int64_t blk = p / kPairsPerBlock;
    const int row = a.expert_off[e] + a.hist[blk * a.E + e] + a.local_rank[p];
    a.sorted_pair[row] = static_cast<int32_t>(p);
    a.pair_row[p] = row;
  }
}

__global__ __launch_bounds__(kPermThreads) void permute_count_kernel(PermArgs a) {
  __shared__ int s_cnt[kPermWaves][kMaxE];
  count_block(a, blockIdx.x, s_cnt);
}

__global__ __launch_bounds__(kPermThreads) void permute_scan_kernel(PermArgs a) {
  __shared__ int s_pad[kMaxE];
  scan_all(a, s_pad);
}

__global__ __launch_bounds__(kPermThreads) void permute_scatter_kernel(PermArgs a) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * kPermThreads + threadIdx.x;
  scatter_range(a, p, p + 1, 1);
}

// All three phases in one workgroup for P <= kPairsPerBlock, with ranks,
// histograms and offsets kept in LDS: the expert ids are read once and
// nothing written here is read back from global memory.
__global__ __launch_bounds__(kPermThreads) void permute_small_kernel(PermArgs a) {
  __shared__ int s_cnt[kPermWaves][kMaxE];   // per-wavefront counts, then per-wavefront bases
  __shared__ int s_tot[kMaxE];               // pairs per expert
  __shared__ int s_end[kMaxE];               // padded sizes, then inclusive padded ends
  __shared__ int s_rank[kPairsPerBlock];     // rank among the wavefront's pairs of one expert
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int i = threadIdx.x; i < kPermWaves * kMaxE; i += kPermThreads) (&s_cnt[0][0])[i] = 0;
  constexpr int kChunks = kPairsPerWave / 64;
  const int64_t base = static_cast<int64_t>(wave) * kPairsPerWave;
  int ex[kChunks];
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {   // every load issues before the first use
    const int64_t p = base + c * 64 + lane;
    const int e = a.idx[p < a.P ? p : 0];
    ex[c] = (p < a.P && e >= 0 && e < a.E) ? e : -1;
  }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int e = ex[c];
    uint64_t todo = __ballot(e >= 0);
    int rank = 0, same = 0;
    while (todo) {
      const int leader = __ffsll(static_cast<long long>(todo)) - 1;
      const int el = __builtin_amdgcn_readlane(e, leader);   // leader is wavefront-uniform
      const uint64_t m = __ballot(e == el);
      if (e == el) {
        rank = __popcll(m & below);
        same = __popcll(m);
      }
      todo &= ~m;
    }
    int r = 0;
    if (e >= 0) r = s_cnt[wave][e] + rank;
    __builtin_amdgcn_wave_barrier();
    if (e >= 0 && rank == same - 1) s_cnt[wave][e] += same;
    __builtin_amdgcn_wave_barrier();
    s_rank[wave * kPairsPerWave + c * 64 + lane] = r;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kMaxE; e += kPermThreads) {
    int run = 0;
    if (e < a.E) {
#pragma unroll
      for (int w = 0; w < kPermWaves; ++w) {
        const int v = s_cnt[w][e];
        s_cnt[w][e] = run;
        run += v;
      }
      a.counts[e] = run;
    }
    s_tot[e] = run;
    s_end[e] = (run + a.TM - 1) / a.TM * a.TM;
  }
  __syncthreads();
  for (int off = 1; off < kMaxE; off <<= 1) {   // inclusive scan, two entries per thread
    int v0 = 0, v1 = 0;
    const int i0 = threadIdx.x, i1 = threadIdx.x + kPermThreads;
    if (i0 >= off) v0 = s_end[i0 - off];
    if (i1 >= off) v1 = s_end[i1 - off];
    __syncthreads();
    s_end[i0] += v0;
    s_end[i1] += v1;
    __syncthreads();
  }
  for (int e = threadIdx.x; e < a.E; e += kPermThreads) {
    const int end = s_end[e];
    const int start = e > 0 ? s_end[e - 1] : 0;
    a.expert_off[e] = start;
    for (int j = 0; j < (end - start) / a.TM; ++j) {
      a.tile_expert[start / a.TM + j] = e;
      a.tile_row[start / a.TM + j] = start + j * a.TM;
    }
    for (int r = start + s_tot[e]; r < end; ++r) a.sorted_pair[r] = -1;
  }
  if (threadIdx.x == 0) {
    a.expert_off[a.E] = s_end[a.E - 1];
    *a.n_tiles = s_end[a.E - 1] / a.TM;
  }
#pragma unroll
  for (int c = 0; c < kChunks; ++c) {
    const int64_t p = base + c * 64 + lane;
    if (p < a.P) {
      const int e = ex[c];
      if (e < 0) {
        a.pair_row[p] = -1;
      } else {
        const int start = e > 0 ? s_end[e - 1] : 0;
        const int row = start + s_cnt[wave][e] + s_rank[wave * kPairsPerWave + c * 64 + lane];
        a.sorted_pair[row] = static_cast<int32_t>(p);
        a.pair_row[p] = row;
      }
    }
  }
}

}  // namespace

int64_t permute_scratch_ints(int64_t P, int E) {
  const int64_t nblk = (P + kPairsPerBlock - 1) / kPairsPerBlock;
  return P + nblk * E;
}

hipError_t launch_permute(const moe_config &cfg, int64_t T, const int32_t *topk_idx,
                          const moe_routing &r, hipStream_t st) {
  PermArgs a;
  a.idx = topk_idx;
  a.P = T * cfg.top_k;
  a.E = cfg.n_routed;
  a.TM = r.tile_m;
  a.nblk = static_cast<int>((a.P + kPairsPerBlock - 1) / kPairsPerBlock);
  a.counts = r.counts;
  a.expert_off = r.expert_off;
  a.sorted_pair = r.sorted_pair;
  a.pair_row = r.pair_row;
  a.tile_expert = r.tile_expert;
  a.tile_row = r.tile_row;
  a.n_tiles = r.n_tiles;
  a.local_rank = r.scratch;
  a.hist = r.scratch + a.P;
  if (a.nblk == 1) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(kPermThreads), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(permute_count_kernel, dim3(a.nblk), dim3(kPermThreads), 0, st, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(kPermThreads), 0, st, a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned g = static_cast<unsigned>((a.P + kPermThreads - 1) / kPermThreads);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(g), dim3(kPermThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace moe
