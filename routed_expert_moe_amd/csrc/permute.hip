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
//
// With 128-row tiles the scan also lists each expert's row chunks for the
// prefill GEMM (write_units below): an expert's rows are cut into chunks of up
// to kChunkTiles 128-row tiles, and a chunk of n tiles is computed as one tile
// of 128*mw rows with mw = chunk_units(n) (1, 2, 4, 4 for n = 1, 2, 3, 4), so
// that one workgroup holds every row of the chunk and reads each weight row
// once.  The table has one entry per 128-row unit of mw (a chunk of mw units),
// in expert order.
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
  int32_t *units;       // [max units][4] chunk table (TM == 128), or nullptr
  int32_t *n_units;     // [1]
  int id_bits;          // bits of the largest expert id (E - 1)
};


// the chunk entries of expert e: rows [off, off + padded), `cnt` of them real;
// entry {first row, end of its real rows, expert, (mw << 8) | unit within the chunk}
__device__ void write_units(const PermArgs &a, int e, int off, int cnt, int padded, int u0) {
  const int n128 = padded / 128;
  const int nch = (n128 + kChunkTiles - 1) / kChunkTiles;
  int u = u0;
  for (int c = 0; c < nch; ++c) {
    const int tiles = min(kChunkTiles, n128 - kChunkTiles * c);
    const int mw = chunk_units(tiles);
    const int row0 = off + 128 * kChunkTiles * c;
    const int real_end = min(row0 + 128 * tiles, off + cnt);
    for (int j = 0; j < mw; ++j, ++u) {
      int32_t *d = a.units + 4 * static_cast<int64_t>(u);
      d[0] = row0;
      d[1] = real_end;
      d[2] = e;
      d[3] = (mw << 8) | j;
    }
  }
}

// inclusive scan of v[0, kMaxE) in LDS: every thread takes two consecutive entries, each
// wavefront scans its 64 pair sums by shuffles, and the wavefront totals are added in
// wavefront order (two barriers; integer sums, so the result is exact)
__device__ void scan_lds(int *v) {
  static_assert(kMaxE == 2 * kPermThreads, "two entries per thread");
  __shared__ int s_wave[kPermWaves];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int lo = v[2 * t], hi = v[2 * t + 1];
  int x = lo + hi;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  for (int w = 0; w < wave; ++w) x += s_wave[w];
  v[2 * t] = x - hi;
  v[2 * t + 1] = x;
  __syncthreads();
}

// the chunk table from counts and padded ends (TM == 128); s_u is LDS scratch of kMaxE
__device__ void build_units(const PermArgs &a, const int *s_cnt_e, const int *s_end, int *s_u) {
  for (int e = threadIdx.x; e < kMaxE; e += kPermThreads) {
    const int start = e > 0 ? s_end[e - 1] : 0;
    s_u[e] = e < a.E ? units_of_tiles((s_end[e] - start) / 128) : 0;
  }
  __syncthreads();
  scan_lds(s_u);
  for (int e = threadIdx.x; e < a.E; e += kPermThreads) {
    const int start = e > 0 ? s_end[e - 1] : 0;
    const int u0 = e > 0 ? s_u[e - 1] : 0;
    write_units(a, e, start, s_cnt_e[e], s_end[e] - start, u0);
  }
  if (threadIdx.x == 0) *a.n_units = s_u[kMaxE - 1];
}

// lanes of the wavefront holding the same expert id as this lane (e >= 0; lanes with e < 0
// are in nobody's set): one ballot per bit of the id, so the cost is log2(E) ballots however
// many distinct experts the 64 lanes hold
__device__ __forceinline__ uint64_t same_expert_lanes(int e, int id_bits) {
  uint64_t same = __ballot(e >= 0);
  for (int b = 0; b < id_bits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  return same;
}

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
    const uint64_t m = same_expert_lanes(e, a.id_bits);
    const int rank = __popcll(m & below), same = __popcll(m);
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
__device__ void scan_all(const PermArgs &a, int *s_pad, int *s_cnt_e, int *s_u) {
  for (int e = threadIdx.x; e < a.E; e += kPermThreads) {
    // exclusive prefix over the count workgroups, 32 histogram entries loaded at a time
    // (one dependent load per entry left a global round trip per workgroup; the V3
    // prefill batch has 32 count workgroups, so one round trip)
    int run = 0;
    constexpr int kBatch = 32;
    for (int b0 = 0; b0 < a.nblk; b0 += kBatch) {
      int v[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        v[i] = b0 + i < a.nblk ? a.hist[static_cast<int64_t>(b0 + i) * a.E + e] : 0;
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (b0 + i < a.nblk) a.hist[static_cast<int64_t>(b0 + i) * a.E + e] = run;
        run += v[i];
      }
    }
    a.counts[e] = run;
    s_cnt_e[e] = run;
    s_pad[e] = (run + a.TM - 1) / a.TM * a.TM;
  }
  for (int e = a.E + threadIdx.x; e < kMaxE; e += kPermThreads) s_pad[e] = 0;
  __syncthreads();
  scan_lds(s_pad);
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
  if (a.units != nullptr) build_units(a, s_cnt_e, s_pad, s_u);
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
  __shared__ int s_cnt_e[kMaxE];
  __shared__ int s_u[kMaxE];
  scan_all(a, s_pad, s_cnt_e, s_u);
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
  __shared__ int s_u[kMaxE];                 // chunk units per expert, then their inclusive scan
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
    const uint64_t m = same_expert_lanes(e, a.id_bits);
    const int rank = __popcll(m & below), same = __popcll(m);
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
  scan_lds(s_end);
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
  if (a.units != nullptr) build_units(a, s_tot, s_end, s_u);
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

// scratch of a routing buffer: local ranks [P], histograms [nblk][E], then the
// chunk table: n_units (padded to 4 ints) and [max units][4] entries.  An
// expert of n 128-row tiles has at most n + 1 units, and sum n <= P/128 + E.
int64_t permute_units_offset(int64_t P, int E) {
  const int64_t nblk = (P + kPairsPerBlock - 1) / kPairsPerBlock;
  return (P + nblk * E + 3) / 4 * 4;   // 16-byte aligned entries
}
int64_t permute_max_units(int64_t P, int E) { return P / 128 + 2 * static_cast<int64_t>(E) + 2; }
int64_t permute_scratch_ints(int64_t P, int E) {
  return permute_units_offset(P, E) + 4 + 4 * permute_max_units(P, E);
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
  a.units = nullptr;
  a.n_units = nullptr;
  a.id_bits = 0;
  while ((1 << a.id_bits) < a.E) ++a.id_bits;   // ids 0 .. E-1 fit in id_bits bits
  if (a.TM == 128) {
    int32_t *u = r.scratch + permute_units_offset(a.P, a.E);
    a.n_units = u;
    a.units = u + 4;
  }
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
