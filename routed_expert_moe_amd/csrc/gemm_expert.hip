// Grouped GEMM of the forward expert FFNs on bf16 MFMA, one expert's rows per tile:
//     C[rows, n] = A[rows, k] * B_e[n, k]^T,  fp32 accumulation, bf16 output.
//
// The routed experts of a prefill batch receive a few hundred rows each
// (DeepSeek-V3 notes page, "DeepSeekMoE" paragraph: fine-grained experts, so
// each expert's FFN sees a small share of the tokens), so the expert weights,
// read in full for every expert, are most of the traffic.  A tile of 128 rows
// leaves an expert with 250 rows to two tiles that each read the whole weight
// matrix and share it through L2 only while they stay in step.  Here one
// workgroup takes a chunk of up to 128 * kChunkTiles rows of one expert (the
// chunk table the dispatch writes) as one tile of M = 128*mw rows by N = 512/mw
// weight rows (mw = chunk_units of the chunk's 128-row tiles), so each weight row
// of a chunk is loaded by exactly one workgroup, while the chunk's activation
// rows are shared by the workgroups of its column blocks, which are consecutive
// in the work list and run side by side on one XCD (its L2 holds them).
//
// Every shape keeps the same work per wavefront: 128 rows (four 32-row blocks)
// by 64 weight rows, as 4 x 2 v_mfma_f32_32x32x16_bf16 blocks (128 fp32
// accumulators per lane, two wavefronts per SIMD).  The eight wavefronts form
// mw row groups by 8/mw column groups; row group m holds the 32-row blocks m,
// m + mw, m + 2 mw, m + 3 mw of the tile, so the blocks of a partly filled tile
// (an expert's last chunk) spread over the four SIMDs.  Blocks past the chunk's
// real rows skip their MFMAs and fragment reads; their A rows load row 0.
//
// Operands go from global memory straight into LDS by buffer_load ... lds.  Rows
// are 128 bytes in LDS; the lane that writes physical chunk p of row r fetches
// logical chunk p ^ ((r >> 1) & 7), which makes the 16-row fragment reads
// conflict-free across the 64 banks.  Measured at V3 prefill, the step time is
// set by the weight stream from HBM (with the weight loads removed the gate/up
// launch takes about as long as with no loads at all), so the pipeline gives the
// weights the most time: with 256 x 256 tiles (mw = 2) a step's operands are
// 32 KiB each, and two A stages plus three B stages (160 KiB) let the weight
// rows load two steps ahead; 128 x 512 tiles (mw = 1) use two stages of 80 KiB.
// With mw = 1 each wavefront loads exactly the weight rows it multiplies (its
// gate rows and the matching up rows for SwiGLU), so a step waits for its own A
// loads, passes the barrier that makes every wavefront's A rows visible, then
// waits for its own weight rows; with mw > 1 weight rows are shared by mw
// wavefronts and a step waits for its loads before the barrier.
//
// The grid is persistent (one workgroup per CU).  Work items are (unit, column
// block) of the routed chunk table, then the dense segment's (the shared
// expert, cut into chunks the same way); the list is split into eight
// contiguous ranges, one per XCD (workgroup b runs on XCD b % 8).
//
// Epilogue: SwiGLU (silu(gate) * up in fp32) or plain; the bf16 tile is staged
// in LDS and written as whole row runs with the non-temporal hint (h and y_pairs are
// read back only after the whole launch, long evicted; 1-2% faster per launch at V3).
// Only rows that hold a real pair (routed) or a token (dense) are written; padding
// rows keep unspecified values.
// A training forward can also keep the SwiGLU's inputs: with c_save set, each
// real row's gate and up pre-activations are stored in fp32 straight from the
// accumulators (16 bytes per lane), so the backward need not recompute them.
#include "common.hpp"
#include <type_traits>

namespace moe {
namespace {

constexpr int BK = 64;                           // K step (bf16 elements = 128 bytes per row)
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowBytes = BK * 2;
constexpr int kStageBytes = 80 * 1024;           // (M + N) * 128 bytes for mw = 1 and 4; 64 KiB for mw = 2
constexpr int kLdsBytes = 2 * kStageBytes;       // 160 KiB
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void lds_void_t;

struct ExpertWork {
  Segment seg[2];          // seg[0] routed (chunk table), seg[1] dense (optional)
  int nseg;
  int nb1[2];              // column blocks of a 512-row (mw = 1) tile, per segment
  const int32_t *units;    // routed chunk table: {row0, real_end, expert, (mw << 8) | unit in chunk}
  const int32_t *n_units;  // [1] entries in use
};

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                           char *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(lds_wave_base), 16, voff, soff, 0, 0);
}
// s_waitcnt immediate for gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
// a pointer held in SGPRs (the buffer descriptors built from it must be wavefront-uniform)
template <typename T>
__device__ __forceinline__ T *uptr(T *p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T *>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_expert_kernel(ExpertWork wk) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, khalf = lane >> 5;
  const int lrow = lane >> 3, pch = lane & 7;    // DMA: row within the 8-row wave load, 16-byte chunk

  // ---- work list: routed units x column blocks, then the dense segment's
  const int units0 = uniform(*wk.n_units);
  const int items0 = units0 * wk.nb1[0];
  int dense_units = 0;
  if (wk.nseg > 1) {
    dense_units = units_of_tiles((wk.seg[1].a_rows + 127) / 128);
  }
  const int items1 = wk.nseg > 1 ? dense_units * wk.nb1[1] : 0;
  const int total = items0 + items1;
  const int nloc = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
  const int chunk = (total + kXcds - 1) / kXcds;
  const int w_end = min(total, (xcd + 1) * chunk);

  for (int w = xcd * chunk + loc; w < w_end; w += nloc) {
    const bool s1 = w >= items0;
    // the segment's fields, picked without indexing the kernel-argument array (a
    // runtime index made the compiler copy it to scratch and treat every field as divergent)
#define SEGF(f) (s1 ? wk.seg[1].f : wk.seg[0].f)
    const void *a_base = uptr(SEGF(a));
    const int64_t lda = SEGF(lda);
    const int32_t *gather = uptr(SEGF(gather));
    const int topk = uniform(SEGF(topk));
    const int a_rows = uniform(SEGF(a_rows));
    const void *b_base = uptr(SEGF(b));
    const int64_t b_stride = SEGF(b_stride);
    const int n_all = uniform(SEGF(n));
    const int K = uniform(SEGF(k));
    void *c_base = uptr(SEGF(c));
    const int64_t ldc = SEGF(ldc);
    float *c_save = uptr(SEGF(c_save));
    const int64_t ld_save = SEGF(ld_save);
#undef SEGF
    const int local = s1 ? w - items0 : w;
    const int nb1 = s1 ? wk.nb1[1] : wk.nb1[0];
    const int u = local / nb1;
    int row0, real_end, expert, mw, uin;
    if (!s1) {
      const int4 d = reinterpret_cast<const int4 *>(wk.units)[u];
      row0 = uniform(d.x);
      real_end = uniform(d.y);
      expert = uniform(d.z);
      mw = uniform(d.w >> 8);
      uin = uniform(d.w & 255);
    } else {
      constexpr int kFull = chunk_units(kChunkTiles);     // units of a full chunk
      const int c = u / kFull;
      const int t128 = (a_rows - 128 * kChunkTiles * c + 127) / 128;
      mw = chunk_units(min(kChunkTiles, t128));
      uin = u - kFull * c;
      row0 = 128 * kChunkTiles * c;
      real_end = min(row0 + 128 * mw, a_rows);
      expert = 0;
    }
    const int nb = local - (u - uin) * nb1;     // column block among the chunk's mw * nb1
    const int half_n = n_all / 2;
    const int ncols = EPI == EPI_SWIGLU ? half_n : n_all;
    const int nk = K / BK;
    const int nblk_all = (real_end - row0 + 31) / 32;      // 32-row blocks holding real rows

    // one item of tile shape MW (compile-time, so the step's loads, waits and fragment
    // addresses carry no branches)
    auto run_item = [&](auto mwc) __attribute__((always_inline)) {
      constexpr int MW = decltype(mwc)::value;
      constexpr int M = 128 * MW, N = 512 / MW;            // tile rows (A) and weight rows (B)
      constexpr int OUT = EPI == EPI_SWIGLU ? N / 2 : N;   // output columns of the tile
      constexpr int NW = 8 / MW;
      constexpr int NA = 2 * MW, NB_L = 8 / MW;           // wave loads of 8 rows per step: A, B
      if (nb * OUT >= ncols) return;                       // the last chunk's blocks past the matrix
      // wavefront roles: row group m (blocks m + MW*i), column group n (64 weight rows)
      const int n_grp = wave % NW;
      const int m_grp = MW == 4 ? ((wave >> 1) == 2 ? 3 : (wave >> 1) == 3 ? 2 : (wave >> 1)) : wave / NW;
      const int nblk = uniform(nblk_all > m_grp ? min(4, (nblk_all - m_grp + MW - 1) / MW) : 0);

      // ---- DMA sources: 32-bit byte offsets from the matrix bases; the K step goes in soffset
      const auto ra = rsrc(a_base, 0xFFFFFFFFu);
      const uint16_t *Bm = static_cast<const uint16_t *>(b_base) + static_cast<int64_t>(expert) * b_stride;
      const auto rb = rsrc(Bm, 0xFFFFFFFFu);
      // A rows behind this lane's A loads: every gathered index is loaded before any is used;
      // tile rows past the chunk's real rows read row 0 (one line for the whole wave load)
      int arow_v[NA];
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int grow = row0 + (wave * NA + i) * 8 + lrow;
        const int gi = min(grow, real_end - 1);
        const int v = gather != nullptr ? gather[gi] : gi;
        arow_v[i] = grow < real_end ? v : (gather != nullptr ? -1 : 0);
      }
      uint32_t voff[NA + NB_L];
      int lrow_of[NA + NB_L];                              // LDS row of each wave load (uniform)
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int r = (wave * NA + i) * 8 + lrow;
        const int v = arow_v[i];
        const int64_t arow = gather != nullptr ? (v >= 0 ? v / topk : 0) : v;
        voff[i] = static_cast<uint32_t>(arow * lda * 2) + (pch ^ swz(r)) * 16;
        lrow_of[i] = (wave * NA + i) * 8;     // row of the A stage
      }
#pragma unroll
      for (int li = 0; li < NB_L; ++li) {
        int r0, brow;
        if (EPI == EPI_SWIGLU) {   // gate rows of the block, then the matching up rows
          r0 = li < NB_L / 2 ? (wave * (NB_L / 2) + li) * 8 : N / 2 + (wave * (NB_L / 2) + li - NB_L / 2) * 8;
          const int r = r0 + lrow;
          const int col = min(nb * OUT + (r % (N / 2)), half_n - 1);
          brow = r < N / 2 ? col : half_n + col;
        } else {
          r0 = (wave * NB_L + li) * 8;
          brow = min(nb * N + r0 + lrow, n_all - 1);
        }
        voff[NA + li] = static_cast<uint32_t>(brow) * static_cast<uint32_t>(K * 2) + (pch ^ swz(r0 + lrow)) * 16;
        lrow_of[NA + li] = r0;                // row of the B stage
      }
#pragma unroll
      for (int i = 0; i < NA + NB_L; ++i) {
        // keep the offset in its register: left alone, the compiler recomputed the gathered
        // A offsets (a sorted_pair load and an integer division) at every step's DMA issue
        asm volatile("" : "+v"(voff[i]));
      }
      // LDS stages.  With MW == 2 (tiles of 256 x 256) a step's operands are 32 KiB each:
      // two A stages and three B stages fill the 160 KiB, so weight rows (streamed from
      // HBM) are loaded two steps ahead and the shared A rows (L2 hits) one step ahead.
      // Otherwise two stages of (M + N) rows, both operands one step ahead.
      constexpr bool kB3 = MW == 2;
      auto a_st = [&](int kt) __attribute__((always_inline)) -> char * {
        return kB3 ? lds + (kt & 1) * (M * kRowBytes) : lds + (kt & 1) * kStageBytes;
      };
      auto b_st = [&](int kt) __attribute__((always_inline)) -> char * {
        return kB3 ? lds + 2 * M * kRowBytes + (kt % 3) * (N * kRowBytes) : a_st(kt) + M * kRowBytes;
      };
      auto issue_a = [&](int kt) __attribute__((always_inline)) {
        char *st = a_st(kt);
        const uint32_t k0 = static_cast<uint32_t>(kt * BK * 2);
#pragma unroll
        for (int i = 0; i < NA; ++i) load_lds16(ra, voff[i], k0, st + lrow_of[i] * kRowBytes);
      };
      auto issue_b = [&](int kt) __attribute__((always_inline)) {
        char *st = b_st(kt);
        const uint32_t k0 = static_cast<uint32_t>(kt * BK * 2);
#pragma unroll
        for (int i = NA; i < NA + NB_L; ++i) load_lds16(rb, voff[i], k0, st + lrow_of[i] * kRowBytes);
      };
      static_assert(!kB3 || 2 * M * kRowBytes + 3 * N * kRowBytes <= kLdsBytes, "three B stages must fit");

      f32x16_t acc[4][2];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

      // LDS rows this lane reads: A rows (m_grp + MW*i)*32 + l32; B rows of sub-tile j
      // (SwiGLU: j = 0 the 32 gate rows of column group n, j = 1 the matching up rows)
      int brow_l[2];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        brow_l[j] = (EPI == EPI_SWIGLU ? j * (N / 2) + n_grp * 32 : n_grp * 64 + j * 32) + l32;

      auto kloop = [&](auto nbc) __attribute__((always_inline)) {
        constexpr int NB = decltype(nbc)::value;
        auto read_frags = [&](const char *sa, const char *sb, int s, auto &af, bf16x8_t (&bf)[2]) __attribute__((always_inline)) {
          const u32x4_t *arows = reinterpret_cast<const u32x4_t *>(sa);
          const u32x4_t *brows = reinterpret_cast<const u32x4_t *>(sb);
          const int c = 2 * s + khalf;
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            const int r = (m_grp + MW * i) * 32 + l32;
            af[i] = __builtin_bit_cast(bf16x8_t, arows[r * 8 + (c ^ swz(r))]);
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int r = brow_l[j];
            bf[j] = __builtin_bit_cast(bf16x8_t, brows[r * 8 + (c ^ swz(r))]);
          }
        };
        // the loads of the steps after kt, issued after step kt's barrier: the stages they
        // fill were last read in step kt-1.  They go out a quarter per K-slice (issue_part
        // q = 0..3, A loads first, then B, as in issue_next, so the waits count the same
        // loads): eight 1 KiB loads per wavefront at once kept the texture unit's address
        // and command FIFOs full on 12-15% of the cycles, stalling the MFMAs queued behind
        // the loads; spread out, the prefill gate/up launch takes ~2% less time.
        auto issue_part = [&](int kt, auto qc) __attribute__((always_inline)) {
          constexpr int q = decltype(qc)::value, L = NA + NB_L;
          constexpr int lo = q * L / 4, hi = (q + 1) * L / 4;
          const bool a_ok = kt + 1 < nk, b_ok = kB3 ? kt + 2 < nk : kt + 1 < nk;
          const int kb = kB3 ? kt + 2 : kt + 1;
#pragma unroll
          for (int i = lo; i < hi; ++i) {
            if (i < NA) {
              if (a_ok) load_lds16(ra, voff[i], static_cast<uint32_t>((kt + 1) * BK * 2), a_st(kt + 1) + lrow_of[i] * kRowBytes);
            } else {
              if (b_ok) load_lds16(rb, voff[i], static_cast<uint32_t>(kb * BK * 2), b_st(kb) + lrow_of[i] * kRowBytes);
            }
          }
        };
        auto issue_next = [&](int kt) __attribute__((always_inline)) {   // all at once
          if (kB3) {
            if (kt + 1 < nk) issue_a(kt + 1);
            if (kt + 2 < nk) issue_b(kt + 2);
          } else if (kt + 1 < nk) {
            issue_a(kt + 1);
            issue_b(kt + 1);
          }
        };
        issue_a(0);
        issue_b(0);
        if (kB3 && nk > 1) issue_b(1);
        for (int kt = 0; kt < nk; ++kt) {
          if constexpr (MW == 1) {
            // this wavefront's A rows (issued before its weight rows) have landed; the
            // barrier makes every wavefront's A rows visible; then its own weight rows
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(NB_L));
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
          } else if constexpr (kB3) {
            // A(kt) was issued before B(kt+1), the only loads allowed to stay in flight
            if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NB_L));
            else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __builtin_amdgcn_s_barrier();
          } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
            __builtin_amdgcn_s_barrier();
          }
          const char *sa = a_st(kt);
          const char *sb = b_st(kt);
          if constexpr (NB == 0) {   // no real rows in this wavefront's blocks: its loads and barriers only
            issue_next(kt);
          } else {
            bf16x8_t af[2][NB], bf[2][2];
            read_frags(sa, sb, 0, af[0], bf[0]);
#pragma unroll
            for (int s = 0; s < BK / 16; ++s) {
              if (s == 0) issue_part(kt, std::integral_constant<int, 0>{});
              if (s == 1) issue_part(kt, std::integral_constant<int, 1>{});
              if (s == 2) issue_part(kt, std::integral_constant<int, 2>{});
              if (s == 3) issue_part(kt, std::integral_constant<int, 3>{});
              if (s + 1 < BK / 16) read_frags(sa, sb, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
              for (int i = 0; i < NB; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)   // weight fragment first: lanes end with 4 consecutive columns
                  acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s & 1][j], af[s & 1][i], acc[i][j], 0, 0, 0);
            }
            // the fragment reads of K-slice s+1 go one by one between the MFMAs of slice s
            constexpr int NM = NB * 2, ND = NB + 2;
#pragma unroll
            for (int s = 0; s < BK / 16; ++s) {
              if (s + 1 < BK / 16) {
#pragma unroll
                for (int q = 0; q < ND; ++q) {
                  if (q < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                  __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                if (NM > ND) __builtin_amdgcn_sched_group_barrier(0x008, NM - ND, 0);
              } else {
                __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);
              }
            }
          }
        }
      };
      switch (nblk) {
        case 0: kloop(std::integral_constant<int, 0>{}); break;
        case 1: kloop(std::integral_constant<int, 1>{}); break;
        case 2: kloop(std::integral_constant<int, 2>{}); break;
        case 3: kloop(std::integral_constant<int, 3>{}); break;
        default: kloop(std::integral_constant<int, 4>{}); break;
      }
      __syncthreads();   // every wavefront is done with both stages

      // ---- epilogue.  acc[i][j][4g + t] is C[tile row (m_grp + MW*i)*32 + l32]
      //      [tile column n_grp*64 + j*32 + 8g + 4*khalf + t]; SwiGLU pairs j = 0 (gate) with j = 1 (up).
      constexpr int LDR = OUT * 2 + 16;           // padded LDS row, bytes
      char *ot = lds;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i >= nblk) break;
        const int lr = (m_grp + MW * i) * 32 + l32;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int lc = n_grp * 32 + 8 * g + 4 * khalf;
            if (c_save != nullptr && row0 + lr < real_end && nb * OUT + lc < ncols) {
              // the pre-activations a and c of this row's four columns, in fp32
              float *dst = c_save + static_cast<int64_t>(row0 + lr) * ld_save + nb * OUT + lc;
              const f32x4_t av = {acc[i][0][4 * g], acc[i][0][4 * g + 1], acc[i][0][4 * g + 2], acc[i][0][4 * g + 3]};
              const f32x4_t cv = {acc[i][1][4 * g], acc[i][1][4 * g + 1], acc[i][1][4 * g + 2], acc[i][1][4 * g + 3]};
              __builtin_nontemporal_store(av, reinterpret_cast<f32x4_t *>(dst));
              __builtin_nontemporal_store(cv, reinterpret_cast<f32x4_t *>(dst + half_n));
            }
            float h[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) h[t] = silu_mul(acc[i][0][4 * g + t], acc[i][1][4 * g + t]);
            uint2 v;
            v.x = pack_bf16x2(h[0], h[1]);
            v.y = pack_bf16x2(h[2], h[3]);
            *reinterpret_cast<uint2 *>(ot + lr * LDR + lc * 2) = v;
            __builtin_amdgcn_sched_barrier(0);   // keep accumulator reads next to their store
          }
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int lc = n_grp * 64 + j * 32 + 8 * g + 4 * khalf;
              uint2 v;
              v.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
              v.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
              *reinterpret_cast<uint2 *>(ot + lr * LDR + lc * 2) = v;
              __builtin_amdgcn_sched_barrier(0);
            }
        }
      }
      __syncthreads();
      constexpr int CPR = OUT / 8;                // 16-byte chunks per output row
      const int col0 = nb * OUT;
      const int nrows = real_end - row0;
      for (int cidx = threadIdx.x; cidx < nrows * CPR; cidx += kThreads) {
        const int lr = cidx / CPR, cc = cidx - lr * CPR;
        const int gcol = col0 + cc * 8;
        if (gcol >= ncols) continue;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ot + lr * LDR + cc * 16);
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(c_base) + static_cast<int64_t>(row0 + lr) * ldc + gcol));
      }
      __syncthreads();   // the next item's loads refill this LDS
      // gfx9 counts stores in vmcnt: drain them so the next item's waits count only its loads
      __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    };
    if (mw == 1) run_item(std::integral_constant<int, 1>{});
    else if (kChunkTiles <= 2 || mw == 2) run_item(std::integral_constant<int, 2>{});
    else run_item(std::integral_constant<int, 4>{});
  }
}

template <int EPI>
hipError_t launch_one(const ExpertWork &wk, int grid, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(&gemm_expert_kernel<EPI>), kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_expert_kernel<EPI>), dim3(grid), dim3(kThreads), kLdsBytes, st, wk);
  return hipGetLastError();
}

}  // namespace

bool gemm_expert_supported(const Segment *segs, int nseg) {
  for (int s = 0; s < nseg; ++s) {
    const Segment &g = segs[s];
    if (g.k % BK != 0 || g.k <= 0 || g.n % 8 != 0 || g.n < 8 || g.ldc % 8 != 0 || g.lda % 8 != 0) return false;
    // 32-bit byte offsets: every weight matrix, and every A matrix, below 4 GiB
    if (static_cast<int64_t>(g.n) * g.k * 2 >= (1ll << 32)) return false;
    if (s == 1 && g.n_tiles_dev != nullptr) return false;   // the second segment is dense
  }
  return nseg >= 1 && segs[0].n_tiles_dev != nullptr;
}

hipError_t launch_gemm_expert(const Segment *segs, int nseg, Epilogue epi, const int32_t *units,
                              const int32_t *n_units, int64_t a_bytes_max, hipStream_t st) {
  if (a_bytes_max >= (1ll << 32)) return hipErrorInvalidValue;
  ExpertWork wk{};
  wk.nseg = nseg;
  wk.units = units;
  wk.n_units = n_units;
  const int out1 = epi == EPI_SWIGLU ? 256 : 512;
  for (int s = 0; s < nseg; ++s) {
    wk.seg[s] = segs[s];
    const int ncols = epi == EPI_SWIGLU ? segs[s].n / 2 : segs[s].n;
    wk.nb1[s] = (ncols + out1 - 1) / out1;
  }
  if (nseg > 1 && segs[1].a_rows <= 0) wk.nseg = 1;
  int grid = device_cu_count() / kXcds * kXcds;
  if (grid < kXcds) grid = kXcds;
  if (epi == EPI_SWIGLU) return launch_one<EPI_SWIGLU>(wk, grid, st);
  return launch_one<EPI_STORE>(wk, grid, st);
}

}  // namespace moe
