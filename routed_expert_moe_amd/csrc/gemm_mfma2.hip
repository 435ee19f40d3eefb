// Grouped GEMM on bf16 MFMA for prefill-sized tiles:
//     C[rows, n] = A[rows, k] * B_e[n, k]^T,  fp32 accumulation.
//
// Workgroup tile 128 (rows of A) x 512 (rows of B) x 64 (K); eight wavefronts
// side by side, each owning all 128 rows and its own 64 rows of B, as 4 x 2
// blocks of v_mfma_f32_32x32x16_bf16 (128 fp32 accumulators per lane, two
// wavefronts per SIMD).  On one dense 65536 x 4096 x 7168 product the kernel
// runs at 1.2-1.4 PFLOP/s (measured); on routed work, where each expert's
// weights are read by only its own few M-tiles, a step waits for weight rows
// from HBM: the two LDS stages (the whole 160 KiB) give each step's loads one
// step to land.  LDS bank conflicts stay under 1% of LDS cycles.
//
// Operands go from global memory straight into LDS with
// global_load_lds_dwordx4 (two 80 KiB stages; all loads of step k+1 are issued
// as step k starts, which gives them the whole step to land).  Each 1 KiB wave load fills eight
// 128-byte LDS rows; the lane that writes physical chunk p of row r fetches
// logical chunk p ^ ((r >> 1) & 7).  An operand read serves 16 lanes at a time,
// 16 consecutive rows at one logical chunk: two rows share each 256-byte bank
// line, and the swizzle sends the 8 rows of each parity to 8 different chunks,
// so the 16 reads cover all 64 banks once.
//
// Each wavefront loads exactly the B rows it multiplies (for SwiGLU its 32
// gate rows and the 32 matching up rows), so B is private to the wavefront and
// only A is shared: a step waits for the wavefront's own A loads (issued before
// its B loads, and vmcnt counts in order), passes the barrier that makes every
// wavefront's A visible, and only then waits for its own B.  A wavefront whose
// weight rows come late then stalls alone while its SIMD partner keeps the
// MFMA busy; waiting for all loads before the barrier made every wavefront of
// the CU wait for the slowest (8% slower gate/up at V3 prefill).
//
// The MFMA takes the weight fragment as its first operand, so each lane ends
// with four consecutive output columns of one row: one 16-byte store for fp32
// output, one 8-byte LDS store for bf16 output, which is then written to
// memory in whole-row 1 KiB runs per wavefront.
//
// The grid is persistent: one workgroup per CU, the work list (routed tiles x
// column blocks, then the dense segment's) cut into eight contiguous ranges,
// one per XCD (workgroup b runs on XCD b % 8).  Inside each run of up to eight
// M-tiles of one expert the list goes column block by column block, so the
// tiles that read one block of an expert's weights start together on one XCD
// and the block comes from HBM once; in tile-major order an expert's tiles
// often landed in different rounds and each re-read the weights.
//
// Two operand layouts:
//   NT  C = A B_e^T, both k-contiguous (the forward).
//   NN  C = A B_e with B_e stored [k][n] (the backward's row-form products):
//       each K step stages 64 k-rows of 512 columns as 1 KiB LDS rows.
// The k-strided tile stores the 64-byte block b of k-row r at block b ^ (r & 3)
// and its MFMA operand (8 consecutive k of one column per lane) is read with
// two ds_read_b64_tr_b16.  The LDS serves those 8-byte reads 32 lanes at a
// time, four k-rows x 64 bytes, which the swizzle puts on four disjoint bank
// ranges.
//
// Routed tiles skip the MFMAs and fragment reads of 32-row blocks that hold
// only padding (an expert's last tile): on a 256-expert, top-8 routing of 8192
// tokens that is 15% of the routed MFMA work.  Skipped blocks store zeros.
//
// Requires K % 64 == 0.  Rows outside the valid range are clamped to a valid
// row; their results are never stored (dense) or never read (routed padding).
#include "common.hpp"
#include <type_traits>

namespace moe {
namespace {

constexpr int BM = 128, BN = 512, BK = 64;
constexpr int kWaves = 8;                               // wavefronts per workgroup, side by side
constexpr int kThreads = 64 * kWaves;
constexpr int NJ = BN / kWaves / 32;                    // 32-row B sub-tiles per wavefront
constexpr int kStages = 2;
constexpr int kRowBytes = BK * 2;                       // 128 B per LDS row
constexpr int kATileBytes = BM * kRowBytes;             // 16 KiB
constexpr int kBTileBytes = BN * kRowBytes;             // 64 KiB
constexpr int kStageBytes = kATileBytes + kBTileBytes;  // 80 KiB
constexpr int kLdsBytes = kStages * kStageBytes;        // 160 KiB
constexpr int kXcds = 8;
constexpr int kGroup = 8;                               // M-tiles whose items interleave
constexpr int kALoads = BM * kRowBytes / 1024 / kWaves;  // wave loads of A per wavefront
constexpr int kBLoads = BN * kRowBytes / 1024 / kWaves;  // wave loads of B per wavefront
constexpr int kLoads = kALoads + kBLoads;                // per wavefront per K step

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

struct Work2 {
  Segment seg[2];
  int nseg;
  int nblk_n[2];
};

__device__ __forceinline__ void load_lds16(const void *g, char *lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t *)(g), (lds_void_t *)(lds_wave_base), 16, 0, 0);
}

// s_waitcnt immediate for gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// two 4 x bf16 transposed reads -> one MFMA operand of 8 bf16
__device__ __forceinline__ bf16x8_t join_tr(v4i16_t lo, v4i16_t hi) {
  const u32x4_t v = {static_cast<uint32_t>(static_cast<uint16_t>(lo[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[1])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(lo[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[3])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(hi[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[1])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(hi[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[3])) << 16)};
  return __builtin_bit_cast(bf16x8_t, v);
}

constexpr int kLayNT = 0, kLayNN = 1;

// byte offset of (k-row r, tile column c) in a k-strided stage of ROW-byte rows
template <int ROW>
__device__ __forceinline__ int kt_off(int r, int c) { return r * ROW + (((c >> 5) ^ (r & 3)) << 6) + ((c * 2) & 63); }

// MFMA operand of tile columns [cb, cb + 32), K slice s from a k-strided stage:
// lane 16g + q addresses k-row kr + q/4, columns cb + 16(g&1) + 4(q%4); lane
// 16g + l receives column cb + 16(g&1) + l of k-rows kr .. kr+3, then kr+4 .. kr+7
template <int ROW>
__device__ __forceinline__ bf16x8_t frag_kt(const char *base, int cb, int s, int lane) {
  const int g = lane >> 4, q = lane & 15;
  const int kr = 16 * s + 8 * (g >> 1) + (q >> 2);
  const int col = cb + 16 * (g & 1) + 4 * (q & 3);
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(base + kt_off<ROW>(kr, col)));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(base + kt_off<ROW>(kr + 4, col)));
  return join_tr(lo, hi);
}

template <int EPI, bool OUT_F32, int LAY>
__global__ __launch_bounds__(kThreads, 1) void gemm_mfma2_kernel(Work2 wk) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, khalf = lane >> 5;
  const int lrow = lane >> 3, pch = lane & 7;    // DMA: row within the 8-row wave load, chunk

  // ---- work list: segment 0 tiles x column blocks, then segment 1
  const int tiles0 = uniform(wk.seg[0].n_tiles_dev ? *wk.seg[0].n_tiles_dev : wk.seg[0].n_tiles_host);
  const int items0 = tiles0 * wk.nblk_n[0];
  const int items1 = wk.nseg > 1 ? wk.seg[1].n_tiles_host * wk.nblk_n[1] : 0;
  const int total = items0 + items1;
  const int nloc = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
  const int chunk = ((total + kXcds - 1) / kXcds + 7) / 8 * 8;   // whole groups stay on one XCD more often
  const int w_end = min(total, (xcd + 1) * chunk);

  for (int w = xcd * chunk + loc; w < w_end; w += nloc) {
    const int si = w < items0 ? 0 : 1;
    const Segment &sg = wk.seg[si];
    const int local = si == 0 ? w : w - items0;
    const bool dense = sg.n_tiles_dev == nullptr;
    // Within a run of up to kGroup M-tiles of one expert (every tile of a dense
    // segment shares one B), items go column block by column block, so the
    // tiles reading the same block of B are adjacent in the list, run side by
    // side on one XCD and fetch that block from HBM once.
    int tile, nb;
    {
      const int nbk = wk.nblk_n[si];
      const int slot = local / nbk;
      int first, last;
      if (dense) {
        first = 0;
        last = sg.n_tiles_host;
      } else {
        const int e = sg.tile_expert[slot];
        first = sg.expert_off[e] / BM;
        last = sg.expert_off[e + 1] / BM;
      }
      const int g0 = first + (slot - first) / kGroup * kGroup;
      const int gs = min(kGroup, last - g0);
      const int lg = local - g0 * nbk;
      nb = uniform(lg / gs);
      tile = uniform(g0 + lg - nb * gs);
    }
    const int row0 = uniform(dense ? tile * BM : sg.tile_row[tile]);
    const int expert = uniform(dense ? 0 : sg.tile_expert[tile]);
    const int K = sg.k;
    const int nk = K / BK;
    const int half_n = sg.n / 2;

    // ---- global sources of this lane's DMA rows
    const uint16_t *A = static_cast<const uint16_t *>(sg.a);
    const uint16_t *asrc[kALoads];
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
      const int r = (wave * kALoads + i) * 8 + lrow;    // A tile row
      const int grow = row0 + r;
      int64_t arow;
      if (sg.gather != nullptr) {
        const int pair = sg.gather[grow];
        arow = pair >= 0 ? pair / sg.topk : 0;
      } else {
        arow = (!dense || grow < sg.a_rows) ? grow : sg.a_rows - 1;
      }
      asrc[i] = A + arow * sg.lda + (pch ^ swz(r)) * 8;
    }
    const uint16_t *Bm = static_cast<const uint16_t *>(sg.b) + static_cast<int64_t>(expert) * sg.b_stride;
    // first B tile row of this wavefront's load i: the rows it multiplies, so B is
    // private to the wavefront (SwiGLU: 32 gate rows, then the 32 matching up rows)
    auto brow0 = [&](int i) -> int {
      if (EPI == EPI_SWIGLU && LAY == kLayNT)
        return i < kBLoads / 2 ? wave * (BN / 2 / kWaves) + 8 * i : BN / 2 + wave * (BN / 2 / kWaves) + 8 * (i - kBLoads / 2);
      return (wave * kBLoads + i) * 8;
    };
    auto bptr = [&](int i, int kt) -> const uint16_t * {
      if (LAY == kLayNN) {   // k-row kr of the step; this lane fills physical 16-byte chunk `lane` of its LDS row
        const int kr = wave * kBLoads + i;
        int col = nb * BN + ((((lane >> 2) ^ (kr & 3)) << 5) | ((lane & 3) << 3));
        if (col > sg.n - 8) col = sg.n - 8;
        return Bm + static_cast<int64_t>(kt * BK + kr) * sg.ldb + col;
      }
      const int r = brow0(i) + lrow;    // B tile row (the rows this wavefront reads)
      int brow;
      if (EPI == EPI_SWIGLU) {
        const int col = nb * (BN / 2) + (r & (BN / 2 - 1));
        const int c = col < half_n ? col : half_n - 1;
        brow = r < BN / 2 ? c : half_n + c;
      } else {
        brow = nb * BN + r;
        if (brow >= sg.n) brow = sg.n - 1;
      }
      return Bm + static_cast<int64_t>(brow) * K + (pch ^ swz(r)) * 8 + kt * BK;
    };
    auto issue_one = [&](int li, int kt) {
      char *st = lds + (kt & 1) * kStageBytes;
      const int k0 = kt * BK;
      if (li < kALoads)
        load_lds16(asrc[li] + k0, st + (wave * kALoads + li) * 1024);
      else
        load_lds16(bptr(li - kALoads, kt), st + kATileBytes + brow0(li - kALoads) * kRowBytes);
    };

    f32x16_t acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // LDS rows read by this lane: A rows i*32 + l32; B rows of sub-tile j
    // SwiGLU: sub-tiles [0, NJ/2) are gate rows, [NJ/2, NJ) the matching up rows
    int brow_l[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      brow_l[j] = (EPI == EPI_SWIGLU ? (j / (NJ / 2)) * (BN / 2) + wave * (NJ / 2) * 32 + (j % (NJ / 2)) * 32
                                     : wave * NJ * 32 + j * 32) + l32;

    // 32-row blocks of this tile that hold real rows: routed padding (sorted_pair < 0)
    // sits at the end of an expert's last tile, and its MFMAs are skipped
    int nblk = 4;
    if (sg.row_pair != nullptr) {
      nblk = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) nblk += sg.row_pair[row0 + 32 * i] >= 0 ? 1 : 0;
    } else if (dense) {
      nblk = min(4, (sg.a_rows - row0 + 31) / 32);
    }
    nblk = uniform(nblk);

    auto kloop = [&](auto nbc) {
      constexpr int NB = decltype(nbc)::value;
      auto read_frags = [&](const char *st, int s, bf16x8_t (&af)[NB], bf16x8_t (&bf)[NJ]) {
        const u32x4_t *As = reinterpret_cast<const u32x4_t *>(st);
        const u32x4_t *Bs = reinterpret_cast<const u32x4_t *>(st + kATileBytes);
        const int c = 2 * s + khalf;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const int r = i * 32 + l32;
          af[i] = __builtin_bit_cast(bf16x8_t, As[r * 8 + (c ^ swz(r))]);
        }
        if (LAY == kLayNN) {
#pragma unroll
          for (int j = 0; j < NJ; ++j) bf[j] = frag_kt<BN * 2>(st + kATileBytes, brow_l[j] - l32, s, lane);
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j) {
            const int r = brow_l[j];
            bf[j] = __builtin_bit_cast(bf16x8_t, Bs[r * 8 + (c ^ swz(r))]);
          }
        }
      };
#pragma unroll
      for (int li = 0; li < kLoads; ++li) issue_one(li, 0);
      for (int kt = 0; kt < nk; ++kt) {
        // stage kt: this wavefront's A rows (issued before its B rows) have landed;
        // the barrier makes every wavefront's A rows visible, then its own B rows
        // (in the k-strided layout every wavefront reads every k-row of B: wait for all)
        if (LAY == kLayNN) __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        else __builtin_amdgcn_s_waitcnt(waitcnt_vm(kBLoads));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        const char *st = lds + (kt & 1) * kStageBytes;
        const bool more = kt + 1 < nk;
        bf16x8_t af[2][NB], bf[2][NJ];
        read_frags(st, 0, af[0], bf[0]);
#pragma unroll
        for (int s = 0; s < BK / 16; ++s) {
          if (more && s == 0) {   // all loads of step kt+1 (the other stage is free)
#pragma unroll
            for (int q = 0; q < kLoads; ++q) issue_one(q, kt + 1);
          }
          if (s + 1 < BK / 16) read_frags(st, s + 1, af[(s + 1) & 1], bf[(s + 1) & 1]);
#pragma unroll
          for (int i = 0; i < NB; ++i)
#pragma unroll
            for (int j = 0; j < NJ; ++j)   // weight fragment first: lanes end with 4 consecutive columns
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s & 1][j], af[s & 1][i], acc[i][j], 0, 0, 0);
        }
        // schedule: the fragment reads of K-slice s+1 go one by one between the MFMAs of
        // slice s, so each wavefront waits on LDS once per slice (left alone, the compiler
        // reused one fragment set and waited every two to four MFMAs)
        constexpr int NM = NB * NJ, ND = NB + (LAY == kLayNN ? 2 : 1) * NJ;
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
    };
    switch (nblk) {
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      default: kloop(std::integral_constant<int, 4>{}); break;
    }
    __syncthreads();   // all waves done with both stages before the next item refills them

    // ---- epilogue.  acc[i][j][4g + t] is C[row i*32 + l32][col j*32 + 8g + 4*khalf + t].
    // bf16 results go through LDS (both stages are free now): each lane writes its
    // 4 consecutive columns as one 8-byte LDS store, then every wavefront writes
    // 1 KiB runs of whole output rows (eight full 128-byte lines per store).
    if (OUT_F32) {
      float *C = static_cast<float *>(sg.c);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int grow = row0 + i * 32 + l32;
        if (dense && grow >= sg.a_rows) continue;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = nb * BN + wave * NJ * 32 + j * 32 + 8 * g + 4 * khalf;
            if (col >= sg.n) continue;
            const f32x4_t v = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
            *reinterpret_cast<f32x4_t *>(C + static_cast<int64_t>(grow) * sg.ldc + col) = v;
          }
      }
    } else {
      constexpr int OUTC = EPI == EPI_SWIGLU ? BN / 2 : BN;   // output columns of the tile
      constexpr int LDR = OUTC * 2 + 16;                       // padded LDS row, bytes
      char *ot = lds;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = i * 32 + l32;
        if (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int jj = 0; jj < NJ / 2; ++jj)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int lc = wave * (NJ / 2) * 32 + jj * 32 + 8 * g + 4 * khalf;
              float h[4];
#pragma unroll
              for (int t = 0; t < 4; ++t) h[t] = silu_mul(acc[i][jj][4 * g + t], acc[i][jj + NJ / 2][4 * g + t]);
              uint2 v;
              v.x = pack_bf16x2(h[0], h[1]);
              v.y = pack_bf16x2(h[2], h[3]);
              *reinterpret_cast<uint2 *>(ot + lr * LDR + lc * 2) = v;
              __builtin_amdgcn_sched_barrier(0);   // keep accumulator reads next to their store
            }
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int lc = wave * NJ * 32 + j * 32 + 8 * g + 4 * khalf;
              uint2 v;
              v.x = pack_bf16x2(acc[i][j][4 * g], acc[i][j][4 * g + 1]);
              v.y = pack_bf16x2(acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]);
              *reinterpret_cast<uint2 *>(ot + lr * LDR + lc * 2) = v;
              __builtin_amdgcn_sched_barrier(0);
            }
        }
      }
      __syncthreads();
      constexpr int CPR = OUTC / 8;                  // 16-byte chunks per row
      const int ncols = EPI == EPI_SWIGLU ? half_n : sg.n;
      const int col0 = nb * OUTC;
      for (int cidx = threadIdx.x; cidx < BM * CPR; cidx += kThreads) {
        const int lr = cidx / CPR, cc = cidx - lr * CPR;
        const int grow = row0 + lr, gcol = col0 + cc * 8;
        if ((dense && grow >= sg.a_rows) || gcol >= ncols) continue;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ot + lr * LDR + cc * 16);
        *reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(sg.c) + static_cast<int64_t>(grow) * sg.ldc + gcol) = v;
      }
      __syncthreads();   // the next item's loads refill this LDS
    }
    // gfx9 counts stores in vmcnt: drain them so the next item's waits count only its loads
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
}

template <int EPI, bool OUT_F32, int LAY = kLayNT>
hipError_t launch_one(const Work2 &wk, int grid, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(&gemm_mfma2_kernel<EPI, OUT_F32, LAY>), kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_mfma2_kernel<EPI, OUT_F32, LAY>), dim3(grid), dim3(kThreads), kLdsBytes, st, wk);
  return hipGetLastError();
}

}  // namespace

bool gemm_mfma2_supported(const Segment *segs, int nseg) {
  for (int s = 0; s < nseg; ++s)
    if (segs[s].k % BK != 0 || segs[s].k <= 0 || segs[s].n % 8 != 0 || segs[s].ldc % 8 != 0) return false;
  return true;
}

namespace {
// the work list of the segments; returns its capacity in items
int64_t fill_work(const Segment *segs, int nseg, Epilogue epi, Work2 &wk) {
  wk.nseg = nseg;
  int64_t cap = 0;
  for (int s = 0; s < nseg; ++s) {
    wk.seg[s] = segs[s];
    const int ncols = epi == EPI_SWIGLU ? segs[s].n / 2 : segs[s].n;
    const int per = epi == EPI_SWIGLU ? BN / 2 : BN;
    wk.nblk_n[s] = (ncols + per - 1) / per;
    cap += static_cast<int64_t>(segs[s].n_tiles_host) * wk.nblk_n[s];
  }
  return cap;
}

int grid_size() {
  const int grid = device_cu_count() / kXcds * kXcds;
  return grid < kXcds ? kXcds : grid;
}
}  // namespace

hipError_t launch_gemm_mfma2(const Segment *segs, int nseg, Epilogue epi, bool out_f32,
                             hipStream_t st) {
  Work2 wk{};
  const int64_t cap = fill_work(segs, nseg, epi, wk);
  if (cap == 0) return hipSuccess;
  if (cap >= (1ll << 31)) return hipErrorInvalidValue;
  const int grid = grid_size();
  if (epi == EPI_SWIGLU) return launch_one<EPI_SWIGLU, false>(wk, grid, st);
  if (out_f32) return launch_one<EPI_STORE, true>(wk, grid, st);
  return launch_one<EPI_STORE, false>(wk, grid, st);
}

bool gemm_mfma2_bt_supported(const Segment *segs, int nseg) {
  for (int s = 0; s < nseg; ++s)
    if (segs[s].k % BK != 0 || segs[s].k <= 0 || segs[s].n % 8 != 0 || segs[s].n < 8 || segs[s].ldc % 4 != 0)
      return false;
  return true;
}

hipError_t launch_gemm_mfma2_bt(const Segment *segs, int nseg, hipStream_t st) {
  Work2 wk{};
  const int64_t cap = fill_work(segs, nseg, EPI_STORE, wk);
  if (cap == 0) return hipSuccess;
  if (cap >= (1ll << 31)) return hipErrorInvalidValue;
  return launch_one<EPI_STORE, true, kLayNN>(wk, grid_size(), st);
}

}  // namespace moe
