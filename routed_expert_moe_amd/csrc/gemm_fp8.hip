// Grouped GEMM for FP8 W8A8 experts (DeepSeek-R1 analysis page, training-process
// hyper-parameters paragraph: FP8 mixed precision, W8A8; DeepSeek-V3 notes page,
// V3 config table: fp8 experts):
//     C[rows, n] = sum over 128-wide K blocks b of  sa[row][b] * sw[n/128][b] * (A_q B_q^T)_b
// with A_q, B_q e4m3 codes, sa the 1 x 128 activation scales and sw the
// 128 x 128 weight block scales, fp32 accumulation.
//
// Same tiling, LDS layout, DMA loads, swizzle and persistent XCD-partitioned
// work list as the bf16 prefill GEMM: a 128 x 512 tile per workgroup, eight
// wavefronts side by side (128 rows x 64 columns each), two 80 KiB stages, but a
// K step of 128 codes (the same 128 bytes per row) and two
// v_mfma_scale_f32_32x32x64_f8f6f4 per block pair (hardware scales fixed at 1).
//
// Block scales: each accumulator holds the running sum divided by the current
// block's combined scale c_b = sa[row][b] * sw[col block][b] (the activation
// scale raised to at least 2^-80 of the row's largest so far, so the ratio below
// stays finite); moving to block b multiplies it by c_{b-1} / c_b before the
// block's MFMAs, and the epilogue multiplies by the last c.  That is exact up to
// one fp32 rounding per block.
//
// The next step's ten 1 KiB tile loads per wavefront go out in four parts, before and
// in the middle of each K-slice's MFMAs: issued at once after the barrier they kept the
// texture unit's address and command FIFOs full on 27-31% of the cycles and the MFMAs
// behind them waiting (gate/up 3.78 -> 3.2-3.3 ms at V3 prefill).  The last step loads
// block nk-1 once more into the free stage instead of branching around the loads, which
// would split the slice's code.
//
// Routed tiles skip the MFMAs, fragment reads and rescaling of 32-row blocks
// that hold only padding (an expert's last tile); those rows come out as zeros.
//
// Epilogues: EPI_STORE rounds to bf16 (the down projection); EPI_SWIGLU forms
// silu(gate) * up in fp32, stages the 128 x 256 tile in LDS and quantises every
// 128-column run of a row to e4m3 with s = max|h| / 448 (1 for a zero run),
// code = RNE(h / s), writing codes and scales.
#include "common.hpp"
#include <type_traits>

namespace moe {
namespace {

constexpr int BM = 128, BN = 512, BK = 128;             // BK in elements = bytes
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int NJ = BN / kWaves / 32;                    // 2 sub-tiles of 32 weight rows per wavefront
constexpr int kRowBytes = BK;                           // 128 B per LDS row
constexpr int kATileBytes = BM * kRowBytes;             // 16 KiB
constexpr int kBTileBytes = BN * kRowBytes;             // 64 KiB
constexpr int kStageBytes = kATileBytes + kBTileBytes;  // 80 KiB
constexpr int kLdsBytes = 2 * kStageBytes;              // 160 KiB
constexpr int kXcds = 8;
constexpr int kGroup = 8;                               // M-tiles whose items interleave
constexpr int kALoads = BM * kRowBytes / 1024 / kWaves; // 2
constexpr int kBLoads = BN * kRowBytes / 1024 / kWaves; // 8
constexpr int kLoads = kALoads + kBLoads;
constexpr int kScaleRegs = 2;                           // weight scales of up to 128 K blocks
constexpr float kE4m3Max = 448.0f;
// Moving the running sums from a block scale c_prev to a much smaller c multiplies them by
// c_prev / c, which for a block of tiny activations (amax ~ 1e-30) after a large one could
// overflow fp32.  So a row's activation scale is raised to at least 2^-80 times the largest
// it had in the earlier blocks: the sums then stay within 2^80 * 448^2 * K * (weight scale
// spread) of the largest term, far below the fp32 range, and a raised block contributes at
// most 2^-80 of what the row's largest block can.
constexpr float kRelFloor = 0x1p-80f;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;
typedef int v8i_t __attribute__((ext_vector_type(8)));

struct WorkF8 {
  Segment seg[2];
  int nseg;
  int nblk_n[2];
};

// Buffer descriptors keep each matrix base in SGPRs, so a DMA source costs one
// 32-bit VGPR offset (loop-invariant) plus the step's K offset as the scalar offset.
constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kRsrcWord3);
}
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                           char *lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(lds_wave_base), 16, voff, soff, 0, 0);
}
constexpr int waitcnt_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(__float_as_uint(v)), l)));
}

// e4m3 code of v (|v| <= 448 by construction of the scale): round to nearest even
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp8_kernel(WorkF8 wk) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, khalf = lane >> 5;
  const int lrow = lane >> 3, pch = lane & 7;

  const int tiles0 = uniform(wk.seg[0].n_tiles_dev ? *wk.seg[0].n_tiles_dev : wk.seg[0].n_tiles_host);
  const int items0 = tiles0 * wk.nblk_n[0];
  const int items1 = wk.nseg > 1 ? wk.seg[1].n_tiles_host * wk.nblk_n[1] : 0;
  const int total = items0 + items1;
  const int nloc = gridDim.x / kXcds;
  const int xcd = blockIdx.x % kXcds, loc = blockIdx.x / kXcds;
  const int chunk = ((total + kXcds - 1) / kXcds + 7) / 8 * 8;
  const int w_end = min(total, (xcd + 1) * chunk);

  for (int w = xcd * chunk + loc; w < w_end; w += nloc) {
    const int si = w < items0 ? 0 : 1;
    const Segment &sg = wk.seg[si];
    const int local = si == 0 ? w : w - items0;
    const bool dense = sg.n_tiles_dev == nullptr;
    // within a run of up to kGroup M-tiles of one expert, column block by column block
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

    // A row (of the A matrix) behind tile row r; padding rows read row 0
    auto a_row = [&](int r) -> int64_t {
      const int grow = row0 + r;
      if (sg.gather != nullptr) {
        const int pair = sg.gather[grow];
        return pair >= 0 ? pair / sg.topk : 0;
      }
      return (!dense || grow < sg.a_rows) ? grow : sg.a_rows - 1;
    };
    // DMA sources: 32-bit byte offsets from the matrix bases (the host checks
    // that every fp8 operand matrix is below 2 GiB)
    // the lane that fills physical chunk pch of LDS row r fetches logical chunk pch ^ swz(r)
    const auto ra = rsrc(sg.a, 0xFFFFFFFFu);
    uint32_t aoff[kALoads];
#pragma unroll
    for (int i = 0; i < kALoads; ++i) {
      const int r = (wave * kALoads + i) * 8 + lrow;
      aoff[i] = static_cast<uint32_t>(a_row(r) * sg.lda) + (pch ^ swz(r)) * 16;
    }
    // weight row behind B tile row r (SwiGLU: [0, 256) gate rows, [256, 512) the matching up rows)
    auto b_row = [&](int r) -> int {
      if (EPI == EPI_SWIGLU) {
        const int col = nb * (BN / 2) + (r & (BN / 2 - 1));
        const int c = col < half_n ? col : half_n - 1;
        return r < BN / 2 ? c : half_n + c;
      }
      const int brow = nb * BN + r;
      return brow < sg.n ? brow : sg.n - 1;
    };
    const uint8_t *Bm = static_cast<const uint8_t *>(sg.b) + static_cast<int64_t>(expert) * sg.b_stride;
    const auto rb = rsrc(Bm, static_cast<uint32_t>(static_cast<int64_t>(sg.n) * K));
    uint32_t boff[kBLoads];
#pragma unroll
    for (int i = 0; i < kBLoads; ++i) {
      const int r = (wave * kBLoads + i) * 8 + lrow;
      boff[i] = static_cast<uint32_t>(b_row(r)) * static_cast<uint32_t>(K) + (pch ^ swz(r)) * 16;
    }
    // part q (of 4) of the kLoads tile loads of step kt into `stage`: A loads first, then B;
    // every wavefront waits for all of them at the next step, so the order needs no care
    auto issue_part = [&](int kt, int stage, int q) {
      char *st = lds + stage * kStageBytes;
      const uint32_t k0 = static_cast<uint32_t>(kt * BK);
#pragma unroll
      for (int l = 0; l < kLoads; ++l) {
        if (l < q * kLoads / 4 || l >= (q + 1) * kLoads / 4) continue;
        if (l < kALoads) load_lds16(ra, aoff[l], k0, st + (wave * kALoads + l) * 1024);
        else load_lds16(rb, boff[l - kALoads], k0, st + kATileBytes + (wave * kBLoads + l - kALoads) * 1024);
      }
    };
    auto issue = [&](int kt) {
      char *st = lds + (kt & 1) * kStageBytes;
      const uint32_t k0 = static_cast<uint32_t>(kt * BK);
#pragma unroll
      for (int i = 0; i < kALoads; ++i) load_lds16(ra, aoff[i], k0, st + (wave * kALoads + i) * 1024);
#pragma unroll
      for (int i = 0; i < kBLoads; ++i) load_lds16(rb, boff[i], k0, st + kATileBytes + (wave * kBLoads + i) * 1024);
    };

    // LDS rows this lane multiplies: A rows i*32 + l32; B rows of sub-tile j
    int brow_l[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      brow_l[j] = (EPI == EPI_SWIGLU ? (j / (NJ / 2)) * (BN / 2) + wave * (NJ / 2) * 32 + (j % (NJ / 2)) * 32
                                     : wave * NJ * 32 + j * 32) + l32;
    // scales: the activation scales of this lane's four output rows (one per i block),
    // the weight scales of the two 32-row sub-tiles (K block b in lane b % 64 of swv[j][b / 64])
    const auto rs = rsrc(sg.a_scale, 0xFFFFFFFFu);
    uint32_t soff_m[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) soff_m[i] = static_cast<uint32_t>(a_row(i * 32 + l32) * sg.a_sld * 4);
    auto ascale = [&](int i, int kb) -> float {
      return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, soff_m[i], kb * 4, 0));
    };
    float swv[NJ][kScaleRegs];
    {
      const float *ws = sg.b_scale + static_cast<int64_t>(expert) * sg.s_stride;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int wrow = b_row(brow_l[j] - l32);   // first weight row of the sub-tile
        const float *srow = ws + static_cast<int64_t>(wrow / 128) * nk;
#pragma unroll
        for (int q = 0; q < kScaleRegs; ++q) swv[j][q] = srow[min(q * 64 + lane, nk - 1)];
      }
    }
    auto wscale = [&](int j, int kb) -> float {
      const float s0 = lane_f32(swv[j][0], kb & 63), s1 = lane_f32(swv[j][1], kb & 63);
      return kb < 64 ? s0 : s1;
    };

    f32x16_t acc[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    auto read_frag = [&](const char *base, int r, int s) -> v8i_t {
      const u32x4_t *rows = reinterpret_cast<const u32x4_t *>(base);
      const int c0 = 4 * s + 2 * khalf;   // 32 bytes = chunks c0, c0+1 of the 128-byte row
      const u32x4_t lo = rows[r * 8 + (c0 ^ swz(r))];
      const u32x4_t hi = rows[r * 8 + ((c0 + 1) ^ swz(r))];
      const v8i_t v = {static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                       static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                       static_cast<int>(hi[2]), static_cast<int>(hi[3])};
      return v;
    };

    // 32-row blocks of this tile that hold real rows (routed padding, sorted_pair < 0,
    // sits at the end of an expert's last tile)
    int nblk = 4;
    if (sg.row_pair != nullptr) {
      nblk = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) nblk += sg.row_pair[row0 + 32 * i] >= 0 ? 1 : 0;
    } else if (dense) {
      nblk = min(4, (sg.a_rows - row0 + 31) / 32);
    }
    nblk = uniform(nblk);

    float sa[4], sa_max[4], c_prev[4][NJ];
    auto kloop = [&](auto nbc) {
      constexpr int NB = decltype(nbc)::value;
      // block 0's scales seed c_prev (the first rescale multiplies zeros by one); the
      // last step's loads fetch block nk-1 again, unused (its tiles into the free stage)
#pragma unroll
      for (int i = 0; i < 4; ++i) sa[i] = sa_max[i] = ascale(i, 0);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const float sw0 = wscale(j, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) c_prev[i][j] = sa[i] * sw0;
      }
      issue(0);
      for (int kt = 0; kt < nk; ++kt) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));   // this step's tiles (and its scales) have landed
        __builtin_amdgcn_s_barrier();
        const char *st = lds + (kt & 1) * kStageBytes;
        const int kn = min(kt + 1, nk - 1);
        // next block's activation scales first, then its tiles: waiting for the
        // scales (older in the in-order queue) never waits for the tiles
        float sa_next[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) sa_next[i] = ascale(i, kn);
        // the other stage: every wavefront finished reading it (the last step loads block
        // nk-1 there once more, unused, so that no branch splits the slice's code)
        // rescale the running sums from block kt-1's scale to block kt's
        float sae[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sae[i] = fmaxf(sa[i], sa_max[i] * kRelFloor);
          sa_max[i] = fmaxf(sa_max[i], sa[i]);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const float sw = wscale(j, kt);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float c = sae[i] * sw;
            if (i >= NB) {   // padding block: keep the scale bookkeeping only
              c_prev[i][j] = c;
              continue;
            }
            const float ratio = c_prev[i][j] * __builtin_amdgcn_rcpf(c);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] *= ratio;
            c_prev[i][j] = c;
          }
        }
#pragma unroll
        for (int s = 0; s < BK / 64; ++s) {
          v8i_t bf[NJ];
#pragma unroll
          for (int j = 0; j < NJ; ++j) bf[j] = read_frag(st + kATileBytes, brow_l[j], s);
#pragma unroll
          for (int i = 0; i < NB; ++i) {
            if (i == 0) issue_part(kn, (kt + 1) & 1, 2 * s);
            if (i == (NB > 1 ? (NB + 1) / 2 : 0)) issue_part(kn, (kt + 1) & 1, 2 * s + 1);
            const v8i_t af = read_frag(st, i * 32 + l32, s);
#pragma unroll
            for (int j = 0; j < NJ; ++j)   // weight fragment first: lanes end with 4 consecutive columns
              acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[j], af, acc[i][j], 0, 0, 0,
                                                                           127, 0, 127);
          }
          // one slice's fragments at a time (hoisting both slices' reads runs out of registers)
          __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sa[i] = sa_next[i];
      }
    };
    switch (nblk) {
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      default: kloop(std::integral_constant<int, 4>{}); break;
    }
    // every load has landed (the last step's into the free stage too) and all waves are done
    // with both stages
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    __syncthreads();

    // ---- epilogue.  acc[i][j][4g + t] * c_prev[i][j] is C[row i*32 + l32][col j*32 + 8g + 4*khalf + t].
    if (EPI == EPI_SWIGLU) {
      constexpr int OUTC = BN / 2;             // 256 output columns
      constexpr int LDR = OUTC * 4 + 16;       // fp32 staging row, bytes (128 x 1040 B = 130 KiB)
      char *ot = lds;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = i * 32 + l32;
#pragma unroll
        for (int jj = 0; jj < NJ / 2; ++jj) {
          const float cg = c_prev[i][jj], cu = c_prev[i][jj + NJ / 2];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int lc = wave * (NJ / 2) * 32 + jj * 32 + 8 * g + 4 * khalf;
            f32x4_t h;
#pragma unroll
            for (int t = 0; t < 4; ++t) h[t] = silu_mul(acc[i][jj][4 * g + t] * cg, acc[i][jj + NJ / 2][4 * g + t] * cu);
            *reinterpret_cast<f32x4_t *>(ot + lr * LDR + lc * 4) = h;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __syncthreads();
      // 128 rows x 2 runs of 128 columns; two threads per run, 64 values each
      {
        const int run = threadIdx.x >> 1, part = threadIdx.x & 1;
        const int lr = run >> 1, cb = run & 1;
        const int grow = row0 + lr;
        const int gcol0 = nb * OUTC + cb * 128;
        const float *src = reinterpret_cast<const float *>(ot + lr * LDR) + cb * 128 + part * 64;
        float amax = 0.0f;
#pragma unroll
        for (int v = 0; v < 64; v += 4) {
          const f32x4_t x = *reinterpret_cast<const f32x4_t *>(src + v);
          amax = fmaxf(amax, fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3]))));
        }
        amax = fmaxf(amax, __shfl_xor(amax, 1));
        const float s = amax > 0.0f ? amax / kE4m3Max : 1.0f;
        const bool store = !(dense && grow >= sg.a_rows) && gcol0 < half_n;
        uint8_t *dst = static_cast<uint8_t *>(sg.c) + static_cast<int64_t>(grow) * sg.ldc + gcol0 + part * 64;
#pragma unroll
        for (int v = 0; v < 64; v += 16) {
          u32x4_t o;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4_t x = *reinterpret_cast<const f32x4_t *>(src + v + 4 * q);
            o[q] = e4m3_pair(x[0] / s, x[1] / s) | (e4m3_pair(x[2] / s, x[3] / s) << 16);
          }
          if (store) *reinterpret_cast<u32x4_t *>(dst + v) = o;
        }
        if (store && part == 0) sg.c_scale[static_cast<int64_t>(grow) * sg.c_sld + gcol0 / 128] = s;
      }
      __syncthreads();   // the next item's loads refill this LDS
    } else {
      constexpr int OUTC = BN;
      constexpr int LDR = OUTC * 2 + 16;
      char *ot = lds;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lr = i * 32 + l32;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const float c = c_prev[i][j];
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int lc = wave * NJ * 32 + j * 32 + 8 * g + 4 * khalf;
            uint2 v;
            v.x = pack_bf16x2(acc[i][j][4 * g] * c, acc[i][j][4 * g + 1] * c);
            v.y = pack_bf16x2(acc[i][j][4 * g + 2] * c, acc[i][j][4 * g + 3] * c);
            *reinterpret_cast<uint2 *>(ot + lr * LDR + lc * 2) = v;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      __syncthreads();
      constexpr int CPR = OUTC / 8;
      const int col0 = nb * OUTC;
      for (int cidx = threadIdx.x; cidx < BM * CPR; cidx += kThreads) {
        const int lr = cidx / CPR, cc = cidx - lr * CPR;
        const int grow = row0 + lr, gcol = col0 + cc * 8;
        if ((dense && grow >= sg.a_rows) || gcol >= sg.n) continue;
        const u32x4_t v = *reinterpret_cast<const u32x4_t *>(ot + lr * LDR + cc * 16);
        *reinterpret_cast<u32x4_t *>(static_cast<uint16_t *>(sg.c) + static_cast<int64_t>(grow) * sg.ldc + gcol) = v;
      }
      __syncthreads();
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
  }
}

template <int EPI>
hipError_t launch_one(const WorkF8 &wk, int grid, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(&gemm_fp8_kernel<EPI>), kLdsBytes, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gemm_fp8_kernel<EPI>), dim3(grid), dim3(kThreads), kLdsBytes, st, wk);
  return hipGetLastError();
}

// ---- activation quantisation: 16 lanes per 128-column run (8 values each, one
// 16-byte load), the run's max over the 16-lane row by DPP moves
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_max16(float v) {
  v = fmaxf(v, dpp_f32<0xB1>(v));    // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f32<0x4E>(v));    // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f32<0x141>(v));   // mirror within 8
  v = fmaxf(v, dpp_f32<0x140>(v));   // mirror within 16
  return v;
}

__global__ __launch_bounds__(256) void quant_act_kernel(const uint16_t *__restrict__ x, int64_t runs,
                                                        int64_t cols, uint8_t *__restrict__ q,
                                                        float *__restrict__ s) {
  const int l16 = threadIdx.x & 15;
  const int64_t run = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  if (run >= runs) return;   // uniform over the 16 lanes of a run (a DPP row)
  const int64_t nb = cols / 128;
  const int64_t row = run / nb, cb = run - row * nb;
  const int64_t at = row * cols + cb * 128 + 8 * l16;
  const u32x4_t v = *reinterpret_cast<const u32x4_t *>(x + at);
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
  }
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(f[i]));
  m = row_max16(m);
  const float sc = m > 0.0f ? m / kE4m3Max : 1.0f;
  uint2 o;
  o.x = e4m3_pair(f[0] / sc, f[1] / sc) | (e4m3_pair(f[2] / sc, f[3] / sc) << 16);
  o.y = e4m3_pair(f[4] / sc, f[5] / sc) | (e4m3_pair(f[6] / sc, f[7] / sc) << 16);
  *reinterpret_cast<uint2 *>(q + at) = o;
  if (l16 == 0) s[row * nb + cb] = sc;
}

}  // namespace

bool gemm_fp8_supported(const Segment *segs, int nseg) {
  for (int s = 0; s < nseg; ++s)
    if (segs[s].k % BK != 0 || segs[s].k <= 0 || segs[s].k > kScaleRegs * 64 * BK || segs[s].n % 128 != 0)
      return false;
  return true;
}

hipError_t launch_gemm_fp8(const Segment *segs, int nseg, Epilogue epi, hipStream_t st) {
  WorkF8 wk{};
  wk.nseg = nseg;
  int64_t cap = 0;
  for (int s = 0; s < nseg; ++s) {
    wk.seg[s] = segs[s];
    const int ncols = epi == EPI_SWIGLU ? segs[s].n / 2 : segs[s].n;
    const int per = epi == EPI_SWIGLU ? BN / 2 : BN;
    wk.nblk_n[s] = (ncols + per - 1) / per;
    cap += static_cast<int64_t>(segs[s].n_tiles_host) * wk.nblk_n[s];
  }
  if (cap == 0) return hipSuccess;
  if (cap >= (1ll << 31)) return hipErrorInvalidValue;
  int grid = device_cu_count() / kXcds * kXcds;
  if (grid < kXcds) grid = kXcds;
  if (epi == EPI_SWIGLU) return launch_one<EPI_SWIGLU>(wk, grid, st);
  return launch_one<EPI_STORE>(wk, grid, st);
}

hipError_t launch_quant_act(const void *x, int64_t rows, int64_t cols, uint8_t *q, float *s,
                            hipStream_t st) {
  const int64_t runs = rows * (cols / 128);
  if (runs == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((runs + 15) / 16)), block(256);
  hipLaunchKernelGGL(quant_act_kernel, grid, block, 0, st, static_cast<const uint16_t *>(x), runs,
                     cols, q, s);
  return hipGetLastError();
}

}  // namespace moe
