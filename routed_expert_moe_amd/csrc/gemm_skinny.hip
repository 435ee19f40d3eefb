// Weight-streaming grouped GEMM for tiles of at most 16 rows (decode-sized
// work): C[16, n] = A[16, k] * B_e[n, k]^T on v_mfma_f32_16x16x32_bf16.
//
// The weights dominate the bytes, so every lane streams whole 16-byte pieces
// of its weight row: within each 128-wide K block, lane (row n = lane%16,
// quarter q = lane/16) owns K positions [32q, 32q+32) of that row.  Because a
// dot product does not care about the order of its terms, the A fragments are
// loaded with the same K permutation, and four MFMAs cover the block.
//
// fp8 weights (OCP e4m3fn, exact in bf16) are widened with v_cvt_pk_f32_fp8,
// each 128-wide K block is accumulated separately and added with its fp32
// block scale: acc += s[n/128][k/128] * partial.
//
// A workgroup (four wavefronts) owns one 16-row tile and a slab of weight
// rows; each wavefront two 16-row weight groups (gate + matching up rows for
// the SwiGLU epilogue, or two consecutive groups).
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kRowsPerWave = 32;                   // two 16-row weight groups
constexpr int kColsPerBlockStore = kWaves * kRowsPerWave;   // 128 output columns
constexpr int kColsPerBlockSwiglu = kWaves * 16;           // 64 output columns

struct Work {
  Segment seg[2];
  int nseg;
  int nblk_n[2];
  int64_t start[3];
};

__device__ __forceinline__ bf16x8_t fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  // e4m3 -> fp32 is exact; every e4m3 value is exact in bf16, so the top half
  // of the fp32 pattern is the bf16 value.
  uint32_t w[4];
  const uint32_t src[2] = {lo, hi};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(src[h]), false);
    const f32x2_t b = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(src[h]), true);
    w[2 * h] = (__float_as_uint(a[0]) >> 16) | (__float_as_uint(a[1]) & 0xFFFF0000u);
    w[2 * h + 1] = (__float_as_uint(b[0]) >> 16) | (__float_as_uint(b[1]) & 0xFFFF0000u);
  }
  const u32x4_t v = {w[0], w[1], w[2], w[3]};
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int EPI, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void gemm_skinny_kernel(Work wk) {
  const int64_t bid = blockIdx.x;
  const int si = (wk.nseg > 1 && bid >= wk.start[1]) ? 1 : 0;
  const Segment &sg = wk.seg[si];
  const int64_t local = bid - wk.start[si];
  const int tile = static_cast<int>(local / wk.nblk_n[si]);
  const int nb = static_cast<int>(local % wk.nblk_n[si]);
  int row0, expert;
  if (sg.n_tiles_dev != nullptr) {
    if (tile >= *sg.n_tiles_dev) return;
    row0 = sg.tile_row[tile];
    expert = sg.tile_expert[tile];
  } else {
    row0 = tile * kSkinnyTileM;
    expert = 0;
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int l16 = lane & 15, q = lane >> 4;
  const int K = sg.k;
  const int half_n = sg.n / 2;
  const bool dense = sg.n_tiles_dev == nullptr;

  // A row of this lane (row l16 of the tile)
  const uint16_t *A = static_cast<const uint16_t *>(sg.a);
  const uint16_t *arow = nullptr;
  {
    const int grow = row0 + l16;
    if (sg.gather != nullptr) {
      const int pair = sg.gather[grow];
      if (pair >= 0) arow = A + static_cast<int64_t>(pair / sg.topk) * sg.lda;
    } else if (!dense || grow < sg.a_rows) {
      arow = A + static_cast<int64_t>(grow) * sg.lda;
    }
  }

  // weight rows of this lane for its two groups
  int wrow[2];
  bool wvalid[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    if (EPI == EPI_SWIGLU) {
      const int col = nb * kColsPerBlockSwiglu + wave * 16 + l16;
      wrow[g] = g == 0 ? col : half_n + col;
      wvalid[g] = col < half_n;
    } else {
      wrow[g] = nb * kColsPerBlockStore + wave * kRowsPerWave + g * 16 + l16;
      wvalid[g] = wrow[g] < sg.n;
    }
  }
  const int64_t eoff = static_cast<int64_t>(expert) * sg.b_stride;
  const float *scale = FP8 ? sg.b_scale + static_cast<int64_t>(expert) * sg.s_stride : nullptr;
  const int kblocks = (K + 127) / 128;
  // scale rows of the two groups (uniform within a 16-row group)
  int srow[2];
  bool gvalid[2];   // wavefront-uniform: the group's first row exists
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    int base;
    if (EPI == EPI_SWIGLU) {
      const int col0 = nb * kColsPerBlockSwiglu + wave * 16;
      base = g == 0 ? col0 : half_n + col0;
      gvalid[g] = col0 < half_n;
    } else {
      base = nb * kColsPerBlockStore + wave * kRowsPerWave + g * 16;
      gvalid[g] = base < sg.n;
    }
    srow[g] = base / 128;
  }

  f32x4_t acc[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int kb = 0; kb < kblocks; ++kb) {
    const int kq = kb * 128 + 32 * q;   // first K position of this lane's quarter
    // A fragments: 4 x 8 bf16 at kq + 8i
    bf16x8_t af[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = kq + 8 * i;
      u32x4_t v = {0, 0, 0, 0};
      if (arow != nullptr && k < K) v = *reinterpret_cast<const u32x4_t *>(arow + k);
      af[i] = __builtin_bit_cast(bf16x8_t, v);
    }
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      bf16x8_t bfr[4];
      if (FP8) {
        const uint8_t *wp = static_cast<const uint8_t *>(sg.b) + eoff + static_cast<int64_t>(wrow[g]) * K + kq;
        u32x4_t v0 = {0, 0, 0, 0}, v1 = {0, 0, 0, 0};
        if (wvalid[g]) {
          v0 = *reinterpret_cast<const u32x4_t *>(wp);
          v1 = *reinterpret_cast<const u32x4_t *>(wp + 16);
        }
        bfr[0] = fp8x8_to_bf16x8(v0[0], v0[1]);
        bfr[1] = fp8x8_to_bf16x8(v0[2], v0[3]);
        bfr[2] = fp8x8_to_bf16x8(v1[0], v1[1]);
        bfr[3] = fp8x8_to_bf16x8(v1[2], v1[3]);
        f32x4_t part = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[i], part, 0, 0, 0);
        const float s = gvalid[g] ? scale[static_cast<int64_t>(srow[g]) * kblocks + kb] : 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[g][r] += s * part[r];
      } else {
        const uint16_t *wp = static_cast<const uint16_t *>(sg.b) + eoff + static_cast<int64_t>(wrow[g]) * K + kq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          u32x4_t v = {0, 0, 0, 0};
          if (wvalid[g] && kq + 8 * i < K) v = *reinterpret_cast<const u32x4_t *>(wp + 8 * i);
          bfr[i] = __builtin_bit_cast(bf16x8_t, v);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[i], acc[g], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds column l16 (a weight row), tile rows 4q + r
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int grow = row0 + 4 * q + r;
    if (dense && grow >= sg.a_rows) continue;
    if (EPI == EPI_SWIGLU) {
      const int col = nb * kColsPerBlockSwiglu + wave * 16 + l16;
      if (col < half_n) {
        const float h = silu_mul(acc[0][r], acc[1][r]);
        static_cast<uint16_t *>(sg.c)[static_cast<int64_t>(grow) * sg.ldc + col] = f32_to_bf16_bits(h);
      }
    } else {
#pragma unroll
      for (int g = 0; g < 2; ++g) {
        const int col = wrow[g];
        if (!wvalid[g]) continue;
        const int64_t o = static_cast<int64_t>(grow) * sg.ldc + col;
        if (OUT_F32)
          static_cast<float *>(sg.c)[o] = acc[g][r];
        else
          static_cast<uint16_t *>(sg.c)[o] = f32_to_bf16_bits(acc[g][r]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const Segment *segs, int nseg, Epilogue epi, bool w_fp8,
                              bool out_f32, hipStream_t st) {
  Work wk{};
  wk.nseg = nseg;
  int64_t total = 0;
  for (int s = 0; s < nseg; ++s) {
    wk.seg[s] = segs[s];
    const int ncols = epi == EPI_SWIGLU ? segs[s].n / 2 : segs[s].n;
    const int per = epi == EPI_SWIGLU ? kColsPerBlockSwiglu : kColsPerBlockStore;
    wk.nblk_n[s] = (ncols + per - 1) / per;
    wk.start[s] = total;
    total += static_cast<int64_t>(segs[s].n_tiles_host) * wk.nblk_n[s];
  }
  wk.start[nseg] = total;
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(total)), block(kThreads);
#define MOE_SKINNY(E_, F_, O_) hipLaunchKernelGGL((gemm_skinny_kernel<E_, F_, O_>), grid, block, 0, st, wk)
  if (epi == EPI_SWIGLU) {
    if (w_fp8) MOE_SKINNY(EPI_SWIGLU, true, false);
    else MOE_SKINNY(EPI_SWIGLU, false, false);
  } else if (out_f32) {
    if (w_fp8) MOE_SKINNY(EPI_STORE, true, true);
    else MOE_SKINNY(EPI_STORE, false, true);
  } else {
    if (w_fp8) MOE_SKINNY(EPI_STORE, true, false);
    else MOE_SKINNY(EPI_STORE, false, false);
  }
#undef MOE_SKINNY
  return hipGetLastError();
}

}  // namespace moe
