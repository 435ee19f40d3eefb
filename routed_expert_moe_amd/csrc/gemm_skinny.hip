// Weight-streaming grouped GEMM for tiles of at most 16 rows (decode-sized
// work): C[16, n] = A[16, k] * B_e[n, k]^T on v_mfma_f32_16x16x32_bf16.
//
// At decode the weights are nearly all of the bytes, so the kernel is built to
// keep HBM busy:
//  * persistent grid (as many workgroups as fit on the CUs at once); every wavefront takes work
//    items (tile, NG 16-row weight groups) from one list that holds only
//    the tiles in use, so no workgroup is launched for an untouched expert;
//  * each wavefront streams its NG groups over the whole K, loading the next
//    one or two 128-wide K blocks while it multiplies block k (NG and the
//    buffer count are set per kernel below so that 64-128 KiB of weights stay
//    in flight per CU, which covers the several-microsecond HBM latency under
//    full load);
//  * within a 128-wide K block, lane (row n = lane%16, quarter q = lane/16)
//    owns 32 K positions of its weight row, chosen so that the four lanes of a
//    row read one contiguous 64-byte run per load; the A fragments use the
//    same K permutation, which a dot product allows, and four MFMAs cover the
//    block.
// fp8 weights (OCP e4m3fn, exact in bf16) are widened with v_cvt_pk_f32_fp8,
// each 128-wide K block is accumulated separately and added times its fp32
// block scale: acc += s[n/128][k/128] * partial.
//
// SwiGLU items pair NG/2 16-row gate groups with the matching up groups; plain
// items take NG consecutive 16-row groups.  Consecutive items share their tile's A rows, and
// the four wavefronts of a workgroup take consecutive items.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// 16-row weight groups per work item and K-block buffers per wavefront.  The
// fp8 kernels are limited by the weight bytes each wavefront keeps in flight,
// so they take as many groups as the registers allow: gate/up (K = model dim,
// long) 8 groups double-buffered at one wavefront per SIMD, down 4 groups
// triple-buffered at two.
template <bool FP8, bool UP> constexpr int kGroups = !FP8 ? 2 : UP ? 8 : 4;
template <bool FP8, bool UP> constexpr int kBufs = FP8 && UP ? 2 : 3;
int groups_per_item(bool fp8, bool up) { return !fp8 ? 2 : up ? 8 : 4; }

struct Work {
  Segment seg[2];
  int nseg;
  int ngp[2];                             // work items per tile
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

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// operands of one 128-wide K block for this lane
template <bool FP8, bool UP>
struct KBlock {
  u32x4_t a[4];                  // A: 4 x 8 bf16
  u32x4_t w[kGroups<FP8, UP>][FP8 ? 2 : 4];     // per group: 32 fp8 (2 x 16 B) or 32 bf16 (4 x 16 B)
};

template <int EPI, bool FP8, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void gemm_skinny_kernel(Work wk) {
  constexpr bool UP = EPI == EPI_SWIGLU;
  constexpr int NG = kGroups<FP8, UP>, HG = NG / 2;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l16 = lane & 15, q = lane >> 4;

  const int tiles0 = uniform(wk.seg[0].n_tiles_dev ? *wk.seg[0].n_tiles_dev : wk.seg[0].n_tiles_host);
  const int items0 = tiles0 * wk.ngp[0];
  const int items1 = wk.nseg > 1 ? wk.seg[1].n_tiles_host * wk.ngp[1] : 0;
  const int total = items0 + items1;
  const int nwaves = gridDim.x * kWaves;

  for (int item = blockIdx.x * kWaves + wave; item < total; item += nwaves) {
    const int si = item < items0 ? 0 : 1;
    const Segment &sg = wk.seg[si];
    const int local = si == 0 ? item : item - items0;
    const int tile = local / wk.ngp[si];
    const int gp = local - tile * wk.ngp[si];
    const bool dense = sg.n_tiles_dev == nullptr;
    const int row0 = uniform(dense ? tile * kSkinnyTileM : sg.tile_row[tile]);
    const int expert = uniform(dense ? 0 : sg.tile_expert[tile]);
    const int K = sg.k;
    const int half_n = sg.n / 2;
    const int kblocks = (K + 127) / 128;

    // A row of this lane (row l16 of the tile); padding rows read as zeros
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
    // weight rows of this lane's groups, and whether each group exists
    int base[NG], wrow[NG];
    bool gvalid[NG], wvalid[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (EPI == EPI_SWIGLU) {
        const int col0 = gp * 16 * HG + (g % HG) * 16;
        base[g] = g < HG ? col0 : half_n + col0;
        gvalid[g] = col0 < half_n;
        wvalid[g] = col0 + l16 < half_n;
      } else {
        base[g] = gp * 16 * NG + g * 16;
        gvalid[g] = base[g] < sg.n;
        wvalid[g] = base[g] + l16 < sg.n;
      }
      wrow[g] = base[g] + l16;
    }
    const int64_t eoff = static_cast<int64_t>(expert) * sg.b_stride;
    const float *scale = FP8 ? sg.b_scale + static_cast<int64_t>(expert) * sg.s_stride : nullptr;

    // K positions of this lane inside a 128-wide block, in MFMA order i = 0..3
    // (8 each).  fp8: two 16-byte pieces at bytes 16q and 64 + 16q, so the four
    // lanes of a row read one contiguous 64-byte run per load; bf16: four pieces
    // at elements 32i/4 + 8q, i.e. bytes 64i + 16q, again contiguous per load.
    auto kpos = [&](int kb, int i) -> int {
      return FP8 ? kb * 128 + (i >> 1) * 64 + 16 * q + (i & 1) * 8 : kb * 128 + 32 * i + 8 * q;
    };
    auto load_kb = [&](int kb, KBlock<FP8, UP> &d) {
      const bool kin = kb < kblocks;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = kpos(kb, i);
        d.a[i] = (arow != nullptr && kin && k < K) ? *reinterpret_cast<const u32x4_t *>(arow + k)
                                                   : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (FP8) {
          const uint8_t *wp = static_cast<const uint8_t *>(sg.b) + eoff + static_cast<int64_t>(wrow[g]) * K;
          const bool ok = wvalid[g] && kin;
          d.w[g][0] = ok ? *reinterpret_cast<const u32x4_t *>(wp + kpos(kb, 0)) : u32x4_t{0, 0, 0, 0};
          d.w[g][1] = ok ? *reinterpret_cast<const u32x4_t *>(wp + kpos(kb, 2)) : u32x4_t{0, 0, 0, 0};
        } else {
          const uint16_t *wp = static_cast<const uint16_t *>(sg.b) + eoff + static_cast<int64_t>(wrow[g]) * K;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = kpos(kb, i);
            d.w[g][i] = (wvalid[g] && kin && k < K) ? *reinterpret_cast<const u32x4_t *>(wp + k)
                                                    : u32x4_t{0, 0, 0, 0};
          }
        }
      }
    };

    f32x4_t acc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto compute_kb = [&](int kb, const KBlock<FP8, UP> &d) {
      bf16x8_t af[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = __builtin_bit_cast(bf16x8_t, d.a[i]);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        if (FP8) {
          const bf16x8_t b0 = fp8x8_to_bf16x8(d.w[g][0][0], d.w[g][0][1]);
          const bf16x8_t b1 = fp8x8_to_bf16x8(d.w[g][0][2], d.w[g][0][3]);
          const bf16x8_t b2 = fp8x8_to_bf16x8(d.w[g][1][0], d.w[g][1][1]);
          const bf16x8_t b3 = fp8x8_to_bf16x8(d.w[g][1][2], d.w[g][1][3]);
          f32x4_t part = {0.f, 0.f, 0.f, 0.f};
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[0], b0, part, 0, 0, 0);
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[1], b1, part, 0, 0, 0);
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[2], b2, part, 0, 0, 0);
          part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[3], b3, part, 0, 0, 0);
          // wavefront-uniform: the group's rows share one 128-row scale block
          const float s = (gvalid[g] && kb < kblocks) ? scale[static_cast<int64_t>(base[g] / 128) * kblocks + kb] : 0.0f;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[g][r] += s * part[r];
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], __builtin_bit_cast(bf16x8_t, d.w[g][i]), acc[g], 0, 0, 0);
        }
      }
    };

    // K-block buffers: with two, block kb+1 loads while kb multiplies; with
    // three, blocks kb+1 and kb+2
    if constexpr (kBufs<FP8, UP> == 2) {
      KBlock<FP8, UP> buf[2];
      load_kb(0, buf[0]);
      for (int kb = 0; kb < kblocks; kb += 2) {
        load_kb(kb + 1, buf[1]);
        compute_kb(kb, buf[0]);
        if (kb + 1 >= kblocks) break;
        load_kb(kb + 2, buf[0]);
        compute_kb(kb + 1, buf[1]);
      }
    } else {
      KBlock<FP8, UP> buf[3];
      load_kb(0, buf[0]);
      load_kb(1, buf[1]);
      for (int kb = 0; kb < kblocks; kb += 3) {
        load_kb(kb + 2, buf[2]);
        compute_kb(kb, buf[0]);
        if (kb + 1 >= kblocks) break;
        load_kb(kb + 3, buf[0]);
        compute_kb(kb + 1, buf[1]);
        if (kb + 2 >= kblocks) break;
        load_kb(kb + 4, buf[1]);
        compute_kb(kb + 2, buf[2]);
      }
    }

    // epilogue: lane holds column l16 of the group (a weight row), tile rows 4q + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int grow = row0 + 4 * q + r;
      if (dense && grow >= sg.a_rows) continue;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) {
          const int col = gp * 16 * HG + hg * 16 + l16;
          if (col < half_n) {
            const float h = silu_mul(acc[hg][r], acc[hg + HG][r]);
            static_cast<uint16_t *>(sg.c)[static_cast<int64_t>(grow) * sg.ldc + col] = f32_to_bf16_bits(h);
          }
        }
      } else {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          if (!wvalid[g]) continue;
          const int64_t o = static_cast<int64_t>(grow) * sg.ldc + wrow[g];
          if (OUT_F32)
            static_cast<float *>(sg.c)[o] = acc[g][r];
          else
            static_cast<uint16_t *>(sg.c)[o] = f32_to_bf16_bits(acc[g][r]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_skinny(const Segment *segs, int nseg, Epilogue epi, bool w_fp8,
                              bool out_f32, hipStream_t st) {
  Work wk{};
  const int NG = groups_per_item(w_fp8, epi == EPI_SWIGLU), HG = NG / 2;
  wk.nseg = nseg;
  int64_t cap = 0;
  for (int s = 0; s < nseg; ++s) {
    wk.seg[s] = segs[s];
    wk.ngp[s] = epi == EPI_SWIGLU ? (segs[s].n / 2 + 16 * HG - 1) / (16 * HG) : (segs[s].n + 16 * NG - 1) / (16 * NG);
    cap += static_cast<int64_t>(segs[s].n_tiles_host) * wk.ngp[s];
  }
  if (cap == 0) return hipSuccess;
  if (cap >= (1ll << 31)) return hipErrorInvalidValue;
  int64_t blocks = (cap + kWaves - 1) / kWaves;
  auto resident = [&](const void *fn) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess || per_cu < 1)
      per_cu = 1;
    return static_cast<int64_t>(device_cu_count()) * per_cu;
  };
#define MOE_SKINNY(E_, F_, O_)                                                                  \
  do {                                                                                          \
    static std::atomic<int64_t> resident_cache[kMaxDevices];                                    \
    const int dev_ = current_device();                                                          \
    int64_t max_blocks = dev_ < kMaxDevices ? resident_cache[dev_].load(std::memory_order_relaxed) : 0; \
    if (max_blocks == 0) {                                                                      \
      max_blocks = resident(reinterpret_cast<const void *>(&gemm_skinny_kernel<E_, F_, O_>));   \
      if (dev_ < kMaxDevices) resident_cache[dev_].store(max_blocks, std::memory_order_relaxed); \
    }                                                                                           \
    const dim3 grid(static_cast<unsigned>(blocks < max_blocks ? blocks : max_blocks)), block(kThreads); \
    hipLaunchKernelGGL((gemm_skinny_kernel<E_, F_, O_>), grid, block, 0, st, wk);                 \
  } while (0)
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
