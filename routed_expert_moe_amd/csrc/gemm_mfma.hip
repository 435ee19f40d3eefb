// Grouped GEMM on bf16 MFMA (v_mfma_f32_32x32x16_bf16) for the expert FFNs and
// the gate logits:  C[rows, n] = A[rows, k] * B_e[n, k]^T, fp32 accumulation.
//
// One workgroup of four wavefronts computes a 128 x 128 tile; each wavefront a
// 64 x 64 quarter as 2 x 2 MFMA blocks of 32 x 32.  K advances 64 at a time
// through two LDS buffers (32 KiB each) whose 16-byte chunks are XOR-swizzled
// by row so the MFMA operand reads spread over the banks.  A rows of a routed
// gate/up tile are gathered from x through sorted_pair (padding rows read as
// zeros), so the expert-sorted activations are never materialised.
//
// SwiGLU epilogue: the 128 B rows of a tile are 64 gate rows (W1) followed by
// the 64 matching up rows (W3); a wavefront holds gate and up accumulators of
// the same output columns in the same lanes and writes silu(g) * u.
#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kChunksPerRow = BK / 8;        // 16-byte chunks per LDS row
constexpr int kTileBytes = BM * BK * 2;      // 16 KiB per operand tile

struct Work {
  Segment seg[2];
  int nseg;
  int nblk_n[2];      // column blocks per tile
  int64_t start[3];   // first workgroup of each segment
  int tile_m;
};

__device__ __forceinline__ int swz(int row, int chunk) { return row * kChunksPerRow + (chunk ^ (row & 7)); }

template <int EPI, bool OUT_F32>
__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(Work wk) {
  __shared__ __attribute__((aligned(16))) u32x4_t lds[2][2][BM * kChunksPerRow];  // [buf][A|B]

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
    row0 = tile * wk.tile_m;
    expert = 0;
  }

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int K = sg.k;
  const int half_n = sg.n / 2;

  // ---- per-thread global source rows (4 A rows, 4 B rows, one 16-byte chunk column)
  const int ch = tid & 7;
  const uint16_t *a_src[4];
  const uint16_t *b_src[4];
  const uint16_t *A = static_cast<const uint16_t *>(sg.a);
  const uint16_t *B = static_cast<const uint16_t *>(sg.b) + static_cast<int64_t>(expert) * sg.b_stride;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (tid >> 3) + 32 * i;
    const int grow = row0 + r;
    const uint16_t *p = nullptr;
    if (sg.gather != nullptr) {
      const int pair = sg.gather[grow];
      if (pair >= 0) p = A + static_cast<int64_t>(pair / sg.topk) * sg.lda;
    } else if (sg.n_tiles_dev != nullptr || grow < sg.a_rows) {
      p = A + static_cast<int64_t>(grow) * sg.lda;
    }
    a_src[i] = p;
    int brow;
    if (EPI == EPI_SWIGLU)
      brow = r < 64 ? nb * 64 + r : half_n + nb * 64 + (r - 64);
    else
      brow = nb * BN + r;
    const bool bvalid = EPI == EPI_SWIGLU ? (nb * 64 + (r & 63)) < half_n : brow < sg.n;
    b_src[i] = bvalid ? B + static_cast<int64_t>(brow) * K : nullptr;
  }

  u32x4_t ra[4], rb[4];
  auto load_tiles = [&](int k0) {
    const int k = k0 + ch * 8;
    const bool kin = k < K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = (a_src[i] != nullptr && kin) ? *reinterpret_cast<const u32x4_t *>(a_src[i] + k)
                                           : u32x4_t{0, 0, 0, 0};
      rb[i] = (b_src[i] != nullptr && kin) ? *reinterpret_cast<const u32x4_t *>(b_src[i] + k)
                                           : u32x4_t{0, 0, 0, 0};
    }
  };
  auto store_tiles = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 3) + 32 * i;
      lds[buf][0][swz(r, ch)] = ra[i];
      lds[buf][1][swz(r, ch)] = rb[i];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // LDS rows read by this lane
  const int l32 = lane & 31, khalf = lane >> 5;
  int arow[2], brow_l[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) arow[i] = wm * 64 + i * 32 + l32;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    brow_l[j] = (EPI == EPI_SWIGLU ? j * 64 + wn * 32 : wn * 64 + j * 32) + l32;

  const int nk = (K + BK - 1) / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) load_tiles((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int c = 2 * s + khalf;
      bf16x8_t af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const u32x4_t v = lds[cur][0][swz(arow[i], c)];
        af[i] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4_t v = lds[cur][1][swz(brow_l[j], c)];
        bfr[j] = __builtin_bit_cast(bf16x8_t, v);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) store_tiles(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue.  Lane holds column l32 of each 32x32 block, rows
  //      8*(r/4) + 4*(lane/32) + r%4 for accumulator r.
  const bool dense = sg.n_tiles_dev == nullptr;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lrow = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
      const int grow = row0 + lrow;
      if (dense && grow >= sg.a_rows) continue;
      if (EPI == EPI_SWIGLU) {
        const int col = nb * 64 + wn * 32 + l32;
        if (col >= half_n) continue;
        const float h = silu_mul(acc[i][0][r], acc[i][1][r]);
        static_cast<uint16_t *>(sg.c)[static_cast<int64_t>(grow) * sg.ldc + col] = f32_to_bf16_bits(h);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = nb * BN + wn * 64 + j * 32 + l32;
          if (col >= sg.n) continue;
          const int64_t o = static_cast<int64_t>(grow) * sg.ldc + col;
          if (OUT_F32)
            static_cast<float *>(sg.c)[o] = acc[i][j][r];
          else
            static_cast<uint16_t *>(sg.c)[o] = f32_to_bf16_bits(acc[i][j][r]);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_mfma(const Segment *segs, int nseg, int tile_m, Epilogue epi,
                            bool out_f32, hipStream_t st) {
  Work wk{};
  wk.nseg = nseg;
  wk.tile_m = tile_m;
  int64_t total = 0;
  for (int s = 0; s < nseg; ++s) {
    wk.seg[s] = segs[s];
    const int ncols = epi == EPI_SWIGLU ? segs[s].n / 2 : segs[s].n;
    const int per = epi == EPI_SWIGLU ? 64 : BN;
    wk.nblk_n[s] = (ncols + per - 1) / per;
    wk.start[s] = total;
    total += static_cast<int64_t>(segs[s].n_tiles_host) * wk.nblk_n[s];
  }
  wk.start[nseg] = total;
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(total)), block(kThreads);
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL((gemm_mfma_kernel<EPI_SWIGLU, false>), grid, block, 0, st, wk);
  else if (out_f32)
    hipLaunchKernelGGL((gemm_mfma_kernel<EPI_STORE, true>), grid, block, 0, st, wk);
  else
    hipLaunchKernelGGL((gemm_mfma_kernel<EPI_STORE, false>), grid, block, 0, st, wk);
  return hipGetLastError();
}

}  // namespace moe
