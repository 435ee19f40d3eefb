// fp32 grouped GEMM on the vector ALUs for fp32 layers:
// C[rows, n] = A[rows, k] * B_e[n, k]^T with fp32 fused multiply-adds.
//
// A workgroup of 256 threads computes a 64 x 64 block of (A rows x B rows);
// each thread 4 rows x 4 B rows (columns tc, tc+16, tc+32, tc+48).  In the
// SwiGLU epilogue B rows 0..31 of the block are gate rows and 32..63 the
// matching up rows, so a thread holds both halves of its two output columns.
#include <math.h>

#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = 64, BNB = 64, BK = 32;
constexpr int kThreads = 256;

struct Work {
  Segment seg[2];
  int nseg;
  int nblk_n[2];
  int64_t start[3];
};

template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(Work wk) {
  __shared__ float As[BK][BM + 1];
  __shared__ float Bs[BK][BNB + 1];

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
    row0 = tile * kF32TileM;
    expert = 0;
  }
  const bool dense = sg.n_tiles_dev == nullptr;
  const int tid = threadIdx.x;
  const int K = sg.k;
  const int half_n = sg.n / 2;
  const float *A = static_cast<const float *>(sg.a);
  const float *B = static_cast<const float *>(sg.b) + static_cast<int64_t>(expert) * sg.b_stride;

  // loader: thread covers rows (tid / 4) and k columns (tid % 4) * 8 .. +8
  const int lr = tid >> 2, lk = (tid & 3) * 8;
  const float *a_src = nullptr;
  {
    const int grow = row0 + lr;
    if (sg.gather != nullptr) {
      const int pair = sg.gather[grow];
      if (pair >= 0) a_src = A + static_cast<int64_t>(pair / sg.topk) * sg.lda;
    } else if (!dense || grow < sg.a_rows) {
      a_src = A + static_cast<int64_t>(grow) * sg.lda;
    }
  }
  const float *b_src = nullptr;
  {
    int brow;
    bool ok;
    if (EPI == EPI_SWIGLU) {
      const int col = nb * 32 + (lr & 31);
      brow = lr < 32 ? col : half_n + col;
      ok = col < half_n;
    } else {
      brow = nb * BNB + lr;
      ok = brow < sg.n;
    }
    if (ok) b_src = B + static_cast<int64_t>(brow) * K;
  }

  const int tr = tid >> 4, tc = tid & 15;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + lk + j;
      As[lk + j][lr] = (a_src != nullptr && k < K) ? a_src[k] : 0.0f;
      Bs[lk + j][lr] = (b_src != nullptr && k < K) ? b_src[k] : 0.0f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][tr * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tc + 16 * j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

  float *C = static_cast<float *>(sg.c);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int grow = row0 + tr * 4 + i;
    if (dense && grow >= sg.a_rows) continue;
    if (EPI == EPI_SWIGLU) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = nb * 32 + tc + 16 * j;
        if (col >= half_n) continue;
        const float g = acc[i][j], u = acc[i][j + 2];
        C[static_cast<int64_t>(grow) * sg.ldc + col] = g / (1.0f + expf(-g)) * u;
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = nb * BNB + tc + 16 * j;
        if (col < sg.n) C[static_cast<int64_t>(grow) * sg.ldc + col] = acc[i][j];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(const Segment *segs, int nseg, int tile_m, Epilogue epi,
                           hipStream_t st) {
  (void)tile_m;
  Work wk{};
  wk.nseg = nseg;
  int64_t total = 0;
  for (int s = 0; s < nseg; ++s) {
    wk.seg[s] = segs[s];
    const int ncols = epi == EPI_SWIGLU ? segs[s].n / 2 : segs[s].n;
    const int per = epi == EPI_SWIGLU ? 32 : BNB;
    wk.nblk_n[s] = (ncols + per - 1) / per;
    wk.start[s] = total;
    total += static_cast<int64_t>(segs[s].n_tiles_host) * wk.nblk_n[s];
  }
  wk.start[nseg] = total;
  if (total == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(total)), block(kThreads);
  if (epi == EPI_SWIGLU)
    hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, grid, block, 0, st, wk);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<EPI_STORE>, grid, block, 0, st, wk);
  return hipGetLastError();
}

}  // namespace moe
