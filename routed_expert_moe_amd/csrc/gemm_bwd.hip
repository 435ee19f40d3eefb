// Grouped GEMMs of the layer's backward pass on bf16 MFMA, fp32 results.
//
// Two forms, both over bf16 operands stored row-major:
//   ROWS   C[r, n] = sum_k A[r, k] B_e[k, n]     (r: rows of a 128-row tile of
//          expert e's rows, or of a dense row range).  dH = dY W2_e,
//          dX = dAB W13_e, and the shared expert's and the gate's
//          counterparts, where the prefill GEMM's k-strided mode does not fit.
//   WGRAD  C_e[m, n] = sum_r A[r, m] B[r, n] over the rows r of expert e (or
//          all rows of a dense segment).  dW2_e = dY_e^T H_e, dW13_e =
//          dAB_e^T Xs_e (x gathered into routed-row order beforehand), and the
//          shared expert's and the gate's weight gradients.
// Both use workgroup tiles of 128 x 128 and four wavefronts in a 2 x 2
// arrangement, each owning 64 x 64 of C as 2 x 2 blocks of
// v_mfma_f32_32x32x16_bf16.
//
// ROWS: K step 32.  Operands are copied into LDS through registers, 16 bytes
// per thread and load:
//  * k-contiguous (A in ROWS) as [row][k], rows padded to 80 bytes, so the
//    16-byte fragment reads of 8 consecutive rows hit distinct banks;
//  * k-strided (B) as [k][col], rows padded to 320 bytes; an MFMA operand (8 consecutive k of one column per lane) is then
//    read with two ds_read_b64_tr_b16: within each 16-lane group, lane q
//    addresses 4 columns of row kb + q/4 and lane l receives column l of rows
//    kb .. kb+3.  The LDS serves these 8-byte reads 32 lanes at a time: four
//    rows x 64 bytes, which a row stride of 256 + 64 bytes puts on four
//    disjoint 16-bank ranges (a 288-byte stride overlapped them, and LDS bank
//    conflicts took a third of the LDS cycles).
// The next step's global loads are issued before the current step's MFMAs.
//
// ROWS block order: workgroup b runs on XCD b % 8, so each XCD is given a
// contiguous range of the work list, and inside each run of up to eight
// M-tiles of one expert the list goes column block by column block: the tiles
// that read one column block of the expert's B run side by side on one XCD and
// share it through L2 (in tile-major order each tile streamed the whole B).
//
// WGRAD: the reduction runs over the group's rows, a few hundred at the V3
// prefill shape, so each workgroup is short and the time goes to load latency
// and to the fp32 stores; the kernel keeps several workgroups per CU and
// streams both operands global -> LDS by DMA (global_load_lds_dwordx4) through
// two stages, each step's loads issued one step ahead, one barrier per step
// (33 KiB of LDS per workgroup, set by the epilogue's staging: four workgroups
// per CU, 5% faster at V3 than a three-stage ring with three).  A stage holds 32 k-rows of 128 columns per operand, 256
// bytes per row with the 64-byte block b of row r at block b ^ (r & 3), read
// with ds_read_b64_tr_b16 (conflict-free for the same reason as above).  A
// step that runs past the group's last row reads clamped rows, and each
// wavefront zeroes the A rows it loaded beyond the end before the barrier.
// C is written with non-temporal stores (nothing in the call reads it back;
// 4% off the V3 backward against plain stores).
//
// Rows past a tile's end are read (clamped to a valid row) but never stored; a
// WGRAD group with no rows stores zeros.  Requires every k-contiguous extent
// and every column count to be a multiple of 8.
#include "backward.hpp"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int kThreads = 256;
constexpr int kXcds = 8;
constexpr int kGroup = 8;                    // M-tiles of one expert whose blocks interleave (ROWS)
constexpr int kLdsRow = 40;                  // [row][k] tile: bf16 per row (32 + 8 pad = 80 bytes)
constexpr int kTileElems = 128 * kLdsRow;
constexpr int kTRow = 160;                   // [k][col] tile: bf16 per row (128 + 32 pad = 320 bytes)
constexpr int kTTileElems = BK * kTRow;

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// a [32 k] x [128 cols] slab of a matrix whose rows are k: thread t takes
// chunks t and t + 256 (row c / 16, columns 8 * (c % 16))
struct SlabT {
  u32x4_t v[2];
};
// a [128 rows] x [32 k] slab of a matrix whose rows are the tile rows: thread t
// takes chunks t and t + 256 (row c / 4, k 8 * (c % 4))
struct SlabK {
  u32x4_t v[2];
};

__device__ __forceinline__ void store_t(uint16_t *s, const SlabT &x, int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + kThreads * j;
    *reinterpret_cast<u32x4_t *>(s + (c >> 4) * kTRow + 8 * (c & 15)) = x.v[j];
  }
}
// MFMA operand of column block [cb, cb + 32) and K slice [ks, ks + 16) from a
// [k][col] tile: lane l gets column cb + l % 32, k = ks + 8 * (l / 32) + 0..7
__device__ __forceinline__ bf16x8_t frag_t(const uint16_t *s, int cb, int ks, int lane) {
  const int g = lane >> 4, q = lane & 15;
  const int col = cb + 16 * (g & 1) + 4 * (q & 3);
  const int kb = ks + 8 * (g >> 1) + (q >> 2);
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(s + kb * kTRow + col));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(s + (kb + 4) * kTRow + col));
  const u32x4_t v = {static_cast<uint32_t>(static_cast<uint16_t>(lo[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[1])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(lo[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[3])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(hi[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[1])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(hi[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[3])) << 16)};
  return __builtin_bit_cast(bf16x8_t, v);
}
__device__ __forceinline__ void store_k(uint16_t *s, const SlabK &x, int tid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int c = tid + kThreads * j;
    *reinterpret_cast<u32x4_t *>(s + (c >> 2) * kLdsRow + 8 * (c & 3)) = x.v[j];
  }
}

__global__ __launch_bounds__(kThreads) void gemm_rows_kernel(BwdGemm g) {
  __shared__ __attribute__((aligned(16))) uint16_t s_a[kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[kTTileElems];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const uint16_t *A = g.a;
  const uint16_t *B = g.b;

  int m0, n0, row_end = 0, k_begin, k_end, e = 0;
  {
    const int nbn = (g.n + BN - 1) / BN;
    const int ntiles = g.n_tiles_dev ? *g.n_tiles_dev : (g.dense_rows + BM - 1) / BM;
    // the grid covers the tile capacity in a multiple of 8 blocks; XCD b % 8 takes
    // the contiguous range [xcd * per, xcd * per + per) of the ntiles * nbn items
    const int per = (ntiles * nbn + kXcds - 1) / kXcds;
    const int slot_x = blockIdx.x / kXcds;
    if (slot_x >= per) return;
    const int item = (blockIdx.x % kXcds) * per + slot_x;
    const int slot = item / nbn;
    if (slot >= ntiles) return;
    int first, last;
    if (g.n_tiles_dev) {
      first = g.tile_first[slot];
      last = first + (g.tile_end[slot] - g.tile_row[first] + BM - 1) / BM;
    } else {
      first = 0;
      last = ntiles;
    }
    const int g0 = first + (slot - first) / kGroup * kGroup;
    const int gs = min(kGroup, last - g0);
    const int lg = item - g0 * nbn;
    const int nbi = lg / gs;
    const int ti = g0 + lg - nbi * gs;
    n0 = nbi * BN;
    if (g.n_tiles_dev) {
      m0 = g.tile_row[ti];
      e = g.tile_expert[ti];
      row_end = g.tile_end[ti];
    } else {
      m0 = ti * BM;
      row_end = g.dense_rows;
    }
    B += static_cast<int64_t>(e) * g.b_estride;
    k_begin = 0;
    k_end = g.k;
  }
  m0 = uniform(m0);
  n0 = uniform(n0);
  k_begin = uniform(k_begin);
  k_end = uniform(k_end);
  const int nk = (k_end - k_begin + BK - 1) / BK;

  // ---- global -> register loads of one K step
  // A: rows m0 + r (clamped below row_end), k contiguous
  auto load_ak = [&](int k0, SlabK &x) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + kThreads * j;
      int r = m0 + (c >> 2);
      if (r >= row_end) r = row_end - 1;
      const int k = k0 + 8 * (c & 3);
      x.v[j] = k < k_end ? *reinterpret_cast<const u32x4_t *>(A + static_cast<int64_t>(r) * g.lda + k)
                         : u32x4_t{0, 0, 0, 0};
    }
  };
  // B (rows are k): columns [n0, n0 + 128) of rows k0 .. k0 + 31
  auto load_t = [&](int k0, SlabT &x) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = tid + kThreads * j;
      const int k = k0 + (c >> 4);
      const int col = n0 + 8 * (c & 15);
      x.v[j] = (col < g.n && k < k_end) ? *reinterpret_cast<const u32x4_t *>(B + static_cast<int64_t>(k) * g.ldb + col)
                                        : u32x4_t{0, 0, 0, 0};
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  SlabK ak;
  SlabT bt;
  auto load = [&](int kt) {
    const int k0 = k_begin + kt * BK;
    load_ak(k0, ak);
    load_t(k0, bt);
  };

  if (nk > 0) load(0);
  for (int kt = 0; kt < nk; ++kt) {
    __syncthreads();   // the previous step's fragment reads are done
    store_k(s_a, ak, tid);
    store_t(s_b, bt, tid);
    __syncthreads();
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8_t af[2], bf[2];
      const int kk = s * 16 + 8 * (lane >> 5);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = *reinterpret_cast<const bf16x8_t *>(s_a + (wm * 64 + i * 32 + (lane & 31)) * kLdsRow + kk);
        bf[i] = frag_t(s_b, wn * 64 + i * 32, s * 16, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- store: acc[i][j][r] is C[m0 + wm*64 + i*32 + 8*(r/4) + 4*(lane/32) + r%4][n0 + wn*64 + j*32 + lane%32]
  float *C = g.c;
  const int mlim = row_end;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      if (n >= g.n) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (m < mlim) C[static_cast<int64_t>(m) * g.ldc + n] = acc[i][j][r];
      }
    }
}

// ---- WGRAD on LDS DMA --------------------------------------------------------
constexpr int WBK = 32, WStages = 2, WRow = 256;   // k-rows per step, ring depth, LDS bytes per k-row
constexpr int WTile = WBK * WRow;                  // 8 KiB per operand per stage
constexpr int WStage = 2 * WTile;
constexpr int WSRow = BN * 4 + 16;                 // epilogue: one staged fp32 row of C, bytes
// the ring, or 64 staged rows of C in the epilogue (33 KiB), whichever is larger
constexpr int WLds = WStages * WStage > 64 * WSRow ? WStages * WStage : 64 * WSRow;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;

__device__ __forceinline__ void dma16(const void *src, char *lds_wave_base) {
  __builtin_amdgcn_global_load_lds((gbl_void_t *)(src), (lds_void_t *)(lds_wave_base), 16, 0, 0);
}
// s_waitcnt immediates for gfx9: vmcnt in bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
constexpr int kWaitLgkm0 = 15 | (3 << 14) | (7 << 4);

// byte offset of (k-row r, tile column c) in a WGRAD stage operand
__device__ __forceinline__ int w_off(int r, int c) { return r * WRow + (((c >> 5) ^ (r & 3)) << 6) + ((c * 2) & 63); }

// operand of tile columns [cb, cb + 32), K slice [16 s, 16 s + 16): lane 16g + q
// addresses k-row kr + q/4, columns cb + 16(g&1) + 4(q%4); lane 16g + l receives
// column cb + 16(g&1) + l of k-rows kr .. kr+3, then kr+4 .. kr+7
__device__ __forceinline__ bf16x8_t frag_w(const char *base, int cb, int s, int lane) {
  const int g = lane >> 4, q = lane & 15;
  const int kr = 16 * s + 8 * (g >> 1) + (q >> 2);
  const int col = cb + 16 * (g & 1) + 4 * (q & 3);
  const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(base + w_off(kr, col)));
  const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t *)(base + w_off(kr + 4, col)));
  const u32x4_t v = {static_cast<uint32_t>(static_cast<uint16_t>(lo[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[1])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(lo[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(lo[3])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(hi[0])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[1])) << 16),
                     static_cast<uint32_t>(static_cast<uint16_t>(hi[2])) | (static_cast<uint32_t>(static_cast<uint16_t>(hi[3])) << 16)};
  return __builtin_bit_cast(bf16x8_t, v);
}

__global__ __launch_bounds__(kThreads) void gemm_wgrad_kernel(BwdGemm g) {
  extern __shared__ __attribute__((aligned(1024))) char wl[];
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int nbm = (g.m + BM - 1) / BM, nbn = (g.n + BN - 1) / BN;
  const int e = uniform(blockIdx.x / (nbm * nbn));
  const int rem = blockIdx.x - e * nbm * nbn;
  const int m0 = uniform((rem / nbn) * BM), n0 = uniform((rem % nbn) * BN);
  const int kbeg = uniform(g.expert_off ? g.expert_off[e] : 0);
  const int kend = uniform(g.expert_off ? g.expert_off[e + 1] : g.dense_rows);
  const int nk = (kend - kbeg + WBK - 1) / WBK;

  // DMA: this wavefront loads k-rows 8 wave .. 8 wave + 7 of each step, four per
  // 1 KiB load; the lane fills physical 16-byte chunk p of k-row 8 wave + 4q + rq
  const int p = lane & 15, rq = lane >> 4;
  const int sw = (((p >> 2) ^ rq) << 5) | ((p & 3) << 3);   // logical column of that chunk
  const int acol = min(m0 + sw, g.m - 8), bcol = min(n0 + sw, g.n - 8);
  auto issue = [&](int kt) {
    char *st = wl + (kt % WStages) * WStage;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int row = min(kbeg + kt * WBK + 8 * wave + 4 * q + rq, kend - 1);
      dma16(g.a + static_cast<int64_t>(row) * g.lda + acol, st + (2 * wave + q) * 1024);
      dma16(g.b + static_cast<int64_t>(row) * g.ldb + bcol, st + WTile + (2 * wave + q) * 1024);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  for (int kt = 0; kt < WStages - 1 && kt < nk; ++kt) issue(kt);
  for (int kt = 0; kt < nk; ++kt) {
    // this wavefront's loads of step kt; those of the later steps already issued
    // (up to WStages - 2 of them, 4 loads each) may stay in flight
    static_assert(WStages >= 2 && WStages <= 3, "the wait below covers rings of two or three stages");
    if (WStages == 3 && kt + 1 < nk) __builtin_amdgcn_s_waitcnt(wait_vm(4));
    else __builtin_amdgcn_s_waitcnt(wait_vm(0));
    char *st = wl + (kt % WStages) * WStage;
    const int kleft = kend - kbeg - kt * WBK;
    if (kleft < WBK) {   // zero the A rows this wavefront loaded past the group's end
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (8 * wave + 4 * q + rq >= kleft)
          *reinterpret_cast<u32x4_t *>(st + (2 * wave + q) * 1024 + lane * 16) = u32x4_t{0, 0, 0, 0};
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    }
    __builtin_amdgcn_s_barrier();
    // the stage step kt-1 used is free: refill it with step kt + WStages - 1
    if (kt + WStages - 1 < nk) issue(kt + WStages - 1);
#pragma unroll
    for (int s = 0; s < WBK / 16; ++s) {
      bf16x8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = frag_w(st, wm * 64 + i * 32, s, lane);
        bf[i] = frag_w(st + WTile, wn * 64 + i * 32, s, lane);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }

  // ---- store through LDS, 64 rows at a time: acc[i][j][r] is C_e[m0 + wm*64 + i*32 +
  // 8*(r/4) + 4*(lane/32) + r%4][n0 + wn*64 + j*32 + lane%32]; then each wavefront
  // writes two 512-byte row runs per 16-byte-per-lane store
  constexpr int SROW = WSRow;
  static_assert(64 * SROW <= WLds, "the staged half of C must fit the workgroup's LDS");
  float *C = g.c + static_cast<int64_t>(e) * g.c_estride;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    __syncthreads();   // the ring (or the previous half) is free
    if (wm == h) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int lr = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int lc = wn * 64 + j * 32 + (lane & 31);
            *reinterpret_cast<float *>(wl + lr * SROW + lc * 4) = acc[i][j][r];
          }
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int lr = it * 8 + (threadIdx.x >> 5), cc = threadIdx.x & 31;
      const int m = m0 + h * 64 + lr, n = n0 + cc * 4;
      if (m < g.m && n < g.n)
        __builtin_nontemporal_store(*reinterpret_cast<const f32x4_t *>(wl + lr * SROW + cc * 16),
                                    reinterpret_cast<f32x4_t *>(C + static_cast<int64_t>(m) * g.ldc + n));
    }
  }
}

}  // namespace

hipError_t launch_gemm_bwd(const BwdGemm &g, int groups, hipStream_t st) {
  if (g.mode == BWD_ROWS) {
    const int nbn = (g.n + BN - 1) / BN;
    const int64_t tiles = g.n_tiles_dev ? g.n_tiles_host : (g.dense_rows + BM - 1) / BM;
    const int64_t blocks = (tiles * nbn + kXcds - 1) / kXcds * kXcds;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_rows_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), 0, st, g);
  } else {
    // 16-byte DMA rows and 16-byte stores of C
    if (g.m < 8 || g.n < 8 || g.lda % 8 || g.ldb % 8 || g.ldc % 4 || g.c_estride % 4) return hipErrorInvalidValue;
    const int64_t blocks = static_cast<int64_t>(groups) * ((g.m + BM - 1) / BM) * ((g.n + BN - 1) / BN);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(gemm_wgrad_kernel, dim3(static_cast<unsigned>(blocks)), dim3(kThreads), WLds, st, g);
  }
  return hipGetLastError();
}

}  // namespace moe
