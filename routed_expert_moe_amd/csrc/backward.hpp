// Declarations of the layer backward's kernels (moe_backward).
#pragma once
#include "common.hpp"

namespace moe {

// ---- backward GEMMs (bf16 operands, fp32 C) --------------------------------
//   BWD_ROWS:  C[r, n] = sum_k A[r, k] B_e[k, n]; rows r of 128-row tiles (tile
//              lists from launch_bwd_tiles) or of [0, dense_rows)
//   BWD_WGRAD: C_e[m, n] = sum_r A[r, m] B[r, n]; r over [expert_off[e],
//              expert_off[e+1]) or [0, dense_rows)
enum BwdMode { BWD_ROWS = 0, BWD_WGRAD = 1 };
struct BwdGemm {
  int32_t mode;
  const uint16_t *a;
  int64_t lda;
  const uint16_t *b;
  int64_t ldb;
  int64_t b_estride;            // ROWS: elements between experts' B
  float *c;
  int64_t ldc;
  int64_t c_estride;            // WGRAD: elements between experts' C
  int32_t m, n, k;              // ROWS: n, k; WGRAD: m, n
  const int32_t *tile_row, *tile_expert, *tile_end, *n_tiles_dev;   // ROWS routed
  const int32_t *tile_first;    // ROWS routed: index of the first tile of each tile's expert
  int32_t n_tiles_host;         // ROWS routed: tile capacity
  int32_t dense_rows;           // dense segment rows (ROWS tiles / WGRAD reduction)
  const int32_t *expert_off;    // WGRAD routed
};
hipError_t launch_gemm_bwd(const BwdGemm &g, int groups, hipStream_t st);
hipError_t launch_bwd_tiles(const int32_t *expert_off, int E, int32_t *tile_row, int32_t *tile_expert,
                            int32_t *tile_end, int32_t *tile_first, int32_t *n_tiles, hipStream_t st);
hipError_t launch_combine_bwd(const void *dout, const void *y, const moe_routing &r, const float *topk_w,
                              int K, int D, void *dy, float *dw, hipStream_t st);
// xs[r] = x[sorted_pair[r] / K] for every used routed row (zeros for padding)
hipError_t launch_gather_rows(const void *x, const moe_routing &r, int K, int D, void *xs, hipStream_t st);
// h = silu(a) c, da = dh c silu'(a), dc = dh silu(a) per row of ab = [a | c]; rows whose
// row_pair entry is negative (padding) get zeros whatever ab holds
hipError_t launch_swiglu_bwd(const float *ab, const float *dh, const int32_t *n_tiles, int tile_m,
                             int64_t rows_host, int I, const int32_t *row_pair, void *h, void *dab,
                             hipStream_t st);
hipError_t launch_gate_bwd(const moe_config &cfg, int64_t T, const float *logits, const int32_t *topk_idx,
                           const int32_t *pair_row, const float *dw, void *dl, hipStream_t st);
hipError_t launch_dx_final(int64_t T, int K, int D, int residual, const void *dout, const float *dx_shared,
                           const float *dx_pairs, const float *dx_gate, const int32_t *pair_row, void *dx,
                           hipStream_t st);

}  // namespace moe
