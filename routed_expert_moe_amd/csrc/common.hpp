// Internal declarations shared by the HIP kernels of the MoE layer (forward and backward).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "moe355.h"

namespace moe {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;

// ---- bf16 <-> fp32 -----------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// round-to-nearest-even fp32 -> bf16 bits (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16_bits(lo)) |
         (static_cast<uint32_t>(f32_to_bf16_bits(hi)) << 16);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// ---- host-side caches of device properties and kernel attributes --------------
// One entry per GPU (the current device at the call), filled on first use; the
// entries are atomics, so concurrent calls from several threads are safe.
constexpr int kMaxDevices = 64;
inline int current_device() {
  int d = 0;
  return hipGetDevice(&d) == hipSuccess ? d : 0;
}
// compute units of the current device
inline int device_cu_count() {
  static std::atomic<int> cache[kMaxDevices];
  const int d = current_device();
  int n = d < kMaxDevices ? cache[d].load(std::memory_order_relaxed) : 0;
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, d) != hipSuccess || n <= 0) n = 256;
  if (d < kMaxDevices) cache[d].store(n, std::memory_order_relaxed);
  return n;
}
// raise a kernel's dynamic LDS limit once per device; `done` is that kernel's bit mask
inline hipError_t ensure_dynamic_lds(const void *fn, int bytes, std::atomic<uint64_t> &done) {
  const int d = current_device();
  const uint64_t bit = d < 64 ? (1ull << d) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// ---- GEMM segment: C[rows, N] (+)= A[rows, K] * B[N, K]^T for one group of rows
// sharing a weight matrix.  A rows may be gathered: row r of a tile holds pair
// p = sorted_pair[r] (p < 0: zero row) whose token is p / topk.
struct Segment {
  const void *a;          // A base (x, h, hs)
  int64_t lda;            // elements
  const int32_t *gather;  // sorted_pair (routed gate_up) or nullptr (rows are direct)
  int32_t topk;           // pair -> token divisor when gathering
  int32_t a_rows;         // rows valid in A when not gathering (dense segment), else unused
  const void *b;          // B base of expert 0 (or the only matrix)
  int64_t b_stride;       // elements between experts' matrices
  const float *b_scale;   // fp8 block scales of expert 0, or nullptr
  int64_t s_stride;       // floats between experts' scale tensors
  int32_t n;              // B rows (output columns; 2*inter for gate_up)
  int32_t k;              // reduction length
  void *c;                // output base
  int64_t ldc;            // elements
  // tiles: routed segments read the tile lists written by moe_permute; dense
  // segments cover rows [0, a_rows) in tiles of tile_m with expert 0.
  // fp8 activations (W8A8): one fp32 scale per A row per 128 columns of K, and
  // for fp8 output the scales written per C row per 128 output columns
  const float *a_scale;   // [A rows, k/128] or nullptr
  int64_t a_sld;          // floats between A rows' scales
  float *c_scale;         // [C rows, out cols/128] or nullptr
  int64_t c_sld;
  const int32_t *tile_row;
  const int32_t *tile_expert;
  const int32_t *expert_off;   // first row of each expert, multiples of tile_m (routed only)
  const int32_t *n_tiles_dev;  // nullptr -> dense
  int32_t n_tiles_host;        // dense tile count, or capacity for routed
  const int32_t *row_pair;     // routed rows' sorted_pair (< 0 marks padding), or nullptr
  int64_t ldb;                 // k-strided B (backward row form): elements per B row
  // SwiGLU epilogue of the prefill expert GEMM: when set, the pre-activations a
  // (columns [0, n/2)) and c (columns [n/2, n)) of every real row also go out in fp32
  float *c_save;
  int64_t ld_save;             // floats between rows of c_save
};

enum Epilogue { EPI_STORE = 0, EPI_SWIGLU = 1 };

// The forward expert GEMM takes an expert's rows in chunks of up to kChunkTiles
// 128-row tiles; a chunk of t tiles runs as one tile of 128 * chunk_units(t) rows
// (1, 2 or 4 units).
constexpr int kChunkTiles = 2;
__host__ __device__ constexpr int chunk_units(int tiles) { return tiles <= 1 ? 1 : tiles <= 2 ? 2 : 4; }
// 128-row units of n128 tiles cut into chunks
__host__ __device__ constexpr int units_of_tiles(int n128) {
  return n128 <= 0 ? 0
                   : chunk_units(kChunkTiles) * ((n128 - 1) / kChunkTiles) +
                         chunk_units(n128 - kChunkTiles * ((n128 - 1) / kChunkTiles));
}

// plan chosen for (cfg, T)
enum Path { PATH_F32 = 0, PATH_MFMA = 1, PATH_SKINNY = 2, PATH_FP8 = 3 };
struct Plan {
  int path;
  int tile_m;
};

// ---- launchers (each returns hipSuccess or the launch error) ----------------
hipError_t launch_gate_route(const moe_config &cfg, int64_t T, const float *logits,
                             const float *bias, int32_t *topk_idx, float *topk_w, float *keys,
                             hipStream_t st);
// logits[T, E] (fp32) = x[T, D] W_g^T on bf16 MFMA; supported: D a multiple of 128,
// x and W_g below 4 GiB each
bool gate_logits_supported(int64_t T, int E, int D);
hipError_t launch_gate_logits(int64_t T, int E, int D, const void *x, const void *w_gate, float *logits,
                              hipStream_t st);
hipError_t launch_gate_logits_gemv(const moe_config &cfg, int64_t T, const void *x,
                                   const void *w_gate, float *logits, hipStream_t st);
hipError_t launch_permute(const moe_config &cfg, int64_t T, const int32_t *topk_idx,
                          const moe_routing &r, hipStream_t st);
// fp8 x fp8 grouped GEMM (W8A8 experts): A codes with 1x128 scales, B codes with
// 128x128 scales; EPI_SWIGLU writes fp8 codes + scales, EPI_STORE bf16.
bool gemm_fp8_supported(const Segment *segs, int nseg);
hipError_t launch_gemm_fp8(const Segment *segs, int nseg, Epilogue epi, hipStream_t st);
hipError_t launch_quant_act(const void *x, int64_t rows, int64_t cols, uint8_t *q, float *s,
                            hipStream_t st);
size_t balance_loss_workspace_bytes(const moe_config &cfg, int64_t T, int seq_len);
hipError_t launch_balance_loss(const moe_config &cfg, int64_t T, int seq_len, const float *logits,
                               const int32_t *topk_idx, float alpha, void *workspace, float *loss,
                               hipStream_t st);
hipError_t launch_bias_update(const moe_config &cfg, int64_t T, const moe_routing &r, float gamma,
                              float *bias, hipStream_t st);
hipError_t launch_combine(const moe_config &cfg, int64_t T, const void *u, const void *z,
                          const void *y, const moe_routing &r, const float *w, void *out,
                          hipStream_t st);

// out_f32: C is fp32 (gate logits) instead of the act dtype
hipError_t launch_gemm_f32(const Segment *segs, int nseg, int tile_m, Epilogue epi,
                           hipStream_t st);
hipError_t launch_gemm_mfma(const Segment *segs, int nseg, int tile_m, Epilogue epi,
                            bool out_f32, hipStream_t st);
bool gemm_mfma2_supported(const Segment *segs, int nseg);
hipError_t launch_gemm_mfma2(const Segment *segs, int nseg, Epilogue epi, bool out_f32,
                             hipStream_t st);
// C[rows, n] (fp32) = A[rows, k] B_e[k, n] with B_e stored [k][n] (ldb elements
// per row), on the prefill GEMM's tiling; routed segments need 128-row routing tiles
bool gemm_mfma2_bt_supported(const Segment *segs, int nseg);
hipError_t launch_gemm_mfma2_bt(const Segment *segs, int nseg, hipStream_t st);
// The forward expert GEMMs on expert-sized tiles: segs[0] routed, its rows cut
// into the chunk table moe_permute writes with 128-row tiles (units, n_units);
// segs[1] (optional) dense.  a_bytes_max bounds every A matrix's size in bytes.
bool gemm_expert_supported(const Segment *segs, int nseg);
hipError_t launch_gemm_expert(const Segment *segs, int nseg, Epilogue epi, const int32_t *units,
                              const int32_t *n_units, int64_t a_bytes_max, hipStream_t st);
// sets the thread-local message moe_last_error() returns; returns s
moe_status set_error(moe_status s, const char *msg);
// where the chunk table sits in a routing buffer's scratch (in int32 entries)
int64_t permute_units_offset(int64_t P, int E);
hipError_t launch_gemm_skinny(const Segment *segs, int nseg, Epilogue epi, bool w_fp8,
                              bool out_f32, hipStream_t st);

constexpr int kMfmaTileM = 128;
constexpr int kSkinnyTileM = 16;
constexpr int kF32TileM = 64;

}  // namespace moe
