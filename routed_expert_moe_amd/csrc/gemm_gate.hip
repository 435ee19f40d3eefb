// Gate logits on bf16 MFMA:  logits[T, E] (fp32) = x[T, D] * W_g[E, D]^T
// (DeepSeek-V3 notes page, gate flow, step 1: the affinity of every token with
// every routed expert's centroid).
//
// The product is short in N (the expert count) and long in K (the model width):
// x (T * D * 2 bytes) is read once and W_g (E * D * 2 bytes, 3.7 MB at V3) stays
// in L2, so the launch is bound by how fast the CUs pull operands out of L2, and
// it needs enough tiles to occupy every CU.  A workgroup takes 64 tokens by BN
// experts (BN = 128, or 64 when E is not a multiple of 128 and at most 256), so
// the V3 prefill batch (T = 8192, E = 256) gives 256 tiles.  The work list is
// split into eight contiguous ranges, one per XCD (workgroup b runs on XCD
// b % 8), so the column blocks of one row tile run side by side on one XCD and
// read the tile's x rows from the same L2.
//
// Eight wavefronts: two K groups of four.  Wavefront (g, m, n) multiplies the
// 32 rows m and the BN/2 columns n of the tile over K-slices 4g .. 4g + 3 of
// every 128-wide K step (v_mfma_f32_32x32x16_bf16, weight fragment first so a
// lane ends with four consecutive columns); the two K groups' partial sums are
// added through LDS at the end.  Splitting K inside the workgroup puts two
// wavefronts on every SIMD without reading any fragment twice.
//
// Operands go global -> LDS by buffer_load ... lds (SGPR buffer descriptors, a
// 32-bit byte offset per lane, the K step in the scalar offset) through three
// stages of 128-wide K steps (256-byte rows), two steps ahead: against six
// stages of 64-wide steps this halves the barriers per K and cut the V3 launch
// by about 8 us.  The lane that writes physical 16-byte chunk p of stage row r
// fetches logical chunk p ^ (r & 15), which makes the 16-row fragment reads
// conflict-free.  Token rows past T and expert rows past E load a clamped
// (valid) row and are never stored.
#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = 64;                 // tokens per tile
constexpr int BK = 128;                // K step (bf16 elements): 256 bytes per row
constexpr int kRowBytes = BK * 2;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 3;
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void lds_void_t;

struct GateWork {
  const void *x;      // [T, D] bf16
  const void *w;      // [E, D] bf16
  float *out;         // [T, E] fp32
  int32_t T, E, D;
  int32_t ncb;        // column blocks of BN experts
  int32_t total;      // tiles: row tiles x column blocks
  int32_t per_xcd;    // tiles per XCD range (grid = 8 * per_xcd)
  int32_t vec;        // rows of out are 16-byte aligned (E % 4 == 0, aligned base): float4 stores
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
__device__ __forceinline__ int swz(int row) { return row & 15; }

// wait until at most `ahead` (0 or 1) K steps of this wavefront's loads (L loads each) are in flight
template <int L>
__device__ __forceinline__ void wait_steps(int ahead) {
  switch (ahead) {
    case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
    default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(L)); break;
  }
}

template <int BN>
constexpr int lds_bytes() { return kStages * (BM + BN) * kRowBytes; }

template <int BN>
__global__ __launch_bounds__(kThreads, 1) void gate_logits_kernel(GateWork g) {
  extern __shared__ __attribute__((aligned(1024))) char lds[];
  constexpr int NJ = BN / 64;                 // 32-column MFMA blocks per wavefront (BN/2 columns)
  constexpr int LB = BN / 32;                 // 4-row weight loads per wavefront per step
  constexpr int L = 2 + LB;                   // loads per wavefront per step (two 4-row x loads)
  constexpr int kStage = (BM + BN) * kRowBytes;
  static_assert(kStages - 2 <= 1, "wait_steps covers one step ahead");
  static_assert(BM == 8 * kWaves, "two 4-row x loads per wavefront per step");

  const int b = blockIdx.x;
  const int item = (b % kXcds) * g.per_xcd + b / kXcds;
  if (item >= g.total) return;                // whole workgroup, before any barrier
  const int rt = item / g.ncb, cb = item - rt * g.ncb;
  const int row0 = rt * BM, n0 = cb * BN;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int l32 = lane & 31, khalf = lane >> 5;
  const int lrow = lane >> 4, pch = lane & 15;
  const int T = g.T, E = g.E, D = g.D;
  const int nk = D / BK;
  const uint32_t row_bytes = static_cast<uint32_t>(D) * 2u;

  // ---- DMA: stage rows [0, BM) are x rows, [BM, BM + BN) weight rows
  const auto ra = rsrc(g.x, static_cast<uint32_t>(T) * row_bytes);
  const auto rb = rsrc(g.w, static_cast<uint32_t>(E) * row_bytes);
  const int ar_ld = wave * 8;                                   // this wavefront's x load rows
  uint32_t va[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
    va[i] = static_cast<uint32_t>(min(row0 + ar_ld + 4 * i + lrow, T - 1)) * row_bytes +
            static_cast<uint32_t>((pch ^ swz(ar_ld + 4 * i + lrow)) * 16);
  uint32_t vb[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int r = (wave * LB + i) * 4 + lrow;                   // weight row within the block
    vb[i] = static_cast<uint32_t>(min(n0 + r, E - 1)) * row_bytes +
            static_cast<uint32_t>((pch ^ swz(BM + r)) * 16);
  }
  auto issue = [&](int kt) __attribute__((always_inline)) {
    char *st = lds + (kt % kStages) * kStage;
    const uint32_t k0 = static_cast<uint32_t>(kt) * kRowBytes;
#pragma unroll
    for (int i = 0; i < 2; ++i) load_lds16(ra, va[i], k0, st + (ar_ld + 4 * i) * kRowBytes);
#pragma unroll
    for (int i = 0; i < LB; ++i) load_lds16(rb, vb[i], k0, st + (BM + (wave * LB + i) * 4) * kRowBytes);
  };

  // ---- fragments: K group kg takes slices 2kg, 2kg + 1 (16-byte chunks 4kg + khalf, 4kg + 2 + khalf)
  const int kg = wave >> 2, wq = wave & 3;
  const int wm = wq >> 1, wn = wq & 1;
  const int arow = wm * 32 + l32;
  int brow[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) brow[j] = BM + wn * (BN / 2) + j * 32 + l32;

  f32x16_t acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;

#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (p < nk) issue(p);
  for (int kt = 0; kt < nk; ++kt) {
    // this wavefront's loads of step kt have landed; the barrier makes every
    // wavefront's visible and tells that every wavefront is done with step kt - 1,
    // whose stage the loads of step kt + kStages - 1 refill
    wait_steps<L>(min(kStages - 2, nk - 1 - kt));
    __builtin_amdgcn_s_barrier();
    if (kt + kStages - 1 < nk) issue(kt + kStages - 1);
    const u32x4_t *rows = reinterpret_cast<const u32x4_t *>(lds + (kt % kStages) * kStage);
    bf16x8_t af[4], bf[4][NJ];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int c = 8 * kg + 2 * s + khalf;
      af[s] = __builtin_bit_cast(bf16x8_t, rows[arow * 16 + (c ^ swz(arow))]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) bf[s][j] = __builtin_bit_cast(bf16x8_t, rows[brow[j] * 16 + (c ^ swz(brow[j]))]);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf[s][j], af[s], acc[j], 0, 0, 0);
  }

  // ---- add the K groups: group 1 parks its sums in LDS (lane-contiguous), group 0 adds and stores
  __syncthreads();   // every wavefront is done with the stages (no loads are in flight)
  float *red = reinterpret_cast<float *>(lds);
  if (kg == 1) {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) red[((wq * NJ + j) * 16 + r) * 64 + lane] = acc[j][r];
  }
  __syncthreads();
  if (kg == 1) return;
  // acc[j][4q + t] is C[tile row wm*32 + l32][tile column wn*BN/2 + j*32 + 8q + 4*khalf + t]
  const int row = row0 + arow;
  if (row >= T) return;
  float *orow = g.out + static_cast<int64_t>(row) * E;
  const bool vec = g.vec != 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) v[t] = acc[j][4 * q + t] + red[((wq * NJ + j) * 16 + 4 * q + t) * 64 + lane];
      const int col = n0 + wn * (BN / 2) + j * 32 + 8 * q + 4 * khalf;
      if (vec && col + 4 <= E) {
        *reinterpret_cast<f32x4_t *>(orow + col) = f32x4_t{v[0], v[1], v[2], v[3]};
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (col + t < E) orow[col + t] = v[t];
      }
    }
}

template <int BN>
hipError_t launch_bn(const GateWork &g, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(&gate_logits_kernel<BN>), lds_bytes<BN>(), lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((gate_logits_kernel<BN>), dim3(kXcds * g.per_xcd), dim3(kThreads), lds_bytes<BN>(), st, g);
  return hipGetLastError();
}

}  // namespace

bool gate_logits_supported(int64_t T, int E, int D) {
  return T >= 1 && E >= 1 && D >= BK && D % BK == 0 && T * D * 2 < (1ll << 32) &&
         static_cast<int64_t>(E) * D * 2 < (1ll << 32);
}

hipError_t launch_gate_logits(int64_t T, int E, int D, const void *x, const void *w_gate, float *logits,
                              hipStream_t st) {
  if (!gate_logits_supported(T, E, D)) return hipErrorInvalidValue;
  GateWork g{};
  g.x = x;
  g.w = w_gate;
  g.out = logits;
  g.T = static_cast<int32_t>(T);
  g.E = E;
  g.D = D;
  g.vec = (E % 4 == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0) ? 1 : 0;
  // 128-wide column blocks when E fills them (or is large); 64 otherwise (E = 160 wastes 17%, not 37%)
  const int bn = (E % 128 == 0 || E > 256) ? 128 : 64;
  g.ncb = (E + bn - 1) / bn;
  const int64_t total = (T + BM - 1) / BM * g.ncb;
  g.total = static_cast<int32_t>(total);
  g.per_xcd = static_cast<int32_t>((total + kXcds - 1) / kXcds);
  return bn == 128 ? launch_bn<128>(g, st) : launch_bn<64>(g, st);
}

}  // namespace moe
