// Host side of the C ABI declared in moe355.h: validation, planning, buffer
// carving and the launch sequence of the layer forward.  Nothing here touches
// device memory except through the kernel launches.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "backward.hpp"

#include <algorithm>

namespace moe {
int64_t permute_scratch_ints(int64_t P, int E);
}

using namespace moe;

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}
moe_status ok() {
  g_err[0] = '\0';
  return MOE_OK;
}
moe_status device_fail(hipError_t e, const char *what) {
  return fail(MOE_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

size_t act_bytes(const moe_config &c) { return c.act_dtype == MOE_F32 ? 4 : 2; }
size_t weight_bytes(const moe_config &c) {
  return c.weight_dtype == MOE_F32 ? 4 : c.weight_dtype == MOE_BF16 ? 2 : 1;
}

Plan plan_for(const moe_config &c, int64_t T) {
  if (c.act_dtype == MOE_F32) return Plan{PATH_F32, kF32TileM};
  if (c.act_quant) return Plan{PATH_FP8, kMfmaTileM};
  if (c.weight_dtype == MOE_FP8_E4M3_B128) return Plan{PATH_SKINNY, kSkinnyTileM};
  const int64_t avg_rows = T * c.top_k / c.n_routed;
  if (avg_rows < 32) return Plan{PATH_SKINNY, kSkinnyTileM};
  return Plan{PATH_MFMA, kMfmaTileM};
}

struct RoutingLayout {
  int tile_m;
  int64_t max_rows, max_tiles, P;
  size_t off_counts, off_expert_off, off_sorted, off_pair_row, off_tile_expert, off_tile_row,
      off_ntiles, off_scratch, off_act_q, off_act_s, total;
};

RoutingLayout routing_layout(const moe_config &c, int64_t T) {
  RoutingLayout L{};
  const Plan p = plan_for(c, T);
  L.tile_m = p.tile_m;
  L.P = T * c.top_k;
  // rows in use: every expert that received a pair pads to a multiple of tile_m, and at
  // most min(P, E) experts receive one
  const int64_t busy = std::min<int64_t>(L.P, c.n_routed);
  L.max_rows = static_cast<int64_t>(round_up(static_cast<size_t>(L.P + busy * (p.tile_m - 1)), p.tile_m));
  L.max_tiles = L.max_rows / p.tile_m;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = round_up(o + bytes, kAlign);
    return at;
  };
  L.off_counts = take(4 * static_cast<size_t>(c.n_routed));
  L.off_expert_off = take(4 * static_cast<size_t>(c.n_routed + 1));
  L.off_sorted = take(4 * static_cast<size_t>(L.max_rows));
  L.off_pair_row = take(4 * static_cast<size_t>(L.P));
  L.off_tile_expert = take(4 * static_cast<size_t>(L.max_tiles));
  L.off_tile_row = take(4 * static_cast<size_t>(L.max_tiles));
  L.off_ntiles = take(4);
  L.off_scratch = take(4 * static_cast<size_t>(permute_scratch_ints(L.P, c.n_routed)));
  if (c.act_quant) {   // fp8 codes of x and their 1 x 128 scales
    L.off_act_q = take(static_cast<size_t>(T) * c.dim);
    L.off_act_s = take(4 * static_cast<size_t>(T) * (c.dim / 128));
  }
  L.total = o;
  return L;
}

struct WorkspaceLayout {
  RoutingLayout rl;
  size_t off_logits, off_idx, off_w, off_routing, off_h, off_hs, off_y, off_z, total;
};

WorkspaceLayout workspace_layout(const moe_config &c, int64_t T) {
  WorkspaceLayout W{};
  W.rl = routing_layout(c, T);
  const size_t ab = act_bytes(c);
  const int64_t SI = static_cast<int64_t>(c.n_shared) * c.inter_dim;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = round_up(o + bytes, kAlign);
    return at;
  };
  W.off_logits = take(4 * static_cast<size_t>(T) * c.n_routed);
  W.off_idx = take(4 * static_cast<size_t>(W.rl.P));
  W.off_w = take(4 * static_cast<size_t>(W.rl.P));
  W.off_routing = take(W.rl.total);
  W.off_h = take(ab * static_cast<size_t>(W.rl.max_rows) * c.inter_dim);
  W.off_hs = take(ab * static_cast<size_t>(T) * SI);
  W.off_y = take(ab * static_cast<size_t>(W.rl.max_rows) * c.dim);
  W.off_z = take(ab * static_cast<size_t>(T) * c.dim);
  W.total = o;
  return W;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

moe_status check_cfg(const moe_config *c) {
  if (c == nullptr) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->dim <= 0 || c->inter_dim <= 0) return fail(MOE_ERR_INVALID_ARG, "dim and inter_dim must be > 0");
  if (c->n_routed <= 0) return fail(MOE_ERR_INVALID_ARG, "n_routed must be > 0");
  if (c->n_shared < 0) return fail(MOE_ERR_INVALID_ARG, "n_shared must be >= 0");
  if (c->n_groups <= 0 || c->n_routed % c->n_groups != 0)
    return fail(MOE_ERR_INVALID_ARG, "n_groups must divide n_routed (got %d, %d)", c->n_groups, c->n_routed);
  if (c->topk_groups < 1 || c->topk_groups > c->n_groups)
    return fail(MOE_ERR_INVALID_ARG, "topk_groups must be in [1, n_groups]");
  const int gsz = c->n_routed / c->n_groups;
  if (c->top_k < 1 || c->top_k > c->topk_groups * gsz)
    return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, topk_groups * n_routed / n_groups]");
  if (!isfinite(c->route_scale) || !(c->route_scale > 0.0f))
    return fail(MOE_ERR_INVALID_ARG, "route_scale must be finite and > 0");
  if (c->score_func != MOE_SCORE_SIGMOID && c->score_func != MOE_SCORE_SOFTMAX)
    return fail(MOE_ERR_INVALID_ARG, "unknown score_func %d", c->score_func);
  if (c->norm_topk < -1 || c->norm_topk > 1) return fail(MOE_ERR_INVALID_ARG, "norm_topk must be -1, 0 or 1");
  if (c->add_residual != 0 && c->add_residual != 1) return fail(MOE_ERR_INVALID_ARG, "add_residual must be 0 or 1");
  const bool pair_ok = (c->act_dtype == MOE_F32 && c->weight_dtype == MOE_F32) ||
                       (c->act_dtype == MOE_BF16 && c->weight_dtype == MOE_BF16) ||
                       (c->act_dtype == MOE_BF16 && c->weight_dtype == MOE_FP8_E4M3_B128);
  if (c->act_dtype < MOE_F32 || c->act_dtype > MOE_BF16 || c->weight_dtype < MOE_F32 ||
      c->weight_dtype > MOE_FP8_E4M3_B128)
    return fail(MOE_ERR_INVALID_ARG, "unknown dtype");
  if (!pair_ok) return fail(MOE_ERR_UNSUPPORTED, "unsupported (act, weight) dtype pair (%d, %d)", c->act_dtype, c->weight_dtype);
  if (c->n_routed > 512) return fail(MOE_ERR_UNSUPPORTED, "n_routed > 512");
  if (c->top_k > 32) return fail(MOE_ERR_UNSUPPORTED, "top_k > 32");
  if (c->n_groups > 64) return fail(MOE_ERR_UNSUPPORTED, "n_groups > 64");
  if (c->dim % 8 != 0 || c->inter_dim % 8 != 0) return fail(MOE_ERR_UNSUPPORTED, "dim and inter_dim must be multiples of 8");
  if (c->weight_dtype == MOE_FP8_E4M3_B128 && (c->dim % 128 != 0 || c->inter_dim % 128 != 0))
    return fail(MOE_ERR_UNSUPPORTED, "fp8 block scales need dim and inter_dim multiples of 128");
  if (c->act_quant != 0 && c->act_quant != 1) return fail(MOE_ERR_INVALID_ARG, "act_quant must be 0 or 1");
  if (c->act_quant) {
    if (c->act_dtype != MOE_BF16 || c->weight_dtype != MOE_FP8_E4M3_B128)
      return fail(MOE_ERR_UNSUPPORTED, "act_quant needs bf16 activations and fp8 weights");
    // the fp8 GEMM keeps one weight row's block scales in two registers per lane
    if (c->dim > 16384 || static_cast<int64_t>(c->inter_dim) * (c->n_shared > 0 ? c->n_shared : 1) > 16384)
      return fail(MOE_ERR_UNSUPPORTED, "act_quant supports reduction lengths (dim, n_shared*inter_dim) up to 16384");
  }
  return MOE_OK;
}

moe_status check_T(const moe_config &c, int64_t T) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T must be >= 0");
  const int64_t rows = T * c.top_k + static_cast<int64_t>(c.n_routed) * 128;
  if (T > (1ll << 31) / 64 || rows >= (1ll << 31))
    return fail(MOE_ERR_UNSUPPORTED, "T too large for 32-bit row indices");
  if (c.act_quant) {   // the fp8 GEMM addresses its operands with 32-bit byte offsets
    const int64_t SI = static_cast<int64_t>(c.n_shared) * c.inter_dim;
    if (T * c.dim >= (1ll << 31) || rows * c.inter_dim >= (1ll << 31) || T * SI >= (1ll << 31))
      return fail(MOE_ERR_UNSUPPORTED, "act_quant: activation matrices must stay below 2 GiB");
  }
  return MOE_OK;
}

moe_status check_bias(const moe_config &c, const float *bias) {
  if (bias != nullptr && c.n_groups > 1 && c.n_routed / c.n_groups < 2)
    return fail(MOE_ERR_INVALID_ARG, "with a bias the group score is a top-2 sum: group size must be >= 2");
  return MOE_OK;
}

}  // namespace

// the thread-local message moe_last_error returns, for entry points in other sources
namespace moe {
moe_status set_error(moe_status s, const char *msg) {
  snprintf(g_err, sizeof(g_err), "%s", msg);
  return s;
}
}  // namespace moe

namespace {

#define MOE_TRY(expr)            \
  do {                           \
    const moe_status s_ = (expr); \
    if (s_ != MOE_OK) return s_; \
  } while (0)

#define MOE_NEED(p, name)                                                       \
  do {                                                                          \
    if ((p) == nullptr) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);   \
    if (!aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name); \
  } while (0)

#define MOE_OPT(p, name)                                                        \
  do {                                                                          \
    if ((p) != nullptr && !aligned16(p))                                        \
      return fail(MOE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);      \
  } while (0)

moe_status check_routing(const moe_config &c, int64_t T, const moe_routing *r) {
  if (r == nullptr) return fail(MOE_ERR_INVALID_ARG, "routing is NULL");
  const RoutingLayout L = routing_layout(c, T);
  if (r->tile_m != L.tile_m || r->max_rows != L.max_rows || r->max_tiles != L.max_tiles)
    return fail(MOE_ERR_INVALID_ARG, "routing was built for another configuration or T");
  if (!r->counts || !r->expert_off || !r->sorted_pair || !r->pair_row || !r->tile_expert ||
      !r->tile_row || !r->n_tiles || !r->scratch)
    return fail(MOE_ERR_INVALID_ARG, "routing has NULL arrays");
  if (c.act_quant && (!r->act_q || !r->act_s))
    return fail(MOE_ERR_INVALID_ARG, "routing was built without act_quant buffers");
  return MOE_OK;
}

// ---- the step implementations (arguments already validated) ---------------
moe_status do_gate(const moe_config &c, int64_t T, const void *x, const void *w_gate,
                   const float *bias, float *logits, int32_t *idx, float *w, float *keys,
                   hipStream_t st) {
  Segment s{};
  s.a = x;
  s.lda = c.dim;
  s.a_rows = static_cast<int32_t>(T);
  s.b = w_gate;
  s.n = c.n_routed;
  s.k = c.dim;
  s.c = logits;
  s.ldc = c.n_routed;
  hipError_t e;
  if (c.act_dtype == MOE_F32) {
    s.n_tiles_host = static_cast<int32_t>((T + kF32TileM - 1) / kF32TileM);
    e = launch_gemm_f32(&s, 1, kF32TileM, EPI_STORE, st);
  } else if (T >= 64) {
    if (gate_logits_supported(T, c.n_routed, c.dim)) {
      e = launch_gate_logits(T, c.n_routed, c.dim, x, w_gate, logits, st);
    } else {
      s.n_tiles_host = static_cast<int32_t>((T + kMfmaTileM - 1) / kMfmaTileM);
      e = launch_gemm_mfma(&s, 1, kMfmaTileM, EPI_STORE, true, st);
    }
  } else {
    e = launch_gate_logits_gemv(c, T, x, w_gate, logits, st);
  }
  if (e != hipSuccess) return device_fail(e, "gate logits launch");
  e = launch_gate_route(c, T, logits, bias, idx, w, keys, st);
  if (e != hipSuccess) return device_fail(e, "gate route launch");
  return ok();
}

// which: 1 = gate/up half, 2 = down half, 3 = both
// ab / abs (optional): the gate/up pre-activations in fp32 ([rows, 2I] routed, [T, 2SI]
// shared); only the prefill expert GEMM writes them, and *saved says whether it ran
moe_status do_ffn(const moe_config &c, int64_t T, const void *x, const moe_routing &r,
                  const moe_weights &w, void *h, void *y, void *hs, void *z, hipStream_t st,
                  int which = 3, float *ab = nullptr, float *abs = nullptr, bool *saved = nullptr) {
  const Plan p = plan_for(c, T);
  const int64_t D = c.dim, I = c.inter_dim, SI = static_cast<int64_t>(c.n_shared) * c.inter_dim;
  const bool fp8 = c.weight_dtype == MOE_FP8_E4M3_B128;
  const bool shared = hs != nullptr && (which == 1 || z != nullptr) && c.n_shared > 0;
  const int32_t dense_tiles = static_cast<int32_t>((T + p.tile_m - 1) / p.tile_m);

  Segment up[2] = {}, dn[2] = {};
  up[0].a = x;
  up[0].lda = D;
  up[0].gather = r.sorted_pair;
  up[0].row_pair = r.sorted_pair;
  up[0].topk = c.top_k;
  up[0].b = w.w13;
  up[0].b_stride = 2 * I * D;
  up[0].b_scale = w.w13_scale;
  up[0].s_stride = fp8 ? (2 * I / 128) * (D / 128) : 0;
  up[0].n = static_cast<int32_t>(2 * I);
  up[0].k = static_cast<int32_t>(D);
  up[0].c = h;
  up[0].ldc = I;
  up[0].tile_row = r.tile_row;
  up[0].tile_expert = r.tile_expert;
  up[0].expert_off = r.expert_off;
  up[0].n_tiles_dev = r.n_tiles;
  up[0].n_tiles_host = r.max_tiles;

  dn[0].a = h;
  dn[0].lda = I;
  dn[0].b = w.w2;
  dn[0].b_stride = D * I;
  dn[0].b_scale = w.w2_scale;
  dn[0].s_stride = fp8 ? (D / 128) * (I / 128) : 0;
  dn[0].n = static_cast<int32_t>(D);
  dn[0].k = static_cast<int32_t>(I);
  dn[0].c = y;
  dn[0].ldc = D;
  dn[0].tile_row = r.tile_row;
  dn[0].tile_expert = r.tile_expert;
  dn[0].expert_off = r.expert_off;
  dn[0].n_tiles_dev = r.n_tiles;
  dn[0].n_tiles_host = r.max_tiles;
  dn[0].row_pair = r.sorted_pair;

  int nseg = 1;
  if (shared) {
    nseg = 2;
    up[1].a = x;
    up[1].lda = D;
    up[1].a_rows = static_cast<int32_t>(T);
    up[1].b = w.sw13;
    up[1].b_scale = w.sw13_scale;
    up[1].n = static_cast<int32_t>(2 * SI);
    up[1].k = static_cast<int32_t>(D);
    up[1].c = hs;
    up[1].ldc = SI;
    up[1].n_tiles_host = dense_tiles;

    dn[1].a = hs;
    dn[1].lda = SI;
    dn[1].a_rows = static_cast<int32_t>(T);
    dn[1].b = w.sw2;
    dn[1].b_scale = w.sw2_scale;
    dn[1].n = static_cast<int32_t>(D);
    dn[1].k = static_cast<int32_t>(SI);
    dn[1].c = z;
    dn[1].ldc = D;
    dn[1].n_tiles_host = dense_tiles;
  }
  if (p.path == PATH_FP8) {
    // W8A8: gate/up read the fp8 codes of x (moe_quant_act) and leave h as fp8
    // codes followed by their scales inside the h buffer; down reads them back
    float *h_s = reinterpret_cast<float *>(static_cast<char *>(h) +
                                           round_up(static_cast<size_t>(r.max_rows) * I, kAlign));
    up[0].a = r.act_q;
    up[0].lda = D;
    up[0].a_scale = r.act_s;
    up[0].a_sld = D / 128;
    up[0].ldc = I;
    up[0].c_scale = h_s;
    up[0].c_sld = I / 128;
    dn[0].lda = I;
    dn[0].a_scale = h_s;
    dn[0].a_sld = I / 128;
    if (shared) {
      float *hs_s = reinterpret_cast<float *>(static_cast<char *>(hs) +
                                              round_up(static_cast<size_t>(T) * SI, kAlign));
      up[1].a = r.act_q;
      up[1].lda = D;
      up[1].a_scale = r.act_s;
      up[1].a_sld = D / 128;
      up[1].ldc = SI;
      up[1].c_scale = hs_s;
      up[1].c_sld = SI / 128;
      dn[1].lda = SI;
      dn[1].a_scale = hs_s;
      dn[1].a_sld = SI / 128;
    }
  }
  if (ab != nullptr) {
    up[0].c_save = ab;
    up[0].ld_save = 2 * I;
    if (shared) {
      up[1].c_save = abs;
      up[1].ld_save = 2 * SI;
    }
  }
  if (saved != nullptr) *saved = false;
  auto run = [&](Segment *segs, Epilogue epi) -> hipError_t {
    switch (p.path) {
      case PATH_F32: return launch_gemm_f32(segs, nseg, p.tile_m, epi, st);
      case PATH_FP8: return launch_gemm_fp8(segs, nseg, epi, st);
      case PATH_MFMA:
        if (r.tile_m == 128 && gemm_expert_supported(segs, nseg)) {
          if (segs == up && saved != nullptr) *saved = true;
          const int32_t *nu = r.scratch + permute_units_offset(T * c.top_k, c.n_routed);
          const int64_t a_bytes = segs == up ? T * D * 2
                                             : std::max<int64_t>(static_cast<int64_t>(r.max_rows) * I, T * SI) * 2;
          return launch_gemm_expert(segs, nseg, epi, nu + 4, nu, a_bytes, st);
        }
        if (gemm_mfma2_supported(segs, nseg)) return launch_gemm_mfma2(segs, nseg, epi, false, st);
        return launch_gemm_mfma(segs, nseg, p.tile_m, epi, false, st);
      default: return launch_gemm_skinny(segs, nseg, epi, fp8, false, st);
    }
  };
  hipError_t e = hipSuccess;
  if (which & 1) e = run(up, EPI_SWIGLU);
  if (e == hipSuccess && (which & 2)) e = run(dn, EPI_STORE);
  if (e != hipSuccess) return device_fail(e, "expert FFN launch");
  return ok();
}

moe_status check_weights(const moe_config &c, const moe_weights *w, bool need_shared) {
  if (w == nullptr) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  MOE_NEED(w->w13, "w13");
  MOE_NEED(w->w2, "w2");
  const bool fp8 = c.weight_dtype == MOE_FP8_E4M3_B128;
  if (fp8) {
    if (w->w13_scale == nullptr || w->w2_scale == nullptr)
      return fail(MOE_ERR_INVALID_ARG, "fp8 weights need w13_scale and w2_scale");
  }
  if (need_shared && c.n_shared > 0) {
    MOE_NEED(w->sw13, "sw13");
    MOE_NEED(w->sw2, "sw2");
    if (fp8 && (w->sw13_scale == nullptr || w->sw2_scale == nullptr))
      return fail(MOE_ERR_INVALID_ARG, "fp8 shared weights need sw13_scale and sw2_scale");
  }
  return MOE_OK;
}


// ---- backward workspace ------------------------------------------------------
struct BwdLayout {
  RoutingLayout rl;
  int64_t tcap;   // 128-row tile capacity
  size_t off_trow, off_texp, off_tend, off_tfirst, off_nt, off_ab, off_dy, off_dh, off_h, off_dab, off_dxp, off_dw,
      off_dl, off_dxg, off_abs, off_dhs, off_hsb, off_dabs, off_dxs, off_xs, total;
};

BwdLayout bwd_layout(const moe_config &c, int64_t T) {
  BwdLayout L{};
  L.rl = routing_layout(c, T);
  const size_t MR = static_cast<size_t>(L.rl.max_rows), D = c.dim, I = c.inter_dim, E = c.n_routed,
               K = c.top_k, SI = static_cast<size_t>(c.n_shared) * c.inter_dim, Tz = static_cast<size_t>(T);
  L.tcap = L.rl.max_rows / 128 + 1 + c.n_routed;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = round_up(o + bytes, kAlign);
    return at;
  };
  L.off_trow = take(4 * static_cast<size_t>(L.tcap));
  L.off_texp = take(4 * static_cast<size_t>(L.tcap));
  L.off_tend = take(4 * static_cast<size_t>(L.tcap));
  L.off_tfirst = take(4 * static_cast<size_t>(L.tcap));
  L.off_nt = take(4);
  L.off_ab = take(4 * MR * 2 * I);
  L.off_dy = take(2 * MR * D);
  L.off_dh = take(4 * MR * I);
  L.off_h = take(2 * MR * I);
  L.off_dab = take(2 * MR * 2 * I);
  L.off_dxp = take(4 * MR * D);
  L.off_dw = take(4 * Tz * K);
  L.off_dl = take(2 * Tz * E);
  L.off_dxg = take(4 * Tz * D);
  L.off_abs = take(4 * Tz * 2 * SI);
  L.off_dhs = take(4 * Tz * SI);
  L.off_hsb = take(2 * Tz * SI);
  L.off_dabs = take(2 * Tz * 2 * SI);
  L.off_dxs = take(4 * Tz * D);
  L.off_xs = take(2 * MR * D);
  L.total = o;
  return L;
}

moe_status check_bwd_cfg(const moe_config &c) {
  if (c.act_dtype != MOE_BF16 || c.weight_dtype != MOE_BF16 || c.act_quant)
    return fail(MOE_ERR_UNSUPPORTED, "the backward pass supports bf16 activations and bf16 weights only");
  if (c.dim % 8 || c.inter_dim % 8 || c.n_routed % 8)
    return fail(MOE_ERR_UNSUPPORTED, "the backward pass needs dim, inter_dim and n_routed multiples of 8");
  return MOE_OK;
}

// Row-form backward product C[rows, n] (fp32) = A[rows, k] B_e[k, n]: on the
// prefill GEMM's k-strided mode where its tiling fits (K a multiple of 64,
// routed rows in 128-row routing tiles), else on the backward GEMM
hipError_t rows_gemm(const BwdGemm &q, const moe_routing *routed, hipStream_t st) {
  Segment s{};
  s.a = q.a;
  s.lda = q.lda;
  s.b = q.b;
  s.b_stride = q.b_estride;
  s.ldb = q.ldb;
  s.n = q.n;
  s.k = q.k;
  s.c = q.c;
  s.ldc = q.ldc;
  if (routed != nullptr) {
    s.tile_row = routed->tile_row;
    s.tile_expert = routed->tile_expert;
    s.expert_off = routed->expert_off;
    s.n_tiles_dev = routed->n_tiles;
    s.n_tiles_host = routed->max_tiles;
    s.row_pair = routed->sorted_pair;
  } else {
    s.a_rows = q.dense_rows;
    s.n_tiles_host = (q.dense_rows + 127) / 128;
  }
  // 16-byte DMA rows: A and B row lengths multiples of 8 elements
  const bool fits = (routed == nullptr || routed->tile_m == 128) && q.lda % 8 == 0 && q.ldb % 8 == 0 &&
                    gemm_mfma2_bt_supported(&s, 1);
  return fits ? launch_gemm_mfma2_bt(&s, 1, st) : launch_gemm_bwd(q, 1, st);
}

// C = A B^T with fp32 output (EPI_STORE) on the forward GEMM the plan picks
hipError_t store_gemm_f32(const Plan &p, Segment *segs, int nseg, hipStream_t st) {
  switch (p.path) {
    case PATH_MFMA:
      if (gemm_mfma2_supported(segs, nseg)) return launch_gemm_mfma2(segs, nseg, EPI_STORE, true, st);
      return launch_gemm_mfma(segs, nseg, p.tile_m, EPI_STORE, true, st);
    case PATH_SKINNY: return launch_gemm_skinny(segs, nseg, EPI_STORE, false, true, st);
    default: return hipErrorNotSupported;
  }
}

// a = W1_e x and c = W3_e x of every routed row ([rows, 2I] fp32: a then c) and, when
// abs != nullptr, of the shared expert on every token ([T, 2SI]), as one fp32 GEMM
hipError_t preact_gemm(const moe_config &c, int64_t T, const void *x, const moe_routing &r,
                       const moe_weights &w, float *ab, float *abs, hipStream_t st) {
  const Plan p = plan_for(c, T);
  const int64_t D = c.dim, I = c.inter_dim, SI = static_cast<int64_t>(c.n_shared) * c.inter_dim;
  Segment up[2] = {};
  up[0].a = x;
  up[0].lda = D;
  up[0].gather = r.sorted_pair;
  up[0].row_pair = r.sorted_pair;
  up[0].topk = c.top_k;
  up[0].b = w.w13;
  up[0].b_stride = 2 * I * D;
  up[0].n = static_cast<int32_t>(2 * I);
  up[0].k = static_cast<int32_t>(D);
  up[0].c = ab;
  up[0].ldc = 2 * I;
  up[0].tile_row = r.tile_row;
  up[0].tile_expert = r.tile_expert;
  up[0].expert_off = r.expert_off;
  up[0].n_tiles_dev = r.n_tiles;
  up[0].n_tiles_host = r.max_tiles;
  int nseg = 1;
  if (abs != nullptr && c.n_shared > 0) {
    nseg = 2;
    up[1].a = x;
    up[1].lda = D;
    up[1].a_rows = static_cast<int32_t>(T);
    up[1].b = w.sw13;
    up[1].n = static_cast<int32_t>(2 * SI);
    up[1].k = static_cast<int32_t>(D);
    up[1].c = abs;
    up[1].ldc = 2 * SI;
    up[1].n_tiles_host = static_cast<int32_t>((T + p.tile_m - 1) / p.tile_m);
  }
  return store_gemm_f32(p, up, nseg, st);
}

}  // namespace

extern "C" {

moe_status moe_validate(const moe_config *cfg) {
  MOE_TRY(check_cfg(cfg));
  return ok();
}

moe_status moe_routing_size(const moe_config *cfg, int64_t T, size_t *bytes) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = routing_layout(*cfg, T).total;
  return ok();
}

moe_status moe_routing_init(const moe_config *cfg, int64_t T, void *buf, size_t bytes,
                            moe_routing *r) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  if (r == nullptr) return fail(MOE_ERR_INVALID_ARG, "routing struct is NULL");
  if (buf == nullptr) return fail(MOE_ERR_INVALID_ARG, "routing buffer is NULL");
  if (reinterpret_cast<uintptr_t>(buf) % kAlign != 0)
    return fail(MOE_ERR_INVALID_ARG, "routing buffer is not 256-byte aligned");
  const RoutingLayout L = routing_layout(*cfg, T);
  if (bytes < L.total) return fail(MOE_ERR_WORKSPACE, "routing buffer too small: %zu < %zu", bytes, L.total);
  char *b = static_cast<char *>(buf);
  r->tile_m = L.tile_m;
  r->max_rows = static_cast<int32_t>(L.max_rows);
  r->max_tiles = static_cast<int32_t>(L.max_tiles);
  r->pad_ = 0;
  r->counts = reinterpret_cast<int32_t *>(b + L.off_counts);
  r->expert_off = reinterpret_cast<int32_t *>(b + L.off_expert_off);
  r->sorted_pair = reinterpret_cast<int32_t *>(b + L.off_sorted);
  r->pair_row = reinterpret_cast<int32_t *>(b + L.off_pair_row);
  r->tile_expert = reinterpret_cast<int32_t *>(b + L.off_tile_expert);
  r->tile_row = reinterpret_cast<int32_t *>(b + L.off_tile_row);
  r->n_tiles = reinterpret_cast<int32_t *>(b + L.off_ntiles);
  r->scratch = reinterpret_cast<int32_t *>(b + L.off_scratch);
  r->act_q = cfg->act_quant ? reinterpret_cast<uint8_t *>(b + L.off_act_q) : nullptr;
  r->act_s = cfg->act_quant ? reinterpret_cast<float *>(b + L.off_act_s) : nullptr;
  return ok();
}

moe_status moe_workspace_size(const moe_config *cfg, int64_t T, size_t *bytes) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = workspace_layout(*cfg, T).total;
  return ok();
}

const char *moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "MOE_ERR_UNKNOWN";
}

const char *moe_last_error(void) { return g_err; }

moe_status moe_gate(const moe_config *cfg, int64_t T, const void *x, const void *w_gate,
                    const float *bias, float *logits, int32_t *topk_idx, float *topk_w,
                    float *keys, void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  MOE_TRY(check_bias(*cfg, bias));
  MOE_NEED(x, "x");
  MOE_NEED(w_gate, "w_gate");
  if (logits == nullptr || topk_idx == nullptr || topk_w == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "logits, topk_idx and topk_w are required");
  if (T == 0) return ok();
  return do_gate(*cfg, T, x, w_gate, bias, logits, topk_idx, topk_w, keys,
                 static_cast<hipStream_t>(stream));
}

moe_status moe_permute(const moe_config *cfg, int64_t T, const int32_t *topk_idx,
                       const moe_routing *r, void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  if (topk_idx == nullptr) return fail(MOE_ERR_INVALID_ARG, "topk_idx is NULL");
  MOE_TRY(check_routing(*cfg, T, r));
  if (T == 0) return ok();
  const hipError_t e = launch_permute(*cfg, T, topk_idx, *r, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "permute launch");
  return ok();
}

moe_status moe_expert_ffn(const moe_config *cfg, int64_t T, const void *x,
                          const moe_routing *r, const moe_weights *w, void *h, void *y_pairs,
                          void *hs, void *z, void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  MOE_NEED(x, "x");
  MOE_TRY(check_routing(*cfg, T, r));
  MOE_TRY(check_weights(*cfg, w, z != nullptr));
  MOE_NEED(h, "h");
  MOE_NEED(y_pairs, "y_pairs");
  if (z != nullptr && cfg->n_shared > 0) {
    MOE_NEED(hs, "hs");
    MOE_NEED(z, "z");
  }
  if (T == 0) return ok();
  return do_ffn(*cfg, T, x, *r, *w, h, y_pairs, hs, z, static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn_save(const moe_config *cfg, int64_t T, const void *x, const moe_routing *r,
                               const moe_weights *w, void *h, void *y_pairs, void *hs, void *z, float *ab,
                               float *abs, void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  MOE_TRY(check_bwd_cfg(*cfg));
  MOE_NEED(x, "x");
  MOE_TRY(check_routing(*cfg, T, r));
  const bool shared = cfg->n_shared > 0;
  MOE_TRY(check_weights(*cfg, w, shared));
  MOE_NEED(h, "h");
  MOE_NEED(y_pairs, "y_pairs");
  if (ab == nullptr || !aligned16(ab)) return fail(MOE_ERR_INVALID_ARG, "ab must be non-NULL and 16-byte aligned");
  if (shared) {
    MOE_NEED(hs, "hs");
    MOE_NEED(z, "z");
    if (abs == nullptr || !aligned16(abs))
      return fail(MOE_ERR_INVALID_ARG, "abs must be non-NULL and 16-byte aligned");
  }
  if (T == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  bool saved = false;
  MOE_TRY(do_ffn(*cfg, T, x, *r, *w, h, y_pairs, shared ? hs : nullptr, shared ? z : nullptr, st, 3, ab,
                 shared ? abs : nullptr, &saved));
  if (!saved) {   // a path whose gate/up GEMM keeps no fp32 copy: one more GEMM writes it
    const hipError_t e = preact_gemm(*cfg, T, x, *r, *w, ab, shared ? abs : nullptr, st);
    if (e != hipSuccess) return device_fail(e, "pre-activation GEMM launch");
  }
  return ok();
}

moe_status moe_expert_up(const moe_config *cfg, int64_t T, const void *x, const moe_routing *r,
                         const moe_weights *w, void *h, void *hs, void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  MOE_NEED(x, "x");
  MOE_TRY(check_routing(*cfg, T, r));
  MOE_TRY(check_weights(*cfg, w, hs != nullptr));
  MOE_NEED(h, "h");
  MOE_OPT(hs, "hs");
  if (T == 0) return ok();
  return do_ffn(*cfg, T, x, *r, *w, h, nullptr, hs, nullptr, static_cast<hipStream_t>(stream), 1);
}

moe_status moe_expert_down(const moe_config *cfg, int64_t T, const moe_routing *r,
                           const moe_weights *w, const void *h, const void *hs, void *y_pairs,
                           void *z, void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  MOE_TRY(check_routing(*cfg, T, r));
  MOE_TRY(check_weights(*cfg, w, z != nullptr));
  MOE_NEED(h, "h");
  MOE_NEED(y_pairs, "y_pairs");
  if (z != nullptr && cfg->n_shared > 0) {
    MOE_NEED(hs, "hs");
    MOE_NEED(z, "z");
  }
  if (T == 0) return ok();
  return do_ffn(*cfg, T, nullptr, *r, *w, const_cast<void *>(h), y_pairs, const_cast<void *>(hs),
                z, static_cast<hipStream_t>(stream), 2);
}

moe_status moe_combine(const moe_config *cfg, int64_t T, const void *u, const void *z,
                       const void *y_pairs, const moe_routing *r, const float *topk_w,
                       void *out, void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  if (cfg->add_residual) MOE_NEED(u, "u");
  MOE_OPT(z, "z");
  MOE_NEED(y_pairs, "y_pairs");
  MOE_NEED(out, "out");
  if (topk_w == nullptr) return fail(MOE_ERR_INVALID_ARG, "topk_w is NULL");
  MOE_TRY(check_routing(*cfg, T, r));
  if (T == 0) return ok();
  const hipError_t e = launch_combine(*cfg, T, u, z, y_pairs, *r, topk_w, out,
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "combine launch");
  return ok();
}

moe_status moe_quant_act(const moe_config *cfg, int64_t T, const void *x, const moe_routing *r,
                         void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  if (!cfg->act_quant) return fail(MOE_ERR_INVALID_ARG, "moe_quant_act needs cfg->act_quant = 1");
  MOE_NEED(x, "x");
  MOE_TRY(check_routing(*cfg, T, r));
  if (T == 0) return ok();
  const hipError_t e = launch_quant_act(x, T, cfg->dim, r->act_q, r->act_s, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "activation quantisation launch");
  return ok();
}

static moe_status check_balance(const moe_config *cfg, int64_t T, int32_t seq_len) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  if (seq_len < 1) return fail(MOE_ERR_INVALID_ARG, "seq_len must be >= 1");
  if (T % seq_len != 0) return fail(MOE_ERR_INVALID_ARG, "T must be a multiple of seq_len");
  return MOE_OK;
}

moe_status moe_balance_loss_workspace_size(const moe_config *cfg, int64_t T, int32_t seq_len,
                                           size_t *bytes) {
  MOE_TRY(check_balance(cfg, T, seq_len));
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = T == 0 ? 0 : balance_loss_workspace_bytes(*cfg, T, seq_len);
  return ok();
}

moe_status moe_balance_loss(const moe_config *cfg, int64_t T, int32_t seq_len, const float *logits,
                            const int32_t *topk_idx, float alpha, void *workspace,
                            size_t workspace_bytes, float *loss, void *stream) {
  MOE_TRY(check_balance(cfg, T, seq_len));
  if (!isfinite(alpha)) return fail(MOE_ERR_INVALID_ARG, "alpha must be finite");
  if (logits == nullptr || topk_idx == nullptr || loss == nullptr)
    return fail(MOE_ERR_INVALID_ARG, "logits, topk_idx and loss must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(topk_idx) |
       reinterpret_cast<uintptr_t>(loss)) % 4 != 0)
    return fail(MOE_ERR_INVALID_ARG, "logits, topk_idx and loss must be 4-byte aligned");
  if (T == 0) return ok();
  const size_t need = balance_loss_workspace_bytes(*cfg, T, seq_len);
  if (workspace == nullptr) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(MOE_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "balance-loss workspace too small: %zu < %zu", workspace_bytes, need);
  const hipError_t e = launch_balance_loss(*cfg, T, seq_len, logits, topk_idx, alpha, workspace, loss,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "balance loss launch");
  return ok();
}

moe_status moe_bias_update(const moe_config *cfg, int64_t T, const moe_routing *r, float gamma,
                           float *bias, void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  if (!isfinite(gamma) || !(gamma >= 0.0f)) return fail(MOE_ERR_INVALID_ARG, "gamma must be finite and >= 0");
  if (bias == nullptr) return fail(MOE_ERR_INVALID_ARG, "bias is NULL");
  if (reinterpret_cast<uintptr_t>(bias) % 4 != 0) return fail(MOE_ERR_INVALID_ARG, "bias is not 4-byte aligned");
  MOE_TRY(check_routing(*cfg, T, r));
  if (T == 0) return ok();
  const hipError_t e = launch_bias_update(*cfg, T, *r, gamma, bias, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_fail(e, "bias update launch");
  return ok();
}

moe_status moe_forward(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                       void *out, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                       void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  MOE_NEED(x, "x");
  MOE_NEED(out, "out");
  if (out == x) return fail(MOE_ERR_INVALID_ARG, "out must not alias x");
  MOE_TRY(check_weights(*cfg, w, true));
  MOE_NEED(w->w_gate, "w_gate");
  MOE_TRY(check_bias(*cfg, w->bias));
  const moe_config &c = *cfg;
  const WorkspaceLayout W = workspace_layout(c, T);
  if (ws == nullptr) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign != 0)
    return fail(MOE_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (ws_bytes < W.total) return fail(MOE_ERR_WORKSPACE, "workspace too small: %zu < %zu", ws_bytes, W.total);
  if (T == 0) return ok();
  hipStream_t st = static_cast<hipStream_t>(stream);
  char *b = static_cast<char *>(ws);
  float *logits = reinterpret_cast<float *>(b + W.off_logits);
  int32_t *idx = topk_idx != nullptr ? topk_idx : reinterpret_cast<int32_t *>(b + W.off_idx);
  float *wt = topk_w != nullptr ? topk_w : reinterpret_cast<float *>(b + W.off_w);
  moe_routing r{};
  MOE_TRY(moe_routing_init(cfg, T, b + W.off_routing, W.rl.total, &r));
  MOE_TRY(do_gate(c, T, x, w->w_gate, w->bias, logits, idx, wt, nullptr, st));
  hipError_t e = launch_permute(c, T, idx, r, st);
  if (e != hipSuccess) return device_fail(e, "permute launch");
  if (c.act_quant) {
    e = launch_quant_act(x, T, c.dim, r.act_q, r.act_s, st);
    if (e != hipSuccess) return device_fail(e, "activation quantisation launch");
  }
  const bool shared = c.n_shared > 0;
  void *h = b + W.off_h, *hs = b + W.off_hs, *y = b + W.off_y, *z = b + W.off_z;
  MOE_TRY(do_ffn(c, T, x, r, *w, h, y, shared ? hs : nullptr, shared ? z : nullptr, st));
  e = launch_combine(c, T, x, shared ? z : nullptr, y, r, wt, out, st);
  if (e != hipSuccess) return device_fail(e, "combine launch");
  return ok();
}


moe_status moe_backward_workspace_size(const moe_config *cfg, int64_t T, size_t *bytes) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  MOE_TRY(check_bwd_cfg(*cfg));
  if (bytes == nullptr) return fail(MOE_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = bwd_layout(*cfg, T).total;
  return ok();
}

// ab_in / abs_in: the pre-activations moe_expert_ffn_save kept, or nullptr to recompute them
static moe_status backward_impl(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                                const moe_routing *r, const int32_t *topk_idx, const float *topk_w,
                                const float *logits, const void *y_pairs, const void *dout,
                                const float *ab_in, const float *abs_in, const moe_grads *g,
                                void *workspace, size_t workspace_bytes, void *stream) {
  MOE_TRY(check_cfg(cfg));
  MOE_TRY(check_T(*cfg, T));
  MOE_TRY(check_bwd_cfg(*cfg));
  const moe_config &c = *cfg;
  const bool shared = c.n_shared > 0;
  MOE_TRY(check_weights(c, w, shared));
  MOE_NEED(w->w_gate, "w_gate");
  MOE_TRY(check_routing(c, T, r));
  if (g == nullptr) return fail(MOE_ERR_INVALID_ARG, "grads is NULL");
  MOE_NEED(x, "x");
  MOE_NEED(topk_idx, "topk_idx");
  MOE_NEED(topk_w, "topk_w");
  MOE_NEED(logits, "logits");
  MOE_NEED(y_pairs, "y_pairs");
  MOE_NEED(dout, "dout");
  MOE_NEED(g->dx, "grads->dx");
  MOE_NEED(g->dw_gate, "grads->dw_gate");
  MOE_NEED(g->dw13, "grads->dw13");
  MOE_NEED(g->dw2, "grads->dw2");
  if (shared) {
    MOE_NEED(g->dsw13, "grads->dsw13");
    MOE_NEED(g->dsw2, "grads->dsw2");
  }
  if ((reinterpret_cast<uintptr_t>(topk_idx) | reinterpret_cast<uintptr_t>(topk_w) |
       reinterpret_cast<uintptr_t>(logits)) % 4 != 0)
    return fail(MOE_ERR_INVALID_ARG, "topk_idx, topk_w and logits must be 4-byte aligned");
  const void *vec[] = {x, w->w_gate, w->w13, w->w2, y_pairs, dout, g->dx, g->dw_gate, g->dw13, g->dw2};
  for (const void *q : vec)
    if (!aligned16(q)) return fail(MOE_ERR_INVALID_ARG, "x, weights, y_pairs, dout and the gradients must be 16-byte aligned");
  if (shared && (!aligned16(w->sw13) || !aligned16(w->sw2) || !aligned16(g->dsw13) || !aligned16(g->dsw2)))
    return fail(MOE_ERR_INVALID_ARG, "shared weights and gradients must be 16-byte aligned");
  if (ab_in != nullptr && (!aligned16(ab_in) || (shared && !aligned16(abs_in))))
    return fail(MOE_ERR_INVALID_ARG, "ab and abs must be non-NULL and 16-byte aligned");
  if (T == 0) return ok();
  const BwdLayout L = bwd_layout(c, T);
  if (workspace == nullptr) return fail(MOE_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0)
    return fail(MOE_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "backward workspace too small: %zu < %zu", workspace_bytes, L.total);

  hipStream_t st = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  auto at = [&](size_t off) { return static_cast<void *>(ws + off); };
  const int64_t D = c.dim, I = c.inter_dim, SI = static_cast<int64_t>(c.n_shared) * c.inter_dim,
                E = c.n_routed, K = c.top_k;
  int32_t *trow = static_cast<int32_t *>(at(L.off_trow)), *texp = static_cast<int32_t *>(at(L.off_texp)),
          *tend = static_cast<int32_t *>(at(L.off_tend)), *tfirst = static_cast<int32_t *>(at(L.off_tfirst)),
          *nt = static_cast<int32_t *>(at(L.off_nt));
  const float *ab = ab_in != nullptr ? ab_in : static_cast<float *>(at(L.off_ab));
  float *dh = static_cast<float *>(at(L.off_dh)),
        *dxp = static_cast<float *>(at(L.off_dxp)), *dw = static_cast<float *>(at(L.off_dw)),
        *dxg = static_cast<float *>(at(L.off_dxg)), *dhs = static_cast<float *>(at(L.off_dhs)),
        *dxs = static_cast<float *>(at(L.off_dxs));
  const float *abs_ = ab_in != nullptr ? abs_in : static_cast<float *>(at(L.off_abs));
  void *dy = at(L.off_dy), *hb = at(L.off_h), *dab = at(L.off_dab), *dl = at(L.off_dl), *hsb = at(L.off_hsb),
       *dabs = at(L.off_dabs), *xs = at(L.off_xs);
  auto bf = [](const void *q) { return static_cast<const uint16_t *>(q); };
  hipError_t e = hipSuccess;
#define MOE_BWD(call, what) \
  do {                      \
    e = (call);             \
    if (e != hipSuccess) return device_fail(e, what); \
  } while (0)

  // 1. a, c of every used row again, unless the forward kept them: [rows, 2I] fp32
  if (ab_in == nullptr)
    MOE_BWD(preact_gemm(c, T, x, *r, *w, static_cast<float *>(at(L.off_ab)),
                        shared ? static_cast<float *>(at(L.off_abs)) : nullptr, st),
            "backward gate/up recompute launch");
  MOE_BWD(launch_bwd_tiles(r->expert_off, c.n_routed, trow, texp, tend, tfirst, nt, st),
          "backward tile list launch");

  // 2. combine: dw, dy
  MOE_BWD(launch_combine_bwd(dout, y_pairs, *r, topk_w, c.top_k, c.dim, dy, dw, st), "combine backward launch");

  // 3. routed experts: dh = dy W2_e, SwiGLU backward, dx_pairs = dab W13_e, dW2, dW13
  BwdGemm rg{};
  rg.mode = BWD_ROWS;
  rg.tile_row = trow;
  rg.tile_expert = texp;
  rg.tile_end = tend;
  rg.tile_first = tfirst;
  rg.n_tiles_dev = nt;
  rg.n_tiles_host = static_cast<int32_t>(L.tcap);
  BwdGemm q = rg;
  q.a = bf(dy);
  q.lda = D;
  q.b = bf(w->w2);
  q.ldb = I;
  q.b_estride = D * I;
  q.c = dh;
  q.ldc = I;
  q.n = static_cast<int32_t>(I);
  q.k = static_cast<int32_t>(D);
  MOE_BWD(rows_gemm(q, r, st), "backward dh launch");
  MOE_BWD(launch_swiglu_bwd(ab, dh, r->n_tiles, r->tile_m, r->max_rows, static_cast<int>(I), r->sorted_pair,
                            hb, dab, st),
          "backward SwiGLU launch");
  q = rg;
  q.a = bf(dab);
  q.lda = 2 * I;
  q.b = bf(w->w13);
  q.ldb = D;
  q.b_estride = 2 * I * D;
  q.c = dxp;
  q.ldc = D;
  q.n = static_cast<int32_t>(D);
  q.k = static_cast<int32_t>(2 * I);
  MOE_BWD(rows_gemm(q, r, st), "backward dx launch");
  BwdGemm wg{};
  wg.mode = BWD_WGRAD;
  wg.expert_off = r->expert_off;
  q = wg;
  q.a = bf(dy);
  q.lda = D;
  q.b = bf(hb);
  q.ldb = I;
  q.c = g->dw2;
  q.ldc = I;
  q.c_estride = D * I;
  q.m = static_cast<int32_t>(D);
  q.n = static_cast<int32_t>(I);
  MOE_BWD(launch_gemm_bwd(q, c.n_routed, st), "backward dW2 launch");
  // dW13_e reads the tokens in routed-row order
  MOE_BWD(launch_gather_rows(x, *r, c.top_k, c.dim, xs, st), "backward token gather launch");
  q = wg;
  q.a = bf(dab);
  q.lda = 2 * I;
  q.b = bf(xs);
  q.ldb = D;
  q.c = g->dw13;
  q.ldc = D;
  q.c_estride = 2 * I * D;
  q.m = static_cast<int32_t>(2 * I);
  q.n = static_cast<int32_t>(D);
  MOE_BWD(launch_gemm_bwd(q, c.n_routed, st), "backward dW13 launch");

  // 4. shared expert: dz = dout
  if (shared) {
    BwdGemm dg{};
    dg.mode = BWD_ROWS;
    dg.dense_rows = static_cast<int32_t>(T);
    q = dg;
    q.a = bf(dout);
    q.lda = D;
    q.b = bf(w->sw2);
    q.ldb = SI;
    q.c = dhs;
    q.ldc = SI;
    q.n = static_cast<int32_t>(SI);
    q.k = static_cast<int32_t>(D);
    MOE_BWD(rows_gemm(q, nullptr, st), "backward shared dh launch");
    MOE_BWD(launch_swiglu_bwd(abs_, dhs, nullptr, 0, T, static_cast<int>(SI), nullptr, hsb, dabs, st),
            "backward shared SwiGLU launch");
    q = dg;
    q.a = bf(dabs);
    q.lda = 2 * SI;
    q.b = bf(w->sw13);
    q.ldb = D;
    q.c = dxs;
    q.ldc = D;
    q.n = static_cast<int32_t>(D);
    q.k = static_cast<int32_t>(2 * SI);
    MOE_BWD(rows_gemm(q, nullptr, st), "backward shared dx launch");
    BwdGemm dw1{};
    dw1.mode = BWD_WGRAD;
    dw1.dense_rows = static_cast<int32_t>(T);
    q = dw1;
    q.a = bf(dout);
    q.lda = D;
    q.b = bf(hsb);
    q.ldb = SI;
    q.c = g->dsw2;
    q.ldc = SI;
    q.m = static_cast<int32_t>(D);
    q.n = static_cast<int32_t>(SI);
    MOE_BWD(launch_gemm_bwd(q, 1, st), "backward shared dW2 launch");
    q = dw1;
    q.a = bf(dabs);
    q.lda = 2 * SI;
    q.b = bf(x);
    q.ldb = D;
    q.c = g->dsw13;
    q.ldc = D;
    q.m = static_cast<int32_t>(2 * SI);
    q.n = static_cast<int32_t>(D);
    MOE_BWD(launch_gemm_bwd(q, 1, st), "backward shared dW13 launch");
  }

  // 5. gate: dlogits, dx_gate = dl W_g, dW_g = dl^T x
  MOE_BWD(launch_gate_bwd(c, T, logits, topk_idx, r->pair_row, dw, dl, st), "gate backward launch");
  {
    BwdGemm dg{};
    dg.mode = BWD_ROWS;
    dg.dense_rows = static_cast<int32_t>(T);
    dg.a = bf(dl);
    dg.lda = E;
    dg.b = bf(w->w_gate);
    dg.ldb = D;
    dg.c = dxg;
    dg.ldc = D;
    dg.n = static_cast<int32_t>(D);
    dg.k = static_cast<int32_t>(E);
    MOE_BWD(rows_gemm(dg, nullptr, st), "gate dx launch");
    BwdGemm gw{};
    gw.mode = BWD_WGRAD;
    gw.dense_rows = static_cast<int32_t>(T);
    gw.a = bf(dl);
    gw.lda = E;
    gw.b = bf(x);
    gw.ldb = D;
    gw.c = g->dw_gate;
    gw.ldc = D;
    gw.m = static_cast<int32_t>(E);
    gw.n = static_cast<int32_t>(D);
    MOE_BWD(launch_gemm_bwd(gw, 1, st), "gate dW launch");
  }

  // 6. the tokens' gradient
  MOE_BWD(launch_dx_final(T, static_cast<int>(K), static_cast<int>(D), c.add_residual, dout,
                          shared ? dxs : nullptr, dxp, dxg, r->pair_row, g->dx, st),
          "backward dx launch");
#undef MOE_BWD
  return ok();
}

moe_status moe_backward(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                        const moe_routing *r, const int32_t *topk_idx, const float *topk_w,
                        const float *logits, const void *y_pairs, const void *dout, const moe_grads *g,
                        void *workspace, size_t workspace_bytes, void *stream) {
  return backward_impl(cfg, T, x, w, r, topk_idx, topk_w, logits, y_pairs, dout, nullptr, nullptr, g,
                       workspace, workspace_bytes, stream);
}

moe_status moe_backward_saved(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                              const moe_routing *r, const int32_t *topk_idx, const float *topk_w,
                              const float *logits, const void *y_pairs, const void *dout,
                              const float *ab, const float *abs, const moe_grads *g, void *workspace,
                              size_t workspace_bytes, void *stream) {
  if (ab == nullptr) return fail(MOE_ERR_INVALID_ARG, "ab is NULL");
  if (cfg != nullptr && cfg->n_shared > 0 && abs == nullptr) return fail(MOE_ERR_INVALID_ARG, "abs is NULL");
  return backward_impl(cfg, T, x, w, r, topk_idx, topk_w, logits, y_pairs, dout, ab, abs, g, workspace,
                       workspace_bytes, stream);
}

}  // extern "C"
