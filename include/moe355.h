/*
 * moe355.h - C ABI of an MI355X (gfx950) forward pass for one DeepSeekMoE layer.
 *
 * The layer (DeepSeek-V3 notes page, 73biji.xyz/llm_pp_dsv3, "DeepSeekMoE"
 * paragraph, total-output equation):
 *
 *     h'_t = u_t + FFN_share(u_t) + sum_{r in S_t} g_{r,t} FFN_r(u_t)
 *
 * with S_t and g chosen by the gate (same page, gate flow in five steps):
 * sigmoid scores (plus a per-expert bias that only steers selection), a
 * group-limited top-k, and the unbiased scores at the chosen experts,
 * renormalised and scaled by route_scale.  The conventional softmax top-k
 * gate of the same paragraph is the other scoring mode.  Every expert FFN is
 * a SwiGLU, W2 (silu(W1 u) * (W3 u)).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers unless a comment says "host".  All buffers
 *    are row-major and dense; "K-contiguous" means the last dimension is the
 *    reduction dimension.
 *  - The caller owns every buffer.  Inputs are read only; outputs are fully
 *    overwritten.  The library allocates no device memory; its only global
 *    state is a per-device cache of device properties and kernel attributes,
 *    filled on first use with atomics, so calls from several threads or on
 *    different streams and devices are independent.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Calls only enqueue work: results are ready when the stream is
 *    synchronised.  Nothing is read back to the host.
 *  - Every argument is validated on the host before anything is enqueued; on
 *    any error status no kernel has been launched.  T == 0 returns MOE_OK and
 *    launches nothing.  A launch failure returns MOE_ERR_DEVICE; a fault inside
 *    a kernel surfaces at the caller's next synchronisation, as with any HIP call.
 *  - moe_last_error() returns a thread-local message for the last failing call.
 *  - Same inputs give bitwise-identical outputs (no atomics on any value path;
 *    every reduction has a fixed order).
 */
#ifndef MOE355_H
#define MOE355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,   /* bad configuration, size or NULL pointer */
  MOE_ERR_UNSUPPORTED = 2,   /* valid layer, but outside this library's kernels */
  MOE_ERR_WORKSPACE = 3,     /* workspace / routing buffer too small */
  MOE_ERR_DEVICE = 4         /* a HIP call or kernel launch failed */
} moe_status;

typedef enum {
  MOE_F32 = 0,               /* IEEE binary32 */
  MOE_BF16 = 1,              /* bfloat16 */
  MOE_FP8_E4M3_B128 = 2      /* OCP e4m3fn codes, one fp32 scale per 128x128 block */
} moe_dtype;

typedef enum {
  MOE_SCORE_SIGMOID = 0,     /* s = sigmoid(W_g u); ranked key s + b */
  MOE_SCORE_SOFTMAX = 1      /* p = softmax(W_g u) over all experts; ranked key = logit (p + b with a bias) */
} moe_score;

/* The layer's hyper-parameters, named as in the DeepSeek-V3 model.py config
 * table on the notes page (dim, n_routed_experts, n_shared_experts, n_expert_groups,
 * n_limited_groups -> topk_groups, n_activated_experts -> top_k, route_scale,
 * moe_inter_dim -> inter_dim, score_func). */
typedef struct moe_config {
  int32_t dim;           /* model width D */
  int32_t n_routed;      /* routed experts E, 1..512 */
  int32_t n_shared;      /* shared experts S >= 0; they act as one SwiGLU of hidden S*inter_dim */
  int32_t n_groups;      /* routing groups G (E % G == 0); 1 = no group limit */
  int32_t topk_groups;   /* groups kept per token, 1..G */
  int32_t top_k;         /* experts per token K, 1..min(32, topk_groups*E/G) */
  int32_t inter_dim;     /* hidden size I of one expert */
  float route_scale;     /* finite, > 0 */
  int32_t score_func;    /* moe_score */
  int32_t norm_topk;     /* -1: sigmoid renormalises the chosen weights, softmax does not; 0/1 force */
  int32_t act_dtype;     /* x, out, w_gate, intermediates: MOE_F32 or MOE_BF16 */
  int32_t weight_dtype;  /* routed + shared expert weights: MOE_F32 (with act F32), MOE_BF16 or
                            MOE_FP8_E4M3_B128 (with act BF16) */
  int32_t add_residual;  /* 1: out includes u_t (the total-output equation); 0: out = FFN terms only */
  int32_t act_quant;     /* 0: the expert GEMMs read activations in act dtype (W8A16 with fp8
                            weights); 1: FP8 W8A8 (DeepSeek-R1 analysis page, training-process
                            hyper-parameters paragraph: FP8 mixed precision, W8A8):
                            x and the SwiGLU output h are quantised to e4m3 with one fp32 scale
                            per row per 128 columns, s = max|a|/448 (1 for a zero block),
                            code = round-to-nearest-even(a/s), right before each expert GEMM.
                            Requires act BF16 and weights FP8_E4M3_B128. */
} moe_config;

/* Expert weights.  fp8 scale tensors are fp32 with one entry per 128x128 block
 * of the matrix they scale (NULL for other dtypes). */
typedef struct moe_weights {
  const void *w_gate;        /* [E, D] act dtype, K-contiguous (one row per routed expert) */
  const float *bias;         /* [E] fp32, or NULL (no bias: group score = max key) */
  const void *w13;           /* [E, 2I, D]: rows [0,I) = W1 (gate proj), [I,2I) = W3 (up proj) */
  const float *w13_scale;    /* fp8: [E, 2I/128, D/128] */
  const void *w2;            /* [E, D, I]  (down proj, K-contiguous) */
  const float *w2_scale;     /* fp8: [E, D/128, I/128] */
  const void *sw13;          /* [2SI, D]: rows [0,SI) gate, [SI,2SI) up; NULL iff S == 0 */
  const float *sw13_scale;   /* fp8: [2SI/128, D/128] */
  const void *sw2;           /* [D, SI] */
  const float *sw2_scale;    /* fp8: [D/128, SI/128] */
} moe_weights;

/* Dispatch state written by moe_permute: the T*K (token, slot) pairs sorted by
 * expert into row ranges padded to a multiple of tile_m.  Pair id p = t*K + k.
 * Build it with moe_routing_init over one caller buffer of moe_routing_size bytes. */
typedef struct moe_routing {
  int32_t tile_m;        /* host: rows per expert tile (chosen by the library for (cfg, T)) */
  int32_t max_rows;      /* host: capacity in rows = T*K + min(T*K, E)*(tile_m-1), rounded up to tile_m */
  int32_t max_tiles;     /* host: capacity of the tile lists = max_rows / tile_m */
  int32_t pad_;
  int32_t *counts;       /* [E]          pairs routed to each expert */
  int32_t *expert_off;   /* [E+1]        first row of each expert (multiples of tile_m);
                                         expert_off[E] = rows in use */
  int32_t *sorted_pair;  /* [max_rows]   pair id held by each row, -1 in padding rows;
                                         within an expert pairs ascend by id (stable) */
  int32_t *pair_row;     /* [T*K]        row of each pair (inverse of sorted_pair) */
  int32_t *tile_expert;  /* [max_tiles]  expert of each tile, tiles in row order */
  int32_t *tile_row;     /* [max_tiles]  first row of each tile */
  int32_t *n_tiles;      /* [1]          tiles in use */
  int32_t *scratch;      /* internal */
  uint8_t *act_q;        /* act_quant only (else NULL): [T, D] e4m3 codes of x, from moe_quant_act */
  float *act_s;          /* act_quant only (else NULL): [T, D/128] fp32 scales of act_q */
} moe_routing;

/* ---- host-only queries (no device access) -------------------------------- */

/* Checks a configuration: E % G == 0, 1 <= topk_groups <= G,
 * 1 <= top_k <= topk_groups*E/G, group size >= 2 when a bias makes the group
 * score a top-2 sum (checked at call time), route_scale finite and > 0,
 * dims > 0.  Returns MOE_ERR_UNSUPPORTED for valid layers outside the
 * kernels' limits: E > 512, top_k > 32, G > 64, dtype pairs other than
 * (F32,F32), (BF16,BF16), (BF16,FP8); D or I not a multiple of 8 (of 128 for fp8). */
moe_status moe_validate(const moe_config *cfg);

/* Bytes of one routing buffer for T tokens (host out-param *bytes). */
moe_status moe_routing_size(const moe_config *cfg, int64_t T, size_t *bytes);

/* Carves a routing buffer (device memory of >= moe_routing_size bytes, 256-byte
 * aligned) into the arrays of *r (host struct).  Host only: nothing is written
 * to the device. */
moe_status moe_routing_init(const moe_config *cfg, int64_t T, void *buf, size_t bytes,
                            moe_routing *r);

/* Bytes of the workspace moe_forward needs for T tokens (host out-param). */
moe_status moe_workspace_size(const moe_config *cfg, int64_t T, size_t *bytes);

const char *moe_status_str(moe_status s);
const char *moe_last_error(void);   /* thread-local; "" after a successful call */

/* ---- the forward pass, step by step ---------------------------------------- */

/* Gate (notes page, gate flow steps 1-5).
 *   x        [T, D] act dtype;  w_gate [E, D] act dtype;  bias [E] fp32 or NULL
 *   logits   [T, E] fp32 out:   x W_g^T with fp32 accumulation
 *   topk_idx [T, K] int32 out:  chosen experts, ascending; ties rank the lower
 *                               expert (and group) index first
 *   topk_w   [T, K] fp32 out:   unbiased score at each chosen expert, renormalised
 *                               (per norm_topk) and times route_scale
 *   keys     [T, E] fp32 out or NULL: the ranked key of every expert before
 *                               group masking (sigmoid: s+b; softmax: logit, or p+b) */
moe_status moe_gate(const moe_config *cfg, int64_t T, const void *x, const void *w_gate,
                    const float *bias, float *logits, int32_t *topk_idx, float *topk_w,
                    float *keys, void *stream);

/* Dispatch (replaces the per-expert gather of the notes page's MoE forward,
 * step 2): histogram of experts over the T*K pairs, exclusive scan of the
 * padded counts, stable scatter into expert-sorted rows, tile lists.
 *   topk_idx [T, K] int32;  r from moe_routing_init.  Entries outside [0, E)
 *   are dropped: they get no row and pair_row = -1. */
moe_status moe_permute(const moe_config *cfg, int64_t T, const int32_t *topk_idx,
                       const moe_routing *r, void *stream);

/* Expert FFNs (notes page, "DeepSeekMoE" paragraph: the routed experts FFN_r and
 * the shared experts FFN_share, each a SwiGLU FFN): for every used row i of
 * expert e holding pair p = t*K + k,
 *   h[i]       = silu(W1_e x_t) * (W3_e x_t)               [max_rows, I] act dtype
 *   y_pairs[i] = W2_e h[i]                                   [max_rows, D] act dtype
 * and, when z != NULL, the shared expert on every token:
 *   hs[t] = silu(SW1 x_t) * (SW3 x_t)  [T, S*I];  z[t] = SW2 hs[t]  [T, D]  act dtype
 * Accumulation is fp32; h, hs, y_pairs and z are rounded once to the act dtype.
 * Padding rows of h and y_pairs hold unspecified values.  r must hold the
 * output of moe_permute for the same T and topk_idx.
 * With act_quant = 1 the GEMMs read x as r->act_q / r->act_s (moe_quant_act),
 * and h / hs hold the SwiGLU output quantised from fp32 in the same 1 x 128
 * format, inside the same buffers: R*C e4m3 codes ([R, C] with R = max_rows,
 * C = I for h; R = T, C = S*I for hs), then at byte offset (R*C rounded up to
 * 256) the fp32 scales [R, C/128].  y_pairs and z stay bf16. */
moe_status moe_expert_ffn(const moe_config *cfg, int64_t T, const void *x,
                          const moe_routing *r, const moe_weights *w, void *h, void *y_pairs,
                          void *hs, void *z, void *stream);

/* Training variant of moe_expert_ffn (notes page, SwiGLU experts; the layer
 * backward below needs the SwiGLU's inputs a = W1_e x_t and c = W3_e x_t of every
 * routed row and, with a shared expert, of every token).  Same arguments and
 * outputs as moe_expert_ffn, bf16 activations and weights only
 * (MOE_ERR_UNSUPPORTED otherwise), and it also writes:
 *   ab  [max_rows, 2I] fp32: row i (routed-row order, as h) holds a in columns
 *       [0, I) and c in [I, 2I), accumulated in fp32 exactly as the backward would
 *       recompute them; padding rows hold unspecified values
 *   abs [T, 2SI] fp32 when n_shared > 0 (hs and z are then required too): the shared
 *       expert's a and c per token; ignored otherwise
 * Both 16-byte aligned, caller-owned.  Pass them to moe_backward_saved. */
moe_status moe_expert_ffn_save(const moe_config *cfg, int64_t T, const void *x, const moe_routing *r,
                               const moe_weights *w, void *h, void *y_pairs, void *hs, void *z,
                               float *ab, float *abs, void *stream);

/* The two halves of moe_expert_ffn (the SwiGLU FFN's gate/up projection with the
 * activation, then its down projection), for callers that schedule or time them
 * separately (same arguments and outputs as above):
 *   moe_expert_up:   h (and hs when hs != NULL) from x
 *   moe_expert_down: y_pairs from h (and z from hs when both are non-NULL) */
moe_status moe_expert_up(const moe_config *cfg, int64_t T, const void *x, const moe_routing *r,
                         const moe_weights *w, void *h, void *hs, void *stream);
moe_status moe_expert_down(const moe_config *cfg, int64_t T, const moe_routing *r,
                           const moe_weights *w, const void *h, const void *hs, void *y_pairs,
                           void *z, void *stream);

/* FP8 W8A8 only (cfg->act_quant = 1): quantise x for the expert GEMMs into
 * r->act_q / r->act_s (1 x 128 blocks, the rule stated at moe_config.act_quant).
 * Call it after moe_routing_init and before moe_expert_up / moe_expert_ffn for
 * the same x; moe_forward calls it itself.  x [T, D] bf16. */
moe_status moe_quant_act(const moe_config *cfg, int64_t T, const void *x, const moe_routing *r,
                         void *stream);

/* Combine (total-output equation): for every token t
 *   out[t] = (add_residual ? u[t] : 0) + (z ? z[t] : 0)
 *            + sum over slots k = 0..K-1 of topk_w[t,k] * y_pairs[pair_row[t*K+k]]
 * summed in fp32 in exactly that order (the gate emits slots in ascending
 * expert order), rounded once to the act dtype.  Pairs that moe_permute
 * dropped (expert index outside [0, E)) contribute nothing.
 *   u [T, D], z [T, D] or NULL, out [T, D]: act dtype;  topk_w [T, K] fp32. */
moe_status moe_combine(const moe_config *cfg, int64_t T, const void *u, const void *z,
                       const void *y_pairs, const moe_routing *r, const float *topk_w,
                       void *out, void *stream);

/* Whole layer (notes page, "DeepSeekMoE" total-output equation
 * h'_t = u_t + FFN_share(u_t) + sum_r g_{r,t} FFN_r(u_t), computed as the MoE
 * forward's steps: gate, per-expert FFNs on the chosen tokens, weighted sum):
 * moe_gate -> moe_permute -> moe_expert_ffn -> moe_combine on one stream, every
 * intermediate in `ws` (>= moe_workspace_size bytes, 256-byte aligned).
 *   x [T, D] act dtype;  out [T, D] act dtype (must not alias x)
 *   topk_idx [T, K] int32 / topk_w [T, K] fp32: optional copies of the routing (NULL = skip) */
moe_status moe_forward(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                       void *out, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                       void *stream);

/* The whole layer with no allocation anywhere, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  Same arguments, results and validation as
 * moe_forward, without `ws`: the workspace is a 64 MiB device array inside this
 * library (each GPU the library runs on holds its own copy until the process
 * ends).  Layers whose moe_workspace_size exceeds 64 MiB (a V3-shaped layer up
 * to a few dozen tokens, larger T for smaller layers) return MOE_ERR_WORKSPACE
 * before any launch.  The array keeps the last call's contents, which no call
 * reads before writing; every call on one GPU uses the same array, so calls that
 * overlap on one GPU (on other streams or from other threads) race. */
moe_status moe_forward_static(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                              void *out, int32_t *topk_idx, float *topk_w, void *stream);

/* Auxiliary-loss-free load balancing, one step (DeepSeek-V3 notes page,
 * "V3 improvement 1": b_i follows each expert's load at speed gamma; DeepSeek-R1
 * analysis page, MoE hyper-parameters paragraph: an overloaded expert's bias is
 * lowered, an underloaded expert's raised).  With load_e = r->counts[e], the
 * pairs of this batch routed to expert e by moe_permute:
 *   bias[e] -= gamma  if load_e * n_routed > T * top_k   (above the mean load)
 *   bias[e] += gamma  if load_e * n_routed < T * top_k   (below it)
 * and an expert exactly at the mean keeps its bias bit for bit.  The comparison
 * is exact (integers); the update is one fp32 addition.
 *   r: the routing moe_permute filled for this T (device counts are read)
 *   bias [n_routed] fp32, device, updated in place (the gate's `bias` input)
 *   gamma: finite, >= 0.  T = 0 is a no-op. */
moe_status moe_bias_update(const moe_config *cfg, int64_t T, const moe_routing *r, float gamma,
                           float *bias, void *stream);

/* Sequence-wise balance loss (DeepSeek-V3 notes page, "V3 improvement 2", the
 * paper's eqs. 17-20), one value per sequence of seq_len consecutive tokens:
 *   loss[q] = alpha * sum_i f_i * P_i,
 *   f_i = n_routed / (top_k * seq_len) * (tokens of the sequence with i in topk_idx),
 *   P_i = (1/seq_len) * sum_t s_{i,t} / sum_j s_{j,t},
 * s = sigmoid(logit) for MOE_SCORE_SIGMOID, the softmax probability for
 * MOE_SCORE_SOFTMAX (the unbiased score; no bias enters).  Sums of s' run in
 * fp64 in a fixed order; the result is rounded once to fp32 and is the same on
 * every run.
 *   logits [T, E] fp32 (moe_gate's logits), topk_idx [T, K] int32,
 *   workspace: device memory of >= moe_balance_loss_workspace_size bytes,
 *     256-byte aligned, owned by the caller; it holds per-chunk partial sums
 *     between the two launches of one call and needs no initial contents;
 *   loss [T / seq_len] fp32 out;  T % seq_len == 0, seq_len >= 1, alpha finite.
 * A workspace that is too small returns MOE_ERR_WORKSPACE before any launch. */
moe_status moe_balance_loss(const moe_config *cfg, int64_t T, int32_t seq_len, const float *logits,
                            const int32_t *topk_idx, float alpha, void *workspace,
                            size_t workspace_bytes, float *loss, void *stream);

/* Bytes of workspace moe_balance_loss needs for (cfg, T, seq_len): about
 * 12 * n_routed * T / 64 (0 when T == 0).  Host only. */
moe_status moe_balance_loss_workspace_size(const moe_config *cfg, int64_t T, int32_t seq_len,
                                           size_t *bytes);

/* ---- the layer backward ------------------------------------------------------ */

/* Gradients of a scalar loss L with upstream gradient dout = dL/d(out), for the
 * layer the forward entry points compute (notes page: total-output equation,
 * gate flow steps 1-5, SwiGLU experts).  The chain rule of those steps:
 *   combine  dw[t,k] = <dout_t, y_pairs[row(t,k)]>,  dy = w[t,k] dout_t
 *   experts  a = W1_e x_t, c = W3_e x_t (recomputed), h = silu(a) c,
 *            dh = dy W2_e, da = dh c silu'(a), dc = dh silu(a),
 *            dW2_e = sum dy h^T, dW1_e = sum da x^T, dW3_e = sum dc x^T,
 *            dx_t += da W1_e + dc W3_e;  the shared expert likewise with dz = dout
 *   gate     ds at the chosen experts from dw through route_scale and the
 *            renormalisation (per norm_topk); dlogits = ds s(1-s) (sigmoid) or
 *            s (ds - <ds, s>) (softmax); dx += dlogits W_g, dW_g = dlogits^T x
 *   residual dx += dout when add_residual.
 * The selection (top-k over s + b, group masking) is piecewise constant: no
 * gradient flows through it, and the bias gets none.  bf16 activations and bf16
 * weights only (MOE_ERR_UNSUPPORTED otherwise); dim, inter_dim and n_routed
 * must be multiples of 8.  GEMMs run on bf16 operands with fp32 accumulation;
 * dy, h, da/dc and dlogits are rounded to bf16 as GEMM operands.
 *   x [T, D], w (w_gate, w13, w2, sw13, sw2 as in the forward), r / topk_idx /
 *   topk_w / logits / y_pairs: exactly what moe_gate, moe_permute and
 *   moe_expert_ffn produced for this batch; dout [T, D] act dtype.
 *   grads: caller-owned outputs, fully overwritten (experts that no token chose
 *   get zero gradients):
 *     dx [T, D] act dtype;  dw_gate [E, D] fp32;  dw13 [E, 2I, D] fp32;
 *     dw2 [E, D, I] fp32;  dsw13 [2SI, D] fp32, dsw2 [D, SI] fp32 (n_shared > 0,
 *     else ignored).
 *   workspace: device memory of >= moe_backward_workspace_size bytes, 256-byte
 *   aligned; no initial contents needed.  Operand pointers 16-byte aligned.
 * Results are the same on every run (no atomics; fixed summation orders). */
typedef struct moe_grads {
  void *dx;
  float *dw_gate;
  float *dw13;
  float *dw2;
  float *dsw13;
  float *dsw2;
} moe_grads;

moe_status moe_backward_workspace_size(const moe_config *cfg, int64_t T, size_t *bytes);
moe_status moe_backward(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                        const moe_routing *r, const int32_t *topk_idx, const float *topk_w,
                        const float *logits, const void *y_pairs, const void *dout,
                        const moe_grads *grads, void *workspace, size_t workspace_bytes,
                        void *stream);

/* moe_backward without the recompute of a and c: ab / abs are what
 * moe_expert_ffn_save wrote for this batch (abs only when n_shared > 0), read
 * only.  Same arguments otherwise, same workspace size, and the same gradients
 * bit for bit as moe_backward. */
moe_status moe_backward_saved(const moe_config *cfg, int64_t T, const void *x, const moe_weights *w,
                              const moe_routing *r, const int32_t *topk_idx, const float *topk_w,
                              const float *logits, const void *y_pairs, const void *dout,
                              const float *ab, const float *abs, const moe_grads *grads,
                              void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE355_H */
