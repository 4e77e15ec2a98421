/* moe.h - C ABI of libmoe.so, the sparse mixture-of-experts feed-forward
 * layer of AFMoE (Arcee Trinity) and MiniMax-M3 on one AMD MI355X (gfx950).
 *
 * The layer (pages: mlxcel issue #845 "add Arcee AFMoE", "Routing detail" and
 * "Checkpoint weight layout"; HF Transformers doc "AFMoE", AfmoeConfig and the
 * expert-routing / shared-expert sections; mlxcel issue #763 "add MiniMax-M3",
 * "Architecture specification", MoE and Activation bullets):
 *
 *   L    = x . W_r^T                         router logits, fp32
 *   s    = sigmoid(L) (or softmax over E)    scores
 *   idx  = top-k of (s + expert_bias)        bias used for selection only;
 *                                            ties -> lower expert index;
 *                                            emitted in that order
 *   w    = route_scale * s[idx] / sum s[idx] route_norm on (without the
 *                                            division when off)
 *   y_e  = W_d[e] . act(W_g[e] . x, W_u[e] . x)
 *   out  = sum_j w_j * y_{idx_j} + sum_s y_shared_s(x)
 *
 * Conventions of every entry point:
 *  - Pointers are DEVICE pointers unless marked "host". The caller owns all
 *    memory. The library allocates nothing and keeps no state between calls;
 *    work happens asynchronously on the given stream.
 *  - Device tensors are 16-byte aligned (the kernels move 16-byte vectors).
 *  - Tensors are row-major and dense. Weights use the [out, in] layout of a
 *    linear layer: gate/up [E_tot, I, H], down [E_tot, H, I], where
 *    E_tot = E + 1 when the shared expert is packed as slot E, else E.
 *  - "dtype" tensors (x, expert weights, h, out) are bf16 or fp32 as
 *    moe_config.dtype says. The router weight and logits are always fp32.
 *  - All argument checks run on the host before any launch; a call that
 *    returns an error has launched nothing. Faults inside kernels surface at
 *    the caller's next synchronisation. Values are not checked (no NaN/Inf
 *    scan).
 *  - T == 0 returns MOE_OK and launches nothing.
 *  - Calls are reentrant. Concurrent calls need distinct workspaces.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* moe_stream_t; /* a hipStream_t; NULL = null stream */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad size, null required pointer, bad flag */
  MOE_ERR_UNSUPPORTED = 2, /* valid config outside what the kernels cover */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than the query reports */
  MOE_ERR_HIP = 4          /* a HIP launch or API call failed */
} moe_status;

/* Scoring function (the router's per-expert scores s from the logits L):
 *   sigmoid: s_e = 1 / (1 + exp(-L_e))               (mlxcel #845 "Routing detail")
 *   softmax: s_e = exp(L_e - max L) / sum_e' exp(L_e' - max L) over the E
 *            routed experts                           (HF "AFMoE" doc, key
 *            features: sigmoid- or softmax-based token-choice routing)
 * Both are formed in fp64 from the fp32 logits; the selection bias, the
 * gather of unbiased scores, route_norm and route_scale follow unchanged. */
typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SOFTMAX = 1 } moe_score_func;

/* Group-limited routing (moe_config.n_group > 1; mlxcel #845 "Routing
 * detail" names group routing and n_group, the rule is read from the
 * DeepSeek MoE family the page derives AFMoE from): the E experts form
 * n_group contiguous groups of E / n_group; a group's score is the sum of
 * its two largest selection keys (fp64, the larger first); the topk_group
 * groups with the largest scores (ties: lower group index) stay eligible and
 * the top-k runs over their experts only. Weights, route_norm and
 * route_scale are unchanged. */

/* Expert activation: SiLU-SwiGLU (HF "AFMoE" doc, hidden_act "silu") or
 * clamp-SwiGLU (mlxcel #763 Activation bullet, hidden_act "swigluoai"):
 *   silu:      a = g * sigmoid(g) * u
 *   swigluoai: a = g' * sigmoid(alpha*g') * (u' + beta),
 *              g' = min(g, limit), u' = clamp(u, -limit, limit)
 * with g the gate projection and u the up projection. */
typedef enum { MOE_ACT_SILU = 0, MOE_ACT_SWIGLUOAI = 1 } moe_hidden_act;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* Storage of the expert weights (routed and shared; the router stays fp32):
 *   MOE_WEIGHTS_DTYPE  as moe_config.dtype
 *   MOE_WEIGHTS_MXFP8  OCP Microscaling (MX) v1.0 MXFP8, the format of the
 *                      MiniMax-M3 MXFP8 export (mlxcel #763 "Validation"):
 *                      each weight is one E4M3 code (uint8; bias 7, largest
 *                      finite 448, 0x7F/0xFF NaN), and every 32 consecutive
 *                      inputs of a weight row share one E8M0 scale byte
 *                      (2^(e-127)); w = e4m3(code) * 2^(e-127). The code
 *                      tensors keep the weights' shapes and layout; the
 *                      scales are passed in moe_mx_scales. Needs dtype bf16
 *                      (activations stay bf16, accumulation fp32; else
 *                      MOE_ERR_UNSUPPORTED).
 *   MOE_WEIGHTS_MXFP4  OCP MX v1.0 MXFP4, read as the format of the 4-bit
 *                      Trinity checkpoints (mlxcel #845 "Checkpoint
 *                      confirmed", "Checkpoint weight layout": 4-bit experts,
 *                      no format given): each weight is one E2M1 code (sign,
 *                      2 exponent bits with bias 1, 1 mantissa bit: values
 *                      +-{0, .5, 1, 1.5, 2, 3, 4, 6}), two per byte along
 *                      the weight row, input 2j in the low nibble of byte j,
 *                      so an [N, K] matrix is [N, K/2] bytes (gate, up
 *                      [E_tot, I, H/2], down [E_tot, H, I/2], shared
 *                      likewise); the same E8M0 scales per 32 inputs in
 *                      moe_mx_scales. Needs dtype bf16, as MXFP8. */
typedef enum {
  MOE_WEIGHTS_DTYPE = 0,
  MOE_WEIGHTS_MXFP8 = 1,
  MOE_WEIGHTS_MXFP4 = 2
} moe_weight_format;

/* E8M0 scales of MX (MXFP8, MXFP4) expert weights, block-major: for an
 * [N, K] weight matrix the scales are [K/32, N] (for every block of 32
 * inputs, the scales of all N rows), stacked like the weights:
 *   gate, up      [E_tot, H/32, I]     down        [E_tot, I/32, H]
 *   shared_gate,  [S, H/32, I_s]       shared_down [S, I_s/32, H]
 *   shared_up                          (NULL when S == 0 or packed: the
 *                                       packed shared expert's scales are
 *                                       slot E of gate/up/down)
 * A checkpoint's [N, K/32] scale tensor is the transpose of this layout. */
typedef struct {
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  const uint8_t* shared_gate;
  const uint8_t* shared_up;
  const uint8_t* shared_down;
  const uint8_t* router;  /* [H/32, E], when router_format is MXFP8     */
} moe_mx_scales;

/* Storage of the router weights:
 *   MOE_ROUTER_F32    fp32 [E, H]
 *   MOE_ROUTER_MXFP8  E4M3 codes [E, H] (uint8) with E8M0 scales per 32
 *                     inputs in moe_mx_scales.router, block-major [H/32, E]:
 *                     the 8-bit router of the 4-bit Trinity checkpoints
 *                     (mlxcel #845 "Checkpoint weight layout": the router
 *                     gate at 8 bits, the rest at 4), read as MXFP8 like the
 *                     experts. The codes are dequantised exactly to fp32 in
 *                     the workspace and the router GEMM runs unchanged. */
typedef enum { MOE_ROUTER_F32 = 0, MOE_ROUTER_MXFP8 = 1 } moe_router_format;

/* Layer configuration (host struct, passed by const pointer). Field names
 * follow the pages' config keys. */
typedef struct {
  int32_t hidden_size;              /* H; multiple of 64                         */
  int32_t num_experts;              /* E routed experts, 1..1024                 */
  int32_t num_experts_per_tok;      /* k, 1..min(E, 32)                          */
  int32_t num_shared_experts;       /* S >= 0, always-on experts                 */
  int32_t moe_intermediate_size;    /* I; multiple of 64                         */
  int32_t shared_intermediate_size; /* I_s; 0 means I; multiple of 64            */
  int32_t shared_packed;            /* 1: the shared expert is slot E of the
                                       stacked tensors, with fixed weight 1.0;
                                       needs S == 1 and I_s == I (mlxcel #763)   */
  int32_t score_func;               /* moe_score_func                            */
  int32_t route_norm;               /* 0/1: renormalise the k gathered scores    */
  float route_scale;                /* route_scale / routed_scaling_factor;
                                       multiplies routed weights only            */
  int32_t hidden_act;               /* moe_hidden_act                            */
  float act_alpha;                  /* swigluoai alpha (1.702)                   */
  float act_limit;                  /* swigluoai limit (7.0)                     */
  float act_beta;                   /* swigluoai beta  (1.0)                     */
  int32_t dtype;                    /* moe_dtype of x, h, out (and the expert
                                       weights when weight_format is DTYPE)     */
  int32_t weight_format;            /* moe_weight_format of the expert weights   */
  int32_t n_group;                  /* group-limited routing: 0 or 1 = off; else
                                       E % n_group == 0, E / n_group >= 2,
                                       n_group <= 64                             */
  int32_t topk_group;               /* groups kept, 1..n_group; k <= topk_group *
                                       E / n_group (used when n_group > 1)       */
  int32_t router_format;            /* moe_router_format of w_router             */
} moe_config;

/* Bytes of device workspace that moe_layer_forward (and every stage entry
 * point) needs for T tokens. bytes: host pointer. The workspace must be
 * 256-byte aligned. */
moe_status moe_workspace_size(const moe_config* cfg, int64_t T, size_t* bytes);

/* Router GEMM: logits[T,E] (fp32) = x[T,H] . w_router[E,H]^T, fp32
 * accumulation. The router is a bias-free linear map (mlxcel #845
 * "Checkpoint weight layout": mlp.router.gate). The result does not depend on
 * timing, and identical router rows give bitwise identical logit columns.
 * w_router: fp32 [E,H], or E4M3 codes [E,H] when router_format is MXFP8 (mx:
 * host pointer to the scales, mx->router; else mx may be NULL).
 * ws, ws_bytes: workspace of at least moe_workspace_size bytes (scratch). */
moe_status moe_router_logits(const moe_config* cfg, int64_t T, const void* x,
                             const void* w_router, const moe_mx_scales* mx, float* logits,
                             void* ws, size_t ws_bytes, moe_stream_t stream);

/* Routing (mlxcel #845 "Routing detail"; mlxcel #763 MoE bullet): sigmoid
 * (or softmax) scores, selection key s + expert_bias formed in fp64, top-k by
 * (key desc, index asc), weights from the unbiased scores, route_norm,
 * route_scale.
 *   logits      [T,E] fp32
 *   expert_bias [E] fp32, or NULL (no bias)
 *   topk_idx    [T,k] int32 out, in selection order
 *   topk_w      [T,k] fp32 out
 *   expert_counts [E] int32 out or NULL: number of rows routed to each expert
 *                 (the array is cleared and filled by this call). */
moe_status moe_route(const moe_config* cfg, int64_t T, const float* logits,
                     const float* expert_bias, int32_t* topk_idx,
                     float* topk_w, int32_t* expert_counts,
                     moe_stream_t stream);

/* Grouping of the T*k (token, slot) rows r = t*k + j by expert: a stable
 * counting sort.
 *   expert_offsets [E+1] out: exclusive scan of the per-expert row counts
 *   sorted_rows    [T*k] out: rows of expert 0 in ascending r, then expert 1..
 *   row_pos        [T*k] out: inverse, row_pos[sorted_rows[p]] = p
 *   ws, ws_bytes: workspace of at least moe_workspace_size bytes. */
moe_status moe_permute(const moe_config* cfg, int64_t T,
                       const int32_t* topk_idx, int32_t* expert_offsets,
                       int32_t* sorted_rows, int32_t* row_pos, void* ws,
                       size_t ws_bytes, moe_stream_t stream);

/* Grouped gate/up projections with the activation fused (stacked expert
 * tensors: mlxcel #845 "Checkpoint weight layout"):
 *   h[p, :]        = act(x[t] . W_g[e]^T, x[t] . W_u[e]^T) for the p-th
 *                    sorted row (t = sorted_rows[p] / k, e its expert)
 *   h_shared[t, s*I_s:(s+1)*I_s] = act(x[t] . Ws_g[s]^T, x[t] . Ws_u[s]^T)
 *   x [T,H]; w_gate, w_up [E_tot,I,H]; ws_gate, ws_up [S,I_s,H] (NULL when
 *   S == 0 or the shared expert is packed: then slot E of w_gate/w_up is
 *   used); mx: host pointer to the scales when weight_format is MXFP8 or MXFP4
 *   (ignored otherwise, may be NULL); h [T*k, I] out; h_shared [T, S*I_s]
 *   out (NULL iff S == 0). */
moe_status moe_grouped_gate_up_swiglu(
    const moe_config* cfg, int64_t T, const void* x, const void* w_gate,
    const void* w_up, const void* ws_gate, const void* ws_up,
    const moe_mx_scales* mx, const int32_t* expert_offsets,
    const int32_t* sorted_rows, void* h, void* h_shared, void* ws,
    size_t ws_bytes, moe_stream_t stream);

/* Grouped down projection with the combine:
 *   acc[t, :]  = sum_s h_shared[t, s] . Ws_d[s]^T          (stored; zeros
 *                                                            when S == 0)
 *   then for every sorted row p (row r = sorted_rows[p], t = r / k):
 *     y_perm == NULL:  acc[t, :] += topk_w[r] * (h[p] . W_d[e]^T)
 *                      (fp32 atomics; summation order varies run to run)
 *     y_perm != NULL:  y_perm[p, :] = h[p] . W_d[e]^T   (dtype, unweighted;
 *                      moe_combine then sums in a fixed order)
 *   h [T*k, I]; w_down [E_tot,H,I]; h_shared [T,S*I_s]; ws_down [S,H,I_s] or
 *   NULL (packed or S == 0); mx as for the gate/up call; topk_w [T,k];
 *   acc [T,H] fp32 out. The shared
 *   experts carry weight exactly 1 and no route_scale (HF "AFMoE" doc:
 *   route_scale scales the routed experts; mlxcel #763: fixed score 1.0). */
moe_status moe_grouped_down(const moe_config* cfg, int64_t T, const void* h,
                            const void* w_down, const void* h_shared,
                            const void* ws_down, const moe_mx_scales* mx,
                            const int32_t* expert_offsets,
                            const int32_t* sorted_rows, const float* topk_w,
                            float* acc, void* y_perm, void* ws,
                            size_t ws_bytes, moe_stream_t stream);

/* Finalise: out[t] = acc[t] (y_perm == NULL), or
 *           out[t] = acc[t] + sum_j topk_w[t,j] * y_perm[row_pos[t*k+j]]
 * summed in j order (y_perm != NULL), cast to dtype. out [T,H]. */
moe_status moe_combine(const moe_config* cfg, int64_t T, const float* acc,
                       const void* y_perm, const int32_t* row_pos,
                       const float* topk_w, void* out, moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * Fused expert FFN of a decode batch: one kernel in place of the grouping,
 * the two grouped GEMMs and the h round trip through memory. An expert's
 * output down(act(gate x, up x)) (mlxcel #845 "Routing detail") is a sum
 * over the columns of h, so it is computed per 128-column slice C of the
 * intermediate width into an fp32 partial plane, and moe_combine_partials
 * adds a row's planes in slice order. moe_layer_forward and
 * moe_block_forward take this path by themselves where it applies.
 *
 * Applies to: dtype bf16 with bf16, MXFP8 or MXFP4 expert weights,
 * hidden_size 512 or 1024 (MXFP4: 1024), moe_intermediate_size and (S > 0)
 * the shared width multiples of 128, num_experts <= 256, T <= 32 and
 * T*k <= 256, and at most 8 slices per workgroup of the launch (one
 * workgroup per compute unit). Elsewhere the three calls return
 * MOE_ERR_UNSUPPORTED. */

/* Bytes of the partial planes for T tokens,
 *   (I/128 * T*k + S*I_s/128 * T) * H * 4.  bytes: host pointer. */
moe_status moe_expert_ffn_size(const moe_config* cfg, int64_t T, size_t* bytes);

/* The partial planes, fp32 [rows][H] each:
 *   routed plane c < I/128, row r = t*k + j (expert e = topk_idx[r]):
 *     parts_c[r, :] = bf16(act(x[t] . W_g[e, C]^T, x[t] . W_u[e, C]^T)) . W_d[e][:, C]^T
 *     with C the columns 128c .. 128c+127 (the activation rounded to bf16
 *     as the grouped path stores h; MX weights as their exact values);
 *   then shared plane a < S*I_s/128, row t: the same for slice a of the
 *     shared experts' concatenated width.
 * x [T,H]; weights as for the grouped calls (ws_* NULL when packed or
 * S == 0); mx: the MX scales (gate, up, down and the shared ones) when
 * weight_format is MXFP8 or MXFP4, else ignored; topk_idx [T,k]: a token's
 * k experts distinct (as moe_route emits them); rows naming an expert
 * outside [0, E) are skipped (their rows of parts are left unwritten).
 * parts: moe_expert_ffn_size bytes. */
moe_status moe_expert_ffn(const moe_config* cfg, int64_t T, const void* x,
                          const void* w_gate, const void* w_up, const void* w_down,
                          const void* ws_gate, const void* ws_up, const void* ws_down,
                          const moe_mx_scales* mx, const int32_t* topk_idx, float* parts,
                          moe_stream_t stream);

/* Finalise from the partial planes:
 *   out[t] = sum_a shared_a[t] + sum_j topk_w[t,j] * (sum_c parts_c[t*k+j])
 * every sum in index order (the result does not depend on timing), cast to
 * dtype. parts from moe_expert_ffn; topk_w [T,k]; out [T,H]. */
moe_status moe_combine_partials(const moe_config* cfg, int64_t T, const float* parts,
                                const float* topk_w, void* out, moe_stream_t stream);

/* The whole layer: router GEMM, routing, grouping, gate/up + activation,
 * down + combine, cast.
 *   x [T,H] dtype; w_router [E,H] fp32 (or MXFP8 codes, router_format);
 *   expert_bias [E] fp32 or NULL;
 *   w_gate, w_up, w_down stacked experts; ws_* separate shared experts or
 *   NULL; mx: scales of MX weights (host pointer) or NULL;
 *   router_logits_in [T,E] or NULL (when given, the router GEMM is
 *   skipped and these logits are routed); router_logits_out [T,E] or NULL;
 *   topk_idx_out [T,k] / topk_w_out [T,k] or NULL; out [T,H] dtype.
 *   deterministic: 0 = fp32 atomic combine, 1 = fixed-order combine. */
moe_status moe_layer_forward(
    const moe_config* cfg, int64_t T, const void* x, const void* w_router,
    const float* expert_bias, const void* w_gate, const void* w_up,
    const void* w_down, const void* ws_gate, const void* ws_up,
    const void* ws_down, const moe_mx_scales* mx, const float* router_logits_in,
    float* router_logits_out, int32_t* topk_idx_out, float* topk_w_out,
    void* out, int32_t deterministic, void* ws, size_t ws_bytes,
    moe_stream_t stream);

/* ---------------------------------------------------------------------------
 * The MoE block: the layer between two RMSNorms, plus the residual
 * (mlxcel #845 "What the original body missed": four norms per layer, the
 * feed-forward half being out = h + post_mlp_norm(mlp(pre_mlp_norm(h)))):
 *
 *   RMSNorm(x)[i] = x[i] / sqrt(sum_i' x[i']^2 / H + eps) * scale[i]
 *   scale = w           (AFMoE; eps = rms_norm_eps, 1e-5 in AfmoeConfig)
 *   scale = w + 1       (Gemma style, MiniMax-M3: mlxcel #763 Norms bullet)
 *
 * The sum of squares is taken in fp32 in a fixed order, so results do not
 * depend on timing. Norm weights are fp32 [H]. H <= 8192 (one workgroup
 * holds a row); larger H returns MOE_ERR_UNSUPPORTED. */
typedef struct {
  float rms_norm_eps; /* eps >= 0, finite                                   */
  int32_t add_one;    /* 0: scale = w; 1: scale = w + 1 (Gemma style)       */
} moe_norm_config;

/* y[T,H] = RMSNorm(x[T,H]) with weight [H] (fp32); x and y in cfg->dtype
 * (only hidden_size and dtype of cfg are used). y may equal x (in place);
 * partial overlap is not allowed. */
moe_status moe_rms_norm(const moe_config* cfg, const moe_norm_config* norm,
                        int64_t T, const void* x, const float* weight, void* y,
                        moe_stream_t stream);

/* Finalise with the post-norm and the residual:
 *   v[t]   = acc[t]                                            (y_perm NULL)
 *          = acc[t] + sum_j topk_w[t,j] * y_perm[row_pos[t*k+j]]  (j order)
 *   out[t] = residual[t] + RMSNorm(v[t]) with post_norm_w
 * v stays fp32 (the layer output is normalised before any rounding);
 * residual and out [T,H] in dtype; out may equal residual (in place). */
moe_status moe_combine_norm_residual(const moe_config* cfg,
                                     const moe_norm_config* norm, int64_t T,
                                     const float* acc, const void* y_perm,
                                     const int32_t* row_pos,
                                     const float* topk_w,
                                     const float* post_norm_w,
                                     const void* residual, void* out,
                                     moe_stream_t stream);

/* Workspace bytes of moe_block_forward: the layer's workspace plus the
 * normalised input rows [T,H] (dtype). */
moe_status moe_block_workspace_size(const moe_config* cfg, int64_t T,
                                    size_t* bytes);

/* The whole block: out = h + RMSNorm_post(layer(RMSNorm_pre(h))).
 *   h [T,H] dtype (the residual stream); pre_norm_w, post_norm_w [H] fp32;
 *   the layer's weights and outputs as in moe_layer_forward, the layer
 *   running on the normalised rows (rounded to dtype); out [T,H] dtype,
 *   may equal h (in place). ws: moe_block_workspace_size bytes. */
moe_status moe_block_forward(
    const moe_config* cfg, const moe_norm_config* norm, int64_t T,
    const void* h, const float* pre_norm_w, const float* post_norm_w,
    const void* w_router, const float* expert_bias, const void* w_gate,
    const void* w_up, const void* w_down, const void* ws_gate,
    const void* ws_up, const void* ws_down, const moe_mx_scales* mx,
    float* router_logits_out,
    int32_t* topk_idx_out, float* topk_w_out, void* out,
    int32_t deterministic, void* ws, size_t ws_bytes, moe_stream_t stream);

const char* moe_status_string(moe_status s);

/* Library version and the GPU architecture the kernels were built for. */
const char* moe_build_info(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
