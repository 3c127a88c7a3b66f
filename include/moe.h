/*
 * moe.h — C ABI of the MI355X (gfx950) token-choice MoE FFN layer forward.
 *
 * One device's share of a Mixture-of-Experts FFN layer (no expert parallelism):
 *   route    logits = x . Wg (+ bias) in fp32, softmax, top-k, gates
 *   assign   capacity-limited slot assignment (drop or dropless), packing
 *   dispatch gather token rows into expert-contiguous buffers
 *   experts  grouped-GEMM FFN (ReLU / GELU / SwiGLU)
 *   combine  gate-weighted sum of expert outputs plus an optional residual
 *
 * Sources (web pages, by title and section):
 *   [EP]     "Expert-parallel MoE training" explainer (blog.vllbc.top, visual
 *            reading): router Wg in R^{HxE} with softmax then top-k, or top-k then
 *            normalise over the selected; capacity = ceil((T*k/E)*cf); drop or
 *            dropless; "position" drop policy; the walk through one MoE layer
 *            (permute, experts, unpermute, gate-weighted sum, residual); gated
 *            experts with gate / up / down matrices (memory calculator).
 *   [DS7508] DeepSpeed discussion #7508 "The MoE spends too much time on the gate
 *            network": capacity ceil((tokens/experts)*cf*k) (10,923 worked value);
 *            the dense one-hot [T,E,C] dispatch mask that blows up; padding-free
 *            execution on the actual tokens per expert.
 *   [SW]     Switch Transformers explainer ("AI 十大论文精讲（七）: Switch
 *            Routing"): §1.1 router logits, softmax, argmax, y = E_i(x) p_i(x);
 *            §1.2 capacity factor, overflow passes through the residual; §2.1
 *            selective precision (router input, logits and softmax in fp32).
 *
 * Conventions (all entry points):
 *   - Ownership: the caller owns every buffer.  The library never allocates,
 *     frees, or synchronises; it only enqueues kernels on `stream`.
 *   - Pointers marked "device" are device (HBM) addresses; moe_config is read on
 *     the host during the call and may be freed afterwards.
 *   - stream: a hipStream_t passed as void* (NULL = the default stream).  Results
 *     are valid once the stream has been synchronised.  No device-to-host copy
 *     happens inside any call: the number of kept rows R stays on the device.
 *   - Errors: every argument check runs on the host before anything is enqueued;
 *     on error nothing is enqueued.  MOE_ERR_HIP means a launch failed (the
 *     message of the failure is available from moe_last_error()).  No exception
 *     crosses the ABI.
 *   - Alignment: 16-byte aligned pointers with H % 8 == 0 and F % 8 == 0 take the
 *     vector paths; every other shape takes a correct scalar path.
 *   - Preconditions: inputs are finite (NaN / Inf behaviour is unspecified).
 *   - Thread safety: calls are independent given distinct plan, workspace and
 *     output buffers.
 *   - Determinism: no floating-point atomics; repeated calls give the same bits.
 *
 * Data layout (row-major, 0-based):
 *   x, residual, y : [T][H]  of dtype
 *   Wg             : [H][E]  fp32 (logits = x . Wg)
 *   bias           : [E]     fp32, may be NULL
 *   W1 (gate/W_in) : [E][F][H] of dtype   (each matrix stored [out][in])
 *   W3 (up)        : [E][F][H] of dtype   (SwiGLU only, else NULL)
 *   W2 (down/W_out): [E][H][F] of dtype
 *   X, Y           : [R_max][H] of dtype, expert-contiguous packed rows;
 *                    rows [offsets[e], offsets[e+1]) belong to expert e.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* bad shape / mode / NULL required pointer */
  MOE_ERR_UNSUPPORTED = 2, /* valid in principle but not provided by this library */
  MOE_ERR_WORKSPACE = 3,   /* ws_bytes smaller than moe_workspace_bytes() */
  MOE_ERR_HIP = 4          /* a HIP launch failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype; /* of x, W1/W3/W2, X, Y, residual, y */

/* Gate values g[t][r] of the k chosen experts ([EP] router; [SW] §1.1):
 *   SOFTMAX_TOPK        p = softmax over all E logits; g_r = p[e_r]          (Switch, DeepSpeed)
 *   SOFTMAX_TOPK_RENORM g_r = p[e_r] / sum_j p[e_j]                         (DeepSeek-style)
 *   TOPK_SOFTMAX        g = softmax over the k chosen logits                (Megatron default)
 * The last two are equal in exact arithmetic (the full denominator cancels). */
typedef enum { MOE_SOFTMAX_TOPK = 0, MOE_SOFTMAX_TOPK_RENORM = 1, MOE_TOPK_SOFTMAX = 2 } moe_gate_mode;

/* Expert FFN: RELU / GELU (exact erf form): y = act(x W_in) W_out;
 * SWIGLU: y = (silu(x W_gate) * (x W_up)) W_down. */
typedef enum { MOE_RELU = 0, MOE_GELU = 1, MOE_SWIGLU = 2 } moe_act;

/* Token fraction f_e of the load-balancing loss alpha * E * sum_e f_e P_e ([EP]
 * router section, auxiliary-loss paragraph; [SW] "Load balance & capacity"):
 *   MOE_AUX_ALL_CHOICES  f_e = demand_e / (T*k): every choice counts, k in the
 *                        denominator (Switch, Megatron-Core, DeepSpeed top-1/top-k)
 *   MOE_AUX_FIRST_CHOICE f_e = (tokens whose first choice is e) / T, no division
 *                        by k (DeepSpeed's top-2 path)
 * P_e is the mean over tokens of softmax(logits)_e in both. */
typedef enum { MOE_AUX_ALL_CHOICES = 0, MOE_AUX_FIRST_CHOICE = 1 } moe_aux_mode;

/* Router score ([EP] router: logits pass through softmax or sigmoid before the
 * top-k).  Both are
 * increasing in the logit, so the choices are the same; with SIGMOID the gate of
 * a choice is its score s = 1/(1+exp(-l)) (MOE_SOFTMAX_TOPK) or s over the sum
 * of the chosen scores (MOE_SOFTMAX_TOPK_RENORM); MOE_TOPK_SOFTMAX is the
 * softmax over the chosen logits either way. */
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_fn;

/* Which over-capacity assignments are dropped ([EP] capacity / drop section):
 *   POSITION  the last ones in choice-major order (r*T + t)
 *   PROBS     per expert, the ones with the smallest gate value; kept: the C
 *             largest gates (equal gates: earlier position first), packed in
 *             position order.  Same as POSITION when nothing is dropped. */
typedef enum { MOE_DROP_POSITION = 0, MOE_DROP_PROBS = 1 } moe_drop_policy;

/* Second choice with k = 2 ([EP] router: GShard uses top-2 and sends a token
 * to its second expert at random, by that expert's weight):
 *   ALWAYS  plain top-k
 *   RANDOM  the second assignment exists iff u_t * (g1 + g2) < 2 * g2 (binary64
 *           on the fp32 gates; GShard's rule), u_t from plan->second_u; an
 *           absent assignment takes no slot, is not counted in demand, gets
 *           dst_row -1, and the first gate is not renormalised. */
typedef enum { MOE_SECOND_ALWAYS = 0, MOE_SECOND_RANDOM = 1 } moe_second_policy;

typedef struct {
  int32_t T;              /* tokens, >= 0 (T = 0 is a valid no-op)            */
  int32_t H;              /* hidden size, >= 1                                 */
  int32_t E;              /* experts, 1 .. 1024                                */
  int32_t k;              /* choices per token, 1 .. min(E, 16)                */
  int32_t F;              /* expert FFN width, >= 1                            */
  int32_t dtype;          /* moe_dtype                                         */
  int32_t gate_mode;      /* moe_gate_mode                                     */
  int32_t act;            /* moe_act                                           */
  int32_t dropless;       /* 1: no capacity limit; 0: capacity from cf         */
  int32_t min_capacity;   /* capacity floor (DeepSpeed-style); 0 = none        */
  double capacity_factor; /* cf > 0 unless dropless                            */
  int32_t aux_mode;       /* moe_aux_mode (used when plan->losses != NULL)      */
  double aux_coeff;       /* alpha of the load-balancing loss, finite          */
  double z_coeff;         /* coefficient of the z-loss, finite                 */
  int32_t score_fn;       /* moe_score_fn                                       */
  int32_t drop_policy;    /* moe_drop_policy                                    */
  int32_t second_policy;  /* moe_second_policy (RANDOM requires k = 2)         */
  int32_t shared_F;       /* width of the shared expert, 0 = none (see moe_shared_expert) */
} moe_config;

/* Routing plan: device arrays, allocated by the caller, written by moe_route. */
typedef struct {
  int32_t *topk_idx;  /* [T][k]  chosen experts; r = 0 is the largest logit, ties to the lower index */
  float *topk_gate;   /* [T][k]  fp32 gate values (moe_gate_mode)                                  */
  int32_t *dst_row;   /* [T][k]  packed row of the assignment in X / Y, or -1 if dropped            */
  int32_t *demand;    /* [E]     assignments per expert before the capacity limit                   */
  int32_t *kept;      /* [E]     min(demand, C)                                                      */
  int32_t *offsets;   /* [E+1]   exclusive prefix sum of kept; offsets[E] = R                        */
  int32_t *row_token; /* [R_max] token of each packed row (rows >= R are not written)                */
  int32_t *n_dropped; /* [1]     T*k - R                                                             */
  float *logits;      /* [T][E]  optional: fp32 router logits are written here when not NULL        */
  double *losses;     /* [2]     optional: when not NULL, moe_route writes the router training terms
                       *         [0] = aux_coeff * E * sum_e f_e P_e   (load balancing, moe_aux_mode)
                       *         [1] = z_coeff * mean_t logsumexp(logits_t)^2   (z-loss)
                       *         ([EP] router section: auxiliary-loss and z-loss paragraphs)        */
  const float *second_u; /* [T] input: uniforms in [0, 1) for MOE_SECOND_RANDOM (the caller draws
                          *     them: the library consumes random numbers, it does not make them);
                          *     required iff second_policy is RANDOM and T > 0                     */
} moe_plan;

/* ---- host-only helpers (no HIP call; usable without a GPU) ------------------ */

/* MOE_OK, or the reason the configuration is rejected. */
moe_status moe_validate(const moe_config *cfg);

/* Expert capacity C = max(min_capacity, ceil(double(T*k) * cf / E)) ([EP] capacity;
 * [DS7508]); -1 when dropless; -2 when the configuration is invalid. */
int64_t moe_capacity(const moe_config *cfg);

/* R_max: T*k when dropless, else min(T*k, E*C); the row count X / Y / row_token
 * must hold.  -1 when the configuration is invalid. */
int64_t moe_max_rows(const moe_config *cfg);

/* Device workspace bytes that moe_route / moe_expert_ffn / moe_forward need, and
 * with shared_F > 0 also moe_shared_expert / moe_forward_shared (0 when the
 * configuration is invalid). */
size_t moe_workspace_bytes(const moe_config *cfg);

const char *moe_status_str(moe_status s);

/* Text of the last MOE_ERR_HIP failure on the calling thread ("" if none). */
const char *moe_last_error(void);

/* ---- stream-ordered entry points ----------------------------------------------- */

/* Route: logits ([SW] §1.1, fp32 per §2.1, defined as the binary64 dot product
 * plus bias rounded once to fp32), top-k selection (larger logit first, ties to
 * the lower expert index), gates (moe_gate_mode), capacity ([EP]; [DS7508]), and
 * slot assignment in choice-major priority — every token's first choice before
 * any second choice, token order inside each ([EP] "position" policy), or by
 * gate value ("probs", moe_drop_policy) — then packing into expert-contiguous
 * rows.  Every choice is the one the defined
 * logits make; logits written to plan->logits are the defined values for the
 * experts that decide a choice and within ~1e-7 relative of them otherwise.
 * With plan->losses set, also the router training terms (see moe_plan).
 * x: device [T][H] dtype.  Wg: device [H][E] fp32.  bias: device [E] fp32 or NULL.
 * plan: every pointer but logits, losses and second_u required (second_u: see
 * moe_second_policy).  ws: device, >= moe_workspace_bytes. */
moe_status moe_route(const moe_config *cfg, const void *x, const float *Wg, const float *bias,
                     const moe_plan *plan, void *ws, size_t ws_bytes, void *stream);

/* moe_route without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments, kernels and results as moe_route; the route
 * scratch is a static device array of the library (96 MiB, one per device, held
 * until the process ends), so the call allocates nothing.  Configurations whose
 * route scratch (the routing part of moe_workspace_bytes) exceeds 96 MiB return
 * MOE_ERR_WORKSPACE with the sizes in moe_last_error().  Every call on a device
 * shares that device's array, which keeps the last call's contents (the kernels
 * initialise everything they read): calls that overlap on one device race and
 * must be ordered by the caller (for example, one stream per device). */
moe_status moe_route_noalloc(const moe_config *cfg, const void *x, const float *Wg, const float *bias,
                             const moe_plan *plan, void *stream);

/* Dispatch ([EP] layer walk-through: group tokens by target expert):
 * X[dst_row[t][r]] = x[t] for every kept assignment (a bit copy).
 * Reads plan->dst_row; X: device [R_max][H] dtype. */
moe_status moe_dispatch(const moe_config *cfg, const void *x, const moe_plan *plan, void *X, void *stream);

/* Expert FFN on the packed rows ([EP] gated experts; [SW] W_in / W_out;
 * [DS7508] padding-free execution on the actual rows per expert): for expert e,
 * rows [offsets[e], offsets[e+1]) of X give the same rows of Y.  bf16 runs use
 * bf16 MFMA with fp32 accumulation; the hidden activation is stored in the
 * workspace in dtype.  Reads plan->offsets only.  W3 required iff SWIGLU. */
moe_status moe_expert_ffn(const moe_config *cfg, const void *X, const moe_plan *plan, const void *W1,
                          const void *W3, const void *W2, void *Y, void *ws, size_t ws_bytes, void *stream);

/* Combine ([EP] unpermute, multiply by the gate, sum, add the residual; [SW] §1.2
 * overflow passes through the residual):
 * y[t] = residual[t] + sum_{r ascending, dst_row >= 0} topk_gate[t][r] * Y[dst_row[t][r]],
 * accumulated in fp32 and rounded once to dtype.  residual: device [T][H] or NULL (= 0).
 * Gates are not renormalised after drops. */
moe_status moe_combine(const moe_config *cfg, const void *Y, const moe_plan *plan, const void *residual,
                       void *y, void *stream);

/* The whole layer on `stream`: moe_route, moe_dispatch, moe_expert_ffn,
 * moe_combine.  Where the expert GEMMs run on the tiled bf16 path (bf16, H % 64
 * == 0, 16-byte aligned buffers), the first GEMM reads the token rows of x
 * through plan->row_token itself and the dispatch copy is not made; with
 * k == 1 there (and F % 64 == 0, 16-byte aligned residual and y) the second GEMM
 * also does the combine, writing y directly with the arithmetic of moe_combine
 * (bit-identical to the separate calls), and Y is not written.  X and Y:
 * device [R_max][H] dtype scratch; their contents afterwards are unspecified.
 * y may be the same buffer as residual and x (the layer applied in place): x is
 * read by launches that precede every write of y, and each element of y is
 * written by the thread that read its residual. */
moe_status moe_forward(const moe_config *cfg, const void *x, const float *Wg, const float *bias, const void *W1,
                       const void *W3, const void *W2, const void *residual, void *y, const moe_plan *plan,
                       void *X, void *Y, void *ws, size_t ws_bytes, void *stream);

/* Bytes of the pre-activations moe_forward_save keeps: m1 * R_max * F * 2, m1 = 2
 * for SwiGLU, else 1 (0 when the configuration is invalid).  Host only. */
size_t moe_saved_act_bytes(const moe_config *cfg);

/* moe_forward for training that keeps the forward's activations for the
 * backward instead of recomputing them (memory for time; the pages leave the
 * choice open): the first expert GEMM also
 * writes its pre-activations of every kept row as bf16, act[0][row][f] = u =
 * X W1_e^T and, for SwiGLU, act[1][row][f] = v = X W3_e^T (act: device
 * [m1][R_max][F], 16-byte aligned, moe_saved_act_bytes; rows past offsets[E]
 * are not written).  Passed to moe_backward with the same plan, they replace
 * its recomputation and give the same gradients bit for bit.  y is as
 * moe_forward's.  Only where the expert GEMMs run on the tiled bf16 path (bf16,
 * H % 64 == 0, F % 8 == 0, 16-byte aligned buffers): MOE_ERR_UNSUPPORTED
 * otherwise; act NULL: MOE_ERR_INVALID_ARG. */
moe_status moe_forward_save(const moe_config *cfg, const void *x, const float *Wg, const float *bias,
                            const void *W1, const void *W3, const void *W2, const void *residual, void *y,
                            const moe_plan *plan, void *X, void *Y, void *act, void *ws, size_t ws_bytes,
                            void *stream);

/* ---- shared expert ([EP] layer walk-through: a dense MLP outside the router
 * and the all-to-all, run on every token, its output added to the routed
 * experts' output; Megatron-Core SharedExpertMLP, DeepSpeed Residual-MoE).  Taken
 * as one more FFN of the routed experts' form: activation cfg->act, width
 * cfg->shared_F (> 0 for these calls), weights Ws1 (and Ws3 iff SwiGLU)
 * [shared_F][H], Ws2 [H][shared_F], all dtype, [out][in] row-major like W1/W2. */

/* Ys[t] = S(x[t]) for every token.  x: device [T][H]; Ys: device [T][H] dtype
 * (bf16 runs: bf16 MFMA, fp32 accumulation, hidden activation rounded to dtype).
 * ws: device, >= moe_workspace_bytes (holds the hidden activation). */
moe_status moe_shared_expert(const moe_config *cfg, const void *x, const void *Ws1, const void *Ws3,
                             const void *Ws2, void *Ys, void *ws, size_t ws_bytes, void *stream);

/* moe_combine plus the shared output: y[t] = residual[t] + sum_r g[t][r] Y[dst_row[t][r]]
 * + Ys[t], in that order in fp32, rounded once to dtype.  Ys: device [T][H] dtype. */
moe_status moe_combine_shared(const moe_config *cfg, const void *Y, const moe_plan *plan, const void *residual,
                              const void *Ys, void *y, void *stream);

/* moe_forward with the shared expert: route, dispatch, routed experts, shared
 * expert (its output kept in the workspace), moe_combine_shared. */
moe_status moe_forward_shared(const moe_config *cfg, const void *x, const float *Wg, const float *bias,
                              const void *W1, const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                              const void *Ws2, const void *residual, void *y, const moe_plan *plan, void *X, void *Y,
                              void *ws, size_t ws_bytes, void *stream);

/* ---- backward ([EP] layer walk-through run backwards; its all-to-all paragraph:
 * the combine's backward has the dispatch's shape and the dispatch's backward the
 * combine's; router section: the load-balancing term reaches the router only
 * through P_e, the z-loss acts on the logits).  The gradient of
 *   L = sum_{t,h} dy[t][h] * y[t][h]  (+ the router training terms when plan->losses != NULL)
 * where y is the routed layer's output (moe_forward without the shared expert),
 * with the routing decision held fixed: the choices, drops and GShard draws of
 * `plan` are constants, roundings are taken as the identity, and a dropped or
 * absent choice gets no gradient from y while still entering the Jacobian of the
 * other gates.  The residual's gradient is dy itself and is not written.  The
 * hidden activations are recomputed from x (no forward buffers are needed), or
 * taken from the pre-activations moe_forward_save kept.
 * bf16 with H and F multiples of 64 and 16-byte aligned x, dy, W1, W3, W2 and
 * ws runs on the matrix cores with bf16 intermediates (the expert weights and
 * activations read as stored); every other case on fp32 strided products with
 * fp32 intermediates (the expert outputs recomputed as well). */
typedef struct {
  float *dx;    /* [T][H]    dL/dx (expert and router paths), fp32, required            */
  float *dWg;   /* [H][E]    dL/dWg, fp32, required                                     */
  float *dbias; /* [E]       dL/dbias, fp32, or NULL                                    */
  float *dW1;   /* [E][F][H] fp32, required                                             */
  float *dW3;   /* [E][F][H] fp32, required iff SwiGLU (else ignored)                   */
  float *dW2;   /* [E][H][F] fp32, required                                             */
  float *dg;    /* [T][k]    dL/dtopk_gate, fp32, or NULL (0 for dropped choices)        */
} moe_grads;

/* Device workspace bytes moe_backward needs (0 when the configuration is invalid). */
size_t moe_backward_workspace_bytes(const moe_config *cfg);

/* x: device [T][H] dtype (the forward's input).  Wg: device [H][E] fp32.  W1, W3,
 * W2: the expert weights (W3 iff SwiGLU).  plan: the routing moe_route made for x
 * (topk_idx, topk_gate, dst_row, demand, offsets, row_token) with plan->logits
 * written; plan->losses != NULL adds the gradients of the training terms of cfg
 * (aux_mode, aux_coeff, z_coeff, score_fn).  dy: device [T][H] dtype.  act: the
 * pre-activations moe_forward_save kept for this x, plan and weights, or NULL to
 * recompute them; used on the matrix-core path (where it must be 16-byte
 * aligned), ignored on the other, whose fp32 intermediates are recomputed.  Every
 * sum is accumulated in fp32 in a fixed order (binary64 inside the per-token
 * gate Jacobian), so results are deterministic.  ws: device, >=
 * moe_backward_workspace_bytes.  The shared expert is not part of this
 * gradient. */
moe_status moe_backward(const moe_config *cfg, const void *x, const float *Wg, const void *W1, const void *W3,
                        const void *W2, const moe_plan *plan, const void *dy, const void *act,
                        const moe_grads *grads, void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
