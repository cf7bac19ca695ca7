/*
 * moe.h -- C ABI of libmoe.so, a capacity-limited sparse mixture-of-experts layer
 * (forward and backward) for AMD Instinct MI355X (gfx950).
 *
 * The layer, as defined on the source pages:
 *   router scores       s = x W_r                      ("Top-k MoE Router with Load
 *                                                        Statistics", score equation)
 *   fp32 softmax, top-k by score with exact ties to the lower expert index, gates
 *   renormalised over the k choices                    (same page, alpha equation;
 *                                                        "Sparse MoE Layer in NumPy",
 *                                                        section 1 traps 1 and 7)
 *   capacity C = ceil(T k cf / E)                       ("Sparse MoE Layer in NumPy",
 *                                                        trap 2; "Module 7", expert_capacity)
 *   position-priority slots: token order, then choice order; over-capacity
 *   assignments are dropped and counted               ("Sparse MoE Layer in NumPy",
 *                                                        trap 3, position_priority_dispatch)
 *   expert MLP on each expert's slot buffer            ("Module 7", swiglu_expert;
 *                                                        llm-atlas "Mixture of Experts",
 *                                                        Expert module)
 *   y = r x + shared(x) + sum over kept choices of gate * expert(x)
 *                                                      ("Sparse MoE Layer in NumPy", trap 4;
 *                                                        router page, y equation)
 *   Switch aux loss E sum_e f_e P_e before any drop, f_e = count_e / (T k),
 *   P_e = mean_t p[t, e]                               ("Sparse MoE Layer in NumPy", trap 6)
 *   backward: dgate, dx, the router-logit gradient through the quotient rule and
 *   the softmax Jacobian, expert (GELU, SwiGLU, linear), shared-expert and router weight
 *   gradients, discrete choices held constant         ("Sparse MoE Layer in NumPy",
 *                                                        trap 7 and section 2)
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" are HIP device pointers (16-byte aligned); the others
 *     are host pointers. The caller allocates every buffer, including the workspace;
 *     the library never allocates or frees device memory.
 *   - Tensors are row-major with unit inner stride; x and dy take a leading dimension
 *     (elements). Expert weights are [E, in, out] row-major; biases [E, out].
 *   - Inputs are never modified. Outputs are fully overwritten, except that rows
 *     c >= used[e] of expert_out / hidden_cache are left unspecified.
 *   - Every call enqueues its kernels on `stream` (a hipStream_t, NULL = the default
 *     stream) and returns without synchronising. Calls on different streams with
 *     different workspaces are independent.
 *   - Arguments are validated on the host before anything is launched; on failure
 *     nothing is written and a status code is returned. MOE_ERR_HIP reports a failed
 *     launch. Caller-supplied expert indices outside [0, E) are data errors found on
 *     the device: moe_dispatch skips them and sets bit 0 of the device error word,
 *     readable with moe_read_error.
 *   - Index outputs are int32; the kept mask is one byte per assignment. An
 *     assignment a = t*k + j is token t's j-th choice.
 *   - Shape limits: 1 <= E <= 1024, 1 <= k <= min(E, 256), T * k < 2^31. bf16 expert
 *     GEMMs need d_model and d_hidden to be multiples of 64; fp32 ones multiples of 16.
 *     bf16 operands are addressed with 32-bit byte offsets from each expert's base, so
 *     x (T rows of ldx), a hidden activation (C rows routed, T rows for the shared
 *     expert, of d_hidden) and one expert's weight matrix must each stay below 4 GiB.
 *     The OUT_IN weight layouts need bf16 experts, the forward, and (moe_forward) the
 *     same layouts for the routed and the shared experts. The combine takes any d_model.
 *     Anything else returns MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* bad size, NULL required pointer, k outside [1, E]     */
  MOE_ERR_UNSUPPORTED = 2,  /* valid but not implemented (shape limits, bf16 backward) */
  MOE_ERR_WORKSPACE = 3,    /* ws_bytes smaller than the matching *_workspace_size    */
  MOE_ERR_HIP = 4           /* a HIP launch or call failed                            */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

typedef enum {
  MOE_EXPERT_LINEAR = 0,    /* o = x W                        ("Sparse MoE Layer in
                               NumPy", section 2 forward einsum); W [E, D, D]          */
  MOE_EXPERT_GELU_MLP = 1,  /* o = GELU_erf(x W1 + b1) W2 + b2 (llm-atlas "Mixture of
                               Experts", Expert); W1 [E,D,F], W2 [E,F,D], b1 [E,F],
                               b2 [E,D]. GELU_erf(z) = z Phi(z), Phi evaluated with an
                               absolute error below 1e-7                               */
  MOE_EXPERT_SWIGLU = 2     /* o = (silu(x Wg) * (x Wu)) Wd   ("Module 7",
                               swiglu_expert); Wg, Wu [E,D,F], Wd [E,F,D], no bias     */
} moe_expert_kind_t;

/* Storage of w_in and w_up (moe_experts_t.w_in_layout) and of w_out (w_out_layout).
   IN_OUT is [E, in, out] as written above (the einsum form of "Sparse MoE Layer in
   NumPy" and "Module 7"); OUT_IN is [E, out, in], each expert's matrix as a torch
   Linear stores its weight (llm-atlas "Mixture of Experts", Expert): W1/Wg/Wu
   [E, F, D], W2/Wd [E, D, F], LINEAR W [E, D, D] transposed. The product is the same;
   OUT_IN is taken by the bf16 forward only. */
typedef enum { MOE_LAYOUT_IN_OUT = 0, MOE_LAYOUT_OUT_IN = 1 } moe_layout_t;

/* A set of experts of one kind and dtype. All pointers are device pointers. */
typedef struct {
  int32_t kind;         /* moe_expert_kind_t                                        */
  int32_t dtype;        /* moe_dtype_t of weights, activations and expert outputs   */
  int32_t num_experts;  /* E (1 for a shared expert)                                */
  int32_t d_model;      /* D                                                        */
  int32_t d_hidden;     /* F; must equal D for LINEAR                               */
  const void* w_in;     /* LINEAR W, GELU W1, SWIGLU Wg                             */
  const void* w_up;     /* SWIGLU Wu, else NULL                                     */
  const void* w_out;    /* GELU W2, SWIGLU Wd, LINEAR NULL                          */
  const void* b_in;     /* GELU b1 (may be NULL = no bias), else NULL               */
  const void* b_out;    /* GELU b2 (may be NULL = no bias), else NULL               */
  int32_t w_in_layout;  /* moe_layout_t of w_in and w_up (0, the zero default:
                           IN_OUT)                                                  */
  int32_t w_out_layout; /* moe_layout_t of w_out (0: IN_OUT, [E, F, D]); ignored for
                           LINEAR experts, which have no w_out                      */
} moe_experts_t;

/*
 * Router variants of "Module 7. Mixture of Experts" (route_logits, dispatch_with_capacity,
 * router_z_loss). The all-zero struct (or a NULL pointer where one is taken) is the
 * default softmax router of the other pages.
 *   scoring          MOE_SCORE_SOFTMAX: gates p[idx] / sum over the k of p[idx].
 *                    MOE_SCORE_SIGMOID: gates sigmoid(s[idx]) / sum over the k of
 *                    sigmoid(s[idx]), evaluated as a softmax of log sigmoid(s) over the k
 *                    chosen experts (finite for any finite logits).
 *   selection_bias   device [E] fp32 or NULL. When given, experts are chosen by the
 *                    fp32 value clean + bias[e] (clean = p or sigmoid(s)), ties to the
 *                    lower index; the gates still come from the clean scores only.
 *                    NULL: chosen by logit.
 *   renormalize_kept 1: after the capacity drop the kept gates of a token are divided
 *                    by their sum (a token with nothing kept gets no expert term).
 *                    Used by moe_forward's combine and by moe_backward.
 *   z_loss           device [1] fp32 or NULL: mean over tokens of (log sum_e exp s)^2.
 *   token_fraction   device [E] fp32 or NULL: f_e = count_e / T, the fraction of tokens
 *                    that chose expert e ("Top-k MoE Router with Load Statistics", f_e
 *                    equation; counts before any drop).
 *   probability_mass device [E] fp32 or NULL: m_e = prob_sum_e / T, the mean softmax
 *                    probability of expert e over the tokens (same page, m_e equation).
 * The aux loss keeps P_e = mean softmax probability and the counts of the selection
 * actually made under every variant.
 */
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_scoring_t;
typedef struct {
  int32_t scoring;
  const float* selection_bias;
  int32_t renormalize_kept;
  float* z_loss;
  float* token_fraction;
  float* probability_mass;
} moe_router_opts_t;

/* Library version string, e.g. "moe-gfx950 0.1". */
const char* moe_version(void);

/* Human-readable name of a status code. */
const char* moe_status_string(int status);

/*
 * Capacity C = ceil(T * k * capacity_factor / E), computed exactly on the given double
 * ("Sparse MoE Layer in NumPy", trap 2). No clamp: capacity_factor = 0 gives 0.
 * Returns -1 if T < 1, k not in [1, E], capacity_factor negative or not finite, or
 * the result does not fit in int32.
 */
int64_t moe_capacity(int64_t T, int32_t k, int32_t E, double capacity_factor);

/*
 * Routing ("Top-k MoE Router with Load Statistics"; "Sparse MoE Layer in NumPy",
 * top_k_gating and trap 6).
 *   x         device, [T, ldx] of x_dtype; read only when w_router != NULL.
 *   w_router  device, [D, E] of x_dtype, or NULL when the logits are supplied.
 *   logits    device, [T, E] fp32. Written (= x W_r, fp32 accumulate) when w_router
 *             is given, else read as the caller's scores.
 *   topk_idx  device, [T, k] int32: experts in descending logit order, exact ties to
 *             the lower index (-0.0 ties +0.0).
 *   topk_gate device, [T, k] fp32: p[idx] / sum over the k of p[idx], p = fp32 softmax.
 *   expert_count device, [E] int32: choices per expert before any drop.
 *   prob_sum  device, [E] fp32: sum over tokens of p[t, e].
 *   aux_loss  device, [1] fp32: E * sum_e (count_e / (T k)) * (prob_sum_e / T).
 *   opts      host pointer to router options, or NULL for the defaults above
 *             (scoring, selection bias and the z-loss output apply here).
 *   ws        device workspace of at least moe_route_workspace_size(T, E) bytes.
 * Non-finite logits violate the precondition; results are then undefined.
 */
size_t moe_route_workspace_size(int32_t T, int32_t E);
moe_status_t moe_route(const void* x, int32_t x_dtype, int64_t ldx, const void* w_router,
                       float* logits, int32_t T, int32_t D, int32_t E, int32_t k,
                       int32_t* topk_idx, float* topk_gate, int32_t* expert_count,
                       float* prob_sum, float* aux_loss, const moe_router_opts_t* opts,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * Position-priority dispatch ("Sparse MoE Layer in NumPy", trap 3 and
 * position_priority_dispatch; "32. Sparse MoE Token Dispatch & Combine", step 2).
 * Equal to visiting assignments a = t*k + j in increasing a and keeping each while its
 * expert has fewer than C kept rows; computed with a device-wide prefix scan.
 *   topk_idx    device, [T, k] int32 (indices outside [0, E) are skipped, flagged).
 *   slot        device, [T, k] int32: position in the expert's buffer, -1 if dropped.
 *   kept        device, [T, k] uint8: 1 if kept.
 *   slot_assign device, [E, C] int32: the assignment a held by each slot, -1 if empty.
 *   expert_used device, [E] int32: min(count, C).
 *   expert_overflow device, [E] int32: count - used.
 *   token_drops device, [T] int32: k minus the number of kept choices of the token.
 *   ws          device workspace, >= moe_dispatch_workspace_size(T, k, E) bytes.
 */
size_t moe_dispatch_workspace_size(int32_t T, int32_t k, int32_t E);
moe_status_t moe_dispatch(const int32_t* topk_idx, int32_t T, int32_t k, int32_t E,
                          int32_t C, int32_t* slot, uint8_t* kept, int32_t* slot_assign,
                          int32_t* expert_used, int32_t* expert_overflow,
                          int32_t* token_drops, void* ws, size_t ws_bytes, void* stream);

/*
 * Expert MLPs on the slot buffers ("Module 7", EducationalMoE expert loop and
 * swiglu_expert; llm-atlas "Mixture of Experts", Expert), as grouped GEMMs.
 * Row r < expert_used[e] of expert e is x[slot_assign[e, r] / k]. With
 * slot_assign == NULL the experts run densely on all T rows (a shared expert:
 * num_experts must be 1, expert_used ignored, outputs are [T, ...]).
 *   x            device, [T, ldx] of ex->dtype.
 *   hidden_cache device, [E, C, F] of ex->dtype (the activation fed to the second
 *                GEMM), or NULL to keep it in the workspace (bf16: in an internal
 *                layout of 32-column pieces, not meant to be read). Ignored for LINEAR.
 *   expert_out   device, [E, C, D] of ex->dtype, ungated.
 *   ws           >= moe_expert_mlp_workspace_size(ex, rows) bytes, rows = C or T.
 */
size_t moe_expert_mlp_workspace_size(const moe_experts_t* ex, int32_t rows);
moe_status_t moe_expert_mlp(const moe_experts_t* ex, const void* x, int64_t ldx, int32_t T,
                            int32_t k, int32_t C, const int32_t* slot_assign,
                            const int32_t* expert_used, void* hidden_cache,
                            void* expert_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Gate-weighted combine ("Sparse MoE Layer in NumPy", trap 4; router page, y
 * equation; "32. Sparse MoE Token Dispatch & Combine", step 6):
 *   y[t] = residual[t] + shared_out[t] + sum_{j = 0..k-1, slot[t,j] >= 0}
 *          topk_gate[t,j] * expert_out[topk_idx[t,j], slot[t,j]]
 * accumulated in fp32 in exactly that order, rounded once to dt. With
 * renormalize_kept = 1 each kept gate is first divided by the token's kept gate sum
 * ("Module 7. Mixture of Experts", dispatch_with_capacity, renormalize_kept_gates).
 *   residual, shared_out  device, [T, D] of dt, each may be NULL (term omitted).
 *   expert_out            device, [E, C, D] of dt (the slot buffers).
 *   slot                  device, [T, k] int32, or NULL: then every choice is kept and
 *                         expert_out holds one output per token and expert, [T, E, D],
 *                         row (t, topk_idx[t, j]) -- the precomputed expert outputs of
 *                         "Top-k MoE Router with Load Statistics" (C is then ignored;
 *                         T * E must be below 2^31).
 * Any D >= 1: rows that split into 16-byte pieces tiling 256 threads (D / 8 for bf16,
 * D / 4 for fp32, dividing 256 or a multiple of it) take the vector kernel, other D a
 * one-element-per-thread kernel with the same summation order.
 * Precondition: 0 <= topk_idx < E and slot < C (violations are skipped).
 */
moe_status_t moe_combine(int32_t dt, const void* residual, const void* shared_out,
                         const void* expert_out, const int32_t* topk_idx,
                         const int32_t* slot, const float* topk_gate, int32_t T,
                         int32_t k, int32_t E, int32_t C, int32_t D,
                         int32_t renormalize_kept, void* y, void* stream);

/* The whole forward pass in one call ("Sparse MoE Layer in NumPy", section 2 forward and
 * section 4 usage; "Module 7. Mixture of Experts", EducationalMoE.forward; llm-atlas
 * "Mixture of Experts", TopKMoE.forward): router scores, routing, capacity dispatch,
 * the routed experts on their slot buffers, the shared expert, the gate-weighted
 * combine onto the residual and the pre-drop aux loss, all enqueued on one stream with
 * no host synchronisation. Each step is the one of the entry point above that names
 * it (moe_route, moe_dispatch, moe_expert_mlp, moe_combine); the outputs are theirs. */
typedef struct {
  const void* x;            /* device [T, ldx], experts.dtype                          */
  int64_t ldx;
  int32_t T;
  const void* w_router;     /* device [D, E] experts.dtype, or NULL: logits are input   */
  float* logits;            /* device [T, E] fp32, written or read (see moe_route)      */
  moe_experts_t experts;    /* routed experts                                          */
  moe_experts_t shared;     /* one always-on SWIGLU expert, or shared.w_in == NULL      */
  int32_t k;
  int32_t capacity;         /* C, e.g. from moe_capacity                               */
  int32_t use_residual;     /* 1: y includes x                                         */
  /* outputs (device) */
  int32_t* topk_idx;        /* [T, k]   */
  float* topk_gate;         /* [T, k]   */
  int32_t* expert_count;    /* [E]      */
  float* prob_sum;          /* [E]      */
  float* aux_loss;          /* [1]      */
  int32_t* slot;            /* [T, k]   */
  uint8_t* kept;            /* [T, k]   */
  int32_t* slot_assign;     /* [E, C]   */
  int32_t* expert_used;     /* [E]      */
  int32_t* expert_overflow; /* [E]      */
  int32_t* token_drops;     /* [T]      */
  void* hidden_cache;       /* [E, C, F] or NULL                                      */
  void* expert_out;         /* [E, C, D], kept for the backward                       */
  void* shared_out;         /* [T, D] or NULL (then kept in the workspace)            */
  void* y;                  /* [T, D]   */
  moe_router_opts_t router; /* router variants; all zero = the default softmax router  */
} moe_forward_args_t;

size_t moe_forward_workspace_size(const moe_forward_args_t* a);
moe_status_t moe_forward(const moe_forward_args_t* a, void* ws, size_t ws_bytes,
                         void* stream);

/*
 * moe_forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation). Same launches, same results as moe_forward. The workspace is a 32 MiB
 * device array inside the library: each GPU the library runs on holds its own copy
 * until the process ends. Requirements beyond moe_forward's: hidden_cache must be
 * given when the experts have a hidden layer and C > 0, shared_out when there is a
 * shared expert (both are then outputs), and moe_forward_workspace_size(a) must not
 * exceed 32 MiB (the routing partials, about T * E / 4 bytes, plus the shared expert's
 * hidden activation, T * d_hidden elements); otherwise MOE_ERR_INVALID_ARG or
 * MOE_ERR_WORKSPACE and nothing is launched. Every call on one GPU uses that GPU's
 * array: calls that are not ordered on one stream race with each other. No contents
 * carry over from one call to the next. Allocates nothing, and makes no allocating
 * library call.
 */
moe_status_t moe_forward_noalloc(const moe_forward_args_t* a, void* stream);

/*
 * Backward of the whole layer ("Sparse MoE Layer in NumPy", section 2 moe_backward and
 * trap 7, for single-linear experts; extended by the chain rule through the GELU and
 * SwiGLU expert MLPs of "Module 7" / llm-atlas "Mixture of Experts", Expert), with the
 * discrete choices (top-k set, kept mask) held constant. For a kept assignment
 * a = (t, j) -> e with expert output o_a (ungated, from the forward) the expert's output
 * gradient is dO_a = g'_a dy_t, g' the effective gate (topk_gate, or with
 * router.renormalize_kept topk_gate / K_t, K_t the token's kept gate sum), and
 *   dgate[a]  = kept_a <dy_t, o_a> (the gradient of topk_gate; with renormalize_kept
 *               taken through the survivor quotient: (d'_a - sum_kept g'_r d'_r) / K_t,
 *               d' = <dy_t, o_a>, 0 for dropped a)
 *   dlogits   = softmax scoring: p * (dp - <p, dp>), dp[t, idx_tj] = dq_tj,
 *               dq_tj = (dgate_tj - sum_r g_tr dgate_tr) / S_t, S_t = sum_r q_tr over the
 *               chosen clean scores q (p or sigmoid(s)); sigmoid scoring: dq_tj q_tj
 *               (1 - q_tj) at the chosen experts, 0 elsewhere; plus aux_grad_scale (E/T)
 *               p (f - <p, f>), f_e = count_e / (T k); plus z_grad_scale (2/T) lse_t p
 *   expert parameter gradients = sums over the expert's kept rows of the MLP's chain
 *               rule with input x_t and output gradient dO_a (LINEAR: dW = x^T dO;
 *               GELU_MLP: Z = x W_in + b_in, dZ = (dO W_out^T) gelu'(Z), dW_in = x^T dZ,
 *               db_in = sum dZ, dW_out = gelu(Z)^T dO, db_out = sum dO; SWIGLU:
 *               A = x W_in, U = x W_up, dH = dO W_out^T, dA = dH U silu'(A),
 *               dU = dH silu(A), dW_in = x^T dA, dW_up = x^T dU, dW_out = (silu(A) U)^T dO);
 *               experts without kept rows get zeros
 *   dx[t]     = r dy_t + sum over kept a in t of the expert's input gradient
 *               (LINEAR: dO W^T; GELU_MLP: dZ W_in^T; SWIGLU: dA W_in^T + dU W_up^T)
 *               + the shared expert's input gradient (ungated: its dO is dy)
 *               + dlogits W_r^T when w_router is given (logits = x W_r); without
 *               w_router the logits are an independent input and dx has no router term
 *   dw_router = x^T dlogits
 * The pre-activations are recomputed from x (nothing but expert_out is kept from the
 * forward). fp32 experts in the IN_OUT layout only (bf16 or OUT_IN returns
 * MOE_ERR_UNSUPPORTED). All reductions run in
 * a fixed order: results are bitwise reproducible.
 */
typedef struct {
  const void* dy;           /* device [T, ld]  */
  const void* x;            /* device [T, ld]  */
  int64_t ld;               /* must equal d_model */
  int32_t T;
  const float* logits;      /* device [T, E]   */
  moe_experts_t experts;
  int32_t k;
  int32_t capacity;
  int32_t use_residual;
  float aux_grad_scale;
  const int32_t* topk_idx;
  const float* topk_gate;
  const int32_t* expert_count;
  const int32_t* slot;
  const int32_t* slot_assign;
  const int32_t* expert_used;
  const void* expert_out;   /* [E, C, D] from the forward */
  /* outputs (device) */
  void* dx;                 /* [T, D]    */
  void* dW;                 /* [E, D, F] gradient of experts.w_in ([E, D, D] for LINEAR) */
  float* dgate;             /* [T, k]    */
  float* dlogits;           /* [T, E]    */
  /* MLP experts: further outputs, required when the kind has the weight */
  void* dW_up;              /* [E, D, F] SWIGLU                                        */
  void* dW_out;             /* [E, F, D] GELU_MLP, SWIGLU                              */
  void* db_in;              /* [E, F]    GELU_MLP with b_in                            */
  void* db_out;             /* [E, D]    GELU_MLP with b_out                           */
  /* shared SwiGLU expert as in the forward, or shared.w_in == NULL */
  moe_experts_t shared;
  void* dshared_w_in;       /* [D, Fs] */
  void* dshared_w_up;       /* [D, Fs] */
  void* dshared_w_out;      /* [Fs, D] */
  /* router weights, or NULL (see dx above); E must be a multiple of 4 */
  const void* w_router;     /* [D, E] */
  void* dw_router;          /* [D, E] */
  /* the forward's router variant (scoring and renormalize_kept are used; the
   * selection is the given topk_idx) and the weight of the z-loss in the loss */
  moe_router_opts_t router;
  float z_grad_scale;
} moe_backward_args_t;

size_t moe_backward_workspace_size(const moe_backward_args_t* a);
moe_status_t moe_backward(const moe_backward_args_t* a, void* ws, size_t ws_bytes,
                          void* stream);

/*
 * Reads (synchronously: waits for `stream`) and returns the device error word kept in
 * a workspace used by moe_dispatch or moe_forward; 0 means no data error. Bit 0: an
 * expert index outside [0, E) was skipped. Returns -1 if the copy failed.
 */
int32_t moe_read_error(const void* ws, void* stream);

/*
 * Per-kernel timing for measurement. When enabled, every entry point brackets each
 * kernel it launches with HIP events recorded on the same stream. moe_profile_read
 * waits for those events and returns, per kernel name, the number of launches and
 * the summed milliseconds; it then clears the record. Not thread-safe.
 */
void moe_profile_enable(int32_t on);
int32_t moe_profile_read(char* names, int32_t name_stride, int32_t* counts, double* total_ms,
                         int32_t max_entries);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
