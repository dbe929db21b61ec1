/*
 * topmoe.h — C ABI of the MI355X (gfx950) MiniMind FFN / top-k MoE forward.
 *
 * Operations (definitions from the MiniMind course, lesson 13 "FFN and MoE",
 * sections 0, 1.2, 1.5, 1.6 and source walkthrough steps 3-6; minimind3
 * chapter 4 "MLP & MoE", sections 4.2-4.4):
 *
 *   dense FFN      y = W_down( SiLU(W_gate x) * W_up x ),  SiLU(z) = z * sigmoid(z)
 *   MoE router     p = softmax(W_router x);  S = TopK(p, k);
 *                  alpha_e = p_e / (sum_{j in S} p_j + 1e-20)
 *   MoE output     y = sum_{e in S} alpha_e * Expert_e(x), each expert a dense FFN
 *   aux loss       aux = E * coef * sum_e load_e * prob_e,
 *                  load_e = (tokens that selected e) / N,  prob_e = mean_t p_{t,e}
 *   z-loss         z_coef * mean_t logsumexp_e(r_te)^2 (router logits r = W_router x)
 *   capacity       each expert takes at most C = ceil(capacity_factor * N * k / E)
 *                  tokens: the first C of its tokens in ascending token order
 *                  (the dispatch order); the others' (token, expert) pairs are
 *                  dropped and add nothing to y
 *                  (the MiniMind study notes' section 10 table names router
 *                  z-loss and expert capacity without defining them; these are
 *                  the standard forms)
 *   backward       the gradients of these with respect to x and every weight:
 *                  the top-k choice and the counts load_e are discrete and
 *                  carry no gradient; the softmax probabilities carry it back
 *                  through alpha and prob_e (minimind3 chapter 4, section
 *                  4.4; MiniMind study notes, section 7 on router training)
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library never allocates, frees or retains them.
 *   - Row-major layouts.  Weights use the nn.Linear [out, in] layout.
 *   - Calls are asynchronous: they validate synchronously on the host, then
 *     enqueue kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *     return.  No host synchronisation, no device-to-host copy.
 *   - On any error nothing is launched and no output is touched.  Errors are
 *     negative status codes (topmoe_strerror gives text).  A HIP launch error
 *     is reported as TOPMOE_ERR_HIP (outputs may then be partly written).
 *   - Results are deterministic: the same inputs give bitwise identical
 *     outputs (no floating-point atomics anywhere).
 *   - `stage_events`, when not NULL, is an array of 2 * stages hipEvent_t
 *     handles (see topmoe_events_create); events 2i and 2i+1 are stamped by
 *     the dispatch of stage i's kernel at its start and end (AMD's
 *     hipExtLaunchKernel start / stop events), so they bracket exactly that
 *     kernel's execution; a stage that launches no kernel records both back
 *     to back.  Pass NULL in production.  Stage counts: TOPMOE_FFN_STAGES,
 *     TOPMOE_MOE_STAGES.
 *
 * dtype
 *   TOPMOE_DTYPE_FP32: x, W_gate, W_up, W_down, y float32; all arithmetic fp32.
 *   TOPMOE_DTYPE_BF16: x, W_gate, W_up, W_down, y bfloat16; fp32 accumulation;
 *                      the SiLU(g)*u intermediate is rounded to bf16; y is
 *                      rounded once (round-to-nearest-even).
 *   The router weight W_router is float32 in both, and routing is fp32.
 *
 * Shape limits: N >= 0 (N == 0 is a no-op apart from zeroed offsets and aux;
 * then x, y, topk_idx, alpha and sorted_token_ids may be NULL),
 * H and I positive multiples of 64, 1 <= E <= 64, 1 <= k <= E,
 * N * max(k, 1) < 2^31, and every GEMM operand below 4 GiB: x (N * H), the
 * intermediate (N * k * I) and one expert's W_gate / W_up / W_down (I * H),
 * counted in bytes of the dtype.
 */
#ifndef TOPMOE_H
#define TOPMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---------------------------------------------------- */
#define TOPMOE_OK                        0
#define TOPMOE_ERR_NULL_ARG             -1  /* a required pointer is NULL            */
#define TOPMOE_ERR_BAD_SHAPE            -2  /* N, H, I, E or k outside the limits     */
#define TOPMOE_ERR_UNSUPPORTED_DTYPE    -3  /* dtype not FP32 / BF16                  */
#define TOPMOE_ERR_WORKSPACE_TOO_SMALL  -4  /* workspace_bytes < *_workspace_bytes()  */
#define TOPMOE_ERR_HIP                  -5  /* a HIP runtime call or launch failed    */
#define TOPMOE_ERR_BAD_ARG              -6  /* aux_coef, z_coef or capacity_factor negative or not
                                               finite; aux_grad or z_grad not finite; unknown
                                               flag bits; misaligned pointer; a launch-shape
                                               override that is not instantiated */
#define TOPMOE_ERR_SCRATCH_TOO_SMALL    -7  /* moe_ffn_fwd_noalloc: the problem's workspace
                                               exceeds the fixed scratch */

/* ---- dtypes ------------------------------------------------------------ */
#define TOPMOE_DTYPE_FP32 0
#define TOPMOE_DTYPE_BF16 1

/* ---- stages (for stage_events) ------------------------------------------ */
#define TOPMOE_FFN_STAGES 2  /* 0 gate/up GEMM + SiLU*up, 1 down GEMM                   */
#define TOPMOE_MOE_STAGES 5  /* 0 router, 1 expert offsets + aux + token scatter,
                                2 grouped gate/up GEMM + SiLU*up, 3 grouped down GEMM
                                + alpha, 4 combine of the k slots (k == 1: empty, or
                                under a capacity the rows of the dropped tokens).
                                Decode-sized inference calls do stage 1 (and, with
                                E <= 16, stage 0) inside the GEMM launches: such a
                                stage launches no kernel                                */
#define TOPMOE_FFN_BWD_STAGES 7  /* 0 weight transposes, 1 x / dy transposes,
                                    2 g, u GEMM (recomputed), 3 dh GEMM + dg, du,
                                    4 dx GEMM, 5 dWg + dWu GEMM, 6 dWd GEMM             */
#define TOPMOE_MOE_BWD_STAGES 12 /* 0 router, 1 offsets + scatter (the forward's routing),
                                    2 weight transposes, 3 grouped x / alpha*dy
                                    transposes, 4 grouped g, u GEMM (recomputed),
                                    5 grouped dh GEMM + dg, du, d alpha, 6 grouped dx GEMM,
                                    7 router backward, 8 dx combine, 9 dW_router,
                                    10 grouped dWg + dWu, 11 grouped dWd               */

/* ---- moe_ffn_fwd flags -------------------------------------------------- */
/* The config's norm_topk_prob = False (lesson 13, walkthrough steps 1 and 5;
 * minimind3 chapter 4, section 4.3 step 2): alpha is the selected
 * probabilities as they are, without renormalisation to sum 1. */
#define TOPMOE_MOE_RAW_TOPK_WEIGHTS 1
/* moe_ffn_bwd only: the workspace already holds the routing, the pairs
 * (g, u) and h^T that moe_ffn_fwd_train wrote into it for the same inputs
 * and arguments, so the router, the permutation and the grouped g, u GEMM
 * (stages 0, 1 and 4) are skipped. */
#define TOPMOE_MOE_BWD_SAVED 2
/* The module outside training (lesson 13, walkthrough step 6: the aux loss
 * is computed only while training; otherwise it is a zero scalar): aux_loss
 * and z_loss are 0 whatever aux_coef and z_coef say, and moe_ffn_bwd passes
 * no gradient through them.  Everything else is unchanged. */
#define TOPMOE_MOE_EVAL 4

/* Workspace needed by ffn_swiglu_fwd: the SiLU(g)*u intermediate [N, I]
 * (dtype-sized elements), 256-byte aligned.  Returns 0 for invalid shapes. */
size_t ffn_workspace_bytes(int64_t N, int64_t H, int64_t I, int dtype);

/* Dense SwiGLU FFN forward (lesson 13, sections 0 and 1.2; walkthrough step 3;
 * minimind3 chapter 4, section 4.2).
 *   x   [N, H]   input tokens (B*S flattened; the caller reshapes)
 *   Wg  [I, H]   gate_proj.weight      Wu [I, H] up_proj.weight
 *   Wd  [H, I]   down_proj.weight
 *   residual [N, H]  optional (NULL = none), same dtype: the block's residual
 *                stream; y = residual + FFN(x) (lesson 13, sections 1.3-1.4:
 *                hidden_states + mlp(...)), summed in fp32 and rounded once.
 *                May alias y (each element is read before it is written).
 *   y   [N, H]   output, same dtype as x; must not alias x or the weights
 *   workspace    device scratch of at least ffn_workspace_bytes(N, H, I, dtype)
 *                bytes, 256-byte aligned; contents on entry are ignored.
 * All tensor pointers must be 16-byte aligned. */
int ffn_swiglu_fwd(const void* x, const void* Wg, const void* Wu, const void* Wd,
                   const void* residual, void* y, int64_t N, int64_t H, int64_t I, int dtype,
                   void* workspace, size_t workspace_bytes,
                   void* stream, void* const* stage_events);

/* Workspace needed by moe_ffn_fwd (routing partials, permutation, the
 * SiLU(g)*u intermediate [N*k, I] and, for k >= 2, the k-slots [N*k, H] of
 * alpha-scaled expert outputs in the dtype).
 * Returns 0 for invalid shapes. */
size_t moe_workspace_bytes(int64_t N, int64_t H, int64_t I, int E, int k, int dtype);

/* Top-k MoE FFN forward (lesson 13, sections 0, 1.5, 1.6 and walkthrough
 * steps 4-6; minimind3 chapter 4, sections 4.3 and 4.4).
 *   x        [N, H]      input tokens (dtype)
 *   Wr       [E, H]      router (gate) weight, float32
 *   Wg, Wu   [E, I, H]   experts' gate_proj / up_proj weights, stacked (dtype)
 *   Wd       [E, H, I]   experts' down_proj weights, stacked (dtype)
 *   residual [N, H]      optional (NULL = none), dtype: y starts from it
 *                        instead of zeros (y = residual + MoE(x), lesson 13,
 *                        sections 1.3-1.4).  May alias y.
 *   aux_coef             router_aux_loss_coef (>= 0); 0 gives aux = 0 exactly,
 *                        which is also the module's value outside training
 *   z_coef               router z-loss coefficient (>= 0); 0 gives z_loss = 0
 *   capacity_factor      expert capacity factor (>= 0); 0 = no capacity (dropless,
 *                        the pages' module); a capacity of N or more drops nothing
 *   flags                0, or TOPMOE_MOE_RAW_TOPK_WEIGHTS and / or TOPMOE_MOE_EVAL
 *   y        [N, H]      output (dtype): y_t = residual_t (or 0) + the sum over
 *                        the selected (and kept) experts in ascending expert id
 *                        of alpha * Expert_e(x_t); with k >= 2 (or a capacity)
 *                        each expert term is first rounded to the dtype (the
 *                        terms the pages' index_add_ adds); the sum is taken in
 *                        fp32 and rounded once
 *   topk_idx [N, k]      int32 selected experts, slot order = probability
 *                        descending, equal probabilities by ascending id
 *                        (dropped pairs included: the router's choice)
 *   alpha    [N, k]      float32 weights in the same slot order: renormalised
 *                        to sum 1 (default) or the raw probabilities (flag);
 *                        not renormalised after drops
 *   aux_loss [1]         float32 load-balancing loss (training-mode value; counts
 *                        every selection, kept or dropped)
 *   z_loss   [1]         optional (NULL = not returned) float32 router z-loss
 *   expert_offsets [E+1] optional (NULL = not returned) int32 exclusive prefix
 *                        sum of per-expert token counts (of the kept tokens)
 *   sorted_token_ids [N*k] optional int32: tokens grouped by expert, ascending
 *                        expert id, ascending token id within an expert (kept
 *                        tokens; the remaining positions hold -1)
 *   workspace            at least moe_workspace_bytes(N, H, I, E, k, dtype)
 *                        bytes, 256-byte aligned; contents on entry ignored.
 * Outputs must not alias inputs or each other.  Tensor pointers must be
 * 16-byte aligned (int32/float32 outputs: 4-byte aligned). */
int moe_ffn_fwd(const void* x, const float* Wr, const void* Wg, const void* Wu,
                const void* Wd, const void* residual, int64_t N, int64_t H, int64_t I,
                int E, int k, float aux_coef, float z_coef, float capacity_factor, int flags,
                int dtype, void* y, int32_t* topk_idx, float* alpha, float* aux_loss,
                float* z_loss, int32_t* expert_offsets, int32_t* sorted_token_ids,
                void* workspace, size_t workspace_bytes,
                void* stream, void* const* stage_events);

/* ---- no allocation ------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the MoE
 * forward with its workspace in a fixed scratch array that the library holds
 * in device memory, one per GPU it runs on, from the first use until the
 * process ends (TOPMOE_NOALLOC_SCRATCH_BYTES: 64 MiB).  Arguments,
 * outputs, errors and results are those of moe_ffn_fwd (the same bits)
 * without the workspace pair; a problem whose moe_workspace_bytes() exceeds
 * the scratch returns TOPMOE_ERR_SCRATCH_TOO_SMALL before anything else
 * happens.  The call allocates nothing: the scratch's device address is
 * looked up once per device (the device current at the call must be the
 * stream's).  All calls on one GPU share its scratch, so calls that overlap
 * on one GPU (other streams, other host threads) race: serialise them.  The
 * scratch keeps the last call's contents; nothing in it needs clearing. */
#define TOPMOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int moe_ffn_fwd_noalloc(const void* x, const float* Wr, const void* Wg, const void* Wu,
                        const void* Wd, const void* residual, int64_t N, int64_t H, int64_t I,
                        int E, int k, float aux_coef, float z_coef, float capacity_factor,
                        int flags, int dtype, void* y, int32_t* topk_idx, float* alpha,
                        float* aux_loss, float* z_loss, int32_t* expert_offsets,
                        int32_t* sorted_token_ids, void* stream, void* const* stage_events);

/* ---- backward ------------------------------------------------------------
 * Gradients of the forward above (same shapes, dtypes and flags).  The
 * forward's intermediate activations are not needed: the backward recomputes
 * them (and, for the MoE, the routing: same kernels, same choices).
 * Gradient outputs are overwritten, not accumulated; weight gradients have
 * the weights' dtype and layout, dW_router is float32.  The gradient with
 * respect to the residual stream of the forward is dy itself (nothing to
 * compute).  In bf16, the recomputed g and u, [dg | du], dg, du, h and
 * alpha*dy are rounded to bf16 before the arithmetic or GEMMs that consume
 * them; all accumulation is fp32. */

/* Workspace needed by ffn_swiglu_bwd: transposed weights [H, 2I] and [I, H],
 * transposed x and dy [H, round64(N)], the pairs (g, u) [N, I], [dg | du]
 * [N, 2I] and dg^T, du^T, h^T [I, round64(N)] (dtype-sized elements).
 * Returns 0 for invalid shapes. */
size_t ffn_bwd_workspace_bytes(int64_t N, int64_t H, int64_t I, int dtype);

/* Dense SwiGLU FFN backward.  With g = x Wg^T, u = x Wu^T, h = SiLU(g) * u,
 * y = h Wd^T and the upstream gradient dy [N, H]:
 *   dWd = dy^T h,  dh = dy Wd,  dg = dh * u * SiLU'(g),  du = dh * SiLU(g),
 *   dWg = dg^T x,  dWu = du^T x,  dx = dg Wg + du Wu,
 *   SiLU'(z) = sigmoid(z) * (1 + z * (1 - sigmoid(z))).
 *   x, Wg, Wu, Wd   as for ffn_swiglu_fwd;  dy [N, H] (dtype)
 *   dx [N, H], dWg [I, H], dWu [I, H], dWd [H, I]   outputs (dtype); N == 0
 *                   gives zero weight gradients (x, dy, dx may then be NULL)
 *   workspace       at least ffn_bwd_workspace_bytes(N, H, I, dtype) bytes,
 *                   256-byte aligned; contents on entry ignored.
 * Outputs must not alias inputs or each other; tensor pointers 16-byte
 * aligned.  Shape limits as for the forward, plus [N, 2I], [H, 2I] and
 * [I, round64(N)] operands below 4 GiB each. */
int ffn_swiglu_bwd(const void* x, const void* Wg, const void* Wu, const void* Wd,
                   const void* dy, void* dx, void* dWg, void* dWu, void* dWd,
                   int64_t N, int64_t H, int64_t I, int dtype,
                   void* workspace, size_t workspace_bytes,
                   void* stream, void* const* stage_events);

/* ---- training: keep g, u for the backward ----------------------------- */
/* The backward recomputes g = x Wg^T and u = x Wu^T (its stage "g, u GEMM")
 * unless the forward kept them.  These forwards compute exactly what
 * ffn_swiglu_fwd / moe_ffn_fwd compute (the same bits in every output) and
 * in the same gate/up GEMM also write the pairs (g, u) and h^T into `saved`,
 * a backward workspace (the MoE forward keeps its routing there as well:
 * selections, probabilities, offsets and the expert-grouped entry lists): at least ffn_bwd_workspace_bytes(N, H, I, dtype) /
 * moe_bwd_workspace_bytes(N, H, I, E, k, dtype) bytes, 256-byte aligned.
 * Pass that same buffer, untouched in between, as the workspace of
 * ffn_swiglu_bwd_saved / moe_ffn_bwd with TOPMOE_MOE_BWD_SAVED for the same
 * inputs and arguments.  Costs the forward the pair and h^T stores (three
 * times h's bytes), saves the backward its largest GEMM but one (and, for
 * the MoE, its routing kernels).  The other
 * arguments, errors and stage events are those of the plain forwards; a
 * NULL `saved` is TOPMOE_ERR_NULL_ARG. */
int ffn_swiglu_fwd_train(const void* x, const void* Wg, const void* Wu, const void* Wd,
                         const void* residual, void* y, int64_t N, int64_t H, int64_t I,
                         int dtype, void* workspace, size_t workspace_bytes,
                         void* saved, size_t saved_bytes,
                         void* stream, void* const* stage_events);
int moe_ffn_fwd_train(const void* x, const float* Wr, const void* Wg, const void* Wu,
                      const void* Wd, const void* residual, int64_t N, int64_t H, int64_t I,
                      int E, int k, float aux_coef, float z_coef, float capacity_factor,
                      int flags, int dtype, void* y, int32_t* topk_idx, float* alpha,
                      float* aux_loss, float* z_loss, int32_t* expert_offsets,
                      int32_t* sorted_token_ids, void* workspace, size_t workspace_bytes,
                      void* saved, size_t saved_bytes,
                      void* stream, void* const* stage_events);
/* ffn_swiglu_bwd on a workspace that ffn_swiglu_fwd_train filled (stage 2
 * skipped, its events zero-length). */
int ffn_swiglu_bwd_saved(const void* x, const void* Wg, const void* Wu, const void* Wd,
                         const void* dy, void* dx, void* dWg, void* dWu, void* dWd,
                         int64_t N, int64_t H, int64_t I, int dtype,
                         void* workspace, size_t workspace_bytes,
                         void* stream, void* const* stage_events);

/* Workspace needed by moe_ffn_bwd: the routing buffers, transposed expert
 * weights [E, H, 2I] and [E, I, H], the per-entry intermediates and
 * gradients, and float32 router buffers.  Returns 0 for invalid shapes. */
size_t moe_bwd_workspace_bytes(int64_t N, int64_t H, int64_t I, int E, int k, int dtype);

/* Top-k MoE FFN backward.  The routing of moe_ffn_fwd(x, Wr, ..., k,
 * aux_coef, flags) is recomputed; for each token t and selected expert e
 * (weight alpha_{t,e}, expert output o = Expert_e(x_t)):
 *   the expert's own backward (as ffn_swiglu_bwd) with upstream alpha * dy_t;
 *   d alpha_{t,e} = dy_t . o;
 *   then dp through alpha = p_S / (sum p_S + 1e-20) (or alpha = p_S with
 *   TOPMOE_MOE_RAW_TOPK_WEIGHTS), plus aux_grad * aux_coef * E * c_e / N^2 on
 *   every p_{t,e} (c_e = tokens routed to e); dr = p * (dp - sum(p * dp))
 *   + z_grad * z_coef * 2 * logsumexp(r_t) * p / N; dW_router = dr^T x and
 *   dx_t += W_router^T dr_t.  A pair dropped by the capacity contributes
 *   neither an expert gradient nor d alpha.
 *   x, Wr, Wg, Wu, Wd, N, H, I, E, k, aux_coef, z_coef, capacity_factor,
 *   flags, dtype    as for moe_ffn_fwd; flags may add TOPMOE_MOE_BWD_SAVED
 *                   (TOPMOE_MOE_EVAL: no gradient through aux_loss, z_loss)
 *   dy [N, H]       upstream gradient of y (dtype)
 *   aux_grad        upstream gradient of aux_loss (1 when it is added to the
 *                   loss as is); finite
 *   z_grad          upstream gradient of z_loss; finite
 *   aux_grad_scale, z_grad_scale
 *                   optional (NULL = 1) float32 device scalars multiplying
 *                   aux_grad / z_grad: an upstream gradient that is still on
 *                   the device (autograd's) is read by the kernel, with no
 *                   host synchronisation.  Their value is not validated.
 *   dx [N, H] (dtype), dWr [E, H] (float32), dWg, dWu [E, I, H], dWd [E, H, I]
 *                   (dtype) outputs; experts no token selected get zero
 *                   gradients.  N == 0 gives all-zero weight gradients.
 *   workspace       at least moe_bwd_workspace_bytes(N, H, I, E, k, dtype)
 *                   bytes, 256-byte aligned; contents on entry ignored.
 * Outputs must not alias inputs or each other; tensor pointers 16-byte
 * aligned. */
int moe_ffn_bwd(const void* x, const float* Wr, const void* Wg, const void* Wu,
                const void* Wd, const void* dy, float aux_grad, float z_grad,
                const float* aux_grad_scale, const float* z_grad_scale,
                int64_t N, int64_t H, int64_t I, int E, int k, float aux_coef, float z_coef,
                float capacity_factor, int flags, int dtype,
                void* dx, float* dWr, void* dWg, void* dWu, void* dWd,
                void* workspace, size_t workspace_bytes,
                void* stream, void* const* stage_events);

/* Human-readable text for a status code (static storage). */
const char* topmoe_strerror(int status);

/* Library ABI version (major * 100 + minor). */
int topmoe_version(void);

/* ---- instrumentation helpers (not on the hot path) ---------------------- */
/* Launch-shape override of one GEMM of the path, for tuning sweeps and tests.
 *   gemm   TOPMOE_TILE_GATEUP (forward gate/up), TOPMOE_TILE_DOWN (forward down
 *          and the backward's dx), TOPMOE_TILE_BWD_GU, TOPMOE_TILE_BWD_DH,
 *          TOPMOE_TILE_WGRAD_GU (dW_g + dW_u), TOPMOE_TILE_WGRAD_D (dW_d)
 *   shape  int[6] {block rows, block columns, wavefront rows, wavefront
 *          columns, LDS row bytes, ring depth}, or NULL to clear the override
 * Returns TOPMOE_ERR_BAD_ARG, changing nothing, if the library does not
 * instantiate that shape for that GEMM.  Initial overrides come from the
 * environment variables TOPMOE_GATEUP_TILE, TOPMOE_DOWN_TILE,
 * TOPMOE_BWDGU_TILE, TOPMOE_BWDDH_TILE, TOPMOE_WGU_TILE, TOPMOE_WD_TILE
 * ("BMxBNxWMxWNxRBxS"), read once, by the first call that plans a launch;
 * while one of them names a shape that is not instantiated, the calls that
 * would use it return TOPMOE_ERR_BAD_ARG before launching anything.  An
 * override applies to every dtype for which the shape is instantiated. */
#define TOPMOE_TILE_GATEUP 0
#define TOPMOE_TILE_DOWN 1
#define TOPMOE_TILE_BWD_GU 2
#define TOPMOE_TILE_BWD_DH 3
#define TOPMOE_TILE_WGRAD_GU 4
#define TOPMOE_TILE_WGRAD_D 5
int topmoe_set_tile_override(int gemm, const int* shape);

/* The launch plan moe_ffn_fwd (inference, flags without effect on it) follows
 * for a problem, computed on the host without touching a GPU: info[i] for
 * i < n receives field i below (-1 past the last).  Returns TOPMOE_OK, or the
 * status moe_ffn_fwd would return for the sizes, dtype or capacity factor
 * (NULL info with n > 0: TOPMOE_ERR_NULL_ARG). */
#define TOPMOE_PATH_ROUTER_LAYOUT 0  /* 0: W_router in LDS, 16 tokens per pass;
                                        1: one token at a time, H split over
                                        four wavefronts; 2: as 0, 16 lanes per token */
#define TOPMOE_PATH_ROUTER_TOKENS 1  /* tokens per router block                  */
#define TOPMOE_PATH_ROUTER_BLOCKS 2  /* router blocks                            */
#define TOPMOE_PATH_UP_BM 3          /* gate/up tile rows, columns, ring depth   */
#define TOPMOE_PATH_UP_BN 4
#define TOPMOE_PATH_UP_RING 5
#define TOPMOE_PATH_DOWN_BM 6        /* down tile rows, columns, ring depth      */
#define TOPMOE_PATH_DOWN_BN 7
#define TOPMOE_PATH_DOWN_RING 8
#define TOPMOE_PATH_DOWN_KSPLIT 9    /* K chunks of the down projection (1: none) */
#define TOPMOE_PATH_INBLOCK 10       /* 1: the GEMMs group the entries themselves
                                        (no permutation launch)                  */
#define TOPMOE_PATH_ROUTER_IN_UP 11  /* 1: the router runs as blocks of the gate/up
                                        launch, which takes every token against
                                        every expert (no router launch)          */
#define TOPMOE_PATH_FIELDS 12
int moe_ffn_fwd_path(int64_t N, int64_t H, int64_t I, int E, int k, float capacity_factor,
                     int dtype, int32_t* info, int n);

/* Create / destroy n timing-enabled hipEvent_t handles. */
int topmoe_events_create(int n, void** events);
int topmoe_events_destroy(int n, void** events);
/* Wait for `stop` and return the elapsed milliseconds between two events. */
int topmoe_event_elapsed_ms(void* start, void* stop, float* ms);

#ifdef __cplusplus
}
#endif
#endif /* TOPMOE_H */
