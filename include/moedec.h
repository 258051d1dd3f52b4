/*
 * moedec.h - C ABI of libmoedec: the routed Mixture-of-Experts FFN step of
 * GLM-5.2-style decode on AMD Instinct MI355X (gfx950).
 *
 * The step, as the pages state it:
 *   - Show HN page "धीमे कंप्यूटर पर GLM 5.2 चलाना" (hi.news.hada.io), section
 *     "implement किए गए मुख्य features": a DeepSeek-V3-style sigmoid router
 *     (noaux_tc correction, routed_scaling_factor, shared expert); int8,
 *     packed int4 and packed int2 weights with one scale per row, dequantised
 *     on use; batch-union MoE (each unique expert of a batch read once and
 *     applied to every position routed to it).
 *   - ideipro.ru, "Энтузиаст запустил GLM-5.2 на ноутбуке с 25 ГБ RAM": 8
 *     experts per token in each MoE layer; packing checked bit for bit.
 *   - same Show HN page, section "disk streaming आधारित MoE execution तरीका":
 *     256 routed experts per layer, about 19 MB per int4 expert.
 * Points the pages leave open are fixed as follows (and documented per call):
 * group score = sum of the two largest bias-corrected scores of a group;
 * corrected scores select, unbiased sigmoid scores weigh; ties go to the lower
 * index; experts are SwiGLU (h = silu(Wg x) * (Wu x), y = Wd h, no biases);
 * shared experts weigh 1; codes are two's complement, lowest column in the
 * lowest bits of its byte; matrices are [out_rows, in] row-major, packed
 * along the input dimension, one fp32 scale per output row.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless stated otherwise; the caller owns and
 *     frees all memory.  The library allocates nothing and never
 *     synchronises: work is enqueued on `stream` (a hipStream_t; NULL = the
 *     null stream) and the call returns at once.  Its only mutable global
 *     state is the static array of moe_expert_down_combine_em_noalloc_q4.
 *   - Struct arguments (moedec_experts, moedec_worklist) are HOST memory read
 *     during the call; their pointer fields are device pointers.
 *   - Arguments are validated before anything is enqueued.  Return values:
 *     MOEDEC_OK, MOEDEC_ERR_INVALID_ARG (null pointer, inconsistent sizes),
 *     MOEDEC_ERR_UNSUPPORTED (valid but outside the kernels' limits below),
 *     MOEDEC_ERR_DEVICE (the HIP runtime reported a launch error).
 *   - Non-finite values: the router ranks a NaN corrected score (s + bias),
 *     and a NaN group score (+inf and -inf in one group), as -inf, ties going
 *     to the lower index, so every slot still gets a distinct valid expert
 *     (Show HN page, implemented features, router item: the plain reading of
 *     a top-k over such scores).  The routing of every other token, and its
 *     outputs, are unaffected.  A token whose x holds a non-finite value
 *     routes by that rule (its scores are NaN); its h and y rows are
 *     unspecified.  Every call stays memory-safe.
 *   - Limits: 1 <= T <= MOEDEC_MAX_TOKENS; n_experts <= MOEDEC_MAX_EXPERTS;
 *     n_group <= 64; top_k <= 32; n_shared <= 8; hidden and inter must be
 *     multiples of 128/bits (one 16-byte group of codes) and at most 16384.
 */
#ifndef MOEDEC_H
#define MOEDEC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOEDEC_OK 0
#define MOEDEC_ERR_INVALID_ARG 1
#define MOEDEC_ERR_UNSUPPORTED 2
#define MOEDEC_ERR_DEVICE 3

#define MOEDEC_MAX_TOKENS 64
#define MOEDEC_MAX_EXPERTS 1024
#define MOEDEC_MAX_DIM 16384

/* A static, never-NULL description of a status code. */
const char* moedec_status_string(int status);

/* ABI version of this header (bumped on any signature change). */
int moedec_abi_version(void);

/*
 * One layer's experts.  Routed experts are 0..n_experts-1, shared experts
 * n_experts..n_experts+n_shared-1; all have the same shape and bit width.
 *   w_gate, w_up : uint8 [(E+S), inter,  hidden*bits/8]   packed codes
 *   w_down       : uint8 [(E+S), hidden, inter*bits/8]
 *   s_gate, s_up : fp32  [(E+S), inter]   one scale per output row
 *   s_down       : fp32  [(E+S), hidden]
 * Weight of row r, column c = code[r][c] * scale[r].
 */
typedef struct moedec_experts {
    int32_t hidden, inter, n_experts, n_shared, bits;
    const uint8_t* w_gate;
    const uint8_t* w_up;
    const uint8_t* w_down;
    const float* s_gate;
    const float* s_up;
    const float* s_down;
} moedec_experts;

/*
 * The batch union: every expert used by the batch, once, with the
 * (token, slot) assignments routed to it.  Written by moe_route_topk, read by
 * the expert calls.  With K = top_k, S = n_shared and
 * max_active = min(n_experts, T*K) + S:
 *   n_active  : int32 [1]               unique experts, shared ones included
 *   expert_id : int32 [max_active]      ascending; shared expert j is E + j
 *   seg       : int32 [max_active + 1]  assign[seg[i] .. seg[i+1]) belong to expert_id[i]
 *   assign    : int32 [T*(K+S)]         assignment index t*(K+S)+slot, ascending
 *                                       within each expert; slots 0..K-1 are the
 *                                       routed slots of token t, K..K+S-1 its shared slots
 * Only the first n_active (+1 for seg) entries are defined after the call,
 * and the first seg[n_active] of assign (T*(K+S) unless top-p dropped slots,
 * which get no assignment).  While moe_route_topk / moe_route_topp run, the
 * n_active word also counts their per-token selection workgroups (it is
 * zeroed by the call itself and holds the expert count once the call ends).
 */
typedef struct moedec_worklist {
    int32_t* n_active;
    int32_t* expert_id;
    int32_t* seg;
    int32_t* assign;
} moedec_worklist;

/*
 * Router (Show HN page, "implemented features", router item; ideipro.ru: top-8).
 *   x        : fp32 [T, H]   token activations
 *   router_w : fp32 [E, H]   router weight, row e = expert e
 *   bias     : fp32 [E]      noaux_tc correction bias (selection only)
 * Computes s[t][e] = sigmoid(router_w[e] . x[t]) and c = s + bias; keeps the
 * topk_group groups (of n_group contiguous groups of E/n_group experts) with
 * the largest top-2 sums of c; picks the top_k largest c among the kept
 * groups' experts, in descending order (ties: lower index); weights
 * w_k = s_k / (sum over the chosen s, taken in slot order) * routed_scaling_factor.
 * Outputs:
 *   scores   : fp32  [T, E]  the sigmoid scores s (unbiased)
 *   topk_idx : int32 [T, top_k]
 *   topk_w   : fp32  [T, top_k]
 *   wl       : the batch union (may be NULL to skip it); n_shared sets its
 *              shared slots
 * Requires E % n_group == 0, E/n_group >= 2, 1 <= topk_group <= n_group,
 * 1 <= top_k <= topk_group*E/n_group.  H must be a multiple of 4.
 */
int moe_route_topk(const float* x, const float* router_w, const float* bias,
                   int T, int H, int E, int n_group, int topk_group, int top_k,
                   int n_shared, float routed_scaling_factor,
                   float* scores, int32_t* topk_idx, float* topk_w,
                   const moedec_worklist* wl, void* stream);

/*
 * moe_route_topk followed by adaptive expert top-p (Show HN page, section
 * "model download और run": the --topp run option, which reads fewer experts;
 * section "community benchmarks": its measured effect).  The pages give no
 * rule; the one implemented: after the top-k selection, order the top_k
 * chosen experts by unbiased score s (descending; a NaN s last; ties to the
 * lower index), add their s in that order in fp32 and keep the shortest
 * prefix whose sum reaches fp32(top_p * total), total being the slot-order
 * fp32 sum of the top_k scores (at least one expert is kept; top_p >= 1
 * keeps all, exactly as moe_route_topk).  Per token, the kept experts move to
 * the first slots in their slot order (corrected score descending) with
 * weights s_k / (slot-order fp32 sum of the kept s) * routed_scaling_factor;
 * the remaining slots hold index -1 and weight 0 and have no assignment in
 * the worklist, so no expert is read for them.  Arguments and outputs as for
 * moe_route_topk; top_p must not be NaN (MOEDEC_ERR_INVALID_ARG).
 */
int moe_route_topp(const float* x, const float* router_w, const float* bias,
                   int T, int H, int E, int n_group, int topk_group, int top_k,
                   int n_shared, float routed_scaling_factor, float top_p,
                   float* scores, int32_t* topk_idx, float* topk_w,
                   const moedec_worklist* wl, void* stream);

/*
 * Gate/up projections and SwiGLU for every assignment of the batch union
 * (Show HN page, "implemented features": dequant-on-use kernels and the
 * batch-union item).  Each active expert's gate and up codes are read once
 * for all tokens routed to it.
 *   x : fp32 [T, H] (the same activations the router saw)
 *   h : fp32 [T*(top_k+S), inter]; row a = assignment a of the worklist gets
 *       silu(s_gate * (Qg x_t)) * (s_up * (Qu x_t))
 * ex->bits must be 4 (q4), 8 (q8) or 2 (q2) to match the suffix.
 */
int moe_expert_gate_up_silu_q4(const float* x, const moedec_experts* ex, const moedec_worklist* wl,
                               int T, int top_k, float* h, void* stream);
int moe_expert_gate_up_silu_q8(const float* x, const moedec_experts* ex, const moedec_worklist* wl,
                               int T, int top_k, float* h, void* stream);
int moe_expert_gate_up_silu_q2(const float* x, const moedec_experts* ex, const moedec_worklist* wl,
                               int T, int top_k, float* h, void* stream);

/*
 * Down projection and weighted combine (Show HN page, "implemented features":
 * router item, shared expert, routed_scaling_factor already in topk_w).
 *   h      : fp32 [T*(top_k+S), inter]  from the gate/up call
 *   topk_w : fp32 [T, top_k]            from moe_route_topk
 *   y      : fp32 [T, H]; y[t] = sum_k topk_w[t][k] * o(t, k) + sum_j o(t, K+j),
 *            o(t, slot) = s_down * (Qd h[t*(K+S)+slot])
 * Every output row is owned by one workgroup that adds the experts in
 * ascending id order: the result is deterministic (no atomics).
 */
int moe_expert_down_combine_q4(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                               const float* topk_w, int T, int top_k, float* y, void* stream);
int moe_expert_down_combine_q8(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                               const float* topk_w, int T, int top_k, float* y, void* stream);
int moe_expert_down_combine_q2(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                               const float* topk_w, int T, int top_k, float* y, void* stream);

/*
 * moe_expert_down_combine in expert-major order, for larger batches (the
 * same result up to the order of the fp32 sums): each expert's down rows are
 * streamed with only that expert's assignments' h staged (rather than every
 * row range with the whole batch's h), each assignment's partial output is
 * written to part, and a second kernel adds them per token in slot order.
 *   part     : fp32 [T*(top_k+S), hidden] scratch the caller owns (every row
 *              of an assignment is overwritten; nothing is read back later)
 *   topk_idx : int32 [T, top_k] from the router, or NULL when every slot has
 *              an assignment; slots with index -1 (top-p) are skipped
 * Other arguments, layouts and errors as for moe_expert_down_combine_q*.
 */
int moe_expert_down_combine_em_q4(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                  const float* topk_w, const int32_t* topk_idx, int T, int top_k, float* part,
                                  float* y, void* stream);
int moe_expert_down_combine_em_q8(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                  const float* topk_w, const int32_t* topk_idx, int T, int top_k, float* part,
                                  float* y, void* stream);
int moe_expert_down_combine_em_q2(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                  const float* topk_w, const int32_t* topk_idx, int T, int top_k, float* part,
                                  float* y, void* stream);

/*
 * moe_expert_down_combine_em_q4 without the part argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The partial outputs go to a
 * static array of MOEDEC_NOALLOC_PART_FLOATS floats (4 MiB) that the library
 * holds on each GPU it runs on until the process ends; the call allocates
 * nothing.  Every call on one GPU shares that GPU's array, so calls that may
 * overlap on one GPU (other streams, other host threads) race and must be
 * serialised by the caller.  Results are those of
 * moe_expert_down_combine_em_q4 bit for bit.  T*(top_k+S)*hidden >
 * MOEDEC_NOALLOC_PART_FLOATS: MOEDEC_ERR_UNSUPPORTED (use the _em call with
 * a caller buffer).  Other arguments, layouts and errors as for
 * moe_expert_down_combine_em_q4.
 */
#define MOEDEC_NOALLOC_PART_FLOATS (1 << 20)
int moe_expert_down_combine_em_noalloc_q4(const float* h, const moedec_experts* ex, const moedec_worklist* wl,
                                          const float* topk_w, const int32_t* topk_idx, int T, int top_k, float* y,
                                          void* stream);

/*
 * The whole layer step in one launch: moe_route_topk (with the worklist),
 * then the gate/up and down calls, fused (same passages as those three calls;
 * Show HN page, "implemented features").  Arguments and outputs are those of
 * the three calls; E = ex->n_experts, H = ex->hidden, S = ex->n_shared.
 * The experts are streamed one after another (shared experts first), each
 * expert's down rows a few experts after its gate/up rows, and activations
 * meet the codes as exact 24-bit integers under one power-of-two scale per
 * token (and per staged h row), so the products are exact but for that
 * rounding (2^-23 of the column's largest magnitude).
 *   x, router_w, bias          : as for moe_route_topk
 *   scores, topk_idx, topk_w   : as for moe_route_topk
 *   wl                         : required; filled as moe_route_topk fills it
 *   h                          : fp32 [T*(top_k+S), inter] (the gate/up result;
 *                                rows from wl's assignment count on hold
 *                                unspecified values)
 *   y                          : fp32 [T, H] (the layer output)
 *   workspace : int32 [MOEDEC_FUSED_WORKSPACE_INTS], device memory the caller
 *       zeroes once before the first call and then leaves to the library; it
 *       holds the arrival counters of the launch's grid-wide exchanges, so
 *       launches that may run at the same time need separate workspaces, and
 *       one workspace serves one GPU (the plain, top-p and residual calls
 *       count on words 1024 .. 1279, the int8-activation call on words
 *       0 .. 511, so the two kinds may share one).  After the call (once the stream has
 *       reached it) workspace[MOEDEC_FUSED_WS_ERROR] != 0 means a wait timed
 *       out: not every workgroup could be resident at once (the GPU was
 *       shared with other work); that call's outputs are invalid and the
 *       workspace must be zeroed again.  workspace[MOEDEC_FUSED_WS_SPIN] > 0
 *       caps each wait at that many polling rounds (0: about two seconds).
 * The scores may differ from moe_route_topk's in the last bits (another
 * summation order); routing and results are otherwise those of the separate
 * calls given the same scores.  Limits: T <= MOEDEC_FUSED_MAX_TOKENS,
 * n_experts <= MOEDEC_FUSED_MAX_EXPERTS, else MOEDEC_ERR_UNSUPPORTED (use the
 * separate calls).
 */
#define MOEDEC_FUSED_WORKSPACE_INTS 4096
#define MOEDEC_FUSED_WS_ERROR 512
#define MOEDEC_FUSED_WS_SPIN 513
#define MOEDEC_FUSED_MAX_TOKENS 16
#define MOEDEC_FUSED_MAX_EXPERTS 512
int moe_layer_fused_q4(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                       int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                       float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                       float* h, float* y, int32_t* workspace, void* stream);
int moe_layer_fused_q8(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                       int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                       float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                       float* h, float* y, int32_t* workspace, void* stream);
int moe_layer_fused_q2(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                       int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                       float* scores, int32_t* topk_idx, float* topk_w, const moedec_worklist* wl,
                       float* h, float* y, int32_t* workspace, void* stream);

/*
 * The fused layer step with the routing of moe_route_topp (adaptive expert
 * top-p): only the kept experts are streamed.  Arguments as for
 * moe_layer_fused_q*, plus top_p (not NaN; >= 1 is the plain top-k call).
 */
int moe_layer_fused_topp_q4(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                            int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                            float top_p, float* scores, int32_t* topk_idx, float* topk_w,
                            const moedec_worklist* wl, float* h, float* y, int32_t* workspace, void* stream);
int moe_layer_fused_topp_q8(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                            int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                            float top_p, float* scores, int32_t* topk_idx, float* topk_w,
                            const moedec_worklist* wl, float* h, float* y, int32_t* workspace, void* stream);
int moe_layer_fused_topp_q2(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                            int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                            float top_p, float* scores, int32_t* topk_idx, float* topk_w,
                            const moedec_worklist* wl, float* h, float* y, int32_t* workspace, void* stream);

/*
 * The fused layer step with Q8_0-style int8 activations (Show HN page,
 * "implemented features": the integer-dot kernel uses Q8_0-style int8
 * activations).  The activations that meet the weights -- each token's x,
 * and each assignment's h times its routing weight -- are quantised in
 * Q8_0's blocks of 32 consecutive input columns, whatever the weights'
 * width: d = absmax / 127, q = rint(v / d) with ties to even, both in IEEE fp32
 * (a zero block: d = 0; a block with a NaN or an infinity: d = NaN, q = 0).
 * Each block's integer dot products are exact and scaled by d.  The result
 * is the layer with those quantised activations (an approximation of the
 * other calls' result, to the blocks' resolution of 1/254 of their largest
 * value).  Arguments, outputs and limits as for moe_layer_fused_topp_q*;
 * also hidden and inter must be multiples of 32, else
 * MOEDEC_ERR_UNSUPPORTED.
 */
int moe_layer_fused_act8_q4(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                            int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                            float top_p, float* scores, int32_t* topk_idx, float* topk_w,
                            const moedec_worklist* wl, float* h, float* y, int32_t* workspace, void* stream);
int moe_layer_fused_act8_q8(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                            int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                            float top_p, float* scores, int32_t* topk_idx, float* topk_w,
                            const moedec_worklist* wl, float* h, float* y, int32_t* workspace, void* stream);
int moe_layer_fused_act8_q2(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                            int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                            float top_p, float* scores, int32_t* topk_idx, float* topk_w,
                            const moedec_worklist* wl, float* h, float* y, int32_t* workspace, void* stream);

/*
 * One layer of a pre-norm residual stack in one launch: x_out = x +
 * MoE(rmsnorm(x)), rmsnorm(x) = x / sqrt(mean(x^2) + eps) per token,
 * weightless.  The pages describe the MoE layer alone; this form is the
 * reading used to chain layers (as moe_residual_rmsnorm between separate
 * calls), fused so that a stack of layers is one launch per layer.  The norm
 * is computed inside the launch (every workgroup, identically), the router and
 * the experts see the normalised tokens, and the last phase adds x.
 *   x     : fp32 [T, H] the residual stream (not normalised)
 *   x_out : fp32 [T, H] may be x itself (every read of x precedes the first
 *           write of x_out); y still receives MoE(rmsnorm(x))
 *   eps   : >= 0, finite
 * Other arguments, outputs and limits as for moe_layer_fused_topp_q*
 * (top_p >= 1: plain top-k).
 */
int moe_layer_fused_resid_q4(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                             int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                             float top_p, float eps, float* x_out, float* scores, int32_t* topk_idx, float* topk_w,
                             const moedec_worklist* wl, float* h, float* y, int32_t* workspace, void* stream);
int moe_layer_fused_resid_q8(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                             int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                             float top_p, float eps, float* x_out, float* scores, int32_t* topk_idx, float* topk_w,
                             const moedec_worklist* wl, float* h, float* y, int32_t* workspace, void* stream);
int moe_layer_fused_resid_q2(const float* x, const float* router_w, const float* bias, const moedec_experts* ex,
                             int T, int n_group, int topk_group, int top_k, float routed_scaling_factor,
                             float top_p, float eps, float* x_out, float* scores, int32_t* topk_idx, float* topk_w,
                             const moedec_worklist* wl, float* h, float* y, int32_t* workspace, void* stream);

/*
 * Packing of codes (ideipro.ru: packing checked bit for bit; Show HN page,
 * "implemented features": int8, packed int4, packed int2).
 *   codes  : int8  [rows, row_len]                 one code per int8
 *   packed : uint8 [rows, row_len*bits/8]
 * Field j of packed byte k holds column k*(8/bits)+j in bits j*bits ..
 * j*bits+bits-1 (two's complement).  pack keeps the low `bits` bits of each
 * code and does not range-check (codes must lie in [-2^(bits-1), 2^(bits-1)-1]);
 * unpack sign-extends.  row_len must be a multiple of 8/bits.
 */
int moe_pack_q4(const int8_t* codes, uint8_t* packed, int64_t rows, int64_t row_len, void* stream);
int moe_unpack_q4(const uint8_t* packed, int8_t* codes, int64_t rows, int64_t row_len, void* stream);
int moe_pack_q8(const int8_t* codes, uint8_t* packed, int64_t rows, int64_t row_len, void* stream);
int moe_unpack_q8(const uint8_t* packed, int8_t* codes, int64_t rows, int64_t row_len, void* stream);
int moe_pack_q2(const int8_t* codes, uint8_t* packed, int64_t rows, int64_t row_len, void* stream);
int moe_unpack_q2(const uint8_t* packed, int8_t* codes, int64_t rows, int64_t row_len, void* stream);

/*
 * Row quantiser: fp32 weight rows -> codes and one fp32 scale per row (Show
 * HN page, "implemented features": the offline converter requantises the
 * dequantised checkpoint into the engine's container; the quantisation item:
 * int8, packed int4, packed int2 with a scale per row).  The pages state no
 * rule; the one implemented: per row s = absmax / qmax (qmax = 127 / 7 / 1,
 * one IEEE fp32 division), code = rint(w / s) with ties to even (IEEE fp32
 * division) clamped to the field.  A row whose s is 0 (all zeros, or absmax
 * so small that s underflows) gets s = 0 and codes 0; a row holding a NaN or
 * an infinity gets s = NaN and codes 0.  Bit-exact and deterministic.
 *   w      : fp32 [rows, row_len], 16-byte aligned; row_len % 4 == 0
 *   codes  : int8 [rows, row_len] (one code per byte, as moe_pack_* reads),
 *            4-byte aligned                       (moe_quantize_rows_q*)
 *   packed : uint8 [rows, row_len*bits/8] in the moe_pack_* layout; 2-byte
 *            aligned for q4, 4-byte for q8        (moe_quantize_pack_rows_q*)
 *   scales : fp32 [rows], 4-byte aligned
 * rows == 0 is a no-op; row_len == 0 writes scales of 0.  The caller owns
 * every buffer; outputs must not overlap w.  Errors: MOEDEC_ERR_INVALID_ARG
 * for negative sizes, row_len % 4 != 0, null or misaligned pointers;
 * MOEDEC_ERR_UNSUPPORTED for more than 2^31 - 1 rows (one workgroup a row).
 */
int moe_quantize_rows_q8(const float* w, int8_t* codes, float* scales, int64_t rows, int64_t row_len, void* stream);
int moe_quantize_rows_q4(const float* w, int8_t* codes, float* scales, int64_t rows, int64_t row_len, void* stream);
int moe_quantize_rows_q2(const float* w, int8_t* codes, float* scales, int64_t rows, int64_t row_len, void* stream);
int moe_quantize_pack_rows_q8(const float* w, uint8_t* packed, float* scales, int64_t rows, int64_t row_len,
                              void* stream);
int moe_quantize_pack_rows_q4(const float* w, uint8_t* packed, float* scales, int64_t rows, int64_t row_len,
                              void* stream);
int moe_quantize_pack_rows_q2(const float* w, uint8_t* packed, float* scales, int64_t rows, int64_t row_len,
                              void* stream);

/*
 * Between stacked MoE layers: x <- x + y (skipped when y is NULL), then
 * xn <- x / sqrt(mean(x^2) + eps) per token (weightless RMSNorm).  The pages
 * describe the MoE layer only; this pre-norm residual form is the reading
 * used for a stack of layers.
 *   x : fp32 [T, H] (updated in place), y : fp32 [T, H] or NULL, xn : fp32 [T, H]
 */
int moe_residual_rmsnorm(float* x, const float* y, float* xn, int T, int H, float eps,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOEDEC_H */
