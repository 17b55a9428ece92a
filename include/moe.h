/*
 * moe.h -- C ABI of the MI355X (gfx950) DeepSeekMoE layer forward, with the
 * training-side pieces next to it: router affinities, the sequence-wise balance loss
 * and its gradient, the backward of the combine, of the gates and of the SwiGLU
 * activation, the input and weight gradients of the experts, and the backward of the
 * router logits.
 *
 * The layer (DeepSeek-V3 technical report summary "深度解读报告", section 2.2):
 *
 *     out_t = [u_t] + sum_{s < Ns} FFN_{E+s}(u_t) + sum_{k < K} g_tk * FFN_{idx_tk}(u_t)
 *
 * with sigmoid affinities s_te = sigmoid(<u_t, W_r[e]>), a per-expert bias b_e
 * added to the affinity for top-K selection only (section 2.3), selection limited
 * to the M best of G expert groups (section 2.4, "node-limited routing": a
 * group's score is the sum of its group_topn best biased affinities), gates
 * g_tk = s_{t,idx_tk} / sum_j s_{t,idx_tj}, SwiGLU experts
 * FFN(u) = W_down (silu(W_gate u) * (W_up u)), and no token dropping.  The
 * devpress page ("DeepSeek-V3 ... 技术解析"), section 1, fixes 256 routed experts,
 * 1 shared expert and 8 routed experts per token; its section 2 fixes the FP8
 * blocks (128x128 for weights, 1x128 for activations).
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless stated otherwise; `moe_config*` and
 *    `moe_expert_weights*` are HOST structs read during the call only.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every
 *    call only enqueues work on `stream`; none synchronises, allocates device
 *    memory, or keeps a pointer after it returns.  Scratch memory comes from the
 *    caller's workspace `ws` of `ws_bytes` bytes (see moe_workspace_bytes), except
 *    for moe_layer_forward_noalloc (a library-held array, see there).
 *  - The caller owns every buffer.  Outputs are fully overwritten.
 *  - Arguments are validated on the host before anything is launched; on any
 *    error nothing is enqueued.  Return codes only (no global error state);
 *    moe_status_string() names a code.  MOE_ERR_HIP reports a failed launch;
 *    faults inside kernels surface at the caller's next synchronisation.
 *  - Calls are thread-safe (the only global state is a per-device cache of the
 *    CU count and of the no-alloc array's address, stored atomically, and that
 *    array itself).  Results are deterministic: no floating-point
 *    atomics; the router's split-K partials are summed in a fixed order.
 *  - Row-major layouts throughout.  Experts are stacked routed-first: experts
 *    0..E-1 are routed, E..E+Ns-1 are the shared experts.
 *
 * Supported dtype combinations (act_dtype, w_dtype): (F32, F32), (BF16, BF16),
 * (BF16, E4M3), (BF16, E4M3_POW2).  Limits: E <= 256, K <= 8, G <= 64; hidden and
 * inter multiples of 128 for BF16/E4M3 weights, of 4 for F32.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,    /* null pointer, inconsistent sizes            */
  MOE_ERR_UNSUPPORTED = 2,         /* valid but outside this library's limits     */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3, /* ws_bytes < moe_workspace_bytes(cfg)          */
  MOE_ERR_HIP = 4                  /* a HIP launch failed                          */
} moe_status;

/* MOE_E4M3_POW2 (expert weights only): E4M3 with every block scale a power of two
 * (what an 8-bit exponent, E8M0, holds); activations are then quantised with
 * power-of-two scales too, and the expert GEMMs apply both in the matrix cores'
 * block-scaled mode.  A cheaper FP8 variant than the pages' arbitrary fp32 block
 * scales (devpress page, section 2, gives the 128x128 / 1x128 block shapes only):
 * its numerics differ from MOE_E4M3's. */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_E4M3 = 2, MOE_E4M3_POW2 = 3 } moe_dtype;

typedef struct {
  int32_t num_tokens;   /* T >= 1                                                  */
  int32_t hidden;       /* h: width of u and of the layer output                   */
  int32_t inter;        /* SwiGLU intermediate width (routed and shared experts)   */
  int32_t num_experts;  /* E = N_r routed experts, 1..256                          */
  int32_t num_shared;   /* N_s shared experts, >= 0                                */
  int32_t top_k;        /* K = K_r routed experts per token, 1..8, <= M*E/G        */
  int32_t num_groups;   /* G expert groups ("nodes"); E % G == 0; G <= 64          */
  int32_t top_groups;   /* M groups kept per token, 1..G                           */
  int32_t group_topn;   /* biased affinities summed into a group score, 1..E/G     */
  moe_dtype act_dtype;  /* F32 | BF16: u, router weight, y_rows and the output     */
  moe_dtype w_dtype;    /* F32 | BF16 | E4M3 | E4M3_POW2: expert weights           */
} moe_config;

/* Expert weights (device pointers), experts stacked routed-first.
 *   w_gate, w_up : [E+Ns, inter, hidden]     w_down : [E+Ns, hidden, inter]
 * in w_dtype.  For E4M3 (OCP e4m3fn codes, one byte each) every 128x128 block
 * carries one fp32 scale, the weight being code_value * scale:
 *   s_gate, s_up : [E+Ns, inter/128, hidden/128]   s_down : [E+Ns, hidden/128, inter/128]
 * (devpress page, section 2: per-128x128-block weight quantisation).  For E4M3_POW2
 * each scale must be a power of two in [2^-126, 2^127] (only its exponent field is
 * used).  The scale pointers must be NULL unless w_dtype is E4M3 or E4M3_POW2. */
typedef struct {
  const void  *w_gate, *w_up, *w_down;
  const float *s_gate, *s_up, *s_down;
} moe_expert_weights;

/* Bytes of device workspace every entry point below may need for `cfg` (the
 * maximum over them; moe_layer_forward needs the most).  Host-only; 0 when cfg
 * is invalid.  The workspace must be 256-byte aligned; its contents on entry
 * are irrelevant and on return undefined. */
size_t moe_workspace_bytes(const moe_config* cfg);

/* Router ("深度解读报告" sections 2.2-2.4): for every token t
 *   s_e = sigmoid(<x_t, w_router[e]>)            (fp32 accumulation)
 *   sb_e = s_e + bias[e]                          (selection only)
 *   keep the top_groups groups with the largest sum of group_topn best sb
 *   topk_idx[t, :] = the top_k experts by sb within the kept groups,
 *                    ordered by (sb descending, expert index ascending);
 *                    exact ties go to the lower group / expert index
 *   topk_gate[t, k] = s_{idx_k} / sum_j s_{idx_j}
 * x [T, hidden] act_dtype; w_router [E, hidden] act_dtype; bias [E] fp32;
 * topk_idx [T, K] int32 out; topk_gate [T, K] fp32 out. */
moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_gate,
                     void* ws, size_t ws_bytes, void* stream);

/* Permute: groups the T*K (token, expert) pairs by expert, tokens ascending
 * within an expert; no pair is dropped ("深度解读报告" section 2.4).
 * topk_idx [T, K] int32 in, every entry in [0, E) and distinct per token
 * (out-of-range entries give undefined results but stay in bounds);
 * expert_load [E] int32 out: pairs per expert, the batch-wide load of section 2.3;
 * expert_offsets [E+1] int32 out: exclusive prefix sum of expert_load;
 * row_token [T*K] int32 out: token of each expert-sorted row;
 * pair_row [T*K] int32 out: row of pair (t, k), indexed t*K + k.
 * Deterministic and atomic-free. */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, int32_t* expert_load,
                       int32_t* expert_offsets, int32_t* row_token, int32_t* pair_row,
                       void* ws, size_t ws_bytes, void* stream);

/* FP8 activation quantisation (devpress page section 2, 1x128 activation tiles;
 * largest e4m3 value 448 from the stapisi blog section 6.2): for every row r and
 * every 128-column block j of x [rows, cols] (act_dtype BF16, cols % 128 == 0)
 *   scales[r, j] = amax / 448 in fp32 (1 when amax == 0); for w_dtype E4M3_POW2
 *                  the smallest power of two s with amax <= 448 s (1 when amax == 0)
 *   q[r, c]      = e4m3 code of round-to-nearest-even(x[r, c] / scales[r, j]),
 *                  saturated to +-448
 * q [rows, cols] uint8 out; scales [rows, cols/128] fp32 out.  Used inside
 * moe_grouped_ffn for E4M3 weights; exposed for stage testing. */
moe_status moe_act_quant_e4m3(const moe_config* cfg, const void* x, int32_t rows, int32_t cols,
                              uint8_t* q, float* scales, void* stream);

/* Grouped expert FFN ("深度解读报告" section 2.2, SwiGLU experts): for each
 * expert-sorted row r of expert e (rows [expert_offsets[e], expert_offsets[e+1]),
 * token row_token[r]) and for the shared rows (row T*K + s*T + t is token t of
 * shared expert E+s):
 *   y_rows[r] = W_down,e (silu(W_gate,e u) * (W_up,e u)),  u = x[token(r)]
 * x [T, hidden] act_dtype; expert_offsets [E+1], row_token [T*K] as produced by
 * moe_permute; y_rows [T*K + T*Ns, hidden] act_dtype out.  fp32 accumulation;
 * the intermediate h is held in act_dtype (BF16/F32) or, for E4M3 weights,
 * re-quantised per 1x128 block to e4m3, like x. */
moe_status moe_grouped_ffn(const moe_config* cfg, const void* x, const int32_t* expert_offsets,
                           const int32_t* row_token, const moe_expert_weights* weights,
                           void* y_rows, void* ws, size_t ws_bytes, void* stream);

/* Combine ("深度解读报告" section 2.2): for every token t
 *   y[t] = [residual[t]] + sum_s y_rows[T*K + s*T + t] + sum_k topk_gate[t,k] * y_rows[pair_row[t*K+k]]
 * summed in fp32 in that order, rounded once to act_dtype.
 * y_rows [T*K + T*Ns, hidden], residual [T, hidden] (nullable), y [T, hidden]. */
moe_status moe_combine(const moe_config* cfg, const void* y_rows, const int32_t* pair_row,
                       const float* topk_gate, const void* residual, void* y, void* stream);

/* Auxiliary-loss-free bias update ("深度解读报告" section 2.3): at the end of a
 * step, from the whole batch's loads, for every expert e (fp32 arithmetic)
 *   expert_load[e] * E > T*K  (overloaded)   ->  bias[e] -= gamma
 *   expert_load[e] * E < T*K  (underloaded)  ->  bias[e] += gamma
 *   otherwise unchanged.
 * expert_load [E] int32 in; bias [E] fp32 in/out; gamma >= 0 (finite). */
moe_status moe_bias_update(const moe_config* cfg, const int32_t* expert_load, float gamma,
                           float* bias, void* stream);

/* Router affinities ("深度解读报告" section 2.2): for every token t and expert e
 *   scores[t, e] = sigmoid(<x_t, w_router[e]>)     (fp32)
 * bit-identical to the affinities moe_route selects on (same logits, same
 * summation order, same sigmoid).  x [T, hidden] act_dtype; w_router [E, hidden]
 * act_dtype; scores [T, E] fp32 out.  The input of moe_balance_loss. */
moe_status moe_router_scores(const moe_config* cfg, const void* x, const void* w_router,
                             float* scores, void* ws, size_t ws_bytes, void* stream);

/* Sequence-wise balance loss ("深度解读报告" section 2.3: beside the bias rule, a
 * sequence-level balance loss L_Bal with a very small coefficient alpha; section 4.4
 * compares sequence-wise with batch-wise auxiliary losses).  The pages print no
 * formula; this is the usual form.  Tokens [q*seq_len, (q+1)*seq_len) form
 * sequence q; for each q and expert e
 *   s'_{t,e} = scores[t, e] / sum_j scores[t, j]
 *   f_e = E / (K * seq_len) * #{t in q : e in topk_idx[t, :]}
 *   P_e = (1 / seq_len) * sum_{t in q} s'_{t,e}
 *   seq_loss[q] = alpha * sum_e f_e P_e
 * seq_len = T gives the batch-wise variant (the step's batch as one sequence).
 * scores [T, E] fp32 (moe_router_scores); topk_idx [T, K] int32 (moe_route;
 * entries outside [0, E) are not counted); seq_loss [T/seq_len] fp32 out;
 * expert_frac [T/seq_len, E] fp32 out (f; nullable); expert_prob [T/seq_len, E]
 * fp32 out (P; nullable); grad_logits [T, E] fp32 out (nullable): the gradient of
 * sum_q seq_loss[q] with respect to the router logits z (scores = sigmoid(z)) with
 * the selection held fixed (it is piecewise constant in z):
 *   alpha / seq_len * (f_e - sum_i f_i s'_{t,i}) / sum_j scores[t, j]
 *     * scores[t, e] * (1 - scores[t, e]).
 * seq_len >= 1 must divide T; alpha >= 0 and finite.  Every sum runs in a fixed
 * order (deterministic). */
moe_status moe_balance_loss(const moe_config* cfg, const float* scores, const int32_t* topk_idx,
                            int32_t seq_len, float alpha, float* seq_loss, float* expert_frac,
                            float* expert_prob, float* grad_logits, void* ws, size_t ws_bytes,
                            void* stream);

/* Backward of the combine ("深度解读报告" section 2.2, differentiated): for every
 * token t, with Y = y_rows of the forward
 *   dgate[t, k] = <dy[t], Y[pair_row[t*K+k]]>            (fp32, fixed summation order)
 *   dy_rows[pair_row[t*K+k]] = topk_gate[t, k] * dy[t]    (fp32 product, one rounding)
 *   dy_rows[T*K + s*T + t]   = dy[t]                      (each shared expert s)
 * The residual's gradient is dy itself.  dy [T, hidden] act_dtype; y_rows
 * [T*K + T*Ns, hidden] act_dtype; pair_row [T*K] int32 as written by moe_permute
 * (negative entries are skipped); topk_gate [T, K] fp32; dgate [T, K] fp32 out;
 * dy_rows [T*K + T*Ns, hidden] act_dtype out (the gradient of y_rows, same layout). */
moe_status moe_combine_backward(const moe_config* cfg, const void* dy, const void* y_rows,
                                const int32_t* pair_row, const float* topk_gate, float* dgate,
                                void* dy_rows, void* stream);

/* Backward of the gates into the router logits ("深度解读报告" sections 2.2-2.3,
 * differentiated): with the selection held fixed, S = sum_k scores[t, idx_k] and
 * g_k = scores[t, idx_k] / S,
 *   grad_logits[t, idx_j] = (dgate[t, j] - sum_k dgate[t, k] g_k) / S
 *                           * scores[t, idx_j] * (1 - scores[t, idx_j])
 * and 0 for the experts not selected; the selection bias gets no gradient (it only
 * decides the selection).  scores [T, E] fp32 (moe_router_scores); topk_idx [T, K]
 * int32 (entries outside [0, E) take no part); dgate [T, K] fp32
 * (moe_combine_backward); grad_logits [T, E] fp32 out, overwritten, or added to when
 * accumulate != 0 (e.g. onto the balance loss's gradient). */
moe_status moe_gate_backward(const moe_config* cfg, const float* scores, const int32_t* topk_idx,
                             const float* dgate, float* grad_logits, int32_t accumulate,
                             void* stream);

/* Backward of the SwiGLU activation of the experts ("深度解读报告" section 2.2,
 * SwiGLU experts h = silu(a) * b with a = W_gate u and b = W_up u, differentiated):
 * for every element of the [rows, inter] arrays
 *   da = dh * b * silu'(a),  silu'(a) = sigmoid(a) * (1 + a * (1 - sigmoid(a)))
 *   db = dh * silu(a)
 * in fp32, one rounding per output.  a, b, dh [rows, inter] act_dtype in (the gate
 * and up pre-activations and the gradient of h); da, db [rows, inter] act_dtype out.
 * rows >= 1.  The forward does not keep a and b: the caller provides them. */
moe_status moe_swiglu_backward(const moe_config* cfg, const void* a, const void* b,
                               const void* dh, int32_t rows, void* da, void* db, void* stream);

/* Bytes of device workspace moe_expert_backward_input and moe_expert_backward need for
 * `cfg` (row-sized buffers and the weight gradients' packed operands).  Host-only;
 * 0 when cfg is invalid or not supported by the backward (BF16 activations and weights
 * only, and T*(K+Ns)*hidden*2 and T*(K+Ns)*inter*4 bytes each below 2^31 - 2^20). */
size_t moe_backward_workspace_bytes(const moe_config* cfg);

/* Input gradient of the grouped SwiGLU experts ("深度解读报告" section 2.2,
 * differentiated), on the forward's row layout: for every grouped row r of expert e
 * (token t as in moe_grouped_ffn), with u = x[t], a = W_gate,e u, b = W_up,e u,
 *   dh = W_down,e^T dy_rows[r];  (da, db) as in moe_swiglu_backward;
 *   dX[r] = W_gate,e^T da + W_up,e^T db;   dx[t] = sum of dX over the token's rows
 * (its K routed rows through pair_row, then its shared rows).  a and b are recomputed
 * (the forward does not keep them); the pre-activations, dh, da | db and dX are held
 * in bf16; fp32 accumulation; dx rounded once.  x [T, hidden], dy_rows [T*K + T*Ns,
 * hidden] (e.g. from moe_combine_backward), dx [T, hidden] out, all BF16;
 * expert_offsets, row_token, pair_row as written by moe_permute; weights as for
 * moe_grouped_ffn (BF16, no scales), read as stored (no transposed copies).
 * Workspace: moe_backward_workspace_bytes(cfg), 256-byte aligned.  The weight
 * gradients: moe_expert_backward. */
moe_status moe_expert_backward_input(const moe_config* cfg, const void* x,
                                     const int32_t* expert_offsets, const int32_t* row_token,
                                     const int32_t* pair_row, const moe_expert_weights* weights,
                                     const void* dy_rows, void* dx, void* ws, size_t ws_bytes,
                                     void* stream);

/* Bytes of device workspace moe_router_backward needs for `cfg` (its own).  Host-only;
 * 0 when cfg is invalid or not supported (BF16 activations, hidden a multiple of 8, and
 * hidden * T and E * T each below about 2^30, with T and E rounded up as below). */
size_t moe_router_backward_workspace_bytes(const moe_config* cfg);

/* Backward of the router logits z = x w_router^T ("深度解读报告" section 2.2, the
 * affinity logits, differentiated) for a logit gradient grad_logits [T, E] fp32 (the
 * sum of moe_gate_backward's and moe_balance_loss's):
 *   dx[t, c]        = sum_e grad_logits[t, e] * w_router[e, c]     [T, hidden] fp32 out
 *   dw_router[e, c] = sum_t grad_logits[t, e] * x[t, c]            [E, hidden] fp32 out
 * On the matrix cores: grad_logits is split into bf16 hi = bf16(g) and lo = bf16(g - hi)
 * (g = hi + lo within 2^-17 |g|), each multiplied exactly by the bf16 operands, fp32
 * accumulation; dw_router sums split-K partials over token ranges in a fixed order
 * (deterministic).  Either output may be NULL, not both.  x [T, hidden] and w_router
 * [E, hidden] BF16.  Workspace: moe_router_backward_workspace_bytes(cfg), 256-byte
 * aligned (about 2 (T + E) hidden + 16 E T + 32 E hidden bytes with E rounded up to 64
 * and T to 128). */
moe_status moe_router_backward(const moe_config* cfg, const void* x, const void* w_router,
                               const float* grad_logits, float* dx, float* dw_router, void* ws,
                               size_t ws_bytes, void* stream);

/* Input and weight gradients of the grouped SwiGLU experts together
 * ("深度解读报告" section 2.2, differentiated): dx as in moe_expert_backward_input
 * (nullable here), and, when dw_gate, dw_up and dw_down are all given (all or none),
 * for every expert e over its rows r (u = x[token of r], h = silu(a) * b)
 *   dw_down[e] = sum_r dy_rows[r]^T h_r       [E+Ns, hidden, inter] fp32 out
 *   dw_gate[e] = sum_r da_r^T u_r             [E+Ns, inter, hidden] fp32 out
 *   dw_up[e]   = sum_r db_r^T u_r             [E+Ns, inter, hidden] fp32 out
 * with a, b recomputed and (da, db) as in moe_swiglu_backward, summed in fp32 in row
 * order (deterministic); experts without rows get zeros.  At least one of dx and the
 * weight gradients must be requested.  Other arguments and the workspace as for
 * moe_expert_backward_input. */
moe_status moe_expert_backward(const moe_config* cfg, const void* x,
                               const int32_t* expert_offsets, const int32_t* row_token,
                               const int32_t* pair_row, const moe_expert_weights* weights,
                               const void* dy_rows, void* dx, float* dw_gate, float* dw_up,
                               float* dw_down, void* ws, size_t ws_bytes, void* stream);

/* The whole layer: moe_route, moe_permute, moe_grouped_ffn and moe_combine
 * enqueued back to back on `stream` with no host synchronisation in between.
 * residual (nullable) is u of "out = u + ..." in section 2.2; NULL gives the MoE
 * branch alone.  topk_idx [T, K], topk_gate [T, K] and expert_load [E] are
 * written as by the stage calls (expert_load feeds moe_bias_update). */
moe_status moe_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                             const float* bias, const moe_expert_weights* weights,
                             const void* residual, void* y, int32_t* topk_idx,
                             float* topk_gate, int32_t* expert_load,
                             void* ws, size_t ws_bytes, void* stream);

/* moe_layer_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels, with the workspace taken from a 64 MiB array that the library holds on
 * each device it runs on, from its load until the process ends.  Accepts exactly the
 * configurations with moe_workspace_bytes(cfg) <= 64 MiB (at hidden 7168, inter
 * 2048, E 256, K 8, one shared expert: up to 365 tokens in BF16, 316 with E4M3
 * weights) and returns MOE_ERR_UNSUPPORTED for larger ones, before anything is
 * enqueued.  Allocates nothing: no hipMalloc, hipFree or allocating library call;
 * the first call on a device looks the array's address up (hipGetSymbolAddress) and
 * caches it.  Every call on a device shares that device's array (its contents on
 * entry are irrelevant: nothing in it needs clearing), so calls that overlap on one
 * device -- concurrent streams or threads -- race and must be serialised by the
 * caller.  Arguments and outputs as for moe_layer_forward. */
moe_status moe_layer_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                                     const float* bias, const moe_expert_weights* weights,
                                     const void* residual, void* y, int32_t* topk_idx,
                                     float* topk_gate, int32_t* expert_load, void* stream);

/* Static string naming a status code ("unknown status" for other values). */
const char* moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
