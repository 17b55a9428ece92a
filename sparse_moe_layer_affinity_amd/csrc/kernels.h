// Internal launchers of the MoE layer kernels (not part of the C ABI).
#pragma once

#include "common.h"

namespace moe {

// Workspace carved out of the caller's buffer (all pieces 256-byte aligned).
struct Workspace {
  float* z;            // [splits, T, E] router logit partials, fp32
  uint64_t* masks;     // [chunks, E] per-64-token-chunk bitmask of the tokens choosing e
  int32_t* base;       // [chunks, E] rows of expert e in earlier chunks
  int32_t* offsets;    // [E+1] expert offsets (layer forward)
  int32_t* row_token;  // [T*K]
  int32_t* pair_row;   // [T*K]
  int32_t* sched_n;    // [1] row blocks of the expert GEMMs
  int4* sched;         // [row-block bound] {group, first row, rows}, largest first
  void* h;             // [rows, inter] act dtype (SwiGLU output of the first GEMM)
  uint8_t* hq;         // [rows, inter] e4m3 codes of h (e4m3 weights)
  float* h_scales;     // [inter/128, rows] (e4m3 weights; transposed)
  uint8_t* xq;         // [T, hidden] e4m3 codes
  float* x_scales;     // [hidden/128, T] (transposed)
  float* xg_scales;    // [hidden/128, rows] x_scales in grouped-row order
  void* y_rows;        // [rows, hidden] act dtype (layer forward)
  float* bal_p;        // [chunks <= T, E] balance loss: partial sums of s' per chunk
  int32_t* bal_c;      // [chunks <= T, E] balance loss: selections per chunk
  float* bal_f;        // [sequences <= T, E] balance loss: f when the caller keeps none
  size_t bytes;        // total bytes of the layout
};

// Transposed, padded operands of the MFMA weight gradients (see wgrad.hip):
// [features][packed rows], every expert's rows padded to a multiple of 64
struct WgradPackWorkspace {
  int32_t* poff;       // [E+Ns+1] padded row offsets
  uint16_t* xt;        // [hidden][packed rows]  u^T (x gathered by row)
  uint16_t* dyt;       // [hidden][packed rows]  dy^T
  uint16_t* dabt;      // [2*inter][packed rows] [da | db]^T
  uint16_t* ht;        // [inter][packed rows]   h^T
};
long long wgrad_packed_rows(const moe_config& c);

// Scratch of the expert backward (its own workspace: row-sized buffers and the packed
// operands of the weight gradients)
struct BackwardWorkspace {
  int32_t* sched_n;    // [1] row blocks of the grouped GEMMs
  int4* sched;         // row blocks {group, first row, rows}, largest first
  float* ones;         // [T*K] unit gates for the final row sum
  uint16_t* ab;        // [rows, 2*inter] recomputed gate | up pre-activations
  uint16_t* dh;        // [rows, inter] gradient of h
  uint16_t* dab;       // [rows, 2*inter] their gradients
  uint16_t* dx_rows;   // [rows, hidden] input gradient of every grouped row
  WgradPackWorkspace pack;  // operands of the weight gradients
  size_t bytes;
};
BackwardWorkspace backward_workspace_layout(const moe_config& c, void* base);

// E4M3 expert weights, with fp32 or power-of-two block scales
inline bool is_fp8(moe_dtype d) { return d == MOE_E4M3 || d == MOE_E4M3_POW2; }

constexpr int kTokChunk = 64;   // tokens per permute chunk (one 64-bit mask)
constexpr int kExpertBM = 320;  // rows per row block of the bf16 expert GEMMs
constexpr int kFp8BT = 320;     // rows per row block of the power-of-two FP8 expert GEMMs (<= kExpertBM)
constexpr int kFp8BT32 = 256;   // rows per row block of the fp32-scale FP8 expert GEMMs

// Upper bound on the row blocks (m-tiles of bm rows) over all groups: every routed
// expert may end in a partial block, the shared experts have T rows each.
inline int expert_row_blocks_upper(const moe_config& c, int bm) {
  const long long TK = 1LL * c.num_tokens * c.top_k;
  long long routed = (TK + 1LL * c.num_experts * (bm - 1)) / bm;
  routed = routed < TK ? routed : TK;
  return int(routed + 1LL * c.num_shared * ((c.num_tokens + bm - 1) / bm));
}
Workspace workspace_layout(const moe_config& c, void* base);

// Split-K factor of the bf16 router-logits GEMM: enough row blocks (kExpertBM rows) x
// splits to fill the chip at small T, each split an even number (at least 8, unless K
// is shorter; never 2 unless K is 128) of 64-wide K stages;
// the fp32 partials are summed in order by the selection kernel.  1 for fp32
// activations.
inline int router_k_chunk(const moe_config& c) {
  const int stages = c.hidden / 64;                       // even: hidden % 128 == 0
  const int blocks = (c.num_tokens + kExpertBM - 1) / kExpertBM;
  int s = 256 / blocks;
  s = s < 1 ? 1 : s;
  int chunk = (stages + s - 1) / s;
  chunk = chunk < 8 ? 8 : chunk;                          // >= 8 stages: fixed costs amortised
  chunk = chunk > stages ? stages : chunk;
  chunk += chunk & 1;                                     // even stage count
  while (stages % chunk == 2) chunk += 2;                 // no two-stage last split
  return chunk * 64;
}
inline int router_splits(const moe_config& c) {
  if (c.act_dtype == MOE_F32) return 1;
  const int chunk = router_k_chunk(c);
  return (c.hidden + chunk - 1) / chunk;
}

hipError_t launch_router_logits(const moe_config& c, const void* x, const void* w, float* z,
                                hipStream_t s);
hipError_t launch_router_select(const moe_config& c, const float* z, const float* bias,
                                int32_t* idx, float* gate, hipStream_t s);
hipError_t launch_permute(const moe_config& c, const int32_t* idx, int32_t* load,
                          int32_t* offsets, int32_t* row_token, int32_t* pair_row,
                          const Workspace& ws, hipStream_t s);
hipError_t launch_router_scores(const moe_config& c, const float* z, float* scores,
                                hipStream_t s);
hipError_t launch_balance_loss(const moe_config& c, const float* scores, const int32_t* idx,
                               int seq_len, float alpha, float* loss, float* frac, float* prob,
                               float* grad, const Workspace& w, hipStream_t s);
hipError_t launch_combine_backward(const moe_config& c, const void* dy, const void* y_rows,
                                   const int32_t* pair_row, const float* gate, float* dgate,
                                   void* dy_rows, hipStream_t s);
hipError_t launch_swiglu_backward(const moe_config& c, const void* a, const void* b,
                                  const void* dh, int rows, void* da, void* db, hipStream_t s);
hipError_t launch_expert_backward(const moe_config& c, const void* x, const int32_t* offsets,
                                  const int32_t* row_token, const int32_t* pair_row,
                                  const moe_expert_weights& wt, const void* dy_rows, void* dx,
                                  float* dw_gate, float* dw_up, float* dw_down,
                                  const BackwardWorkspace& ws, hipStream_t s);
hipError_t launch_expert_wgrad_mfma(const moe_config& c, const void* x, const int32_t* offsets,
                                    const int32_t* row_token, const void* dy_rows,
                                    const uint16_t* ab, const uint16_t* dab, float* dw_gate,
                                    float* dw_up, float* dw_down, const WgradPackWorkspace& ws,
                                    hipStream_t s);
// Scratch of the router backward (its own workspace): the logit gradient split in
// bf16 hi and lo parts in both layouts, W_r^T twice side by side, x^T, and the split-K
// partials of dW_r.  Ep = E rounded up to 64, Tp = T rounded up to 128 (at least 256).
struct RouterBwdWorkspace {
  uint16_t* dzs;   // [T][2 Ep]   hi | lo
  uint16_t* dzt;   // [2 Ep][Tp]  hi rows, then lo rows
  uint16_t* wt2;   // [H][2 Ep]   W_r^T | W_r^T
  uint16_t* xt;    // [H][Tp]     x^T
  float* part;     // [S][2 Ep][H]
  int Ep, Tp, S, kc;   // kc: tokens per split
  size_t bytes;
};
RouterBwdWorkspace router_bwd_workspace_layout(const moe_config& c, void* base);
hipError_t launch_router_backward(const moe_config& c, const void* x, const void* w_router,
                                  const float* dz, float* dx, float* dw,
                                  const RouterBwdWorkspace& ws, hipStream_t st);
hipError_t launch_gate_backward(const moe_config& c, const float* scores, const int32_t* idx,
                                const float* dgate, float* grad, int accumulate, hipStream_t s);
hipError_t launch_act_quant(const void* x, int rows, int cols, uint8_t* q, float* scales,
                            hipStream_t s, bool transposed = false, bool pow2 = false);
hipError_t launch_grouped_ffn(const moe_config& c, const void* x, const int32_t* offsets,
                              const int32_t* row_token, const moe_expert_weights& w,
                              void* y_rows, const Workspace& ws, hipStream_t s);
hipError_t launch_grouped_ffn_fp8(const moe_config& c, const void* x, const int32_t* offsets,
                                  const int32_t* row_token, const moe_expert_weights& w,
                                  void* y_rows, const Workspace& ws, hipStream_t s);
hipError_t launch_gather_scales(const moe_config& c, const float* scales, const int32_t* row_token,
                                int kblocks, float* out, hipStream_t s);
hipError_t launch_combine(const moe_config& c, const void* y_rows, const int32_t* pair_row,
                          const float* gate, const void* residual, void* y, hipStream_t s);
hipError_t launch_bias_update(const moe_config& c, const int32_t* load, float gamma,
                              float* bias, hipStream_t s);

}  // namespace moe
