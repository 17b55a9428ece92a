// C ABI of the MoE layer library: host-side validation, workspace layout, and the
// launch sequences.  Every check runs before anything is enqueued.
#include <math.h>

#include <atomic>

#include "kernels.h"

namespace moe {

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

static size_t act_bytes(const moe_config& c) { return c.act_dtype == MOE_F32 ? 4 : 2; }

Workspace workspace_layout(const moe_config& c, void* base) {
  const size_t T = c.num_tokens, E = c.num_experts, K = c.top_k, Ns = c.num_shared;
  const size_t H = c.hidden, I = c.inter;
  const size_t TK = T * K, rows = TK + T * Ns;
  const size_t chunks = (T + kTokChunk - 1) / kTokChunk;
  const bool fp8 = is_fp8(c.w_dtype);
  Workspace w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  w.z = static_cast<float*>(take(size_t(router_splits(c)) * T * E * 4));
  w.masks = static_cast<uint64_t*>(take(chunks * E * 8));
  w.base = static_cast<int32_t*>(take(chunks * E * 4));
  w.offsets = static_cast<int32_t*>(take((E + 1) * 4));
  w.row_token = static_cast<int32_t*>(take(TK * 4));
  w.pair_row = static_cast<int32_t*>(take(TK * 4));
  w.sched_n = static_cast<int32_t*>(take(4));
  // room for the smallest row blocks any expert GEMM schedules (256 rows)
  w.sched = static_cast<int4*>(take(size_t(expert_row_blocks_upper(c, kFp8BT32)) * 16));
  w.h = take(rows * I * act_bytes(c));
  w.hq = fp8 ? static_cast<uint8_t*>(take(rows * I)) : nullptr;
  w.h_scales = fp8 ? static_cast<float*>(take(rows * (I / 128) * 4)) : nullptr;
  w.xq = fp8 ? static_cast<uint8_t*>(take(T * H)) : nullptr;
  w.x_scales = fp8 ? static_cast<float*>(take(T * (H / 128) * 4)) : nullptr;
  w.xg_scales = fp8 ? static_cast<float*>(take(rows * (H / 128) * 4)) : nullptr;
  w.y_rows = take(rows * H * act_bytes(c));
  w.bal_p = static_cast<float*>(take(T * E * 4));
  w.bal_c = static_cast<int32_t*>(take(T * E * 4));
  w.bal_f = static_cast<float*>(take(T * E * 4));
  w.bytes = off;
  return w;
}

BackwardWorkspace backward_workspace_layout(const moe_config& c, void* base) {
  const size_t T = c.num_tokens, K = c.top_k, Ns = c.num_shared, E = c.num_experts;
  const size_t H = c.hidden, I = c.inter;
  const size_t rows = T * K + T * Ns, G = E + Ns;
  BackwardWorkspace w{};
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + off : nullptr;
    off += align256(bytes);
    return r;
  };
  w.sched_n = static_cast<int32_t*>(take(4));
  w.sched = static_cast<int4*>(take(size_t(expert_row_blocks_upper(c, kExpertBM)) * 16));
  w.ones = static_cast<float*>(take(T * K * 4));
  w.ab = static_cast<uint16_t*>(take(rows * 2 * I * 2));
  w.dh = static_cast<uint16_t*>(take(rows * I * 2));
  w.dab = static_cast<uint16_t*>(take(rows * 2 * I * 2));
  w.dx_rows = static_cast<uint16_t*>(take(rows * H * 2));
  const size_t packed = size_t(wgrad_packed_rows(c));
  w.pack.poff = static_cast<int32_t*>(take((G + 1) * 4));
  w.pack.xt = static_cast<uint16_t*>(take(H * packed * 2));
  w.pack.dyt = static_cast<uint16_t*>(take(H * packed * 2));
  w.pack.dabt = static_cast<uint16_t*>(take(2 * I * packed * 2));
  w.pack.ht = static_cast<uint16_t*>(take(I * packed * 2));
  w.bytes = off;
  return w;
}

static bool valid_dtype(moe_dtype d) {
  return d == MOE_F32 || d == MOE_BF16 || d == MOE_E4M3 || d == MOE_E4M3_POW2;
}

static moe_status validate(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_tokens < 1 || c->hidden < 1 || c->inter < 1 || c->num_experts < 1 ||
      c->num_shared < 0 || c->top_k < 1 || c->num_groups < 1)
    return MOE_ERR_INVALID_ARGUMENT;
  if (!valid_dtype(c->act_dtype) || !valid_dtype(c->w_dtype)) return MOE_ERR_INVALID_ARGUMENT;
  if (c->num_experts % c->num_groups != 0) return MOE_ERR_INVALID_ARGUMENT;
  const int per_group = c->num_experts / c->num_groups;
  if (c->top_groups < 1 || c->top_groups > c->num_groups) return MOE_ERR_INVALID_ARGUMENT;
  if (c->top_k > c->top_groups * per_group) return MOE_ERR_INVALID_ARGUMENT;
  if (c->group_topn < 1 || c->group_topn > per_group) return MOE_ERR_INVALID_ARGUMENT;
  // limits of this implementation
  if (c->num_experts > 256 || c->top_k > 8 || c->num_groups > 64 || c->group_topn > 8 ||
      c->num_shared > 64)
    return MOE_ERR_UNSUPPORTED;
  const bool f32 = c->act_dtype == MOE_F32 && c->w_dtype == MOE_F32;
  const bool bf16 = c->act_dtype == MOE_BF16 && c->w_dtype == MOE_BF16;
  const bool fp8 = c->act_dtype == MOE_BF16 && is_fp8(c->w_dtype);
  if (!(f32 || bf16 || fp8)) return MOE_ERR_UNSUPPORTED;
  if (f32 && (c->hidden % 4 || c->inter % 4)) return MOE_ERR_UNSUPPORTED;
  if (!f32 && (c->hidden % 128 || c->inter % 128)) return MOE_ERR_UNSUPPORTED;
  const long long rows = 1LL * c->num_tokens * (c->top_k + c->num_shared);
  if (rows >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  const long long widest = c->hidden > c->inter ? c->hidden : c->inter;
  if (f32 && rows * widest >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  if (1LL * c->num_tokens * c->num_experts >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;
  // MFMA kernels address x, h and each expert matrix through 32-bit buffer offsets
  // below 2^31 (2^31 itself marks rows to read as zero)
  const long long lim = (1LL << 31) - (1LL << 20);
  if (!f32 && (2LL * c->num_tokens * c->hidden > lim || 2LL * rows * c->inter > lim ||
               2LL * c->hidden * c->inter > lim))
    return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static moe_status check_ws(const moe_config& c, const void* ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_INVALID_ARGUMENT;
  if (reinterpret_cast<uintptr_t>(ws) % 256) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < workspace_layout(c, nullptr).bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return MOE_OK;
}

static moe_status check_weights(const moe_config& c, const moe_expert_weights* w) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_INVALID_ARGUMENT;
  const bool fp8 = is_fp8(c.w_dtype);
  const bool have = w->s_gate && w->s_up && w->s_down;
  const bool none = !w->s_gate && !w->s_up && !w->s_down;
  if (fp8 ? !have : !none) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

static moe_status from_hip(hipError_t e) {
  if (e == hipSuccess) return MOE_OK;
  if (e == hipErrorNotSupported) return MOE_ERR_UNSUPPORTED;
  return MOE_ERR_HIP;
}

// Workspace of moe_layer_forward_noalloc: one array per device, resident from the
// library's load until the process ends, shared by every such call on that device.
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

// Device address of this device's `scratch`, looked up once per device (with that
// device current) and cached; the array's name in host code is only a stand-in for
// the symbol.  nullptr if the lookup fails.
static void* noalloc_scratch() {
  static std::atomic<void*> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  void* p = cached[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
  cached[dev].store(p, std::memory_order_release);
  return p;
}

#define MOE_TRY(expr)                      \
  do {                                     \
    moe_status st_ = (expr);               \
    if (st_ != MOE_OK) return st_;         \
  } while (0)

}  // namespace moe

using namespace moe;

extern "C" {

size_t moe_workspace_bytes(const moe_config* cfg) {
  if (validate(cfg) != MOE_OK) return 0;
  return workspace_layout(*cfg, nullptr).bytes;
}

moe_status moe_route(const moe_config* cfg, const void* x, const void* w_router,
                     const float* bias, int32_t* topk_idx, float* topk_gate, void* ws,
                     size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  if (!x || !w_router || !bias || !topk_idx || !topk_gate) return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_ws(*cfg, ws, ws_bytes));
  const Workspace w = workspace_layout(*cfg, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(from_hip(launch_router_logits(*cfg, x, w_router, w.z, s)));
  return from_hip(launch_router_select(*cfg, w.z, bias, topk_idx, topk_gate, s));
}

moe_status moe_router_scores(const moe_config* cfg, const void* x, const void* w_router,
                             float* scores, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  if (!x || !w_router || !scores) return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_ws(*cfg, ws, ws_bytes));
  const Workspace w = workspace_layout(*cfg, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(from_hip(launch_router_logits(*cfg, x, w_router, w.z, s)));
  return from_hip(launch_router_scores(*cfg, w.z, scores, s));
}

moe_status moe_balance_loss(const moe_config* cfg, const float* scores, const int32_t* topk_idx,
                            int32_t seq_len, float alpha, float* seq_loss, float* expert_frac,
                            float* expert_prob, float* grad_logits, void* ws, size_t ws_bytes,
                            void* stream) {
  MOE_TRY(validate(cfg));
  if (!scores || !topk_idx || !seq_loss) return MOE_ERR_INVALID_ARGUMENT;
  if (seq_len < 1 || cfg->num_tokens % seq_len != 0) return MOE_ERR_INVALID_ARGUMENT;
  if (!(alpha >= 0.0f) || isinf(alpha)) return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_ws(*cfg, ws, ws_bytes));
  const Workspace w = workspace_layout(*cfg, ws);
  return from_hip(launch_balance_loss(*cfg, scores, topk_idx, seq_len, alpha, seq_loss,
                                      expert_frac, expert_prob, grad_logits, w,
                                      static_cast<hipStream_t>(stream)));
}

moe_status moe_combine_backward(const moe_config* cfg, const void* dy, const void* y_rows,
                                const int32_t* pair_row, const float* topk_gate, float* dgate,
                                void* dy_rows, void* stream) {
  MOE_TRY(validate(cfg));
  if (!dy || !y_rows || !pair_row || !topk_gate || !dgate || !dy_rows)
    return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_combine_backward(*cfg, dy, y_rows, pair_row, topk_gate, dgate, dy_rows,
                                          static_cast<hipStream_t>(stream)));
}

// The expert backward: bf16 activations and weights; dy_rows and the [rows, 2*inter]
// intermediates are GEMM operands addressed through 32-bit buffer offsets.
static moe_status validate_backward(const moe_config* c) {
  MOE_TRY(validate(c));
  if (c->act_dtype != MOE_BF16 || c->w_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  const long long rows = 1LL * c->num_tokens * (c->top_k + c->num_shared);
  const long long lim = (1LL << 31) - (1LL << 20);
  if (2LL * rows * c->hidden > lim || 4LL * rows * c->inter > lim) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_backward_workspace_bytes(const moe_config* cfg) {
  if (validate_backward(cfg) != MOE_OK) return 0;
  return backward_workspace_layout(*cfg, nullptr).bytes;
}

moe_status moe_expert_backward(const moe_config* cfg, const void* x,
                               const int32_t* expert_offsets, const int32_t* row_token,
                               const int32_t* pair_row, const moe_expert_weights* weights,
                               const void* dy_rows, void* dx, float* dw_gate, float* dw_up,
                               float* dw_down, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate_backward(cfg));
  if (!x || !expert_offsets || !row_token || !pair_row || !dy_rows)
    return MOE_ERR_INVALID_ARGUMENT;
  const bool dw_all = dw_gate && dw_up && dw_down, dw_none = !dw_gate && !dw_up && !dw_down;
  if (!(dw_all || dw_none) || (!dx && dw_none)) return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_weights(*cfg, weights));
  if (!ws || reinterpret_cast<uintptr_t>(ws) % 256) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < backward_workspace_layout(*cfg, nullptr).bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const BackwardWorkspace w = backward_workspace_layout(*cfg, ws);
  return from_hip(launch_expert_backward(*cfg, x, expert_offsets, row_token, pair_row, *weights,
                                         dy_rows, dx, dw_gate, dw_up, dw_down, w,
                                         static_cast<hipStream_t>(stream)));
}

moe_status moe_expert_backward_input(const moe_config* cfg, const void* x,
                                     const int32_t* expert_offsets, const int32_t* row_token,
                                     const int32_t* pair_row, const moe_expert_weights* weights,
                                     const void* dy_rows, void* dx, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (!dx) return MOE_ERR_INVALID_ARGUMENT;
  return moe_expert_backward(cfg, x, expert_offsets, row_token, pair_row, weights, dy_rows, dx,
                             nullptr, nullptr, nullptr, ws, ws_bytes, stream);
}

static moe_status validate_router_backward(const moe_config* c) {
  MOE_TRY(validate(c));
  if (c->act_dtype != MOE_BF16 || c->hidden % 8) return MOE_ERR_UNSUPPORTED;
  const RouterBwdWorkspace w = router_bwd_workspace_layout(*c, nullptr);
  const long long lim = (1LL << 31) - (1LL << 20);
  if (2LL * c->hidden * w.Tp > lim || 4LL * w.Ep * w.Tp > lim) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

size_t moe_router_backward_workspace_bytes(const moe_config* cfg) {
  if (validate_router_backward(cfg) != MOE_OK) return 0;
  return router_bwd_workspace_layout(*cfg, nullptr).bytes;
}

moe_status moe_router_backward(const moe_config* cfg, const void* x, const void* w_router,
                               const float* grad_logits, float* dx, float* dw_router, void* ws,
                               size_t ws_bytes, void* stream) {
  MOE_TRY(validate_router_backward(cfg));
  if (!x || !w_router || !grad_logits || (!dx && !dw_router)) return MOE_ERR_INVALID_ARGUMENT;
  if (!ws || reinterpret_cast<uintptr_t>(ws) % 256) return MOE_ERR_INVALID_ARGUMENT;
  if (ws_bytes < router_bwd_workspace_layout(*cfg, nullptr).bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  const RouterBwdWorkspace w = router_bwd_workspace_layout(*cfg, ws);
  return from_hip(launch_router_backward(*cfg, x, w_router, grad_logits, dx, dw_router, w,
                                         static_cast<hipStream_t>(stream)));
}

moe_status moe_swiglu_backward(const moe_config* cfg, const void* a, const void* b,
                               const void* dh, int32_t rows, void* da, void* db, void* stream) {
  MOE_TRY(validate(cfg));
  if (!a || !b || !dh || !da || !db || rows < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (1LL * rows * cfg->inter >= (1LL << 40)) return MOE_ERR_UNSUPPORTED;
  return from_hip(launch_swiglu_backward(*cfg, a, b, dh, rows, da, db,
                                         static_cast<hipStream_t>(stream)));
}

moe_status moe_gate_backward(const moe_config* cfg, const float* scores, const int32_t* topk_idx,
                             const float* dgate, float* grad_logits, int32_t accumulate,
                             void* stream) {
  MOE_TRY(validate(cfg));
  if (!scores || !topk_idx || !dgate || !grad_logits) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_gate_backward(*cfg, scores, topk_idx, dgate, grad_logits, accumulate != 0,
                                       static_cast<hipStream_t>(stream)));
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, int32_t* expert_load,
                       int32_t* expert_offsets, int32_t* row_token, int32_t* pair_row, void* ws,
                       size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  if (!topk_idx || !expert_load || !expert_offsets || !row_token || !pair_row)
    return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_ws(*cfg, ws, ws_bytes));
  const Workspace w = workspace_layout(*cfg, ws);
  return from_hip(launch_permute(*cfg, topk_idx, expert_load, expert_offsets, row_token,
                                 pair_row, w, static_cast<hipStream_t>(stream)));
}

moe_status moe_act_quant_e4m3(const moe_config* cfg, const void* x, int32_t rows, int32_t cols,
                              uint8_t* q, float* scales, void* stream) {
  MOE_TRY(validate(cfg));
  if (cfg->act_dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!x || !q || !scales || rows < 1 || cols < 128 || cols % 128)
    return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_act_quant(x, rows, cols, q, scales, static_cast<hipStream_t>(stream), false,
                                   cfg->w_dtype == MOE_E4M3_POW2));
}

moe_status moe_grouped_ffn(const moe_config* cfg, const void* x, const int32_t* expert_offsets,
                           const int32_t* row_token, const moe_expert_weights* weights,
                           void* y_rows, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(validate(cfg));
  if (!x || !expert_offsets || !row_token || !y_rows) return MOE_ERR_INVALID_ARGUMENT;
  MOE_TRY(check_weights(*cfg, weights));
  MOE_TRY(check_ws(*cfg, ws, ws_bytes));
  const Workspace w = workspace_layout(*cfg, ws);
  return from_hip(launch_grouped_ffn(*cfg, x, expert_offsets, row_token, *weights, y_rows, w,
                                     static_cast<hipStream_t>(stream)));
}

moe_status moe_combine(const moe_config* cfg, const void* y_rows, const int32_t* pair_row,
                       const float* topk_gate, const void* residual, void* y, void* stream) {
  MOE_TRY(validate(cfg));
  if (!y_rows || !pair_row || !topk_gate || !y) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_combine(*cfg, y_rows, pair_row, topk_gate, residual, y,
                                 static_cast<hipStream_t>(stream)));
}

moe_status moe_bias_update(const moe_config* cfg, const int32_t* expert_load, float gamma,
                           float* bias, void* stream) {
  MOE_TRY(validate(cfg));
  if (!expert_load || !bias || !(gamma >= 0.0f) || isinf(gamma)) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_bias_update(*cfg, expert_load, gamma, bias,
                                     static_cast<hipStream_t>(stream)));
}

static moe_status check_layer_args(const moe_config* cfg, const void* x, const void* w_router,
                                   const float* bias, const moe_expert_weights* weights,
                                   const void* y, const int32_t* topk_idx,
                                   const float* topk_gate, const int32_t* expert_load) {
  MOE_TRY(validate(cfg));
  if (!x || !w_router || !bias || !y || !topk_idx || !topk_gate || !expert_load)
    return MOE_ERR_INVALID_ARGUMENT;
  return check_weights(*cfg, weights);
}

moe_status moe_layer_forward(const moe_config* cfg, const void* x, const void* w_router,
                             const float* bias, const moe_expert_weights* weights,
                             const void* residual, void* y, int32_t* topk_idx, float* topk_gate,
                             int32_t* expert_load, void* ws, size_t ws_bytes, void* stream) {
  MOE_TRY(check_layer_args(cfg, x, w_router, bias, weights, y, topk_idx, topk_gate, expert_load));
  MOE_TRY(check_ws(*cfg, ws, ws_bytes));
  const Workspace w = workspace_layout(*cfg, ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  MOE_TRY(from_hip(launch_router_logits(*cfg, x, w_router, w.z, s)));
  MOE_TRY(from_hip(launch_router_select(*cfg, w.z, bias, topk_idx, topk_gate, s)));
  MOE_TRY(from_hip(launch_permute(*cfg, topk_idx, expert_load, w.offsets, w.row_token,
                                  w.pair_row, w, s)));
  MOE_TRY(from_hip(launch_grouped_ffn(*cfg, x, w.offsets, w.row_token, *weights, w.y_rows, w, s)));
  return from_hip(launch_combine(*cfg, w.y_rows, w.pair_row, topk_gate, residual, y, s));
}

moe_status moe_layer_forward_noalloc(const moe_config* cfg, const void* x, const void* w_router,
                                     const float* bias, const moe_expert_weights* weights,
                                     const void* residual, void* y, int32_t* topk_idx,
                                     float* topk_gate, int32_t* expert_load, void* stream) {
  MOE_TRY(check_layer_args(cfg, x, w_router, bias, weights, y, topk_idx, topk_gate, expert_load));
  if (workspace_layout(*cfg, nullptr).bytes > kNoallocScratchBytes) return MOE_ERR_UNSUPPORTED;
  void* ws = noalloc_scratch();
  if (!ws) return MOE_ERR_HIP;
  return moe_layer_forward(cfg, x, w_router, bias, weights, residual, y, topk_idx, topk_gate,
                           expert_load, ws, kNoallocScratchBytes, stream);
}

const char* moe_status_string(moe_status status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

}  // extern "C"
