// Combine, auxiliary-loss-free bias update and 1x128 FP8 activation quantisation.
#include "kernels.h"

namespace moe {

// ---- combine ("深度解读报告" section 2.2) -------------------------------------
// y[t] = [u_t] + sum_s y_rows[shared row of t] + sum_k g_tk * y_rows[pair_row[t,k]],
// fp32 in that order, one rounding at the end.  One workgroup per token; each
// thread owns 16-byte column vectors, so every row read is fully coalesced.  The
// token's K routed rows (K <= 8) are loaded together before any is added, so a
// thread has all its row loads in flight at once; the additions keep the order.
constexpr int kCombineMaxK = 8;

__device__ __forceinline__ void add_bf16x8(float acc[8], uint4 p, float g, bool scaled) {
  const uint32_t wds[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_bits_to_f32(wds[i] & 0xffffu), hi = bf16_bits_to_f32(wds[i] >> 16);
    acc[2 * i] = scaled ? fmaf(g, lo, acc[2 * i]) : acc[2 * i] + lo;
    acc[2 * i + 1] = scaled ? fmaf(g, hi, acc[2 * i + 1]) : acc[2 * i + 1] + hi;
  }
}

__global__ __launch_bounds__(256) void combine_bf16(const uint16_t* __restrict__ y_rows,
                                                    const int32_t* __restrict__ pair_row,
                                                    const float* __restrict__ gate,
                                                    const uint16_t* __restrict__ residual,
                                                    uint16_t* __restrict__ y, int T, int K,
                                                    int Ns, int H) {
  const int t = blockIdx.x;
  const size_t TK = size_t(T) * K;
  int row[kCombineMaxK];
  float g[kCombineMaxK];
#pragma unroll
  for (int k = 0; k < kCombineMaxK; ++k) {
    row[k] = k < K ? pair_row[size_t(t) * K + k] : -1;
    g[k] = k < K ? gate[size_t(t) * K + k] : 0.f;
  }
  for (int v = threadIdx.x; v < H / 8; v += 256) {
    const size_t col = size_t(v) * 8;
    uint4 p[kCombineMaxK];
#pragma unroll
    for (int k = 0; k < kCombineMaxK; ++k)
      if (row[k] >= 0) p[k] = *reinterpret_cast<const uint4*>(y_rows + size_t(row[k]) * H + col);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    if (residual)
      add_bf16x8(acc, *reinterpret_cast<const uint4*>(residual + size_t(t) * H + col), 1.f, false);
    for (int s = 0; s < Ns; ++s)
      add_bf16x8(acc, *reinterpret_cast<const uint4*>(y_rows + (TK + size_t(s) * T + t) * H + col),
                 1.f, false);
#pragma unroll
    for (int k = 0; k < kCombineMaxK; ++k)
      if (row[k] >= 0) add_bf16x8(acc, p[k], g[k], true);
    *reinterpret_cast<uint4*>(y + size_t(t) * H + col) =
        make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  }
}

__global__ __launch_bounds__(256) void combine_f32(const float* __restrict__ y_rows,
                                                   const int32_t* __restrict__ pair_row,
                                                   const float* __restrict__ gate,
                                                   const float* __restrict__ residual,
                                                   float* __restrict__ y, int T, int K, int Ns,
                                                   int H) {
  const int t = blockIdx.x;
  const size_t TK = size_t(T) * K;
  for (int v = threadIdx.x; v < H / 4; v += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (residual) {
      float4 p = reinterpret_cast<const float4*>(residual + size_t(t) * H)[v];
      acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
    }
    for (int s = 0; s < Ns; ++s) {
      float4 p = reinterpret_cast<const float4*>(y_rows + (TK + size_t(s) * T + t) * H)[v];
      acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
    }
    for (int k = 0; k < K; ++k) {
      const int r = pair_row[size_t(t) * K + k];
      if (r < 0) continue;
      const float g = gate[size_t(t) * K + k];
      float4 p = reinterpret_cast<const float4*>(y_rows + size_t(r) * H)[v];
      acc.x = fmaf(g, p.x, acc.x); acc.y = fmaf(g, p.y, acc.y);
      acc.z = fmaf(g, p.z, acc.z); acc.w = fmaf(g, p.w, acc.w);
    }
    reinterpret_cast<float4*>(y + size_t(t) * H)[v] = acc;
  }
}

hipError_t launch_combine(const moe_config& c, const void* y_rows, const int32_t* pair_row,
                          const float* gate, const void* residual, void* y, hipStream_t s) {
  if (c.act_dtype == MOE_F32) {
    hipLaunchKernelGGL(combine_f32, dim3(c.num_tokens), dim3(256), 0, s,
                       static_cast<const float*>(y_rows), pair_row, gate,
                       static_cast<const float*>(residual), static_cast<float*>(y),
                       c.num_tokens, c.top_k, c.num_shared, c.hidden);
  } else {
    hipLaunchKernelGGL(combine_bf16, dim3(c.num_tokens), dim3(256), 0, s,
                       static_cast<const uint16_t*>(y_rows), pair_row, gate,
                       static_cast<const uint16_t*>(residual), static_cast<uint16_t*>(y),
                       c.num_tokens, c.top_k, c.num_shared, c.hidden);
  }
  return hipGetLastError();
}

// ---- scale gather: [kblocks, T] token-order scales to grouped-row order -------
// out[kb, r] = scales[kb, token of r]: routed rows (below T*K) through row_token, the
// shared experts' rows in token order.
__global__ __launch_bounds__(256) void gather_scales(const float* __restrict__ scales,
                                                     const int32_t* __restrict__ row_token,
                                                     int T, int TK, int rows,
                                                     float* __restrict__ out) {
  const int r = blockIdx.x * 256 + threadIdx.x, kb = blockIdx.y;
  if (r >= rows) return;
  const int t = r < TK ? row_token[r] : (r - TK) % T;
  out[size_t(kb) * rows + r] = scales[size_t(kb) * T + t];
}

hipError_t launch_gather_scales(const moe_config& c, const float* scales, const int32_t* row_token,
                                int kblocks, float* out, hipStream_t s) {
  const int T = c.num_tokens, TK = T * c.top_k, rows = TK + T * c.num_shared;
  hipLaunchKernelGGL(gather_scales, dim3(unsigned(ceil_div(rows, 256)), unsigned(kblocks)), dim3(256),
                     0, s, scales, row_token, T, TK, rows, out);
  return hipGetLastError();
}

// ---- bias update ("深度解读报告" section 2.3) ---------------------------------
// Mean load is T*K/E; compared in integers.  Plain fp32 add / subtract.
__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ load,
                                                          float gamma, int E, long long total,
                                                          float* __restrict__ bias) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= E) return;
  const long long scaled = 1LL * load[e] * E;
  float b = bias[e];
  if (scaled > total) b = __fsub_rn(b, gamma);
  else if (scaled < total) b = __fadd_rn(b, gamma);
  bias[e] = b;
}

hipError_t launch_bias_update(const moe_config& c, const int32_t* load, float gamma,
                              float* bias, hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(ceil_div(c.num_experts, 256)), dim3(256), 0, s,
                     load, gamma, c.num_experts, 1LL * c.num_tokens * c.top_k, bias);
  return hipGetLastError();
}

// ---- 1x128 e4m3 activation quantisation (devpress page, section 2) ----------
// Each lane owns 8 consecutive columns (one 16-byte load); 16 lanes cover one
// 128-column block and a wave four blocks.  amax by butterfly max inside the 16
// lanes; scale = amax / 448 (1 if amax == 0); code = RNE-saturate(x / scale).
// Scales go to [rows, cols/128] (the C ABI's layout) or, transposed, to [cols/128, rows]
// (the expert GEMM's workspace copies: one K block's scales of consecutive rows are
// then adjacent).  pow2: scale = the smallest power of two s with amax <= 448 s, and
// at least 2^-126 (a normal float32, whose exponent field is its 8-bit exponent code):
// with amax = m 2^e, m in [0.5, 1), and 448 = 0.875 2^9, s = 2^(e-9) if m <= 0.875,
// else 2^(e-8); the quotient x / s is then exact.
// A grid of a few workgroups per CU walks the blocks with a stride, each wave taking
// kQuantUnroll groups of four blocks per step with all their loads issued first.
constexpr int kQuantUnroll = 4;

__global__ __launch_bounds__(256) void act_quant_e4m3(const uint16_t* __restrict__ x, int rows,
                                                      int cols, uint8_t* __restrict__ q,
                                                      float* __restrict__ scales, int transposed,
                                                      int pow2) {
  // block counts stay below 2^31 (checked by the launcher): 32-bit index arithmetic
  const uint32_t bpr = uint32_t(cols) / 128u;                   // blocks per row
  const uint32_t nblk = uint32_t(rows) * bpr;
  const int l16 = threadIdx.x & 15;
  // block of group u of this lane in step it: ((it * grid + wg) * 4 + wave) * U + u, then
  // * 4 + the lane's quarter
  const uint32_t wave_id = blockIdx.x * 4u + (threadIdx.x >> 6);
  const uint32_t waves = gridDim.x * 4u;
  for (uint32_t base = wave_id * kQuantUnroll; base < (nblk + 3u) / 4u; base += waves * kQuantUnroll) {
    uint4 p[kQuantUnroll];
    uint32_t blk[kQuantUnroll];
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      blk[u] = (base + u) * 4u + ((threadIdx.x >> 4) & 3u);
      p[u] = make_uint4(0, 0, 0, 0);
      if (blk[u] < nblk) {
        const uint32_t r = blk[u] / bpr, j = blk[u] - r * bpr;
        p[u] = *reinterpret_cast<const uint4*>(x + size_t(r) * cols + size_t(j) * 128 + size_t(l16) * 8);
      }
    }
#pragma unroll
    for (int u = 0; u < kQuantUnroll; ++u) {
      const uint32_t wd[4] = {p[u].x, p[u].y, p[u].z, p[u].w};
      float v[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(wd[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_f32(wd[i] >> 16);
      }
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
      for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
      if (blk[u] >= nblk) continue;
      float s = 1.0f;
      if (amax > 0.f) {
        if (pow2) {
          int e;
          const float m = frexpf(amax, &e);
          s = ldexpf(1.0f, max(m <= 0.875f ? e - 9 : e - 8, -126));
        } else {
          s = __fdiv_rn(amax, 448.0f);
        }
      }
      // x / s: an IEEE division (pow2: the product with 1/s, exact for a power of two)
      uint32_t c[8];
      const float rs = 1.0f / s;
#pragma unroll
      for (int i = 0; i < 8; ++i) c[i] = f32_to_e4m3_rne_sat(pow2 ? v[i] * rs : __fdiv_rn(v[i], s));
      const uint32_t r = blk[u] / bpr, j = blk[u] - r * bpr;
      const size_t off = size_t(r) * cols + size_t(j) * 128 + size_t(l16) * 8;
      *reinterpret_cast<uint2*>(q + off) =
          make_uint2(c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                     c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24));
      if (l16 == 0) scales[transposed ? size_t(j) * rows + r : size_t(r) * bpr + j] = s;
    }
  }
}

hipError_t launch_act_quant(const void* x, int rows, int cols, uint8_t* q, float* scales,
                            hipStream_t s, bool transposed, bool pow2) {
  const long long blocks = 1LL * rows * (cols / 128);
  if (blocks >= (1LL << 31)) return hipErrorNotSupported;
  // 16 blocks per workgroup and step; at most 8 workgroups per CU (2048 on MI355X)
  const long long need = (blocks + 16 * kQuantUnroll - 1) / (16 * kQuantUnroll);
  const unsigned grid = unsigned(need < 2048 ? need : 2048);
  hipLaunchKernelGGL(act_quant_e4m3, dim3(grid), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), rows, cols, q, scales, transposed ? 1 : 0,
                     pow2 ? 1 : 0);
  return hipGetLastError();
}

}  // namespace moe
