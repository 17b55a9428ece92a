// Router: sigmoid affinities, selection-only bias, group-limited top-K, gates.
//
// "DeepSeek-V3 Technical Report 深度解读报告", section 2.2 (sigmoid affinity,
// gates normalised over the selected experts), section 2.3 (bias b_i added to the
// affinity for top-K selection only), section 2.4 (at most M nodes per token,
// chosen by the sum of the highest affinities on each node).
//
// Logits z = x W_r^T come from the grouped GEMM (bf16 MFMA, fp32 accumulation) or,
// for fp32 activations, from a plain VALU dot-product kernel.  Selection runs one
// wave64 per token: each lane holds up to 4 experts (expert e lives in lane e % 64,
// slot e / 64), groups are scored by single lanes out of LDS, and the top-K is K
// rounds of a wave-wide (value desc, index asc) argmax over butterfly shuffles.
#include "kernels.h"

namespace moe {

hipError_t launch_gemm_router_bf16(const moe_config& c, const uint16_t* x, const uint16_t* w,
                                   float* z, hipStream_t s);

// fp32 logits: one thread per (token, expert), sequential fp32 FMA over hidden.
__global__ __launch_bounds__(256) void router_logits_f32(const float* __restrict__ x,
                                                         const float* __restrict__ w, int T,
                                                         int E, int H, float* __restrict__ z) {
  int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= T * E) return;
  int t = i / E, e = i % E;
  const float4* xr = reinterpret_cast<const float4*>(x + size_t(t) * H);
  const float4* wr = reinterpret_cast<const float4*>(w + size_t(e) * H);
  float acc = 0.f;
  for (int k = 0; k < H / 4; ++k) {
    float4 a = xr[k], b = wr[k];
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    acc = fmaf(a.w, b.w, acc);
  }
  z[i] = acc;
}

constexpr int kSelWaves = 4;
constexpr int kSelBatch = 8;    // split-K partials loaded per round trip

// (value desc, index asc) ordering used for every selection decision.
__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(kSelWaves * 64) void router_select(
    const float* __restrict__ z, int splits, const float* __restrict__ bias, int T, int E, int G,
    int M, int topn, int K, int32_t* __restrict__ idx_out, float* __restrict__ gate_out) {
  __shared__ float sb_lds[kSelWaves][256];
  __shared__ float s_lds[kSelWaves][256];
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  const int t = blockIdx.x * kSelWaves + w;
  const bool active = t < T;
  const int n = E / G;

  // logits = the split-K partials summed in split order (one partial unless split);
  // up to kSelBatch partials of the lane's four experts are loaded together ahead of
  // the in-order adds, so one round trip covers the usual split counts
  float zz[4];
  const size_t stride = size_t(T) * E;
  const size_t tofs = size_t(active ? t : 0) * E;
  auto part = [&](int p, int j) {
    const int e = l + 64 * j;
    return (active && e < E) ? z[size_t(p) * stride + tofs + e] : 0.0f;
  };
#pragma unroll
  for (int j = 0; j < 4; ++j) zz[j] = part(0, j);
  for (int p0 = 1; p0 < splits; p0 += kSelBatch) {
    float pv[kSelBatch][4];
#pragma unroll
    for (int i = 0; i < kSelBatch; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) pv[i][j] = p0 + i < splits ? part(p0 + i, j) : 0.0f;
#pragma unroll
    for (int i = 0; i < kSelBatch; ++i)
      if (p0 + i < splits) {
#pragma unroll
        for (int j = 0; j < 4; ++j) zz[j] += pv[i][j];
      }
  }

  // affinities and biased affinities (fp32)
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = l + 64 * j;
    v[j] = -INFINITY;
    if (active && e < E) {
      float s = 1.0f / (1.0f + expf(-zz[j]));
      float sb = s + bias[e];
      s_lds[w][e] = s;
      sb_lds[w][e] = sb;
      v[j] = sb;
    }
  }
  __syncthreads();
  if (!active) return;

  // stage 1: group score = sum of the topn largest biased affinities (largest first);
  // a two-slot running maximum when topn <= 2 (the same two values, duplicates kept)
  float gscore = -INFINITY;
  if (l < G && topn <= 2) {
    float t0 = -INFINITY, t1 = -INFINITY;
    for (int i = 0; i < n; ++i) {
      const float x = sb_lds[w][l * n + i];
      t1 = x > t0 ? t0 : (x > t1 ? x : t1);
      t0 = x > t0 ? x : t0;
    }
    gscore = topn == 2 ? 0.0f + t0 + t1 : 0.0f + t0;
  } else if (l < G) {
    float top[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) top[i] = -INFINITY;
    for (int i = 0; i < n; ++i) {
      float x = sb_lds[w][l * n + i];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (x > top[q]) { float tmp = top[q]; top[q] = x; x = tmp; }
      }
    }
    float acc = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q < topn) acc += top[q];
    gscore = acc;
  }
  // rank of my group among all G (score desc, index asc); keep the M best
  int rank = 0;
  for (int j = 0; j < G; ++j) {
    float o = __shfl(gscore, j);
    if (better(o, j, gscore, l)) ++rank;
  }
  const uint64_t kept = __ballot(l < G && rank < M);

  // stage 2: top-K biased affinities among the kept groups' experts
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = l + 64 * j;
    if (e >= E || !((kept >> (e / n)) & 1ull)) v[j] = -INFINITY;
  }
  int my_e = -1;
  for (int k = 0; k < K; ++k) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = l + 64 * j;
      if (v[j] != -INFINITY && better(v[j], e, bv, bi)) { bv = v[j]; bi = e; }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oi = __shfl_xor(bi, off);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if (l == k) my_e = bi;
    if (l == (bi & 63)) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == (bi >> 6)) v[j] = -INFINITY;
    }
  }

  // gates: unbiased affinities normalised over the selection, summed in k order
  float sk = (l < K) ? s_lds[w][my_e] : 0.0f;
  float sum = 0.0f;
  for (int k = 0; k < K; ++k) sum += __shfl(sk, k);
  if (l < K) {
    idx_out[size_t(t) * K + l] = my_e;
    gate_out[size_t(t) * K + l] = sk / sum;
  }
}

hipError_t launch_router_logits(const moe_config& c, const void* x, const void* w, float* z,
                                hipStream_t s) {
  if (c.act_dtype == MOE_F32) {
    int n = c.num_tokens * c.num_experts;
    hipLaunchKernelGGL(router_logits_f32, dim3(ceil_div(n, 256)), dim3(256), 0, s,
                       static_cast<const float*>(x), static_cast<const float*>(w),
                       c.num_tokens, c.num_experts, c.hidden, z);
    return hipGetLastError();
  }
  return launch_gemm_router_bf16(c, static_cast<const uint16_t*>(x),
                                 static_cast<const uint16_t*>(w), z, s);
}

hipError_t launch_router_select(const moe_config& c, const float* z, const float* bias,
                                int32_t* idx, float* gate, hipStream_t s) {
  hipLaunchKernelGGL(router_select, dim3(ceil_div(c.num_tokens, kSelWaves)),
                     dim3(kSelWaves * 64), 0, s, z, router_splits(c), bias, c.num_tokens, c.num_experts,
                     c.num_groups, c.top_groups, c.group_topn, c.top_k, idx, gate);
  return hipGetLastError();
}

}  // namespace moe
