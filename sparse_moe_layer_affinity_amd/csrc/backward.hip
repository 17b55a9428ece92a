// Backward of the combine, of the gates and of the SwiGLU activation.
//
// "DeepSeek-V3 Technical Report 深度解读报告", section 2.2: the layer output adds the
// shared experts' outputs and the routed experts' outputs weighted by the gates
// g_k = s_k / sum_j s_j over the selected experts; section 2.3: the bias only
// decides the selection.  Differentiating those formulas:
//   dg_tk = <dy_t, Y[pair_row(t, k)]>,  dY[pair_row(t, k)] = g_tk dy_t,
//   dY[shared row of t] = dy_t,
//   dz_tj = (dg_j - sum_k dg_k g_k) / S * s_j (1 - s_j) on the selected experts,
//   0 elsewhere (S = sum of the selected s); no gradient reaches the bias.
//
// combine_backward: one workgroup per token, each thread owns column vectors (16
// bytes of bf16 or fp32) v = tid, tid + 256, ...; the token's K routed rows are
// loaded together; the K dot products are summed per thread in column order, then
// over each wave by a fixed butterfly and over the four waves in order (fixed order,
// deterministic).  gate_backward: one wave per token.  swiglu_backward: elementwise
// over the [rows, inter] pre-activations of the SwiGLU experts.
#include "kernels.h"

namespace moe {

constexpr int kBwdMaxK = 8;

template <typename T>
struct Vec;
template <>
struct Vec<uint16_t> {                      // 8 bf16
  static constexpr int N = 8;
  uint4 raw;
  __device__ void load(const uint16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
  __device__ float get(int i) const {
    const uint32_t words[4] = {raw.x, raw.y, raw.z, raw.w};
    const uint32_t b = words[i / 2];
    return bf16_bits_to_f32(i % 2 ? b >> 16 : b & 0xffffu);
  }
  __device__ static void store_scaled(uint16_t* p, const Vec& v, float g) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = g * v.get(i);
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                              pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
  __device__ static void store_copy(uint16_t* p, const Vec& v) {
    *reinterpret_cast<uint4*>(p) = v.raw;
  }
  __device__ static void store_vals(uint16_t* p, const float f[8]) {
    *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                                              pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
};
template <>
struct Vec<float> {                         // 4 fp32
  static constexpr int N = 4;
  float4 raw;
  __device__ void load(const float* p) { raw = *reinterpret_cast<const float4*>(p); }
  __device__ float get(int i) const {
    return i == 0 ? raw.x : i == 1 ? raw.y : i == 2 ? raw.z : raw.w;
  }
  __device__ static void store_scaled(float* p, const Vec& v, float g) {
    *reinterpret_cast<float4*>(p) =
        make_float4(g * v.raw.x, g * v.raw.y, g * v.raw.z, g * v.raw.w);
  }
  __device__ static void store_copy(float* p, const Vec& v) {
    *reinterpret_cast<float4*>(p) = v.raw;
  }
  __device__ static void store_vals(float* p, const float f[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};

template <typename T>
__global__ __launch_bounds__(256) void combine_backward(
    const T* __restrict__ dy, const T* __restrict__ y_rows, const int32_t* __restrict__ pair_row,
    const float* __restrict__ gate, int Ttok, int K, int Ns, int H, float* __restrict__ dgate,
    T* __restrict__ dy_rows) {
  using V = Vec<T>;
  __shared__ float part[4][kBwdMaxK];
  const int t = blockIdx.x;
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  const size_t TK = size_t(Ttok) * K;
  int row[kBwdMaxK];
  float g[kBwdMaxK], dot[kBwdMaxK];
#pragma unroll
  for (int k = 0; k < kBwdMaxK; ++k) {
    row[k] = k < K ? pair_row[size_t(t) * K + k] : -1;
    g[k] = k < K ? gate[size_t(t) * K + k] : 0.f;
    dot[k] = 0.f;
  }
  for (int v = threadIdx.x; v < H / V::N; v += 256) {
    const size_t col = size_t(v) * V::N;
    V d, y[kBwdMaxK];
    d.load(dy + size_t(t) * H + col);
#pragma unroll
    for (int k = 0; k < kBwdMaxK; ++k)
      if (row[k] >= 0) y[k].load(y_rows + size_t(row[k]) * H + col);
#pragma unroll
    for (int k = 0; k < kBwdMaxK; ++k) {
      if (row[k] < 0) continue;
#pragma unroll
      for (int i = 0; i < V::N; ++i) dot[k] = fmaf(d.get(i), y[k].get(i), dot[k]);
      V::store_scaled(dy_rows + size_t(row[k]) * H + col, d, g[k]);
    }
    for (int s = 0; s < Ns; ++s) V::store_copy(dy_rows + (TK + size_t(s) * Ttok + t) * H + col, d);
  }
#pragma unroll
  for (int k = 0; k < kBwdMaxK; ++k) {
    float x = dot[k];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    if (l == 0) part[w][k] = x;
  }
  __syncthreads();
  if (threadIdx.x < K)
    dgate[size_t(t) * K + threadIdx.x] =
        ((part[0][threadIdx.x] + part[1][threadIdx.x]) + part[2][threadIdx.x]) + part[3][threadIdx.x];
}

constexpr int kGateWaves = 4;

__global__ __launch_bounds__(kGateWaves * 64) void gate_backward(
    const float* __restrict__ scores, const int32_t* __restrict__ idx,
    const float* __restrict__ dgate, int T, int E, int K, int accumulate,
    float* __restrict__ grad) {
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  const int t = blockIdx.x * kGateWaves + w;
  if (t >= T) return;                       // no barrier below: whole waves leave
  // lane k < K: the k-th selected expert, its affinity and its gate gradient;
  // entries outside [0, E) take no part
  int e = -1;
  float s = 0.f, dg = 0.f;
  if (l < K) {
    e = idx[size_t(t) * K + l];
    if (e >= 0 && e < E) {
      s = scores[size_t(t) * E + e];
      dg = dgate[size_t(t) * K + l];
    } else {
      e = -1;
    }
  }
  float total = 0.f;
  for (int k = 0; k < K; ++k) total += __shfl(s, k);          // S, in k order
  float dot = 0.f;
  for (int k = 0; k < K; ++k) dot += __shfl(dg, k) * (__shfl(s, k) / total);
  const float dz = e >= 0 ? (dg - dot) / total * (s * (1.f - s)) : 0.f;
  float out[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) out[j] = 0.f;
  for (int k = 0; k < K; ++k) {
    const int ek = __shfl(e, k);
    const float dk = __shfl(dz, k);
    if (ek >= 0 && (ek & 63) == l) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == (ek >> 6)) out[j] = dk;
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int ee = l + 64 * j;
    if (ee < E) {
      float* p = grad + size_t(t) * E + ee;
      *p = accumulate ? *p + out[j] : out[j];
    }
  }
}

// SwiGLU backward, elementwise over contiguous [rows, inter] arrays: for h = silu(a) b,
//   da = dh b silu'(a),  silu'(a) = sigmoid(a) (1 + a (1 - sigmoid(a))),  db = dh silu(a)
// in fp32, one rounding per output; 16-byte vectors, grid-stride.
template <typename T>
__global__ __launch_bounds__(256) void swiglu_backward(const T* __restrict__ a,
                                                       const T* __restrict__ b,
                                                       const T* __restrict__ dh,
                                                       T* __restrict__ da, T* __restrict__ db,
                                                       size_t n_vec) {
  using V = Vec<T>;
  for (size_t v = size_t(blockIdx.x) * 256 + threadIdx.x; v < n_vec;
       v += size_t(gridDim.x) * 256) {
    const size_t at = v * V::N;
    V av, bv, hv;
    av.load(a + at);
    bv.load(b + at);
    hv.load(dh + at);
    float fa[V::N], fb[V::N];
#pragma unroll
    for (int i = 0; i < V::N; ++i) {
      const float x = av.get(i);
      const float sg = 1.0f / (1.0f + expf(-x));
      const float dsilu = sg * (1.0f + x * (1.0f - sg));
      fa[i] = hv.get(i) * bv.get(i) * dsilu;
      fb[i] = hv.get(i) * (x * sg);
    }
    V::store_vals(da + at, fa);
    V::store_vals(db + at, fb);
  }
}

hipError_t launch_swiglu_backward(const moe_config& c, const void* a, const void* b,
                                  const void* dh, int rows, void* da, void* db, hipStream_t st) {
  const bool f32 = c.act_dtype == MOE_F32;
  const size_t n_vec = size_t(rows) * c.inter / (f32 ? 4 : 8);
  const size_t want = (n_vec + 255) / 256;
  const unsigned blocks = unsigned(want < 8192 ? want : 8192);
  if (f32)
    hipLaunchKernelGGL(swiglu_backward<float>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const float*>(a), static_cast<const float*>(b),
                       static_cast<const float*>(dh), static_cast<float*>(da),
                       static_cast<float*>(db), n_vec);
  else
    hipLaunchKernelGGL(swiglu_backward<uint16_t>, dim3(blocks), dim3(256), 0, st,
                       static_cast<const uint16_t*>(a), static_cast<const uint16_t*>(b),
                       static_cast<const uint16_t*>(dh), static_cast<uint16_t*>(da),
                       static_cast<uint16_t*>(db), n_vec);
  return hipGetLastError();
}

hipError_t launch_combine_backward(const moe_config& c, const void* dy, const void* y_rows,
                                   const int32_t* pair_row, const float* gate, float* dgate,
                                   void* dy_rows, hipStream_t st) {
  if (c.act_dtype == MOE_F32)
    hipLaunchKernelGGL(combine_backward<float>, dim3(c.num_tokens), dim3(256), 0, st,
                       static_cast<const float*>(dy), static_cast<const float*>(y_rows), pair_row,
                       gate, c.num_tokens, c.top_k, c.num_shared, c.hidden, dgate,
                       static_cast<float*>(dy_rows));
  else
    hipLaunchKernelGGL(combine_backward<uint16_t>, dim3(c.num_tokens), dim3(256), 0, st,
                       static_cast<const uint16_t*>(dy), static_cast<const uint16_t*>(y_rows),
                       pair_row, gate, c.num_tokens, c.top_k, c.num_shared, c.hidden, dgate,
                       static_cast<uint16_t*>(dy_rows));
  return hipGetLastError();
}

hipError_t launch_gate_backward(const moe_config& c, const float* scores, const int32_t* idx,
                                const float* dgate, float* grad, int accumulate, hipStream_t st) {
  hipLaunchKernelGGL(gate_backward, dim3(ceil_div(c.num_tokens, kGateWaves)),
                     dim3(kGateWaves * 64), 0, st, scores, idx, dgate, c.num_tokens,
                     c.num_experts, c.top_k, accumulate, grad);
  return hipGetLastError();
}

}  // namespace moe
