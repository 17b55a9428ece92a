// Backward of the layer: the combine, the gates, the SwiGLU activation, the experts'
// input and weight gradients, and the router logits.
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
// over the [rows, inter] pre-activations of the SwiGLU experts.  The experts' input
// gradient runs the forward's expert GEMM in its [K][N] weight mode (the weights read
// as they are stored, fragments transposed on their way out of LDS); their weight
// gradients run on the matrix cores (wgrad.hip, each expert's row range read on the
// device).  The router logits' backward runs on the matrix cores too: the fp32 logit
// gradient is split into two bf16 parts (hi + lo, within 2^-17 of it) stacked along the
// contraction, so bf16 MFMAs with fp32 accumulation keep about fp32 accuracy.
#include <algorithm>

#include "gemm_common.h"

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

// SwiGLU backward, elementwise over [rows, cols] arrays with their own row pitches:
// for h = silu(a) b,
//   da = dh b silu'(a),  silu'(a) = sigmoid(a) (1 + a (1 - sigmoid(a))),  db = dh silu(a)
// in fp32, one rounding per output; 16-byte vectors, grid-stride.
struct SwigluArgs {
  const void *a, *b, *dh;
  void *da, *db;
  long long lda, ldb, ldh, ldda, lddb;   // row pitches in elements
  int rows, cols;
};

template <typename T>
__global__ __launch_bounds__(256) void swiglu_backward(SwigluArgs p) {
  using V = Vec<T>;
  const size_t per_row = size_t(p.cols) / V::N;
  const size_t n_vec = per_row * p.rows;
  for (size_t v = size_t(blockIdx.x) * 256 + threadIdx.x; v < n_vec;
       v += size_t(gridDim.x) * 256) {
    const size_t r = v / per_row, col = (v % per_row) * V::N;
    V av, bv, hv;
    av.load(static_cast<const T*>(p.a) + r * p.lda + col);
    bv.load(static_cast<const T*>(p.b) + r * p.ldb + col);
    hv.load(static_cast<const T*>(p.dh) + r * p.ldh + col);
    float fa[V::N], fb[V::N];
#pragma unroll
    for (int i = 0; i < V::N; ++i) {
      const float x = av.get(i);
      const float sg = 1.0f / (1.0f + expf(-x));
      const float dsilu = sg * (1.0f + x * (1.0f - sg));
      fa[i] = hv.get(i) * bv.get(i) * dsilu;
      fb[i] = hv.get(i) * (x * sg);
    }
    V::store_vals(static_cast<T*>(p.da) + r * p.ldda + col, fa);
    V::store_vals(static_cast<T*>(p.db) + r * p.lddb + col, fb);
  }
}

static hipError_t launch_swiglu(bool f32, const SwigluArgs& p, hipStream_t st) {
  const size_t n_vec = size_t(p.rows) * p.cols / (f32 ? 4 : 8);
  const size_t want = (n_vec + 255) / 256;
  const unsigned blocks = unsigned(want < 8192 ? want : 8192);
  if (f32) hipLaunchKernelGGL(swiglu_backward<float>, dim3(blocks), dim3(256), 0, st, p);
  else hipLaunchKernelGGL(swiglu_backward<uint16_t>, dim3(blocks), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_swiglu_backward(const moe_config& c, const void* a, const void* b,
                                  const void* dh, int rows, void* da, void* db, hipStream_t st) {
  const long long I = c.inter;
  return launch_swiglu(c.act_dtype == MOE_F32,
                       SwigluArgs{a, b, dh, da, db, I, I, I, I, I, rows, c.inter}, st);
}

__global__ __launch_bounds__(256) void fill_f32(float* __restrict__ p, int n, float v) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = v;
}

// bf16 bits of v, round to nearest even
__device__ __forceinline__ uint32_t bf16_rne(float v) { return pack_bf16x2(v, 0.0f) & 0xffffu; }

// The logit gradient dz [T][E] (fp32) as hi = bf16(dz) and lo = bf16(dz - hi), so that
// dz = hi + lo within 2^-17 |dz|, in both layouts the two products read: dzs [T][2 Ep]
// (hi in columns 0.., lo from column Ep) and dzt [2 Ep][Tp] (hi rows, then lo rows),
// zeros in the padding (experts E..Ep-1, tokens T..Tp-1).  64 x 64 tiles through LDS.
__global__ __launch_bounds__(256) void router_dz_split(const float* __restrict__ dz, int T, int E,
                                                       int Ep, int Tp, uint16_t* __restrict__ dzs,
                                                       uint16_t* __restrict__ dzt) {
  __shared__ uint32_t tile[64][65];          // hi | lo << 16, [token][expert]
  const int t0 = blockIdx.y * 64, e0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int t = t0 + i, e = e0 + tx;
    const float v = t < T && e < E ? dz[size_t(t) * E + e] : 0.0f;
    const uint32_t hi = bf16_rne(v);
    const uint32_t lo = bf16_rne(v - bf16_bits_to_f32(hi));
    tile[i][tx] = hi | (lo << 16);
    if (t < T) {
      dzs[size_t(t) * 2 * Ep + e] = uint16_t(hi);
      dzs[size_t(t) * 2 * Ep + Ep + e] = uint16_t(lo);
    }
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int e = e0 + i, t = t0 + tx;
    const uint32_t v = tile[tx][i];
    dzt[size_t(e) * Tp + t] = uint16_t(v & 0xffffu);
    dzt[size_t(Ep + e) * Tp + t] = uint16_t(v >> 16);
  }
}

// dst[c][col0 + r] = src[r][c] for r < R, zero for R <= r < Rp: src [R][C] bf16 (C a
// multiple of 8), dst rows of ld elements, Rp a multiple of 64.  64 x 64 tiles:
// 16-byte reads along source rows, 16-byte writes along destination rows (each
// gathered from 8 LDS rows); the LDS pitch of 72 elements keeps rows 16-byte aligned.
__global__ __launch_bounds__(256) void transpose_pad_bf16(const uint16_t* __restrict__ src, int R,
                                                          int C, uint16_t* __restrict__ dst,
                                                          long long ld, int col0) {
  constexpr int kPitch = 72;
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kPitch];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int lane8 = (threadIdx.x % 8) * 8, row = threadIdx.x / 8;     // row 0..31
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int i = row + 32 * pass, r = r0 + i, cc = c0 + lane8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < R && cc < C) v = *reinterpret_cast<const uint4*>(src + size_t(r) * C + cc);
    *reinterpret_cast<uint4*>(&tile[i * kPitch + lane8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int j = row + 32 * pass, cc = c0 + j;                        // source column j
    uint16_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = tile[(lane8 + q) * kPitch + j];
    if (cc < C)
      *reinterpret_cast<uint4*>(dst + size_t(cc) * ld + col0 + r0 + lane8) =
          make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                     e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
  }
}

// dw[e][c] = sum over splits s of part[s][e][c], then of part[s][Ep + e][c] (the hi and
// the lo products), in that fixed order.
__global__ __launch_bounds__(256) void router_dw_reduce(const float4* __restrict__ part, int S,
                                                        long long split_stride4,
                                                        long long lo_off4, long long n4,
                                                        float4* __restrict__ dw) {
  const long long i = blockIdx.x * 256LL + threadIdx.x;
  if (i >= n4) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int h = 0; h < 2; ++h)
    for (int s = 0; s < S; ++s) {
      const float4 v = part[s * split_stride4 + h * lo_off4 + i];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
  dw[i] = acc;
}

RouterBwdWorkspace router_bwd_workspace_layout(const moe_config& c, void* base) {
  RouterBwdWorkspace w{};
  const long long T = c.num_tokens, E = c.num_experts, H = c.hidden;
  w.Ep = int((E + 63) / 64 * 64);
  w.Tp = int(std::max<long long>(256, (T + 127) / 128 * 128));
  // split-K of dW over the tokens: every split a multiple of 128 and at least 256 long
  for (w.S = 4; w.S > 1; --w.S) {
    w.kc = (ceil_div(w.Tp, w.S) + 127) / 128 * 128;
    if (w.kc >= 256 && w.Tp - (w.S - 1) * w.kc >= 256) break;
  }
  if (w.S == 1) w.kc = w.Tp;
  char* p = static_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* r = p ? p + off : nullptr;
    off += (bytes + 255) / 256 * 256;
    return r;
  };
  const size_t Ep2 = 2 * size_t(w.Ep);
  w.dzs = static_cast<uint16_t*>(take(size_t(T) * Ep2 * 2));
  w.dzt = static_cast<uint16_t*>(take(Ep2 * w.Tp * 2));
  w.wt2 = static_cast<uint16_t*>(take(size_t(H) * Ep2 * 2));
  w.xt = static_cast<uint16_t*>(take(size_t(H) * w.Tp * 2));
  w.part = static_cast<float*>(take(size_t(w.S) * Ep2 * H * 4));
  w.bytes = off;
  return w;
}

// Backward of the router logits z = x W_r^T for a logit gradient dz [T, E] (fp32), on
// the expert GEMM kernel's fp32-output mode (operands contiguous along the contraction):
//   dx = [hi | lo] [W_r ; W_r]      [T, H]: A = dzs [T][2 Ep], B = wt2 [H][2 Ep]
//   dW = hi^T x + lo^T x            [E, H]: A = dzt [2 Ep][Tp], B = x^T [H][Tp], split-K
//        partials [S][2 Ep][H] summed in a fixed order
hipError_t launch_router_backward(const moe_config& c, const void* x, const void* w_router,
                                  const float* dz, float* dx, float* dw,
                                  const RouterBwdWorkspace& ws, hipStream_t st) {
  const int T = c.num_tokens, E = c.num_experts, H = c.hidden;
  const int Ep = ws.Ep, Tp = ws.Tp;
  hipLaunchKernelGGL(router_dz_split, dim3(Ep / 64, Tp / 64), dim3(256), 0, st, dz, T, E, Ep, Tp,
                     ws.dzs, ws.dzt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const auto* wr = static_cast<const uint16_t*>(w_router);
  const dim3 tgrid_w(ceil_div(H, 64), Ep / 64);
  if (dx) {
    hipLaunchKernelGGL(transpose_pad_bf16, tgrid_w, dim3(256), 0, st, wr, E, H, ws.wt2,
                       2LL * Ep, 0);
    hipLaunchKernelGGL(transpose_pad_bf16, tgrid_w, dim3(256), 0, st, wr, E, H, ws.wt2,
                       2LL * Ep, Ep);
    GemmArgs a{};
    a.A = ws.dzs;
    a.a_rows = T;
    a.T = T;
    a.K = 2 * Ep;
    a.B0 = ws.wt2;
    a.N = H;
    a.C = dx;
    a.ldc = H;
    a.n_tiles = ceil_div(H, 256);
    if ((err = launch_gemm_f32(a, 1, st)) != hipSuccess) return err;
  }
  if (dw) {
    hipLaunchKernelGGL(transpose_pad_bf16, dim3(ceil_div(H, 64), Tp / 64), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), T, H, ws.xt, (long long)Tp, 0);
    GemmArgs b{};
    b.A = ws.dzt;
    b.a_rows = 2 * Ep;
    b.T = 2 * Ep;
    b.K = Tp;
    b.B0 = ws.xt;
    b.N = H;
    b.C = ws.part;
    b.ldc = H;
    b.n_tiles = ceil_div(H, 256);
    b.k_chunk = ws.S > 1 ? ws.kc : 0;
    b.c_split_stride = 2LL * Ep * H;
    if ((err = launch_gemm_f32(b, ws.S, st)) != hipSuccess) return err;
    const long long n4 = 1LL * E * H / 4;
    hipLaunchKernelGGL(router_dw_reduce, dim3(unsigned((n4 + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<const float4*>(ws.part), ws.S, 2LL * Ep * H / 4,
                       1LL * Ep * H / 4, n4, reinterpret_cast<float4*>(dw));
    err = hipGetLastError();
  }
  return err;
}

// Input gradient of the grouped SwiGLU experts (bf16), on the forward's row layout:
//   a | b   = gathered x rows times W_gate^T | W_up^T      (recomputed, plain GEMMs)
//   dh      = dy_rows times W_down                         (W_down [H][I] read as [K][N])
//   da | db = SwiGLU backward of (a, b, dh)
//   dX      = [da | db] times [W_gate ; W_up]              (both [I][H], stacked along K)
//   dx      = sum of dX over each token's rows              (the combine, unit gates)
hipError_t launch_expert_backward(const moe_config& c, const void* x, const int32_t* offsets,
                                  const int32_t* row_token, const int32_t* pair_row,
                                  const moe_expert_weights& wt, const void* dy_rows, void* dx,
                                  float* dw_gate, float* dw_up, float* dw_down,
                                  const BackwardWorkspace& ws, hipStream_t s) {
  const int T = c.num_tokens, K = c.top_k, Ns = c.num_shared;
  const int H = c.hidden, I = c.inter, TK = T * K, rows = TK + T * Ns;
  hipError_t err = launch_build_schedule(c, offsets, kExpertBM, ws.sched, ws.sched_n, s);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(fill_f32, dim3(ceil_div(TK, 256)), dim3(256), 0, s, ws.ones, TK, 1.0f);
  const auto* wg = static_cast<const uint16_t*>(wt.w_gate);
  const auto* wu = static_cast<const uint16_t*>(wt.w_up);
  const auto* wd = static_cast<const uint16_t*>(wt.w_down);

  GemmArgs a{};
  a.sched = ws.sched;
  a.sched_n = ws.sched_n;
  a.T = T;
  a.TK = TK;
  // a and b, recomputed with the row gather of the forward
  a.A = static_cast<const uint16_t*>(x);
  a.row_token = row_token;
  a.gather = 1;
  a.a_rows = T;
  a.b_stride = 1LL * I * H;
  a.ldc = 2 * I;
  a.N = I;
  a.K = H;
  a.n_tiles = ceil_div(I, 256);
  a.B0 = wg;
  a.C = ws.ab;
  if ((err = launch_grouped_plain_bf16(c, a, s)) != hipSuccess) return err;
  a.B0 = wu;
  a.C = ws.ab + I;
  if ((err = launch_grouped_plain_bf16(c, a, s)) != hipSuccess) return err;
  // dh = dy_rows W_down
  GemmArgs d = a;
  d.A = static_cast<const uint16_t*>(dy_rows);
  d.row_token = nullptr;
  d.gather = 0;
  d.a_rows = rows;
  d.B0 = wd;
  d.b_stride = 1LL * I * H;
  d.C = ws.dh;
  d.ldc = I;
  d.N = I;
  d.K = H;
  d.k_split = H;
  d.n_tiles = ceil_div(I, 256);
  if ((err = launch_grouped_kn_bf16(c, d, s)) != hipSuccess) return err;
  // da | db
  const long long I2 = 2LL * I;
  err = launch_swiglu(false, SwigluArgs{ws.ab, ws.ab + I, ws.dh, ws.dab, ws.dab + I, I2, I2, I,
                                        I2, I2, rows, I}, s);
  if (err != hipSuccess) return err;
  if (dw_down) {
    // dW_down = dy^T h, dW_gate = da^T u, dW_up = db^T u over each expert's rows, on the
    // matrix cores (wgrad.hip)
    err = launch_expert_wgrad_mfma(c, x, offsets, row_token, dy_rows, ws.ab, ws.dab, dw_gate,
                                   dw_up, dw_down, ws.pack, s);
    if (err != hipSuccess) return err;
  }
  if (!dx) return hipSuccess;
  // dX = [da | db] [W_gate ; W_up]
  GemmArgs q = d;
  q.A = ws.dab;
  q.B0 = wg;
  q.B1 = wu;
  q.b_stride = 1LL * I * H;
  q.C = ws.dx_rows;
  q.ldc = H;
  q.N = H;
  q.K = 2 * I;
  q.k_split = I;
  q.n_tiles = ceil_div(H, 256);
  if ((err = launch_grouped_kn_bf16(c, q, s)) != hipSuccess) return err;
  // dx: every row of the token with weight one
  return launch_combine(c, ws.dx_rows, pair_row, ws.ones, nullptr, dx, s);
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
