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
// device); the router logits' backward runs in router_wgrad (fp32 logit gradient, VALU).
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

// The router logits' backward on the VALU: one fp32 output tile (128 x 128, 8 x 8 per
// thread; 64 x 64 for small outputs) per workgroup, summed over the rows r of one row
// group in row order (fp32 FMAs):
//   C[m][n] = sum_r A(r, m) * B[r][n]
// A(r, m) = Af[r][m] (row-major fp32) or Af[m][r] (stored transposed); B bf16 rows.
enum { kWgAf32 = 1, kWgAf32T = 2 };
struct WgradArgs {
  const float* Af;
  long long lda;
  const uint16_t* B;
  long long ldb;
  int rows, M, N;
  float* C;                                 // [M][N]
};

__device__ __forceinline__ void bf16x4_to_f32(uint2 raw, float f[4]) {
  f[0] = bf16_bits_to_f32(raw.x & 0xffffu);
  f[1] = bf16_bits_to_f32(raw.x >> 16);
  f[2] = bf16_bits_to_f32(raw.y & 0xffffu);
  f[3] = bf16_bits_to_f32(raw.y >> 16);
}

template <int AMODE, int kT>
__global__ __launch_bounds__(256) void router_wgrad(WgradArgs p) {
  constexpr int kU = kT / 16, kPitch = kT + 4;        // kU x kU outputs per thread
  __shared__ __attribute__((aligned(16))) float As[16][kPitch];
  __shared__ __attribute__((aligned(16))) float Bs[16][kPitch];
  const int m0 = blockIdx.y * kT, n0 = blockIdx.x * kT;
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lr = tid / 16, lc = (tid % 16) * kU;     // loader: row lr, kU columns from lc
  float acc[kU][kU];
#pragma unroll
  for (int i = 0; i < kU; ++i)
#pragma unroll
    for (int j = 0; j < kU; ++j) acc[i][j] = 0.0f;
  for (int rb = 0; rb < p.rows; rb += 16) {
    const int r = rb + lr;
    float av[kU], bv[kU];
#pragma unroll
    for (int i = 0; i < kU; ++i) av[i] = bv[i] = 0.0f;
    // N, and M for the row-major A, are multiples of 8: a group of kU elements is wholly
    // inside or outside; the transposed A (M = tokens) is guarded per row
    if (r < p.rows && m0 + lc < p.M) {
      if (AMODE == kWgAf32) {
#pragma unroll
        for (int q = 0; q < kU / 4; ++q) {
          const float4 f =
              *reinterpret_cast<const float4*>(p.Af + size_t(r) * p.lda + m0 + lc + 4 * q);
          av[4 * q] = f.x; av[4 * q + 1] = f.y; av[4 * q + 2] = f.z; av[4 * q + 3] = f.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < kU; ++i)
          av[i] = m0 + lc + i < p.M ? p.Af[size_t(m0 + lc + i) * p.lda + r] : 0.0f;
      }
    }
    if (r < p.rows && n0 + lc < p.N) {
      const uint16_t* pb = p.B + size_t(r) * p.ldb + n0 + lc;
#pragma unroll
      for (int q = 0; q < kU / 4; ++q)
        bf16x4_to_f32(*reinterpret_cast<const uint2*>(pb + 4 * q), bv + 4 * q);
    }
    __syncthreads();                        // the previous chunk's reads are done
#pragma unroll
    for (int q = 0; q < kU / 4; ++q) {
      *reinterpret_cast<float4*>(&As[lr][lc + 4 * q]) =
          make_float4(av[4 * q], av[4 * q + 1], av[4 * q + 2], av[4 * q + 3]);
      *reinterpret_cast<float4*>(&Bs[lr][lc + 4 * q]) =
          make_float4(bv[4 * q], bv[4 * q + 1], bv[4 * q + 2], bv[4 * q + 3]);
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      float a[kU], b[kU];
#pragma unroll
      for (int q = 0; q < kU / 4; ++q) {
        const float4 fa = *reinterpret_cast<const float4*>(&As[k][ty * kU + 4 * q]);
        const float4 fb = *reinterpret_cast<const float4*>(&Bs[k][tx * kU + 4 * q]);
        a[4 * q] = fa.x; a[4 * q + 1] = fa.y; a[4 * q + 2] = fa.z; a[4 * q + 3] = fa.w;
        b[4 * q] = fb.x; b[4 * q + 1] = fb.y; b[4 * q + 2] = fb.z; b[4 * q + 3] = fb.w;
      }
#pragma unroll
      for (int i = 0; i < kU; ++i)
#pragma unroll
        for (int j = 0; j < kU; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
  }
  if (n0 + tx * kU >= p.N) return;
#pragma unroll
  for (int i = 0; i < kU; ++i)
    if (m0 + ty * kU + i < p.M) {
      float4* q = reinterpret_cast<float4*>(p.C + size_t(m0 + ty * kU + i) * p.N + n0 + tx * kU);
#pragma unroll
      for (int u = 0; u < kU / 4; ++u)
        q[u] = make_float4(acc[i][4 * u], acc[i][4 * u + 1], acc[i][4 * u + 2], acc[i][4 * u + 3]);
    }
}

template <int AMODE, int TILE = 128>
static hipError_t launch_router_wgrad(const WgradArgs& p, hipStream_t st) {
  hipLaunchKernelGGL((router_wgrad<AMODE, TILE>), dim3(ceil_div(p.N, TILE), ceil_div(p.M, TILE)),
                     dim3(256), 0, st, p);
  return hipGetLastError();
}

// Backward of the router logits z = x W_r^T for a logit gradient dz [T, E] (fp32):
//   dx = dz W_r  [T, H]   (rows r = experts, A = dz read transposed)
//   dW = dz^T x  [E, H]   (rows r = tokens)
// each as one row group through the weight-gradient kernel, fp32 sums in row order.
hipError_t launch_router_backward(const moe_config& c, const void* x, const void* w_router,
                                  const float* dz, float* dx, float* dw, hipStream_t st) {
  const int T = c.num_tokens, E = c.num_experts, H = c.hidden;
  WgradArgs w{};
  w.Af = dz;
  w.lda = E;
  w.ldb = H;
  w.N = H;
  hipError_t err = hipSuccess;
  if (dx) {
    w.rows = E;
    w.M = T;
    w.B = static_cast<const uint16_t*>(w_router);
    w.C = dx;
    if ((err = launch_router_wgrad<kWgAf32T>(w, st)) != hipSuccess) return err;
  }
  if (dw) {
    w.rows = T;
    w.M = E;
    w.B = static_cast<const uint16_t*>(x);
    w.C = dw;
    // few output tiles (E x H): 64 x 64 tiles keep more workgroups in flight
    if ((err = launch_router_wgrad<kWgAf32, 64>(w, st)) != hipSuccess) return err;
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
