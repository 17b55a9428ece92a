// Grouped expert GEMMs of the MoE layer on gfx950.
//
// "DeepSeek-V3 Technical Report 深度解读报告", section 2.2: every token passes the
// shared expert(s) and its K routed experts; each expert is a SwiGLU FFN
// W_down (silu(W_gate u) * (W_up u)).  Rows are grouped by expert (see permute),
// the shared experts appended as groups E..E+Ns-1 holding all T tokens, so the
// whole layer is two grouped GEMMs:
//   GEMM1  h[r]      = silu(x[tok(r)] W_gate,e^T) * (x[tok(r)] W_up,e^T)   (gather on load)
//   GEMM2  y_rows[r] = h[r] W_down,e^T
// Both operands are K-contiguous (x and h rows, weight rows), which is exactly the
// operand layout of the MFMA: no transposes anywhere.
//
// bf16 kernel: v_mfma_f32_16x16x32_bf16, fp32 accumulation.  A workgroup owns a
// BM x BN tile of one expert; the K loop stages 64-wide A and B slices through
// padded LDS (row pitch 72 bf16 keeps the 16-lane fragment reads on distinct banks)
// with the next slice's global loads in flight during the MFMAs.  GEMM1's B tile
// stacks BN/2 gate rows over the matching BN/2 up rows and every wave owns the
// same columns of both halves, so the SwiGLU epilogue runs in registers.
// Tile order: (expert, n-tile, m-tile) with m innermost, and the linear
// workgroup id is remapped so that each of the 8 XCDs (workgroups are dispatched
// round-robin over them) walks one contiguous stretch of that order: m-tiles of
// one weight tile, and n-tiles of one expert's rows, then share the XCD's L2.
#include "kernels.h"

namespace moe {

struct GemmArgs {
  const uint16_t* A;         // bf16 activations: x [T, K] (gather) or [rows, K]
  const int32_t* row_token;  // gather map of routed rows (gather only)
  const int32_t* offsets;    // [E+1] expert offsets (nullptr: single group of T rows)
  const int32_t* tile_off;   // [G+1] m-tile prefix per group (nullptr: single group)
  const uint16_t* B0;        // weights [G][N][K] bf16 (GEMM1: gate)
  const uint16_t* B1;        // GEMM1: up
  long long b_stride;        // elements per expert
  void* C;                   // output [rows, ldc]
  int ldc, N, K;             // N = output columns (GEMM1: intermediate columns)
  int E, T, TK, G;           // routed experts, tokens, T*K, groups (E + Ns)
  int n_tiles;
  int gather;
};

enum { kPlainBf16 = 0, kGatedBf16 = 1, kPlainF32 = 2 };

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_bf16(GemmArgs a) {
  constexpr int NT = WM * WN * 64;
  constexpr int BK = 64;
  constexpr int LD = BK + 8;                  // padded LDS row pitch (bf16 elements)
  constexpr int WTM = BM / WM, WTN = BN / WN; // wave tile: rows x B-rows
  constexpr int NI = WTM / 16, NJ = WTN / 16;
  constexpr int CA = BM * (BK / 8) / NT;      // 16-byte chunks per thread per slice
  constexpr int CB = BN * (BK / 8) / NT;
  constexpr int BN_OUT = MODE == kGatedBf16 ? BN / 2 : BN;
  static_assert(CA * NT == BM * (BK / 8) && CB * NT == BN * (BK / 8), "tile/threads");
  static_assert(MODE != kGatedBf16 || NJ % 2 == 0, "gated tiles pair gate/up blocks");

  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LD];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LD];

  // ---- tile decode --------------------------------------------------------
  const int total_m = a.tile_off ? a.tile_off[a.G] : ceil_div(a.T, BM);
  const int total = total_m * a.n_tiles;
  const int b = blockIdx.x;
  if (b >= total) return;
  const int per = total / kXcds, rem = total % kXcds;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;

  int g, nt, mt, r0, r1;
  if (a.tile_off) {
    int lo = 0, hi = a.G;
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (a.tile_off[mid] * a.n_tiles <= logical) lo = mid; else hi = mid;
    }
    g = lo;
    const int mtiles = a.tile_off[g + 1] - a.tile_off[g];
    const int local = logical - a.tile_off[g] * a.n_tiles;
    nt = local / mtiles;
    mt = local % mtiles;
    group_rows(a.offsets, g, a.E, a.T, a.TK, r0, r1);
  } else {
    g = 0;
    nt = logical / total_m;
    mt = logical % total_m;
    r0 = 0;
    r1 = a.T;
  }
  const int m0 = r0 + mt * BM;
  const int mvalid = min(BM, r1 - m0);
  const int n0 = nt * BN_OUT;

  const int tid = threadIdx.x;
  const int K = a.K;

  // ---- per-thread global source pointers ----------------------------------
  const uint16_t* pa[CA];
  const uint16_t* pb[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int c = tid + i * NT;
    const int row = min(c >> 3, mvalid - 1);      // padding rows re-read the last valid row
    const int r = m0 + row;
    const int src = a.gather ? row_token_of(a.row_token, r, a.T, a.TK) : r;
    pa[i] = a.A + size_t(src) * K + (c & 7) * 8;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int c = tid + i * NT;
    const int brow = c >> 3;
    const uint16_t* base = a.B0;
    int n = n0 + brow;
    if (MODE == kGatedBf16 && brow >= BN / 2) {
      base = a.B1;
      n = n0 + brow - BN / 2;
    }
    n = min(n, a.N - 1);
    pb[i] = base + size_t(g) * a.b_stride + size_t(n) * K + (c & 7) * 8;
  }

  uint4 ra[CA], rb[CB];
  auto load_slice = [&](int k0) {
#pragma unroll
    for (int i = 0; i < CA; ++i) ra[i] = *reinterpret_cast<const uint4*>(pa[i] + k0);
#pragma unroll
    for (int i = 0; i < CB; ++i) rb[i] = *reinterpret_cast<const uint4*>(pb[i] + k0);
  };
  auto store_slice = [&]() {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(&As[(c >> 3) * LD + (c & 7) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int c = tid + i * NT;
      *reinterpret_cast<uint4*>(&Bs[(c >> 3) * LD + (c & 7) * 8]) = rb[i];
    }
  };

  const int w = tid >> 6, l = tid & 63;
  const int wm = w / WN, wn = w % WN;
  int brow0[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (MODE == kGatedBf16) {
      brow0[j] = j < NJ / 2 ? wn * (WTN / 2) + j * 16 : BN / 2 + wn * (WTN / 2) + (j - NJ / 2) * 16;
    } else {
      brow0[j] = wn * WTN + j * 16;
    }
  }

  f32x4_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  load_slice(0);
  for (int kt = 0; kt < nk; ++kt) {
    store_slice();
    __syncthreads();
    if (kt + 1 < nk) load_slice((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t af[NI], bfr[NJ];
      const int koff = ks * 32 + (l >> 4) * 8;
#pragma unroll
      for (int i = 0; i < NI; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(&As[(wm * WTM + i * 16 + (l & 15)) * LD + koff]);
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(&Bs[(brow0[j] + (l & 15)) * LD + koff]);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  // ---- epilogue: lane l holds rows (l/16)*4 + q, column l%16 of each 16x16 block
#pragma unroll
  for (int i = 0; i < NI; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rl = wm * WTM + i * 16 + (l >> 4) * 4 + q;
      if (rl >= mvalid) continue;
      const size_t row = size_t(m0 + rl);
      if (MODE == kGatedBf16) {
#pragma unroll
        for (int j = 0; j < NJ / 2; ++j) {
          const int col = n0 + wn * (WTN / 2) + j * 16 + (l & 15);
          const float gt = acc[i][j][q], up = acc[i][j + NJ / 2][q];
          const float hv = gt / (1.0f + expf(-gt)) * up;
          if (col < a.N) static_cast<uint16_t*>(a.C)[row * a.ldc + col] = f32_to_bf16_bits(hv);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int col = n0 + wn * WTN + j * 16 + (l & 15);
          if (col >= a.N) continue;
          if (MODE == kPlainF32)
            static_cast<float*>(a.C)[row * a.ldc + col] = acc[i][j][q];
          else
            static_cast<uint16_t*>(a.C)[row * a.ldc + col] = f32_to_bf16_bits(acc[i][j][q]);
        }
      }
    }
  }
}

// m-tile prefix over groups for two tile heights, one workgroup (G <= 512).
__global__ __launch_bounds__(512) void build_tiles(const int32_t* __restrict__ offsets, int E,
                                                   int Ns, int T, int TK, int bm1, int bm2,
                                                   int32_t* __restrict__ t1,
                                                   int32_t* __restrict__ t2) {
  __shared__ int s1[512], s2[512];
  const int g = threadIdx.x, G = E + Ns;
  int c1 = 0, c2 = 0;
  if (g < G) {
    int r0, r1;
    group_rows(offsets, g, E, T, TK, r0, r1);
    c1 = ceil_div(r1 - r0, bm1);
    c2 = ceil_div(r1 - r0, bm2);
  }
  s1[g] = c1;
  s2[g] = c2;
  __syncthreads();
  for (int d = 1; d < 512; d <<= 1) {
    int a1 = g >= d ? s1[g - d] : 0, a2 = g >= d ? s2[g - d] : 0;
    __syncthreads();
    s1[g] += a1;
    s2[g] += a2;
    __syncthreads();
  }
  if (g < G) {
    t1[g] = s1[g] - c1;
    t2[g] = s2[g] - c2;
  }
  if (g == G - 1) {
    t1[G] = s1[g];
    t2[G] = s2[g];
  }
}

// ---- fp32 path (small fp32 workloads): one thread per output element ---------
__device__ __forceinline__ int group_of_row(const int32_t* offsets, int r, int E, int T, int TK) {
  if (r >= TK) return E + (r - TK) / T;
  int lo = 0, hi = E;                     // largest e with offsets[e] <= r
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(256) void gemm1_f32(const float* __restrict__ x,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ row_token,
                                                 const float* __restrict__ wg,
                                                 const float* __restrict__ wu, int rows, int E,
                                                 int T, int TK, int H, int I,
                                                 float* __restrict__ h) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * I) return;
  const int r = i / I, n = i % I;
  const int e = group_of_row(offsets, r, E, T, TK);
  const float* xr = x + size_t(row_token_of(row_token, r, T, TK)) * H;
  const float* g = wg + (size_t(e) * I + n) * H;
  const float* u = wu + (size_t(e) * I + n) * H;
  float ag = 0.f, au = 0.f;
  for (int k = 0; k < H; ++k) {
    ag = fmaf(xr[k], g[k], ag);
    au = fmaf(xr[k], u[k], au);
  }
  h[i] = ag / (1.0f + expf(-ag)) * au;
}

__global__ __launch_bounds__(256) void gemm2_f32(const float* __restrict__ h,
                                                 const int32_t* __restrict__ offsets,
                                                 const float* __restrict__ wd, int rows, int E,
                                                 int T, int TK, int H, int I,
                                                 float* __restrict__ y) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * H) return;
  const int r = i / H, n = i % H;
  const int e = group_of_row(offsets, r, E, T, TK);
  const float* hr = h + size_t(r) * I;
  const float* d = wd + (size_t(e) * H + n) * I;
  float acc = 0.f;
  for (int k = 0; k < I; ++k) acc = fmaf(hr[k], d[k], acc);
  y[i] = acc;
}

// ---- launch configuration ---------------------------------------------------
constexpr int kBM = 128, kBN = 128, kWM = 2, kWN = 2;

static int m_tiles_upper(const moe_config& c, int bm) {
  const long long TK = 1LL * c.num_tokens * c.top_k;
  long long routed = (TK + 1LL * c.num_experts * (bm - 1)) / bm;
  routed = routed < TK ? routed : TK;
  return int(routed + 1LL * c.num_shared * ceil_div(c.num_tokens, bm));
}

hipError_t launch_gemm_router_bf16(const moe_config& c, const uint16_t* x, const uint16_t* w,
                                   float* z, hipStream_t s) {
  GemmArgs a{};
  a.A = x;
  a.B0 = w;
  a.b_stride = 0;
  a.C = z;
  a.ldc = c.num_experts;
  a.N = c.num_experts;
  a.K = c.hidden;
  a.E = 0;
  a.T = c.num_tokens;
  a.TK = 0;
  a.G = 1;
  a.n_tiles = ceil_div(c.num_experts, kBN);
  const int grid = ceil_div(c.num_tokens, kBM) * a.n_tiles;
  hipLaunchKernelGGL((grouped_gemm_bf16<kBM, kBN, kWM, kWN, kPlainF32>), dim3(grid),
                     dim3(kWM * kWN * 64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_grouped_ffn(const moe_config& c, const void* x, const int32_t* offsets,
                              const int32_t* row_token, const moe_expert_weights& w,
                              void* y_rows, const Workspace& ws, hipStream_t s) {
  const int T = c.num_tokens, E = c.num_experts, Ns = c.num_shared;
  const int TK = T * c.top_k, G = E + Ns, rows = TK + T * Ns;
  const int H = c.hidden, I = c.inter;
  if (c.w_dtype == MOE_F32) {
    hipLaunchKernelGGL(gemm1_f32, dim3(ceil_div(rows * I, 256)), dim3(256), 0, s,
                       static_cast<const float*>(x), offsets, row_token,
                       static_cast<const float*>(w.w_gate), static_cast<const float*>(w.w_up),
                       rows, E, T, TK, H, I, static_cast<float*>(ws.h));
    hipLaunchKernelGGL(gemm2_f32, dim3(ceil_div(rows * H, 256)), dim3(256), 0, s,
                       static_cast<const float*>(ws.h), offsets,
                       static_cast<const float*>(w.w_down), rows, E, T, TK, H, I,
                       static_cast<float*>(y_rows));
    return hipGetLastError();
  }
  if (c.w_dtype != MOE_BF16) return hipErrorNotSupported;
  hipLaunchKernelGGL(build_tiles, dim3(1), dim3(512), 0, s, offsets, E, Ns, T, TK, kBM, kBM,
                     ws.tiles1, ws.tiles2);
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(x);
  a.row_token = row_token;
  a.offsets = offsets;
  a.tile_off = ws.tiles1;
  a.B0 = static_cast<const uint16_t*>(w.w_gate);
  a.B1 = static_cast<const uint16_t*>(w.w_up);
  a.b_stride = 1LL * I * H;
  a.C = ws.h;
  a.ldc = I;
  a.N = I;
  a.K = H;
  a.E = E;
  a.T = T;
  a.TK = TK;
  a.G = G;
  a.n_tiles = ceil_div(I, kBN / 2);
  a.gather = 1;
  hipLaunchKernelGGL((grouped_gemm_bf16<kBM, kBN, kWM, kWN, kGatedBf16>),
                     dim3(m_tiles_upper(c, kBM) * a.n_tiles), dim3(kWM * kWN * 64), 0, s, a);
  GemmArgs d = a;
  d.A = static_cast<const uint16_t*>(ws.h);
  d.row_token = nullptr;
  d.gather = 0;
  d.tile_off = ws.tiles2;
  d.B0 = static_cast<const uint16_t*>(w.w_down);
  d.B1 = nullptr;
  d.b_stride = 1LL * H * I;
  d.C = y_rows;
  d.ldc = H;
  d.N = H;
  d.K = I;
  d.n_tiles = ceil_div(H, kBN);
  hipLaunchKernelGGL((grouped_gemm_bf16<kBM, kBN, kWM, kWN, kPlainBf16>),
                     dim3(m_tiles_upper(c, kBM) * d.n_tiles), dim3(kWM * kWN * 64), 0, s, d);
  return hipGetLastError();
}

}  // namespace moe
