// Weight gradients of the grouped SwiGLU experts on the matrix cores.
//
// "DeepSeek-V3 Technical Report 深度解读报告", section 2.2: each expert is a SwiGLU FFN
// W_down (silu(W_gate u) * (W_up u)); differentiated over the expert's rows r
// (u = x[token of r], a = W_gate u, b = W_up u, h = silu(a) b):
//   dW_gate[e] = sum_r da_r u_r^T,  dW_up[e] = sum_r db_r u_r^T,  dW_down[e] = sum_r dy_r h_r^T.
// The contraction runs over an expert's rows, a ragged range the host does not know
// (the offsets live on the device).  The MFMA wants both operands contiguous along
// the contraction, so the operands are first packed transposed: for every expert its
// rows become columns of a [features][padded rows] array, each expert's segment
// padded with zeros to a multiple of 64 rows (the padded offsets are prefix-summed on
// the device).  Then one GEMM per output family:
//   C_e[m][n] = sum_{k < P_e} A[m][poff_e + k] * B[n][poff_e + k]
// with (A, B) = ([da | db]^T, u^T) for dW_gate | dW_up (M = 2 inter) and (dy^T, h^T)
// for dW_down, fp32 accumulation in the fixed K order of the rows (deterministic).
//
// GEMM tile 256 x 256, four waves of 128 x 128 (4 x 4 v_mfma_f32_32x32x16_bf16
// accumulators in AGPRs, the MFMA computing the transposed tile so that a lane holds
// four adjacent output columns of one row; the tile leaves through LDS as whole
// 512-byte row segments).  K advances 64 rows
// per stage through two 64 KB LDS buffers filled by buffer loads in LDS mode; rows
// are 128 bytes, chunk c of row r in slot c ^ (r & 7) ^ ((r >> 3) & 1) (conflict-free
// fragment reads).  One workgroup per (expert, tile); the shared experts' tiles
// (the long contractions) are dispatched first.  Experts without rows get zeros.
#include "gemm_common.h"

namespace moe {

constexpr int kWgPad = 64;          // rows per padded segment unit

// poff[g] = sum over groups g' < g of roundup(rows of g', 64), g <= G (one workgroup,
// G <= 512): routed group e has offsets[e+1] - offsets[e] rows, a shared group T
__global__ __launch_bounds__(512) void wgrad_offsets(const int32_t* __restrict__ offsets, int E,
                                                     int Ns, int T, int32_t* __restrict__ poff) {
  __shared__ int pre[512];
  const int t = threadIdx.x, G = E + Ns;
  int v = 0;
  if (t < G) {
    const int r = t < E ? offsets[t + 1] - offsets[t] : T;
    v = (r + kWgPad - 1) / kWgPad * kWgPad;
  }
  pre[t] = v;
  __syncthreads();
  for (int d = 1; d < 512; d <<= 1) {
    const int u = t >= d ? pre[t - d] : 0;
    __syncthreads();
    pre[t] += u;
    __syncthreads();
  }
  if (t < G) poff[t + 1] = pre[t];
  if (t == 0) poff[0] = 0;
}

// Transposed packing of one operand: dst[c][poff_g + j] = value of grouped row
// r0_g + j, column c (c < C), for j < rows of g, zero for the padding.
//   kPackRows:   src[r][col0 + c]
//   kPackGather: src[token of r][col0 + c]          (x, gathered like the forward)
//   kPackSwiglu: silu(a) * b, a = src[r][col0 + c], b = src[r][col1 + c] (h, rounded
//                to bf16 once)
// 64 x 64 tiles through LDS (pitch 72), 16-byte vectors on both sides.
enum { kPackRows = 0, kPackGather = 1, kPackSwiglu = 2 };
struct PackArgs {
  const uint16_t* src;
  long long ld_src;
  int col0, col1, C;
  uint16_t* dst;
  long long ld_dst;
  const int32_t* poff;
  const int32_t* offsets;
  const int32_t* row_token;
  int T, TK, E, G;
};

template <int MODE>
__global__ __launch_bounds__(256) void wgrad_pack(PackArgs q) {
  constexpr int kPitch = 72;
  __shared__ __attribute__((aligned(16))) uint16_t tile[64 * kPitch];
  const int p0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  if (p0 >= q.poff[q.G]) return;
  int lo = 0, hi = q.G;                       // largest g with poff[g] <= p0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (q.poff[mid] <= p0) lo = mid; else hi = mid;
  }
  const int g = lo;
  int r0, r1;
  group_rows(q.offsets, g, q.E, q.T, q.TK, r0, r1);
  const int j0 = p0 - q.poff[g];
  const int lane8 = (threadIdx.x % 8) * 8, row = threadIdx.x / 8;     // row 0..31
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int i = row + 32 * pass, cc = c0 + lane8;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (j0 + i < r1 - r0 && cc < q.C) {
      int r = r0 + j0 + i;
      if (MODE == kPackGather) r = row_token_of(q.row_token, r, q.T, q.TK);
      const uint16_t* s = q.src + size_t(r) * q.ld_src;
      v = *reinterpret_cast<const uint4*>(s + q.col0 + cc);
      if (MODE == kPackSwiglu) {
        const uint4 b = *reinterpret_cast<const uint4*>(s + q.col1 + cc);
        const uint32_t av[4] = {v.x, v.y, v.z, v.w}, bv[4] = {b.x, b.y, b.z, b.w};
        uint32_t hv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a0 = bf16_bits_to_f32(av[e] & 0xffffu), a1 = bf16_bits_to_f32(av[e] >> 16);
          const float b0 = bf16_bits_to_f32(bv[e] & 0xffffu), b1 = bf16_bits_to_f32(bv[e] >> 16);
          hv[e] = pack_bf16x2(silu_fast(a0) * b0, silu_fast(a1) * b1);
        }
        v = make_uint4(hv[0], hv[1], hv[2], hv[3]);
      }
    }
    *reinterpret_cast<uint4*>(&tile[i * kPitch + lane8]) = v;
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int jc = row + 32 * pass, cc = c0 + jc;          // source column jc
    uint16_t e[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) e[u] = tile[(lane8 + u) * kPitch + jc];
    if (cc < q.C)
      *reinterpret_cast<uint4*>(q.dst + size_t(cc) * q.ld_dst + p0 + lane8) =
          make_uint4(e[0] | (uint32_t(e[1]) << 16), e[2] | (uint32_t(e[3]) << 16),
                     e[4] | (uint32_t(e[5]) << 16), e[6] | (uint32_t(e[7]) << 16));
  }
}

struct WgMfmaArgs {
  const uint16_t* A;       // [M][ld] bf16, contraction contiguous
  const uint16_t* B;       // [N][ld] bf16
  long long ld;            // elements per packed row
  const int32_t* poff;     // [G+1] padded row offsets (multiples of 64)
  float* C0;               // rows m < M0: C0[g][m][n]
  float* C1;               // rows m >= M0: C1[g][m - M0][n]
  int M0;
  long long cstride;       // floats per group in C0 and C1 (M0 * N)
  int M, N, E, G;
  int n_tiles;             // ceil(N / 256)
};

__global__ __launch_bounds__(256) void wgrad_mfma(WgMfmaArgs p) {
  constexpr int BM = 256, BN = 256, ROWB = 128;
  constexpr uint32_t kBOff = BM * ROWB;                  // B rows follow A rows in a stage
  constexpr uint32_t kStage = (BM + BN) * ROWB;          // 64 KB
  __shared__ __attribute__((aligned(1024))) uint4 lds[2 * kStage / 16];
  const int g = (int(blockIdx.y) + p.E) % p.G;           // shared experts first
  const int mt = int(blockIdx.x) / p.n_tiles, nt = int(blockIdx.x) % p.n_tiles;
  const int m0 = mt * BM, n0 = nt * BN;
  const int k0 = p.poff[g];
  const int nk = (p.poff[g + 1] - k0) / 64;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const uint32_t row_bytes = uint32_t(p.ld) * 2u;
  const int mrows = min(BM, p.M - m0), nrows = min(BN, p.N - n0);
  const __amdgpu_buffer_rsrc_t rsrc_a =
      make_rsrc(p.A + size_t(m0) * p.ld + k0, uint32_t(mrows) * row_bytes);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      make_rsrc(p.B + size_t(n0) * p.ld + k0, uint32_t(nrows) * row_bytes);
  // this wave loads rows 64 w .. 64 w + 63 of A and of B: instruction j puts rows
  // 64 w + 8 j + (l >> 3), lane l into slot l & 7, which holds chunk
  // (l & 7) ^ (l >> 3) ^ (j & 1)
  uint32_t voff_a[8], voff_b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r = 64 * w + 8 * j + (l >> 3);
    const uint32_t chunk = uint32_t((l & 7) ^ (l >> 3) ^ (j & 1)) * 16u;
    voff_a[j] = r < mrows ? uint32_t(r) * row_bytes + chunk : kOob;
    voff_b[j] = r < nrows ? uint32_t(r) * row_bytes + chunk : kOob;
  }
  const uint32_t lds_base = uint32_t(uintptr_t(&lds[0]));
  auto issue = [&](int ks) __attribute__((always_inline)) {
    const uint32_t buf = lds_base + uint32_t(ks & 1) * kStage + uint32_t(64 * w) * ROWB;
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16(rsrc_a, voff_a[j], uint32_t(ks) * ROWB, buf + j * 1024u);
#pragma unroll
    for (int j = 0; j < 8; ++j) dma16(rsrc_b, voff_b[j], uint32_t(ks) * ROWB, buf + kBOff + j * 1024u);
  };

  // wave tile: rows wm * 128 .. of A (output rows), rows wn * 128 .. of B (columns)
  const int wm = w >> 1, wn = w & 1;
  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  uint32_t sl[4];
#pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) sl[s4] = uint32_t((2 * s4 + (l >> 5)) ^ (l & 7) ^ ((l >> 3) & 1)) * 16u;
  const uint32_t a_lane = uint32_t(wm * 128 + (l & 31)) * ROWB;
  const uint32_t b_lane = kBOff + uint32_t(wn * 128 + (l & 31)) * ROWB;
  auto frag = [&](uint32_t byte) __attribute__((always_inline)) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(
                                            reinterpret_cast<const char*>(lds) + byte));
  };

  if (nk > 0) issue(0);
  for (int k = 0; k < nk; ++k) {
    wait_vmcnt<0>();
    stage_barrier();                         // stage k is in LDS; buffer (k + 1) & 1 is free
    if (k + 1 < nk) issue(k + 1);
    const uint32_t buf = uint32_t(k & 1) * kStage;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      bf16x8_t fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = frag(buf + a_lane + uint32_t(i * 32) * ROWB + sl[s4]);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = frag(buf + b_lane + uint32_t(j * 32) * ROWB + sl[s4]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[j], fa[i], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue.  Value r of lane l of block (i, j) is output row wm*128 + 32 i + (l & 31),
  // column wn*128 + 32 j + 8 (r >> 2) + 4 (l >> 5) + (r & 3).  Each wave stages one
  // 32 x 128 fp32 strip at a time (its rows 32 i ..) in its own 16.5 KB of LDS (row
  // pitch 132 floats), then stores it as whole 512-byte row segments: each store
  // instruction writes two rows.
  stage_barrier();                           // every wave is done with the operand buffers
  constexpr int kPitch = 132;
  float* stg = reinterpret_cast<float*>(lds) + w * (32 * kPitch);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(stg + (l & 31) * kPitch + 32 * j + 8 * q + 4 * (l >> 5)) =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                        acc[i][j][4 * q + 3]);
    const int n = n0 + wn * 128 + 4 * (l & 31);
#pragma unroll
    for (int rr = 0; rr < 32; rr += 2) {
      const int row = rr + (l >> 5);
      const int m = m0 + wm * 128 + 32 * i + row;
      const float4 v = *reinterpret_cast<const float4*>(stg + row * kPitch + 4 * (l & 31));
      if (m < p.M && n < p.N) {
        float* crow = m < p.M0 ? p.C0 + size_t(g) * p.cstride + size_t(m) * p.N
                               : p.C1 + size_t(g) * p.cstride + size_t(m - p.M0) * p.N;
        *reinterpret_cast<float4*>(crow + n) = v;
      }
    }
  }
}

// Rows of the packed, padded row space: every group padded to a multiple of 64.
long long wgrad_packed_rows(const moe_config& c) {
  const long long T = c.num_tokens, K = c.top_k, Ns = c.num_shared, G = c.num_experts + Ns;
  return (T * (K + Ns) + kWgPad * G + 63) / 64 * 64;
}

hipError_t launch_expert_wgrad_mfma(const moe_config& c, const void* x, const int32_t* offsets,
                                    const int32_t* row_token, const void* dy_rows,
                                    const uint16_t* ab, const uint16_t* dab, float* dw_gate,
                                    float* dw_up, float* dw_down, const WgradPackWorkspace& ws,
                                    hipStream_t s) {
  const int T = c.num_tokens, K = c.top_k, Ns = c.num_shared, E = c.num_experts, G = E + Ns;
  const int H = c.hidden, I = c.inter, TK = T * K;
  const long long ld = wgrad_packed_rows(c);
  hipLaunchKernelGGL(wgrad_offsets, dim3(1), dim3(512), 0, s, offsets, E, Ns, T, ws.poff);
  PackArgs q{};
  q.poff = ws.poff;
  q.offsets = offsets;
  q.row_token = row_token;
  q.T = T;
  q.TK = TK;
  q.E = E;
  q.G = G;
  q.ld_dst = ld;
  const dim3 blk(256);
  const int pblocks = int(ld / 64);
  // u^T (x gathered), dy^T, [da | db]^T, h^T
  q.src = static_cast<const uint16_t*>(x);
  q.ld_src = H;
  q.col0 = 0;
  q.C = H;
  q.dst = ws.xt;
  hipLaunchKernelGGL(wgrad_pack<kPackGather>, dim3(ceil_div(H, 64), pblocks), blk, 0, s, q);
  q.src = static_cast<const uint16_t*>(dy_rows);
  q.dst = ws.dyt;
  hipLaunchKernelGGL(wgrad_pack<kPackRows>, dim3(ceil_div(H, 64), pblocks), blk, 0, s, q);
  q.src = dab;
  q.ld_src = 2LL * I;
  q.C = 2 * I;
  q.dst = ws.dabt;
  hipLaunchKernelGGL(wgrad_pack<kPackRows>, dim3(ceil_div(2 * I, 64), pblocks), blk, 0, s, q);
  q.src = ab;
  q.col0 = 0;
  q.col1 = I;
  q.C = I;
  q.dst = ws.ht;
  hipLaunchKernelGGL(wgrad_pack<kPackSwiglu>, dim3(ceil_div(I, 64), pblocks), blk, 0, s, q);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  WgMfmaArgs p{};
  p.ld = ld;
  p.poff = ws.poff;
  p.E = E;
  p.G = G;
  // dW_gate | dW_up: A = [da | db]^T (2I rows), B = u^T (H rows)
  p.A = ws.dabt;
  p.B = ws.xt;
  p.M = 2 * I;
  p.N = H;
  p.M0 = I;
  p.C0 = dw_gate;
  p.C1 = dw_up;
  p.cstride = 1LL * I * H;
  p.n_tiles = ceil_div(H, 256);
  hipLaunchKernelGGL(wgrad_mfma, dim3(ceil_div(2 * I, 256) * p.n_tiles, G), blk, 0, s, p);
  // dW_down: A = dy^T (H rows), B = h^T (I rows)
  p.A = ws.dyt;
  p.B = ws.ht;
  p.M = H;
  p.N = I;
  p.M0 = H;
  p.C0 = dw_down;
  p.C1 = dw_down;
  p.cstride = 1LL * H * I;
  p.n_tiles = ceil_div(I, 256);
  hipLaunchKernelGGL(wgrad_mfma, dim3(ceil_div(H, 256) * p.n_tiles, G), blk, 0, s, p);
  return hipGetLastError();
}

}  // namespace moe
