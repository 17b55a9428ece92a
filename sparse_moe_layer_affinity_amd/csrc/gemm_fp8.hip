// FP8 (OCP e4m3) grouped expert GEMMs with fp32 block scales.
//
// "DeepSeek-V3 ... 技术解析" (devpress), section 2: weights are quantised per
// 128x128 block and activations per 1x128 tile; products run in FP8 and are
// promoted to FP32 every 128 elements of K.  Here that promotion is exact per
// block: for every 128-wide K block kb,
//     acc[n][t] += (sum_k qw[n][k] qa[t][k]) * s_w[n/128][kb] * s_a[t][kb]
// with the inner sum from one v_mfma_scale_f32_16x16x128_f8f6f4 (its own E8M0
// scales left at 1.0: the block scales are arbitrary fp32 values, which the
// hardware scale operands cannot carry).
//
// MI355X layout choice: the MFMA rows are weight rows and its columns tokens (the
// transpose of the bf16 kernel), so the four outputs a lane holds (rows 4*(l/16)+q,
// column l%16) share one token and one 128-row weight block, and the per-block
// rescale is one multiplier per lane: four FMAs per MFMA, on the VALU while the
// matrix core runs the next MFMA.  Accumulators therefore live in VGPRs.
//
// Tile: 256 weight rows (GEMM1: 128 gate rows over the matching 128 up rows) x
// 128 tokens; 4 waves, each 128 weight rows x 64 tokens = 8 x 4 MFMA blocks.
// K advances one 128-byte scale block per slice through two swizzled LDS buffers
// (48 KB each), the next slice's buffer loads in flight during the MFMAs.
#include "gemm_common.h"

namespace moe {

struct Fp8Args {
  const uint8_t* A;          // e4m3 activations: xq [T, K] (gather) or hq [rows, K]
  const float* a_scales;     // [a_rows, K/128]
  const int32_t* row_token;  // gather map of routed rows (gather only)
  const int32_t* offsets;    // [E+1]
  const int32_t* tile_off;   // [G+1] m-tile prefix (128 tokens per m-tile)
  const uint8_t* B0;         // e4m3 weights [G][N][K] (GEMM1: gate)
  const uint8_t* B1;         // GEMM1: up
  const float* S0;           // weight block scales [G][N/128][K/128] (GEMM1: gate)
  const float* S1;           // GEMM1: up
  long long b_stride;        // bytes per expert (N*K)
  long long s_stride;        // floats per expert
  uint16_t* C;               // bf16 output [rows, ldc]
  int ldc, N, K;
  int E, T, TK, G;
  int n_tiles;
  int gather;
  int a_rows;
};

template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_fp8(Fp8Args a) {
  constexpr int NT = 256;
  constexpr int BT = 128;                // tokens per tile
  constexpr int BW = 256;                // weight rows per tile
  constexpr int ROWS = BW + BT;          // LDS rows of 128 bytes (one K block)
  constexpr int CH = ROWS * 8 / NT;      // 16-byte chunks per thread per slice (12)
  constexpr int CW = BW * 8 / NT;        // of which weight chunks (8)
  constexpr int BN_OUT = MODE == kGatedBf16 ? BW / 2 : BW;
  __shared__ uint4 lds[2][ROWS * 8];

  // ---- tile decode: (expert, n-tile, m-tile), m innermost, XCD-contiguous ------
  const int total_m = a.tile_off[a.G];
  const int total = total_m * a.n_tiles;
  const int b = blockIdx.x;
  if (b >= total) return;
  const int per = total / kXcds, rem = total % kXcds;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + slot;
  int lo = 0, hi = a.G;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (a.tile_off[mid] * a.n_tiles <= logical) lo = mid; else hi = mid;
  }
  const int g = lo;
  const int mtiles = a.tile_off[g + 1] - a.tile_off[g];
  const int local = logical - a.tile_off[g] * a.n_tiles;
  const int nt = local / mtiles, mt = local % mtiles;
  int r0, r1;
  group_rows(a.offsets, g, a.E, a.T, a.TK, r0, r1);
  const int m0 = r0 + mt * BT;
  const int mvalid = min(BT, r1 - m0);
  const int n0 = nt * BN_OUT;
  const int tid = threadIdx.x;
  const int K = a.K, KBLK = a.K / 128;

  // ---- buffer descriptors and per-lane offsets ----------------------------------
  const __amdgpu_buffer_rsrc_t ra_src = make_rsrc(a.A, uint32_t(a.a_rows) * uint32_t(K));
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(a.a_scales, uint32_t(a.a_rows) * KBLK * 4u);
  const uint32_t b_bytes = uint32_t(a.N) * uint32_t(K);
  const __amdgpu_buffer_rsrc_t rb0 = make_rsrc(a.B0 + size_t(g) * a.b_stride, b_bytes);
  const __amdgpu_buffer_rsrc_t rb1 =
      MODE == kGatedBf16 ? make_rsrc(a.B1 + size_t(g) * a.b_stride, b_bytes) : rb0;
  const int trow = tid >> 3, kc0 = tid & 7;
  // weight chunk i (< CW) is weight row trow + 32 i of the tile (gated: i >= CW/2 up)
  constexpr int CWH = MODE == kGatedBf16 ? CW / 2 : CW;
  const uint32_t ob = uint32_t(n0 + trow) * uint32_t(K) + kc0 * 16;
  const uint32_t ob_step = 32u * uint32_t(K);
  // token chunk i (CW..CH-1) is tile row trow + 32 (i - CW)
  uint32_t oa[CH - CW];
#pragma unroll
  for (int i = 0; i < CH - CW; ++i) {
    const int row = trow + 32 * i;
    uint32_t o = kOob;
    if (row < mvalid) {
      const int r = m0 + row;
      const int src = a.gather ? row_token_of(a.row_token, r, a.T, a.TK) : r;
      o = uint32_t(src) * uint32_t(K) + kc0 * 16;
    }
    oa[i] = o;
  }
  const int st_base = trow * 8 + lds_slot(trow, kc0);

  uint4 rw[CW], rt[CH - CW];
  auto load_slice = [&](int kb) __attribute__((always_inline)) {
    const int kofs = kb * 128;
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int ih = i < CWH ? i : i - CWH;
      rw[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
          i < CWH ? rb0 : rb1, ob + uint32_t(ih) * ob_step, kofs, 0));
    }
#pragma unroll
    for (int i = 0; i < CH - CW; ++i)
      rt[i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(ra_src, oa[i], kofs, 0));
  };
  auto store_slice = [&](uint4* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CW; ++i) buf[st_base + i * NT] = rw[i];
#pragma unroll
    for (int i = 0; i < CH - CW; ++i) buf[BW * 8 + st_base + i * NT] = rt[i];
  };

  // ---- wave geometry: 2 (weight rows) x 2 (tokens) ------------------------------
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  const int wn = w & 1, wt = w >> 1;
  int w_row[8];                            // LDS row of this lane in weight block ib
#pragma unroll
  for (int ib = 0; ib < 8; ++ib) {
    int r;
    if (MODE == kGatedBf16) r = ib < 4 ? wn * 64 + ib * 16 : 128 + wn * 64 + (ib - 4) * 16;
    else r = wn * 128 + ib * 16;
    w_row[ib] = (r + (l & 15)) * 8;
  }
  const int t_row = (BW + wt * 64 + (l & 15)) * 8;       // + jb * 128
  const int slot0 = lds_slot(l & 15, 2 * (l >> 4)), slot1 = lds_slot(l & 15, 2 * (l >> 4) + 1);

  // activation scale offsets (floats) of this lane's 4 tokens; invalid rows read zero
  uint32_t osa[4];
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int row = wt * 64 + jb * 16 + (l & 15);
    uint32_t o = kOob;
    if (row < mvalid) {
      const int r = m0 + row;
      const int src = a.gather ? row_token_of(a.row_token, r, a.T, a.TK) : r;
      o = uint32_t(src) * uint32_t(KBLK) * 4u;
    }
    osa[jb] = o;
  }
  // weight block scales: this wave's weight rows lie in one 128-row block (per matrix)
  // (a wave past N in a partial tile computes zeros: clamp its scale block in range)
  const int nblk0 = min((MODE == kGatedBf16 ? n0 : n0 + wn * 128) / 128, ceil_div(a.N, 128) - 1);
  const float* sw0 = a.S0 + size_t(g) * a.s_stride + size_t(nblk0) * KBLK;
  const float* sw1 = MODE == kGatedBf16 ? a.S1 + size_t(g) * a.s_stride + size_t(n0 / 128) * KBLK
                                        : sw0;

  f32x4_t acc[8][4];
#pragma unroll
  for (int ib = 0; ib < 8; ++ib)
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) acc[ib][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const uint4* buf, int kb) __attribute__((always_inline)) {
    float sa[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
      sa[jb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rsa, osa[jb], kb * 4, 0));
    const float s_w0 = sw0[kb], s_w1 = sw1[kb];
    i32x8_t tf[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const uint4 lo4 = buf[t_row + jb * 128 + slot0], hi4 = buf[t_row + jb * 128 + slot1];
      tf[jb] = i32x8_t{int(lo4.x), int(lo4.y), int(lo4.z), int(lo4.w),
                       int(hi4.x), int(hi4.y), int(hi4.z), int(hi4.w)};
    }
#pragma unroll
    for (int ib = 0; ib < 8; ++ib) {
      const uint4 lo4 = buf[w_row[ib] + slot0], hi4 = buf[w_row[ib] + slot1];
      const i32x8_t wf = i32x8_t{int(lo4.x), int(lo4.y), int(lo4.z), int(lo4.w),
                                 int(hi4.x), int(hi4.y), int(hi4.z), int(hi4.w)};
      const float s_w = (MODE == kGatedBf16 && ib >= 4) ? s_w1 : s_w0;
#pragma unroll
      for (int jb = 0; jb < 4; ++jb) {
        const f32x4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            wf, tf[jb], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        const float s = sa[jb] * s_w;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[ib][jb][q] = fmaf(p[q], s, acc[ib][jb][q]);
      }
    }
  };

  const int nk = KBLK;
  load_slice(0);
  store_slice(lds[0]);
  if (nk > 1) load_slice(1);
  lds_barrier();
  for (int kb = 0; kb < nk; ++kb) {
    uint4* cur = lds[kb & 1];
    uint4* nxt = lds[(kb + 1) & 1];
    compute(cur, kb);
    if (kb + 1 < nk) store_slice(nxt);
    if (kb + 2 < nk) load_slice(kb + 2);
    lds_barrier();
  }

  // ---- epilogue: lane l holds weight rows 4*(l/16)+q of each block, token l%16 ----
#pragma unroll
  for (int jb = 0; jb < 4; ++jb) {
    const int rl = wt * 64 + jb * 16 + (l & 15);
    if (rl >= mvalid) continue;
    uint16_t* crow = a.C + size_t(m0 + rl) * a.ldc;
    if (MODE == kGatedBf16) {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) {
        const int col = n0 + wn * 64 + ib * 16 + 4 * (l >> 4);
        if (col >= a.N) continue;
        uint32_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = f32_to_bf16_bits(silu_fast(acc[ib][jb][q]) * acc[ib + 4][jb][q]);
        *reinterpret_cast<uint2*>(crow + col) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
    } else {
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) {
        const int col = n0 + wn * 128 + ib * 16 + 4 * (l >> 4);
        if (col >= a.N) continue;
        uint32_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = f32_to_bf16_bits(acc[ib][jb][q]);
        *reinterpret_cast<uint2*>(crow + col) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
      }
    }
  }
}

static int m_tiles_upper_fp8(const moe_config& c, int bm) {
  const long long TK = 1LL * c.num_tokens * c.top_k;
  long long routed = (TK + 1LL * c.num_experts * (bm - 1)) / bm;
  routed = routed < TK ? routed : TK;
  return int(routed + 1LL * c.num_shared * ceil_div(c.num_tokens, bm));
}

hipError_t launch_build_tiles(const moe_config& c, const int32_t* offsets, int bm1, int bm2,
                              int32_t* t1, int32_t* t2, hipStream_t s);

hipError_t launch_grouped_ffn_fp8(const moe_config& c, const void* x, const int32_t* offsets,
                                  const int32_t* row_token, const moe_expert_weights& w,
                                  void* y_rows, const Workspace& ws, hipStream_t s) {
  const int T = c.num_tokens, E = c.num_experts, Ns = c.num_shared;
  const int TK = T * c.top_k, G = E + Ns, rows = TK + T * Ns;
  const int H = c.hidden, I = c.inter;
  hipError_t err = launch_act_quant(x, T, H, ws.xq, ws.x_scales, s);
  if (err != hipSuccess) return err;
  err = launch_build_tiles(c, offsets, 128, 128, ws.tiles1, ws.tiles2, s);
  if (err != hipSuccess) return err;
  Fp8Args a{};
  a.A = ws.xq;
  a.a_scales = ws.x_scales;
  a.row_token = row_token;
  a.offsets = offsets;
  a.tile_off = ws.tiles1;
  a.B0 = static_cast<const uint8_t*>(w.w_gate);
  a.B1 = static_cast<const uint8_t*>(w.w_up);
  a.S0 = w.s_gate;
  a.S1 = w.s_up;
  a.b_stride = 1LL * I * H;
  a.s_stride = 1LL * (I / 128) * (H / 128);
  a.C = static_cast<uint16_t*>(ws.h);
  a.ldc = I;
  a.N = I;
  a.K = H;
  a.E = E;
  a.T = T;
  a.TK = TK;
  a.G = G;
  a.n_tiles = ceil_div(I, 128);
  a.gather = 1;
  a.a_rows = T;
  hipLaunchKernelGGL(grouped_gemm_fp8<kGatedBf16>, dim3(m_tiles_upper_fp8(c, 128) * a.n_tiles),
                     dim3(256), 0, s, a);
  err = launch_act_quant(ws.h, rows, I, ws.hq, ws.h_scales, s);
  if (err != hipSuccess) return err;
  Fp8Args d = a;
  d.A = ws.hq;
  d.a_scales = ws.h_scales;
  d.row_token = nullptr;
  d.gather = 0;
  d.a_rows = rows;
  d.tile_off = ws.tiles2;
  d.B0 = static_cast<const uint8_t*>(w.w_down);
  d.B1 = nullptr;
  d.S0 = w.s_down;
  d.S1 = nullptr;
  d.b_stride = 1LL * H * I;
  d.s_stride = 1LL * (H / 128) * (I / 128);
  d.C = static_cast<uint16_t*>(y_rows);
  d.ldc = H;
  d.N = H;
  d.K = I;
  d.n_tiles = ceil_div(H, 256);
  hipLaunchKernelGGL(grouped_gemm_fp8<kPlainBf16>, dim3(m_tiles_upper_fp8(c, 128) * d.n_tiles),
                     dim3(256), 0, s, d);
  return hipGetLastError();
}

}  // namespace moe
