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
// rescale is one multiplier per lane: four FMAs per MFMA.  The accumulators live in
// VGPRs (the VALU adds into them), and this file is compiled with MFMA results in
// VGPRs as well, so no copies out of AGPRs.  Each wave runs its MFMAs and rescales as
// a software pipeline: the products of weight block ib-1 are rescaled between the
// MFMAs of block ib (each product read four MFMAs after its MFMA was issued, so the
// VALU never waits on the matrix core and no wait states are needed).
//
// Tiles: 256 weight rows x 256 tokens for both GEMMs (GEMM1: 128 gate rows over the
// matching 128 up rows, so a tile holds 128 h columns, one whole 1x128 block, and h is
// quantised to e4m3 in its epilogue), 8 waves (two per SIMD: one wave's rescale FMAs
// run while the other's MFMAs hold the matrix core) of 128 weight rows x 64 tokens =
// 8 x 4 MFMA blocks, 128 accumulators per lane.  Row blocks are 256 rows; an expert
// with more splits into a pair of blocks (the last pair evenly), and a pair's two
// blocks take adjacent slots of one XCD n-tile by n-tile, so they stream each weight
// tile side by side through that L2.  Against 256 x 160 tiles this loads a quarter
// fewer bytes per MFMA.  K advances one 128-byte scale block per stage.  Operands and
// scales go global -> LDS with buffer loads in LDS mode into two stage buffers each,
// one workgroup barrier per stage, after which stage k+1's loads go out into the
// buffers stage k-1 left; a stage's token fragments and scales are read into registers
// at its start.
#include "gemm_common.h"

namespace moe {


template <int MODE>
__global__ __launch_bounds__(512) void grouped_gemm_fp8(Fp8Args a) {
  constexpr bool GATED = MODE == kGatedBf16;
  // 256 weight rows (gated: 128 gate over the matching 128 up rows, 128 h columns: one
  // 1x128 block of h) x 256 tokens (one row block)
  constexpr int BW = 256, BT = kFp8BT32, ROWB = 128;
  constexpr int WSTAGE = BW * ROWB, TSTAGE = BT * ROWB;   // 32 KB each
  constexpr int NTB = 4;                                  // 16-token blocks per wave (64 tokens)
  // LDS: two token and two weight stage buffers, two token-scale buffers (waves 0..3,
  // 256 bytes each) and two weight-scale buffers (waves 4..7, 256 bytes each: 4 and 5
  // one block scale each, 6 and 7 a dummy), the epilogue's amax exchange
  constexpr uint32_t kTOff = 0;
  constexpr uint32_t kWOff = 2 * TSTAGE;
  constexpr uint32_t kSaOff = kWOff + 2 * WSTAGE;
  constexpr uint32_t kSaStage = 1024;
  constexpr uint32_t kSwOff = kSaOff + 2 * kSaStage;
  constexpr uint32_t kSwStage = 1024;
  constexpr uint32_t kAmOff = kSwOff + 2 * kSwStage;
  constexpr uint32_t kLdsBytes = kAmOff + 8 * 64 * 4;
  __shared__ __attribute__((aligned(1024))) uint4 lds[kLdsBytes / 16];

  // ---- tile decode: pairs of adjacent schedule positions (one expert's two blocks of
  // a split, or two lone blocks) dealt to the XCDs in snake order, the n-tiles of the
  // pair's two blocks interleaved on consecutive slots of one XCD, so the two blocks of
  // an expert stream each weight tile side by side through that XCD's L2 -------------
  const int b = blockIdx.x;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int per = 2 * a.n_tiles;
  const int rp = slot / per, rem = slot - rp * per;
  const int nt = rem >> 1;
  const int q = rp * kXcds + ((rp & 1) ? kXcds - 1 - xcd : xcd);
  const int pos = 2 * q + (rem & 1);
  if (pos >= *a.sched_n) return;
  const int4 blk = a.sched[pos];
  const int g = blk.x, m0 = blk.y, mvalid = blk.z;
  const int n0 = nt * (GATED ? BW / 2 : BW);
  const int tid = threadIdx.x;
  const int K = a.K, KBLK = a.K / 128;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;

  // ---- this wave's share of every stage: weight rows 32 w .., token rows 32 w .. ----
  // gated: stage rows 0..127 are gate rows n0.., 128..255 the matching up rows
  const bool up = GATED && w >= 4;
  const int wrow0 = GATED ? n0 + 32 * (w & 3) : n0 + 32 * w;
  const __amdgpu_buffer_rsrc_t rsrc_w =
      make_rsrc((up ? a.B1 : a.B0) + size_t(g) * a.b_stride, uint32_t(a.N) * uint32_t(K));
  const __amdgpu_buffer_rsrc_t rsrc_t = make_rsrc(a.A, uint32_t(a.a_rows) * uint32_t(K));
  // stage row 32 w + 8 j + (l >> 3), j = 0..3 (bit 3 of the row is j & 1): loads j and
  // j + 2 are 16 rows apart, a uniform offset that rides in the scalar operand
  uint32_t voff_w[2], voff_t[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t chunk = uint32_t((l & 7) ^ (l >> 3) ^ j) * 16u;
    voff_w[j] = uint32_t(wrow0 + 8 * j + (l >> 3)) * uint32_t(K) + chunk;   // rows >= N read zero
  }
  // shared-expert tiles map rows to consecutive tokens; routed rows gather
  const bool lookup = a.gather && m0 < a.TK;
  const int tbase = !a.gather ? m0 : (lookup ? 0 : (m0 - a.TK) % a.T);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int trow = 32 * w + 8 * j + (l >> 3);
    const uint32_t chunk = uint32_t((l & 7) ^ (l >> 3) ^ (j & 1)) * 16u;
    const int src = trow < mvalid ? (lookup ? a.row_token[m0 + trow] : tbase + trow) : 0;
    voff_t[j] = trow < mvalid ? uint32_t(src) * uint32_t(K) + chunk : kOob;
  }
  // one scale load per wave per stage: waves 0..3 the token scales of rows 64 w + lane
  // (in grouped-row order), waves 4 and 5 one weight block scale each (lane 0; gated:
  // the gate and the up block; plain: the tile's two 128-row blocks, clamped in range:
  // a block past N only feeds outputs that are never stored), 6 and 7 nothing useful
  __amdgpu_buffer_rsrc_t rsrc_s;
  uint32_t voff_s = kOob;
  if (w < 4) {
    rsrc_s = make_rsrc(a.a_scales, uint32_t(a.scale_rows) * KBLK * 4u);
    const int row = 64 * w + l;
    if (row < mvalid) voff_s = uint32_t(m0 + row) * 4u;
  } else {
    const bool sup = GATED && w == 5;
    const int blk_n = min(GATED ? n0 / 128 : n0 / 128 + (w - 4), ceil_div(a.N, 128) - 1);
    rsrc_s = make_rsrc((sup ? a.S1 : a.S0) + size_t(g) * a.s_stride, uint32_t(a.s_stride) * 4u);
    if (l == 0 && w < 6) voff_s = uint32_t(blk_n * KBLK) * 4u;
  }
  // K block ks of the scales: token scales [K/128, scale_rows], weight scales [.., K/128]
  const uint32_t s_step = w < 4 ? uint32_t(a.scale_rows) * 4u : 4u;
  const uint32_t lds_base = uint32_t(uintptr_t(&lds[0]));
  const uint32_t wave_w = lds_base + kWOff + uint32_t(w) * (WSTAGE / 8);
  const uint32_t wave_t = lds_base + kTOff + uint32_t(w) * (TSTAGE / 8);
  const uint32_t wave_s = lds_base + (w < 4 ? kSaOff + 256u * w : kSwOff + 256u * (w - 4));
  const uint32_t s_par = w < 4 ? kSaStage : kSwStage;

  auto load_w = [&](int ks) __attribute__((always_inline)) {
    const uint32_t dst = wave_w + uint32_t(ks & 1) * WSTAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(rsrc_w, voff_w[j & 1], uint32_t(ks) * ROWB + uint32_t(j >> 1) * 16u * uint32_t(K),
            dst + j * 1024u);
  };
  // token rows of stage ks and its scales (buffers ks & 1)
  auto load_t = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(rsrc_t, voff_t[j], uint32_t(ks) * ROWB, wave_t + uint32_t(ks & 1) * TSTAGE + j * 1024u);
    dma4(rsrc_s, voff_s, uint32_t(ks) * s_step,
         __builtin_amdgcn_readfirstlane(wave_s + uint32_t(ks & 1) * s_par));
  };

  // ---- wave geometry: 2 (weight rows, 128 each) x 4 (tokens, 64 each) -------------
  const int wn = w & 1, wt = w >> 1;
  // LDS rows of this lane: weight block ib at w_lane + w_blk(ib) (gated: blocks 0..3
  // gate rows, 4..7 the matching up rows), token block jb at t_row + 16 jb; the lane's
  // two K chunks 2 (l >> 4) and 2 (l >> 4) + 1, XOR-swizzled (the second is the first ^ 16)
  const int t_row = wt * 64 + (l & 15);
  const uint32_t sl0 = uint32_t((2 * (l >> 4)) ^ (l & 7) ^ ((l >> 3) & 1)) * 16u;
  const uint32_t w_lane = uint32_t((GATED ? wn * 64 : wn * 128) + (l & 15)) * ROWB + sl0;
  const uint32_t t_lane = uint32_t(t_row) * ROWB + sl0;
  auto w_blk = [](int ib) constexpr {
    return uint32_t(GATED ? (ib < 4 ? ib * 16 : 128 + (ib - 4) * 16) : ib * 16) * ROWB;
  };

  // token blocks of this wave that hold rows: the MFMAs of empty ones are skipped
  const int njb = min(NTB, max(0, (mvalid - wt * 64 + 15) >> 4));
  auto body = [&](auto njb_tag) __attribute__((always_inline)) {
    constexpr int NJB = decltype(njb_tag)::value;
    constexpr int NJ1 = NJB > 0 ? NJB : 1;
    f32x4_t acc[8][NJ1];
  #pragma unroll
    for (int ib = 0; ib < 8; ++ib)
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb) acc[ib][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // fragment at lane byte lb (first chunk; the second is lb ^ 16) plus offset off
    auto lds_frag = [&](uint32_t lb, uint32_t off) __attribute__((always_inline)) {
      const char* base = reinterpret_cast<const char*>(lds);
      const uint4 lo4 = *reinterpret_cast<const uint4*>(base + lb + off);
      const uint4 hi4 = *reinterpret_cast<const uint4*>(base + (lb ^ 16u) + off);
      return i32x8_t{int(lo4.x), int(lo4.y), int(lo4.z), int(lo4.w),
                     int(hi4.x), int(hi4.y), int(hi4.z), int(hi4.w)};
    };
    auto lds_f32 = [&](uint32_t byte) __attribute__((always_inline)) {
      return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lds) + byte);
    };

    // One barrier per stage k: stage k's tokens, scales and weights are in LDS, and
    // every wave is done with stage k-1, whose buffers take stage k+1.  A stage's token
    // fragments and scales go into registers at its start; the MFMAs of weight block ib
    // run while the products of block ib-1 are rescaled (each product read NJB MFMAs
    // after its MFMA was issued).
    const int nk = KBLK;
    load_t(0);
    load_w(0);
    for (int k = 0; k < nk; ++k) {
      wait_vmcnt<0>();
      stage_barrier();
      if (k + 1 < nk) {
        load_t(k + 1);
        load_w(k + 1);
      }
      const uint32_t wb = kWOff + uint32_t(k & 1) * WSTAGE;
      const uint32_t tb = kTOff + uint32_t(k & 1) * TSTAGE;
      const uint32_t sp = uint32_t(k & 1);
      i32x8_t tf[NJ1];
      float s[2][NJ1];                                   // s_a * s_w per weight half
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb) tf[jb] = lds_frag(t_lane, tb + uint32_t(16 * jb) * ROWB);
      const float s_w0 = lds_f32(kSwOff + sp * kSwStage + (GATED ? 0u : 256u * wn));
      const float s_w1 = GATED ? lds_f32(kSwOff + sp * kSwStage + 256u) : s_w0;
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const float s_a = lds_f32(kSaOff + sp * kSaStage + uint32_t(t_row + 16 * jb) * 4u);
        s[0][jb] = s_a * s_w0;
        s[1][jb] = s_a * s_w1;
      }
      i32x8_t wfb[2];
      f32x4_t pt[2][NJ1];
      if constexpr (NJB > 0) wfb[0] = lds_frag(w_lane + wb, w_blk(0));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NJB > 0) {
        static_for<0, 8>([&](auto ib_tag) __attribute__((always_inline)) {
          constexpr int ib = decltype(ib_tag)::value;
          if constexpr (ib + 1 < 8) wfb[(ib + 1) & 1] = lds_frag(w_lane + wb, w_blk(ib + 1));
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int jb = 0; jb < NJB; ++jb) {
            pt[ib & 1][jb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                wfb[ib & 1], tf[jb], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
            if constexpr (ib > 0) {
              constexpr int h = (GATED && ib - 1 >= 4) ? 1 : 0;
  #pragma unroll
              for (int qq = 0; qq < 4; ++qq)
                acc[ib - 1][jb][qq] = fmaf(pt[(ib - 1) & 1][jb][qq], s[h][jb], acc[ib - 1][jb][qq]);
            }
          }
          if constexpr (ib > 0) {
            // issue order: one MFMA (mask 0x008), then the four VALU FMAs (0x002) of the
            // product NJB MFMAs back, NJB times
  #pragma unroll
            for (int jb = 0; jb < NJB; ++jb) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        });
        constexpr int h7 = GATED ? 1 : 0;
  #pragma unroll
        for (int jb = 0; jb < NJB; ++jb)
  #pragma unroll
          for (int qq = 0; qq < 4; ++qq) acc[7][jb][qq] = fmaf(pt[1][jb][qq], s[h7][jb], acc[7][jb][qq]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- epilogue: lane l holds weight rows 4*(l/16)+q of each block, token l%16 ----
    if constexpr (GATED) {
      // h quantised to e4m3 per 1x128 block here; staging in the two token buffers
      fp8_epilogue_hquant<NJB, 2, 4, 64>(acc, w, l, m0, mvalid, n0, a.Q, a.ldc, a.QS, a.scale_rows,
                                         reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + kAmOff),
                                         reinterpret_cast<uint32_t*>(lds), false);
    } else {
      // bf16 rows through LDS: each wave stages its 64 tokens x 128 columns (16 KB, in
      // the operand buffers, free once every wave is past the barrier) as rows of 256
      // bytes, 16-byte chunk c of row r in slot c ^ (r & 15), then stores whole 16-byte
      // chunks of four rows per instruction (a row's 256 bytes contiguous)
      stage_barrier();
      char* const stg = reinterpret_cast<char*>(lds) + w * 16384;
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const int r = jb * 16 + (l & 15);
  #pragma unroll
        for (int ib = 0; ib < 8; ++ib) {
          const int cc = 2 * ib + (l >> 5);                // 16-byte chunk of the row
          const f32x4_t& v = acc[ib][jb];
          *reinterpret_cast<uint2*>(stg + r * 256 + ((cc ^ (r & 15)) << 4) + ((l >> 4) & 1) * 8) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      const int cc = l & 15;
      const int col = n0 + wn * 128 + cc * 8;
  #pragma unroll
      for (int r0 = 0; r0 < 16 * NJB; r0 += 4) {
        const int r = r0 + (l >> 4);
        const int rl = wt * 64 + r;
        const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 256 + ((cc ^ (r & 15)) << 4));
        if (rl < mvalid && col < a.N)
          *reinterpret_cast<uint4*>(a.C + size_t(m0 + rl) * a.ldc + col) = v;
      }
    }
  };
  if (njb >= 4) body(std::integral_constant<int, 4>{});
  else if (njb == 3) body(std::integral_constant<int, 3>{});
  else if (njb == 2) body(std::integral_constant<int, 2>{});
  else if (njb == 1) body(std::integral_constant<int, 1>{});
  else body(std::integral_constant<int, 0>{});
}

hipError_t launch_build_schedule(const moe_config& c, const int32_t* offsets, int bm, int4* sched,
                                 int32_t* sched_n, hipStream_t s);

// the power-of-two-scale kernel (gemm_fp8p2.hip): 256 weight rows x 320 tokens per tile
hipError_t launch_gemm_fp8p2(const Fp8Args& a, bool gated, int n_tiles_blocks, hipStream_t s);

hipError_t launch_grouped_ffn_fp8(const moe_config& c, const void* x, const int32_t* offsets,
                                  const int32_t* row_token, const moe_expert_weights& w,
                                  void* y_rows, const Workspace& ws, hipStream_t s) {
  const int T = c.num_tokens, Ns = c.num_shared;
  const int TK = T * c.top_k, rows = TK + T * Ns;
  const int H = c.hidden, I = c.inter;
  const bool pow2 = c.w_dtype == MOE_E4M3_POW2;
  hipError_t err = launch_act_quant(x, T, H, ws.xq, ws.x_scales, s, true, pow2);
  if (err != hipSuccess) return err;
  // the x scales in grouped-row order, so each stage's scale loads are contiguous
  err = launch_gather_scales(c, ws.x_scales, row_token, H / 128, ws.xg_scales, s);
  if (err != hipSuccess) return err;
  // row blocks: of up to 320 rows for the power-of-two kernel, 256 for this one
  const int bm = pow2 ? kFp8BT : kFp8BT32;
  err = launch_build_schedule(c, offsets, bm, ws.sched, ws.sched_n, s);
  if (err != hipSuccess) return err;
  const int nblk = expert_row_blocks_upper(c, bm);
  const int rounds = ceil_div(nblk, kXcds);
  // this kernel's grid: pairs of positions, two slots per n-tile
  const int pair_rounds = ceil_div(ceil_div(nblk, 2), kXcds);
  // GEMM1: gated; both kernels' tiles hold 128 h columns, a whole 1x128 block, and
  // quantise h to e4m3 (codes + scales) in their epilogue
  Fp8Args a{};
  a.A = ws.xq;
  a.a_scales = ws.xg_scales;
  a.row_token = row_token;
  a.sched = ws.sched;
  a.sched_n = ws.sched_n;
  a.B0 = static_cast<const uint8_t*>(w.w_gate);
  a.B1 = static_cast<const uint8_t*>(w.w_up);
  a.S0 = w.s_gate;
  a.S1 = w.s_up;
  a.b_stride = 1LL * I * H;
  a.s_stride = 1LL * (I / 128) * (H / 128);
  a.Q = ws.hq;
  a.QS = ws.h_scales;
  a.ldc = I;
  a.N = I;
  a.K = H;
  a.T = T;
  a.TK = TK;
  a.n_tiles = ceil_div(I, 128);
  a.gather = 1;
  a.a_rows = T;
  a.scale_rows = rows;
  if (pow2) {
    err = launch_gemm_fp8p2(a, true, rounds * kXcds * a.n_tiles, s);
    if (err != hipSuccess) return err;
  } else {
    hipLaunchKernelGGL(grouped_gemm_fp8<kGatedBf16>, dim3(pair_rounds * kXcds * 2 * a.n_tiles), dim3(512), 0, s, a);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  // GEMM2: plain, on the e4m3 h
  Fp8Args d = a;
  d.A = ws.hq;
  d.a_scales = ws.h_scales;
  d.row_token = nullptr;
  d.gather = 0;
  d.a_rows = rows;
  d.scale_rows = rows;
  d.B0 = static_cast<const uint8_t*>(w.w_down);
  d.B1 = nullptr;
  d.S0 = w.s_down;
  d.S1 = nullptr;
  d.b_stride = 1LL * H * I;
  d.s_stride = 1LL * (H / 128) * (I / 128);
  d.C = static_cast<uint16_t*>(y_rows);
  d.Q = nullptr;
  d.QS = nullptr;
  d.ldc = H;
  d.N = H;
  d.K = I;
  if (pow2) {
    d.n_tiles = ceil_div(H, 256);
    return launch_gemm_fp8p2(d, false, rounds * kXcds * d.n_tiles, s);
  }
  d.n_tiles = ceil_div(H, 256);
  hipLaunchKernelGGL(grouped_gemm_fp8<kPlainBf16>, dim3(pair_rounds * kXcds * 2 * d.n_tiles), dim3(512), 0, s, d);
  return hipGetLastError();
}

}  // namespace moe
