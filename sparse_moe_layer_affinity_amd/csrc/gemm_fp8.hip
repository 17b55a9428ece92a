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
// VGPRs as well, so no copies out of AGPRs.
//
// Tiles.  GEMM2 (plain): 128 weight rows x 320 tokens (an expert's whole row block, as
// in the bf16 kernel, so its weights stream from HBM once), 8 waves (two per SIMD: one
// wave's rescale FMAs run while the other's MFMAs hold the matrix core) of 64 weight
// rows x 80 tokens = 4 x 5 MFMA blocks.  GEMM1 (gated): 256 weight rows (128 gate rows
// over the matching 128 up rows) x 160 tokens, the same 64 x 80 per wave: a tile holds
// 128 h columns, one whole 1x128 block, so h is quantised to e4m3 in its epilogue; a row
// block of more than 160 rows is split evenly between two tiles in adjacent slots of
// one XCD, which stay in step over the same weight tiles in L2.  K advances one
// 128-byte scale block per stage.  Operands and scales go global -> LDS with buffer
// loads in LDS mode, one workgroup barrier per stage, after which stage k+2's tokens and
// weights go out.  Weights (streamed from HBM) cycle through three stage buffers; tokens
// (mostly L2 hits) and scales through two, and from there into one of two register
// sets a stage early, so their LDS reads overlap the MFMAs.  Row blocks come from the
// same largest-first XCD schedule as the bf16 kernel.
#include "gemm_common.h"

namespace moe {


template <int MODE>
__global__ __launch_bounds__(512) void grouped_gemm_fp8(Fp8Args a) {
  constexpr bool GATED = MODE == kGatedBf16;
  // gated: 256 weight rows (128 gate over the matching 128 up rows: 128 h columns, one
  // 1x128 block of h) x 160 tokens (half a row block); plain: 128 weight rows x 320
  constexpr int BW = GATED ? 256 : 128, BT = GATED ? kFp8BT / 2 : kFp8BT, ROWB = 128;
  constexpr int WSTAGE = BW * ROWB, TSTAGE = BT * ROWB;   // gated 32 KB, 20 KB; plain 16, 40
  constexpr int SW = 3;                                   // weight stage buffers
  constexpr int NTB = 5;                                  // 16-token blocks per wave (80 tokens)
  constexpr int WN = GATED ? 4 : 2;                       // waves along the weight rows
  constexpr int NWL = BW / 64;                            // weight loads (8 rows each) per wave
  constexpr int NTL = GATED ? 3 : 5;                      // token loads per wave
  constexpr int NSA = (BT + 63) / 64;                     // waves loading the token scales
  // LDS: the two token buffers, the weight ring, the two token-scale and the two
  // weight-scale buffers (waves NSA.. write 256 bytes each, those past the weight
  // scales a dummy); gated: the dummy token loads of waves 4..7 and the epilogue's amax
  // exchange
  constexpr uint32_t kTOff = 0;
  constexpr uint32_t kWOff = 2 * TSTAGE;
  constexpr uint32_t kSaOff = kWOff + SW * WSTAGE;
  constexpr uint32_t kSaStage = 256 * NSA;
  constexpr uint32_t kSwOff = kSaOff + 2 * kSaStage;
  constexpr uint32_t kSwStage = 256 * (8 - NSA);
  constexpr uint32_t kDumOff = kSwOff + 2 * kSwStage;
  constexpr uint32_t kAmOff = kDumOff + (GATED ? 1024 : 0);
  constexpr uint32_t kLdsBytes = kAmOff + (GATED ? 8 * 80 * 4 : 0);
  constexpr int BN_OUT = GATED ? BW / 2 : BW;             // output columns: 128
  __shared__ __attribute__((aligned(1024))) uint4 lds[kLdsBytes / 16];

  // ---- tile decode: row blocks dealt to the XCDs in snake order, a block's n-tiles
  // consecutive on one XCD (see the bf16 expert GEMM); gated: the two halves of a
  // block's n-tile in adjacent slots of one XCD, so they share its weight tiles in L2 --
  const int b = blockIdx.x;
  const int xcd = b % kXcds, slot0 = b / kXcds;
  const int half = GATED ? (slot0 & 1) : 0;
  const int slot = GATED ? (slot0 >> 1) : slot0;
  const int round = slot / a.n_tiles, nt = slot % a.n_tiles;
  const int pos = round * kXcds + ((round & 1) ? kXcds - 1 - xcd : xcd);
  if (pos >= *a.sched_n) return;
  const int4 blk = a.sched[pos];
  // gated: a block of more than 160 rows splits evenly (the first half rounded up to 16
  // rows), so the two halves do the same MFMA work and stay in step over the weights
  const int rows0 = GATED && blk.z > BT ? (((blk.z + 1) / 2 + 15) & ~15) : blk.z;
  const int g = blk.x, m0 = blk.y + half * rows0, mvalid = half ? blk.z - rows0 : rows0;
  if (mvalid <= 0) return;
  const int n0 = nt * BN_OUT;
  const int tid = threadIdx.x;
  const int K = a.K, KBLK = a.K / 128;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;

  // ---- this wave's share of every stage: weight rows 8 NWL w .., tokens ------------
  // A tile row lies in the tile's base for every load of this wave, so the lane offsets
  // are per-wave constants.  Gated: stage rows 0..127 are gate rows n0.., 128..255 the
  // matching up rows.
  const bool up = GATED && w >= 4;
  const int wrow0 = GATED ? n0 + 32 * (w & 3) : n0 + 16 * w;
  const __amdgpu_buffer_rsrc_t rsrc_w =
      make_rsrc((up ? a.B1 : a.B0) + size_t(g) * a.b_stride, uint32_t(a.N) * uint32_t(K));
  const __amdgpu_buffer_rsrc_t rsrc_t = make_rsrc(a.A, uint32_t(a.a_rows) * uint32_t(K));
  uint32_t voff_w[NWL], voff_t[NTL];
#pragma unroll
  for (int j = 0; j < NWL; ++j) {
    // stage row 8 NWL w + 8 j + (l >> 3): bit 3 of the row is j & 1 (NWL is even)
    const uint32_t chunk = uint32_t((l & 7) ^ (l >> 3) ^ (j & 1)) * 16u;
    voff_w[j] = uint32_t(wrow0 + 8 * j + (l >> 3)) * uint32_t(K) + chunk;   // rows >= N read zero
  }
  // shared-expert tiles map rows to consecutive tokens; routed rows gather
  const bool lookup = a.gather && m0 < a.TK;
  const int tbase = !a.gather ? m0 : (lookup ? 0 : (m0 - a.TK) % a.T);
  auto src_of = [&](int row) { return lookup ? a.row_token[m0 + row] : tbase + row; };
  // plain: wave w loads stage rows 40 w + 8 j (j < 5); gated: 8-row group 8 j + w (rows
  // 8 (8 j + w) ..), of which waves 4..7 have no third (their third load is a dummy,
  // every lane out of range, so the load counts stay uniform)
  auto trow_of = [&](int j) { return GATED ? 8 * (8 * j + w) + (l >> 3) : 40 * w + 8 * j + (l >> 3); };
#pragma unroll
  for (int j = 0; j < NTL; ++j) {
    const int trow = trow_of(j);
    const int grp = GATED ? 8 * j + w : 5 * w + j;       // bit 3 of the row
    const uint32_t chunk = uint32_t((l & 7) ^ (l >> 3) ^ (grp & 1)) * 16u;
    const bool real = !GATED || j < 2 || w < 4;
    voff_t[j] = real && trow < mvalid ? uint32_t(src_of(trow)) * uint32_t(K) + chunk : kOob;
  }
  // one scale load per wave per stage: waves 0..NSA-1 the token scales of tokens
  // 64 w + lane, the next two one weight block scale each (lane 0; gated: gate and up,
  // plain: the tile's block and nothing), the rest nothing useful (every lane out of
  // range; the load counts stay uniform)
  __amdgpu_buffer_rsrc_t rsrc_s;
  uint32_t voff_s = kOob;
  if (w < NSA) {
    rsrc_s = make_rsrc(a.a_scales, uint32_t(a.scale_rows) * KBLK * 4u);
    const int row = 64 * w + l;
    if (row < mvalid) voff_s = uint32_t(m0 + row) * 4u;
  } else {
    const bool sup = GATED && w == NSA + 1;
    rsrc_s = make_rsrc((sup ? a.S1 : a.S0) + size_t(g) * a.s_stride, uint32_t(a.s_stride) * 4u);
    if (l == 0 && (w == NSA || sup)) voff_s = uint32_t((n0 / 128) * KBLK) * 4u;
  }
  // K block ks of the scales: token scales [K/128, scale_rows], weight scales [.., K/128]
  const uint32_t s_step = w < NSA ? uint32_t(a.scale_rows) * 4u : 4u;
  const uint32_t lds_base = uint32_t(uintptr_t(&lds[0]));
  const uint32_t wave_w = lds_base + kWOff + uint32_t(w) * (WSTAGE / 8);
  const uint32_t wave_s = lds_base + (w < NSA ? kSaOff + 256u * w : kSwOff + 256u * (w - NSA));
  const uint32_t s_par = w < NSA ? kSaStage : kSwStage;
  // LDS byte of token load j in buffer 0 (gated dummies: one shared area, no parity)
  auto tdst = [&](int j) -> uint32_t {
    if (GATED) return j == 2 && w >= 4 ? lds_base + kDumOff : lds_base + kTOff + uint32_t(8 * j + w) * 1024u;
    return lds_base + kTOff + uint32_t(w) * (TSTAGE / 8) + uint32_t(j) * 1024u;
  };
  auto tpar = [&](int j) -> uint32_t { return GATED && j == 2 && w >= 4 ? 0u : uint32_t(TSTAGE); };

  auto load_w = [&](int ks) __attribute__((always_inline)) {
    const uint32_t dst = wave_w + uint32_t(ks % SW) * WSTAGE;
#pragma unroll
    for (int j = 0; j < NWL; ++j) dma16(rsrc_w, voff_w[j], uint32_t(ks) * ROWB, dst + uint32_t(j) * 1024u);
  };
  // token rows of stage ks and its scales, into buffer ks & 1 (NTL + 1 loads)
  auto load_t = [&](int ks) __attribute__((always_inline)) {
    const uint32_t par = uint32_t(ks & 1);
#pragma unroll
    for (int j = 0; j < NTL; ++j)
      dma16(rsrc_t, voff_t[j], uint32_t(ks) * ROWB, __builtin_amdgcn_readfirstlane(tdst(j) + par * tpar(j)));
    dma4(rsrc_s, voff_s, uint32_t(ks) * s_step, __builtin_amdgcn_readfirstlane(wave_s + par * s_par));
  };

  // ---- wave geometry: WN (weight rows) x 8 / WN (tokens, 80 each) -----------------
  const int wn = w % WN, wt = w / WN;
  // LDS row of this lane in weight block ib (gated: gate blocks 0, 1, up blocks 2, 3)
  // and token block jb, and its two K chunks
  int w_row[4];
#pragma unroll
  for (int ib = 0; ib < 4; ++ib) {
    int r;
    if (GATED) r = ib < 2 ? wn * 32 + ib * 16 : BW / 2 + wn * 32 + (ib - 2) * 16;
    else r = wn * 64 + ib * 16;
    w_row[ib] = r + (l & 15);
  }
  const int t_row = wt * 80 + (l & 15);                   // + 16 jb
  const int c0 = 2 * (l >> 4);
  const uint32_t sl0 = uint32_t(c0 ^ (l & 7) ^ ((l >> 3) & 1)) * 16u;
  const uint32_t sl1 = uint32_t((c0 + 1) ^ (l & 7) ^ ((l >> 3) & 1)) * 16u;

  // token blocks of this wave that hold rows: the MFMAs of empty ones are skipped
  const int njb = min(NTB, max(0, (mvalid - wt * 80 + 15) >> 4));
  auto body = [&](auto njb_tag) __attribute__((always_inline)) {
    constexpr int NJB = decltype(njb_tag)::value;
    f32x4_t acc[4][NJB > 0 ? NJB : 1];
  #pragma unroll
    for (int ib = 0; ib < 4; ++ib)
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb) acc[ib][jb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto lds_frag = [&](uint32_t row_byte) __attribute__((always_inline)) {
      const char* base = reinterpret_cast<const char*>(lds) + row_byte;
      const uint4 lo4 = *reinterpret_cast<const uint4*>(base + sl0);
      const uint4 hi4 = *reinterpret_cast<const uint4*>(base + sl1);
      return i32x8_t{int(lo4.x), int(lo4.y), int(lo4.z), int(lo4.w),
                     int(hi4.x), int(hi4.y), int(hi4.z), int(hi4.w)};
    };
    auto lds_f32 = [&](uint32_t byte) __attribute__((always_inline)) {
      return *reinterpret_cast<const float*>(reinterpret_cast<const char*>(lds) + byte);
    };

    // Token fragments and scales of a stage are read into registers one stage early
    // (two register sets), so the reads of stage k+1 run under stage k's MFMAs.  Per
    // stage k, two barriers:
    //   P_k  stage k's weights and stage k+1's tokens and scales are in LDS (loaded two
    //        stages / one and a half stages ahead); weights k+2 go out into the buffer
    //        stage k-1 left
    //   R_k  every wave holds stage k+1's tokens and scales: that buffer takes stage k+3
    // K is a multiple of 128: nk >= 1.
    const int nk = KBLK;
    i32x8_t tf[2][NJB > 0 ? NJB : 1];
    float s[2][2][NJB > 0 ? NJB : 1];                    // per set: s_a * s_w per weight half
    auto read_tokens = [&](auto set_tag, int ks) __attribute__((always_inline)) {
      constexpr int S = decltype(set_tag)::value;
      const uint32_t tp = uint32_t(ks & 1);
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
        tf[S][jb] = lds_frag(kTOff + tp * TSTAGE + uint32_t(t_row + 16 * jb) * ROWB);
      const float s_w0 = lds_f32(kSwOff + tp * kSwStage);
      const float s_w1 = MODE == kGatedBf16 ? lds_f32(kSwOff + tp * kSwStage + 256u) : s_w0;
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const float s_a = lds_f32(kSaOff + tp * kSaStage + uint32_t(t_row + 16 * jb) * 4u);
        s[S][0][jb] = s_a * s_w0;
        s[S][1][jb] = s_a * s_w1;
      }
    };
    // weight block ib of stage ks against the stage's tokens (register set S); each
    // product is rescaled as soon as it is back, the other wave on the SIMD keeping the
    // matrix core busy meanwhile
    auto block_row = [&](auto set_tag, int ks, int ib) __attribute__((always_inline)) {
      constexpr int S = decltype(set_tag)::value;
      if constexpr (NJB > 0) {
        const i32x8_t wf = lds_frag(kWOff + uint32_t(ks % SW) * WSTAGE + uint32_t(w_row[ib]) * ROWB);
        const int h = (MODE == kGatedBf16 && ib >= 2) ? 1 : 0;
  #pragma unroll
        for (int jb = 0; jb < NJB; ++jb) {
          const f32x4_t p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wf, tf[S][jb], f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
  #pragma unroll
          for (int q = 0; q < 4; ++q) acc[ib][jb][q] = fmaf(p[q], s[S][h][jb], acc[ib][jb][q]);
        }
      }
    };
    // prologue: tokens and weights of stages 0 and 1 (in that order), stage 0's token
    // fragments
    load_t(0);
    load_w(0);
    if (nk > 1) {
      load_t(1);
      load_w(1);
      wait_vmcnt<2 * NWL + NTL + 1>();
    } else {
      wait_vmcnt<NWL>();
    }
    stage_barrier();
    read_tokens(std::integral_constant<int, 0>{}, 0);
    auto stage = [&](auto set_tag, int k) __attribute__((always_inline)) {
      constexpr int S = decltype(set_tag)::value;
      using N = std::integral_constant<int, 1 - S>;
      // one barrier per stage: stage k's weights and stage k+1's tokens are in LDS
      // (only the weights of k+1, issued last, may stay in flight), and every wave is
      // done with stage k-1 (weights k-1, tokens k read a stage early), whose buffers
      // take stage k+2's tokens and weights
      if (k + 1 < nk) wait_vmcnt<NWL>();
      else wait_vmcnt<0>();
      stage_barrier();
      if (k + 2 < nk) {
        load_t(k + 2);
        load_w(k + 2);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (k + 1 < nk) read_tokens(N{}, k + 1);
      block_row(set_tag, k, 0);
      __builtin_amdgcn_sched_barrier(0);
      block_row(set_tag, k, 1);
      block_row(set_tag, k, 2);
      block_row(set_tag, k, 3);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int k = 0; k < nk; k += 2) {
      stage(std::integral_constant<int, 0>{}, k);
      if (k + 1 < nk) stage(std::integral_constant<int, 1>{}, k + 1);
    }

    // ---- epilogue: lane l holds weight rows 4*(l/16)+q of each block, token l%16 ----
    if constexpr (GATED) {
      // h quantised to e4m3 per 1x128 block here; staging in the two token buffers
      fp8_epilogue_hquant<NJB, WN, 2>(acc, w, l, m0, mvalid, n0, a.Q, a.ldc, a.QS, a.scale_rows,
                                      reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + kAmOff),
                                      reinterpret_cast<uint32_t*>(lds), false);
    } else {
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const int rl = wt * 80 + jb * 16 + (l & 15);
        if (rl >= mvalid) continue;
        uint16_t* crow = a.C + size_t(m0 + rl) * a.ldc;
  #pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          const int col = n0 + wn * 64 + ib * 16 + 4 * (l >> 4);
          if (col >= a.N) continue;
          const f32x4_t& v = acc[ib][jb];
          *reinterpret_cast<uint2*>(crow + col) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
      }
    }
  };
  if (njb >= 5) body(std::integral_constant<int, 5>{});
  else if (njb >= 3) body(std::integral_constant<int, 4>{});
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
  err = launch_build_schedule(c, offsets, kFp8BT, ws.sched, ws.sched_n, s);
  if (err != hipSuccess) return err;
  const int rounds = ceil_div(expert_row_blocks_upper(c, kFp8BT), kXcds);
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
    // 256-weight-row tiles over the two 160-row halves of each block
    hipLaunchKernelGGL(grouped_gemm_fp8<kGatedBf16>, dim3(rounds * kXcds * a.n_tiles * 2), dim3(512), 0, s, a);
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
  d.n_tiles = ceil_div(H, 128);
  hipLaunchKernelGGL(grouped_gemm_fp8<kPlainBf16>, dim3(rounds * kXcds * d.n_tiles), dim3(512), 0, s, d);
  return hipGetLastError();
}

}  // namespace moe
