// FP8 expert GEMMs with power-of-two block scales (the MOE_E4M3_POW2 weights).
//
// The same GEMMs as the FP8 kernel with fp32 block scales ("DeepSeek-V3 ... 技术解析"
// (devpress), section 2: 128x128 weight blocks, 1x128 activation blocks), but every
// scale is a power of two, so the matrix cores apply both scales of a 128-wide K block
// themselves (v_mfma_scale_f32_16x16x128_f8f6f4 with 8-bit exponents: the weights'
// one per 128-row block, each lane's token's for the tokens; all four 32-wide parts
// of the block carry the same one) and accumulate in place.  With no rescale on the
// VALU the accumulators can live in AGPRs (this file is compiled without the
// VGPR-form MFMA flag), which leaves room for a tile twice as wide in weights as the
// fp32-scale kernel's: 256 weight rows (GEMM1: 128 gate rows over the matching 128 up
// rows) x 320 tokens, 8 waves (two per SIMD), each 128 weight rows x 80 tokens =
// 8 x 5 MFMA blocks, 160 accumulators per lane.  Twice the weight rows per token row
// loaded halves the token bytes per flop.
//
// K advances one 128-byte block per stage, with one barrier per stage.  Weights (from
// HBM, 32 KB a stage), tokens (mostly L2 hits, 40 KB) and their scales have two stage
// buffers each: right after the barrier that publishes stage k, stage k+1's loads go
// into the buffers stage k-1 left, and stage k's fragments are read while they fly;
// within the stage each weight block's fragment is read while the MFMAs of the block
// before it run.  Row blocks come from the largest-first XCD schedule of the bf16
// kernel.
#include "gemm_common.h"

namespace moe {

// Block-scaled MFMA with its accumulator in AGPRs (or VGPRs: the "v" forms), written
// out: the compiler gives an MFMA builtin VGPR accumulators at two waves per SIMD, and
// 160 of them do not fit beside the fragments; at two waves per SIMD it grants 128
// AGPRs, so token blocks 0..3 accumulate in AGPRs and block 4 in VGPRs.  The first MFMA
// of a tile takes an inline zero as SrcC (a
// write of the accumulator just before an MFMA that reads it would need wait states
// the compiler does not insert around inline assembly); every accumulator is read by
// the next MFMA on it only 40 MFMAs later; mfma_p2_drain covers the result latency
// before the epilogue reads them.
__device__ __forceinline__ void mfma_p2(f32x4_t& c, const i32x8_t& a, const i32x8_t& b, int ea, int eb) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(c) : "v"(a), "v"(b), "v"(ea), "v"(eb));
}
__device__ __forceinline__ void mfma_p2_first(f32x4_t& c, const i32x8_t& a, const i32x8_t& b, int ea, int eb) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
               : "=a"(c) : "v"(a), "v"(b), "v"(ea), "v"(eb));
}
__device__ __forceinline__ void mfma_p2v(f32x4_t& c, const i32x8_t& a, const i32x8_t& b, int ea, int eb) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+v"(c) : "v"(a), "v"(b), "v"(ea), "v"(eb));
}
__device__ __forceinline__ void mfma_p2v_first(f32x4_t& c, const i32x8_t& a, const i32x8_t& b, int ea, int eb) {
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, 0, %3, %4 op_sel_hi:[0,0,0]"
               : "=&v"(c) : "v"(a), "v"(b), "v"(ea), "v"(eb));
}

template <int MODE>
__global__ __launch_bounds__(512) void grouped_gemm_fp8p2(Fp8Args a) {
  constexpr int BW = 256, BT = kFp8BT, ROWB = 128;
  constexpr int WSTAGE = BW * ROWB, TSTAGE = BT * ROWB;   // 32 KB, 40 KB
  constexpr int SW = 2;                                   // weight stage buffers
  constexpr int NTB = BT / 64;                            // 16-token blocks per wave: 5
  // LDS: two token buffers, two weight buffers, two token-scale and two weight-scale
  // buffers (waves 5..7 write 256 bytes each, wave 7's are a dummy)
  constexpr uint32_t kTOff = 0;                           // two token stage buffers
  constexpr uint32_t kWOff = 2 * TSTAGE;
  constexpr uint32_t kSaOff = kWOff + SW * WSTAGE;
  constexpr uint32_t kSaStage = 4 * BT;                   // 1280 B
  constexpr uint32_t kSwOff = kSaOff + 2 * kSaStage;
  constexpr uint32_t kSwStage = 768;
  constexpr uint32_t kAmOff = kSwOff + 2 * kSwStage;      // the epilogue's amax exchange
  constexpr int BN_OUT = MODE == kGatedBf16 ? BW / 2 : BW;
  __shared__ __attribute__((aligned(1024))) uint4 lds[(kAmOff + 8 * 80 * 4) / 16];

  // ---- tile decode (as the fp32-scale FP8 kernel) -------------------------------------
  const int b = blockIdx.x;
  const int xcd = b % kXcds, slot = b / kXcds;
  const int round = slot / a.n_tiles, nt = slot % a.n_tiles;
  const int pos = round * kXcds + ((round & 1) ? kXcds - 1 - xcd : xcd);
  if (pos >= *a.sched_n) return;
  const int4 blk = a.sched[pos];
  const int g = blk.x, m0 = blk.y, mvalid = blk.z;
  const int n0 = nt * BN_OUT;
  const int tid = threadIdx.x;
  const int K = a.K, KBLK = a.K / 128;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;

  // ---- this wave's share of every stage: weight rows 32 w .., token rows 40 w .. ----
  // gated: stage rows 0..127 are gate rows n0.., 128..255 the matching up rows
  const bool up = MODE == kGatedBf16 && w >= 4;
  const int wrow0 = MODE == kGatedBf16 ? n0 + 32 * (w & 3) : n0 + 32 * w;
  const __amdgpu_buffer_rsrc_t rsrc_w =
      make_rsrc((up ? a.B1 : a.B0) + size_t(g) * a.b_stride, uint32_t(a.N) * uint32_t(K));
  const __amdgpu_buffer_rsrc_t rsrc_t = make_rsrc(a.A, uint32_t(a.a_rows) * uint32_t(K));
  // stage row 32 w + 8 j + (l >> 3), j = 0..3 (bit 3 of the row is j & 1): loads j and
  // j + 2 are 16 rows apart, a uniform offset that rides in the scalar operand
  uint32_t voff_w[2], voff_t[NTB];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t chunk = uint32_t((l & 7) ^ (l >> 3) ^ j) * 16u;
    voff_w[j] = uint32_t(wrow0 + 8 * j + (l >> 3)) * uint32_t(K) + chunk;   // rows >= N read zero
  }
  // shared-expert tiles map rows to consecutive tokens; routed rows gather
  const bool lookup = a.gather && m0 < a.TK;
  const int tbase = !a.gather ? m0 : (lookup ? 0 : (m0 - a.TK) % a.T);
#pragma unroll
  for (int j = 0; j < NTB; ++j) {
    // stage row 40 w + 8 j + (l >> 3): bit 3 of the row is (5 w + j) & 1
    const int trow = 40 * w + 8 * j + (l >> 3);
    const uint32_t chunk = uint32_t((l & 7) ^ (l >> 3) ^ ((5 * w + j) & 1)) * 16u;
    const int src = trow < mvalid ? (lookup ? a.row_token[m0 + trow] : tbase + trow) : 0;
    voff_t[j] = trow < mvalid ? uint32_t(src) * uint32_t(K) + chunk : kOob;
  }
  // one scale load per wave per stage: waves 0..4 the token scales of rows 64 w + lane
  // (in grouped-row order), waves 5 and 6 one weight block scale each (lane 0; gated:
  // the gate and the up block; plain: the tile's two 128-row blocks, clamped in range:
  // a block past N only feeds outputs that are never stored), wave 7 nothing useful
  __amdgpu_buffer_rsrc_t rsrc_s;
  uint32_t voff_s = kOob;
  if (w < 5) {
    rsrc_s = make_rsrc(a.a_scales, uint32_t(a.scale_rows) * KBLK * 4u);
    const int row = 64 * w + l;
    if (row < mvalid) voff_s = uint32_t(m0 + row) * 4u;
  } else {
    const bool sup = MODE == kGatedBf16 && w == 6;
    const int blk_n = min(MODE == kGatedBf16 ? n0 / 128 : n0 / 128 + (w - 5), ceil_div(a.N, 128) - 1);
    rsrc_s = make_rsrc((sup ? a.S1 : a.S0) + size_t(g) * a.s_stride, uint32_t(a.s_stride) * 4u);
    if (l == 0 && w < 7) voff_s = uint32_t(blk_n * KBLK) * 4u;
  }
  const uint32_t s_step = w < 5 ? uint32_t(a.scale_rows) * 4u : 4u;
  const uint32_t lds_base = uint32_t(uintptr_t(&lds[0]));
  const uint32_t wave_w = lds_base + kWOff + uint32_t(w) * (WSTAGE / 8);
  const uint32_t wave_t = lds_base + kTOff + uint32_t(w) * (TSTAGE / 8);
  const uint32_t wave_s = lds_base + (w < 5 ? kSaOff + 256u * w : kSwOff + 256u * (w - 5));
  const uint32_t s_par = w < 5 ? kSaStage : kSwStage;

  auto load_w = [&](int ks) __attribute__((always_inline)) {
    const uint32_t dst = wave_w + uint32_t(ks % SW) * WSTAGE;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      dma16(rsrc_w, voff_w[j & 1], uint32_t(ks) * ROWB + uint32_t(j >> 1) * 16u * uint32_t(K),
            dst + j * 1024u);
  };
  // token rows of stage ks and its scales (buffers ks & 1)
  auto load_t = [&](int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NTB; ++j)
      dma16(rsrc_t, voff_t[j], uint32_t(ks) * ROWB, wave_t + uint32_t(ks & 1) * TSTAGE + j * 1024u);
    dma4(rsrc_s, voff_s, uint32_t(ks) * s_step,
         __builtin_amdgcn_readfirstlane(wave_s + uint32_t(ks & 1) * s_par));
  };

  // ---- wave geometry: 2 (weight rows) x 4 (tokens) --------------------------------
  const int wn = w & 1, wt = w >> 1;
  // LDS bytes of this lane's first K chunk in weight block 0 / token block 0; block ib /
  // jb adds a constant (gated: blocks 4..7 are the up rows, 128 further), and the second
  // chunk is the first one ^ 16 (chunk 2 (l >> 4) + 1, XOR-swizzled the same way)
  const int t_row = wt * 80 + (l & 15);
  const uint32_t sl0 = uint32_t((2 * (l >> 4)) ^ (l & 7) ^ ((l >> 3) & 1)) * 16u;
  const uint32_t w_lane = uint32_t((MODE == kGatedBf16 ? wn * 64 : wn * 128) + (l & 15)) * ROWB + sl0;
  const uint32_t t_lane = uint32_t(t_row) * ROWB + sl0;
  auto w_blk = [](int ib) constexpr {
    return uint32_t(MODE == kGatedBf16 ? (ib < 4 ? ib * 16 : 128 + (ib - 4) * 16) : ib * 16) * ROWB;
  };

  const int njb = min(NTB, max(0, (mvalid - wt * 80 + 15) >> 4));
  auto body = [&](auto njb_tag) __attribute__((always_inline)) {
    constexpr int NJB = decltype(njb_tag)::value;
    f32x4_t acc[8][NJB > 0 ? NJB : 1];                 // defined by the first stage's MFMAs

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
    // 8-bit exponent code of a power-of-two float32, in every byte of the operand
    auto e8 = [](float v) { return int(((__float_as_uint(v) >> 23) & 0xffu) * 0x01010101u); };

    // prologue: stage 0 (tokens, scales, weights), published
    const int nk = KBLK;
    load_t(0);
    load_w(0);
    wait_vmcnt<0>();
    stage_barrier();
    auto stage = [&](int k, auto first_tag) __attribute__((always_inline)) {
      constexpr bool FIRST = decltype(first_tag)::value;
      const uint32_t wb = kWOff + uint32_t(k & 1) * WSTAGE;
      const uint32_t tb = kTOff + uint32_t(k & 1) * TSTAGE;
      const uint32_t sp = uint32_t(k & 1);
      // every wave is past stage k-1: its buffers take stage k+1
      if (k + 1 < nk) {
        load_t(k + 1);
        load_w(k + 1);
      }
      // token fragments and exponents of stage k into registers
      i32x8_t tf[NJB > 0 ? NJB : 1];
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb) tf[jb] = lds_frag(t_lane, tb + uint32_t(16 * jb) * ROWB);
      int ea[NJB > 0 ? NJB : 1], ew[2];
      ew[0] = e8(lds_f32(kSwOff + sp * kSwStage + (MODE == kGatedBf16 ? 0u : 256u * wn)));
      ew[1] = MODE == kGatedBf16 ? e8(lds_f32(kSwOff + sp * kSwStage + 256u)) : ew[0];
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb)
        ea[jb] = e8(lds_f32(kSaOff + sp * kSaStage + uint32_t(t_row + 16 * jb) * 4u));
      // the exponents were written by the VALU: wait states before an MFMA reads them
      asm volatile("s_nop 4" ::: "memory");
      i32x8_t wfb[2];
      if constexpr (NJB > 0) wfb[0] = lds_frag(w_lane + wb, w_blk(0));
  #pragma unroll
      for (int ib = 0; ib < 8; ++ib) {
        if constexpr (NJB > 0) {
          if (ib + 1 < 8) wfb[(ib + 1) & 1] = lds_frag(w_lane + wb, w_blk(ib + 1));
          __builtin_amdgcn_sched_barrier(0);
          const i32x8_t& wf = wfb[ib & 1];
          const int h = (MODE == kGatedBf16 && ib >= 4) ? 1 : 0;
  #pragma unroll
          for (int jb = 0; jb < NJB; ++jb) {
            if (jb < 4) {
              if constexpr (FIRST) mfma_p2_first(acc[ib][jb], wf, tf[jb], ew[h], ea[jb]);
              else mfma_p2(acc[ib][jb], wf, tf[jb], ew[h], ea[jb]);
            } else {
              if constexpr (FIRST) mfma_p2v_first(acc[ib][jb], wf, tf[jb], ew[h], ea[jb]);
              else mfma_p2v(acc[ib][jb], wf, tf[jb], ew[h], ea[jb]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (k + 1 < nk) {
        // publish stage k+1
        wait_vmcnt<0>();
        stage_barrier();
      }
    };
    stage(0, std::true_type{});
    for (int k = 1; k < nk; ++k) stage(k, std::false_type{});
  #pragma unroll
    for (int ib = 0; ib < 8; ++ib) {
      if constexpr (NJB == 5)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[ib][0]), "+a"(acc[ib][1]), "+a"(acc[ib][2]), "+a"(acc[ib][3]), "+v"(acc[ib][4]));
      else if constexpr (NJB == 4)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[ib][0]), "+a"(acc[ib][1]), "+a"(acc[ib][2]), "+a"(acc[ib][3]));
      else if constexpr (NJB == 2)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[ib][0]), "+a"(acc[ib][1]));
      else if constexpr (NJB == 1)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc[ib][0]));
    }

    // ---- epilogue: lane l holds weight rows 4*(l/16)+q of each block, token l%16 ----
    if constexpr (MODE == kGatedBf16) {
      if (a.Q) {
        // staging in the two token buffers (80 KB)
        fp8_epilogue_hquant<NJB, 2, 4>(acc, w, l, m0, mvalid, n0, a.Q, a.ldc, a.QS, a.scale_rows,
                                 reinterpret_cast<float*>(reinterpret_cast<char*>(lds) + kAmOff),
                                 reinterpret_cast<uint32_t*>(lds), true);
        return;
      }
    }
    if constexpr (MODE == kGatedBf16) {
  #pragma unroll
      for (int jb = 0; jb < NJB; ++jb) {
        const int rl = wt * 80 + jb * 16 + (l & 15);
        if (rl >= mvalid) continue;
        uint16_t* crow = a.C + size_t(m0 + rl) * a.ldc;
  #pragma unroll
        for (int ib = 0; ib < 4; ++ib) {
          const int col = n0 + wn * 64 + ib * 16 + 4 * (l >> 4);
          if (col >= a.N) continue;
          float hv[4];
  #pragma unroll
          for (int q = 0; q < 4; ++q) hv[q] = silu_fast(acc[ib][jb][q]) * acc[ib + 4][jb][q];
          *reinterpret_cast<uint2*>(crow + col) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        }
      }
    } else {
      // bf16 rows through LDS: each wave stages up to 64 of its tokens x 128 columns
      // (16 KB, in the operand buffers, free once every wave is past the barrier) as rows
      // of 256 bytes, 16-byte chunk c of row r in slot c ^ (r & 15), then stores whole
      // 16-byte chunks of four rows per instruction; a fifth token block goes through the
      // same area in a second pass
      stage_barrier();
      char* const stg = reinterpret_cast<char*>(lds) + w * 16384;
      auto pass = [&](auto jb0_tag, auto jb1_tag) __attribute__((always_inline)) {
        constexpr int JB0 = decltype(jb0_tag)::value, JB1 = decltype(jb1_tag)::value;
  #pragma unroll
        for (int jb = JB0; jb < JB1; ++jb) {
          const int r = (jb - JB0) * 16 + (l & 15);
  #pragma unroll
          for (int ib = 0; ib < 8; ++ib) {
            const int cc = 2 * ib + (l >> 5);
            const f32x4_t& v = acc[ib][jb];
            *reinterpret_cast<uint2*>(stg + r * 256 + ((cc ^ (r & 15)) << 4) + ((l >> 4) & 1) * 8) =
                make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
          }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const int cc = l & 15;
        const int col = n0 + wn * 128 + cc * 8;
  #pragma unroll
        for (int r0 = 0; r0 < 16 * (JB1 - JB0); r0 += 4) {
          const int r = r0 + (l >> 4);
          const int rl = wt * 80 + JB0 * 16 + r;
          const uint4 v = *reinterpret_cast<const uint4*>(stg + r * 256 + ((cc ^ (r & 15)) << 4));
          if (rl < mvalid && col < a.N)
            *reinterpret_cast<uint4*>(a.C + size_t(m0 + rl) * a.ldc + col) = v;
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      };
      pass(std::integral_constant<int, 0>{}, std::integral_constant<int, (NJB < 4 ? NJB : 4)>{});
      if constexpr (NJB > 4) pass(std::integral_constant<int, 4>{}, std::integral_constant<int, NJB>{});
    }
  };
  if (njb >= 5) body(std::integral_constant<int, 5>{});
  else if (njb >= 3) body(std::integral_constant<int, 4>{});
  else if (njb == 2) body(std::integral_constant<int, 2>{});
  else if (njb == 1) body(std::integral_constant<int, 1>{});
  else body(std::integral_constant<int, 0>{});
}

hipError_t launch_gemm_fp8p2(const Fp8Args& a, bool gated, int n_tiles_blocks, hipStream_t s) {
  if (gated)
    hipLaunchKernelGGL(grouped_gemm_fp8p2<kGatedBf16>, dim3(n_tiles_blocks), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(grouped_gemm_fp8p2<kPlainBf16>, dim3(n_tiles_blocks), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
