// Shared pieces of the grouped GEMM kernels (bf16 and FP8).
#pragma once

#include <type_traits>

#include "kernels.h"

namespace moe {

struct GemmArgs {
  const uint16_t* A;         // bf16 activations: x [T, K] (gather) or [rows, K]
  const int32_t* row_token;  // gather map of routed rows (gather only)
  const int4* sched;         // row blocks {group, first row, rows}, largest first
                             // (expert GEMMs; nullptr: one group of T rows)
  const int32_t* sched_n;    // number of row blocks
  const uint16_t* B0;        // weights [G][N][K] bf16 (GEMM1: gate)
  const uint16_t* B1;        // GEMM1: up
  long long b_stride;        // elements per expert
  void* C;                   // output [rows, ldc]
  int ldc, N, K;             // N = output columns (GEMM1: intermediate columns)
  int T, TK;                 // tokens, T*K (gather: rows below TK are routed)
  int n_tiles;
  int gather;
  int a_rows;                // rows of A (bounds of the activation buffer)
  int k_chunk;               // split-K: K elements per blockIdx.y (router only)
  long long c_split_stride;  // split-K: elements between the partial outputs
  int k_split;               // [K][N] weights: K rows taken from B0 (the rest from B1)
};

hipError_t launch_build_schedule(const moe_config& c, const int32_t* offsets, int bm, int4* sched,
                                 int32_t* sched_n, hipStream_t s);
hipError_t launch_grouped_plain_bf16(const moe_config& c, const GemmArgs& a, hipStream_t s);
// The same on weights stored [K][N] (B0: K rows 0..k_split-1, B1 the rest; b_stride
// elements per expert in each), no transposed copy needed.
hipError_t launch_grouped_kn_bf16(const moe_config& c, const GemmArgs& a, hipStream_t s);
// One group of a.T rows, fp32 output C = A B^T (A [a.T][K], B [N][K] bf16), split-K over
// `splits` ranges of a.k_chunk (0: one range) into partials a.c_split_stride apart.
// Every range at least 256 long (or every range 128), K a multiple of 128.
hipError_t launch_gemm_f32(const GemmArgs& a, int splits, hipStream_t s);

// Arguments of the FP8 expert GEMMs (e4m3 operands, 128x128 / 1x128 block scales).
struct Fp8Args {
  const uint8_t* A;          // e4m3 activations: xq [T, K] (gather) or hq [rows, K]
  const float* a_scales;     // [K/128, scale_rows] (transposed), in the GEMM's row order
  const int32_t* row_token;  // gather map of routed rows (gather only)
  const int4* sched;         // row blocks {group, first row, rows}, largest first
  const int32_t* sched_n;    // number of row blocks
  const uint8_t* B0;         // e4m3 weights [G][N][K] (GEMM1: gate)
  const uint8_t* B1;         // GEMM1: up
  const float* S0;           // weight block scales [G][N/128][K/128] (GEMM1: gate)
  const float* S1;           // GEMM1: up
  long long b_stride;        // bytes per expert (N*K)
  long long s_stride;        // floats per expert
  uint16_t* C;               // bf16 output [rows, ldc] (plain mode; gated without Q)
  uint8_t* Q;                // gated: e4m3 codes of h [rows, ldc], quantised in the epilogue
  float* QS;                 // gated: their 1x128 scales [ldc/128, scale_rows]
  int ldc, N, K;
  int T, TK;
  int n_tiles;
  int gather;
  int a_rows;
  int scale_rows;            // rows of a_scales (the grouped rows)
};

enum { kPlainBf16 = 0, kGatedBf16 = 1, kPlainF32 = 2, kPlainKN = 3 };


__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

constexpr uint32_t kOob = 0x80000000u;   // a buffer offset past every range: reads zero

// ---- direct global -> LDS loads ("buffer_load_dwordx4 ... lds") ---------------------
// Lane i of one instruction writes its 16 bytes at LDS byte M0 + 16 i.  Issued from
// inline assembly so the compiler does not fence them; callers wait with
// wait_vmcnt<n>() (this wave's n most recent loads may still be in flight) and
// publish with stage_barrier().
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                      uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_byte) : "memory", "m0");
}
// 4-byte variant: lane i's dword lands at M0 + 4 i
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                     uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "s"(lds_byte) : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// LDS reads of this wave complete, then the workgroup barrier; no global fence
__device__ __forceinline__ void stage_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// silu(a) = a / (1 + e^-a) from the hardware exp2 and reciprocal (each about 1 ulp
// in fp32); h is rounded to bf16 (relative step 2^-9) right after.
__device__ __forceinline__ float silu_fast(float a) {
  const float e = __builtin_amdgcn_exp2f(-a * 1.4426950408889634f);
  return a * __builtin_amdgcn_rcpf(1.0f + e);
}

}  // namespace moe

namespace moe {

// GEMM1 epilogue of the FP8 expert GEMMs with 256 weight rows per tile (128 gate rows
// over the matching 128 up rows) and 16x16x128 MFMA blocks (lane l holds weight rows
// 4 (l >> 4) + q of each 16-row block, token l & 15): h = silu(gate) * up, rounded once
// to bf16, then quantised per token over the tile's 128 h columns -- one 1x128 block
// ("DeepSeek-V3 ... 技术解析" (devpress), section 2) -- with the arithmetic of
// act_quant_e4m3: scale amax / 448 (pow2: the smallest power of two s >= 2^-126 with
// amax <= 448 s), code = RNE-saturate(h / scale).  The 8 waves are WN column groups
// (wn = w % WN) by 8 / WN token groups of 80 (wt = w / WN); each wave holds NIB 16-wide
// blocks of h columns: gate accumulators acc[ib], up accumulators acc[ib + NIB].
// Pass 1 reads each accumulator once, writes the bf16 h to the wave's LDS staging area
// (8 waves x TPW tokens x 16 NIB columns, NIB x TPW / 8 KB; the caller's operand
// buffers, free once every wave has passed the barrier at the start) and its per-token
// amax to amax_lds (8 x TPW floats); after a second workgroup barrier pass 2 combines the WN
// column groups' amax and quantises from LDS.  Every wave of the workgroup calls this
// (two barriers).  Codes go to hq [rows][ldq] (4 bytes per lane and block), scales to
// hs [ldq / 128][scale_rows] at block n0 / 128.
template <int NJB, int WN, int NIB, int TPW = 80, class Acc>
__device__ __forceinline__ void fp8_epilogue_hquant(const Acc& acc, int w, int l, int m0,
                                                    int mvalid, int n0, uint8_t* hq, int ldq,
                                                    float* hs, int scale_rows, float* amax_lds,
                                                    uint32_t* stage, bool pow2) {
  static_assert(WN * NIB * 16 == 128, "a tile holds one 128-wide block of h");
  const int wn = w % WN, wt = w / WN;
  // staging: wave w, token block jb, block ib: 64 lanes x 2 dwords (lane l's four bf16)
  uint2* st = reinterpret_cast<uint2*>(stage) + size_t(w) * ((TPW / 16) * NIB * 64);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // operand buffers free
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    float a = 0.f;
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      float hv[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) hv[q] = silu_fast(acc[ib][jb][q]) * acc[ib + NIB][jb][q];
      const uint32_t lo = pack_bf16x2(hv[0], hv[1]), hi = pack_bf16x2(hv[2], hv[3]);
      st[(jb * NIB + ib) * 64 + l] = make_uint2(lo, hi);
      a = fmaxf(a, fmaxf(fmaxf(fabsf(bf16_bits_to_f32(lo & 0xffffu)), fabsf(bf16_bits_to_f32(lo >> 16))),
                         fmaxf(fabsf(bf16_bits_to_f32(hi & 0xffffu)), fabsf(bf16_bits_to_f32(hi >> 16)))));
    }
    a = fmaxf(a, __shfl_xor(a, 16));
    a = fmaxf(a, __shfl_xor(a, 32));
    if ((l >> 4) == 0) amax_lds[w * TPW + jb * 16 + (l & 15)] = a;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    const int tk = jb * 16 + (l & 15);
    float a = amax_lds[(wt * WN) * TPW + tk];
#pragma unroll
    for (int i = 1; i < WN; ++i) a = fmaxf(a, amax_lds[(wt * WN + i) * TPW + tk]);
    float s = 1.0f;
    if (a > 0.f) {
      if (pow2) {
        int e;
        const float m = frexpf(a, &e);
        s = ldexpf(1.0f, max(m <= 0.875f ? e - 9 : e - 8, -126));
      } else {
        s = __fdiv_rn(a, 448.0f);
      }
    }
    const int rl = wt * TPW + tk;
    if (rl >= mvalid) continue;
    uint8_t* qrow = hq + size_t(m0 + rl) * ldq;
    const float rs = 1.0f / s;                           // exact for a power of two
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      const uint2 hb = st[(jb * NIB + ib) * 64 + l];
      const float v[4] = {bf16_bits_to_f32(hb.x & 0xffffu), bf16_bits_to_f32(hb.x >> 16),
                          bf16_bits_to_f32(hb.y & 0xffffu), bf16_bits_to_f32(hb.y >> 16)};
      const int col = n0 + wn * (16 * NIB) + ib * 16 + 4 * (l >> 4);
      uint32_t c = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        c |= f32_to_e4m3_rne_sat(pow2 ? v[q] * rs : __fdiv_rn(v[q], s)) << (8 * q);
      *reinterpret_cast<uint32_t*>(qrow + col) = c;
    }
    if (wn == 0 && (l >> 4) == 0) hs[size_t(n0 / 128) * scale_rows + m0 + rl] = s;
  }
}

}  // namespace moe
