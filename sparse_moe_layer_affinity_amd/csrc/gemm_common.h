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
};

hipError_t launch_build_schedule(const moe_config& c, const int32_t* offsets, int bm, int4* sched,
                                 int32_t* sched_n, hipStream_t s);
hipError_t launch_grouped_plain_bf16(const moe_config& c, const GemmArgs& a, hipStream_t s);

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
  uint16_t* C;               // bf16 output [rows, ldc]
  int ldc, N, K;
  int T, TK;
  int n_tiles;
  int gather;
  int a_rows;
  int scale_rows;            // rows of a_scales (the grouped rows)
};

enum { kPlainBf16 = 0, kGatedBf16 = 1, kPlainF32 = 2 };


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
