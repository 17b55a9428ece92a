// Device-side helpers shared by the gfx950 kernels of the MoE layer library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

constexpr int kWave = 64;
constexpr int kXcds = 8;           // MI355X: 8 XCDs, workgroups dispatched round-robin

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Two fp32 values to packed bf16 (x0 in the low half), round to nearest even, by the
// hardware conversion (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float x0, float x1) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x0, x1}, bf16x2_t));
}

// fp32 -> OCP e4m3fn code: round to nearest even, saturate to +-448, keep the sign
// of values that round to zero, NaN -> 0x7F.  Branch-free (every lane takes the same
// path): below 2^-6 the code is the value on the subnormal grid of 2^-9, RNE; above,
// the code is the fp32 bit pattern's exponent and top three mantissa bits, rounded to
// nearest even by adding 0x7FFFF plus the kept lsb before the shift (a carry moves
// into the exponent), rebiased by (127 - 7) << 3 = 960; magnitudes at or above 448
// give 0x7E.
__device__ __forceinline__ uint32_t f32_to_e4m3_rne_sat(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  const uint32_t sub = uint32_t(rintf(__uint_as_float(a) * 512.0f));   // used if a < 2^-6
  const uint32_t an = a < 0x43e00000u ? a : 0x43e00000u;
  const uint32_t nrm = ((an + 0x7ffffu + ((an >> 20) & 1u)) >> 20) - 960u;
  // both candidates exist before the selection (otherwise the compiler turns it back
  // into a divergent branch around each computation)
  asm volatile("" :: "v"(sub), "v"(nrm));
  const uint32_t code = sign | (a < 0x3c800000u ? sub : (nrm > 0x7Eu ? 0x7Eu : nrm));
  return a > 0x7f800000u ? 0x7Fu : code;
}

// Value of an e4m3fn code (codes 0x7F / 0xFF never reach the kernels: the
// quantiser saturates and weight codes are finite by contract).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  float mag = e == 0 ? float(m) * (1.0f / 512.0f)
                     : __uint_as_float(((e + 120u) << 23) | (m << 20));
  return (c & 0x80u) ? -mag : mag;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Row range of expert-group g in the grouped row space: routed expert e < E owns
// rows [offsets[e], offsets[e+1]); shared expert E+s owns the T rows starting at
// T*K + s*T, in token order.
__device__ __forceinline__ void group_rows(const int32_t* offsets, int g, int E, int T, int TK,
                                           int& r0, int& r1) {
  if (g < E) {
    r0 = offsets[g];
    r1 = offsets[g + 1];
  } else {
    r0 = TK + (g - E) * T;
    r1 = r0 + T;
  }
}

// Token whose activation feeds grouped row r.
__device__ __forceinline__ int row_token_of(const int32_t* row_token, int r, int T, int TK) {
  return r < TK ? row_token[r] : (r - TK) % T;
}

}  // namespace moe
