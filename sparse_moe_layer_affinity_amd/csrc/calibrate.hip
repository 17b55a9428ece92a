// Calibration kernels for the measurements (not part of the layer): what this
// device sustains for plain HBM read and write streams and for back-to-back MFMAs, to quote
// the expert GEMMs' rates against measured ceilings next to the datasheet peaks.
// Built into its own library (libmoe_calib.so); only the benchmark loads it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

// Every lane streams 16-byte vectors, eight in flight, grid-stride over the buffer;
// the XOR of everything read is written per thread so no load is dropped.
__global__ __launch_bounds__(256) void read_stream(const uint4* __restrict__ p, size_t n16,
                                                   uint4* __restrict__ out) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  uint4 acc = make_uint4(0, 0, 0, 0);
  for (; i + 7 * stride < n16; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p[i + u * stride];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      acc.x ^= v[u].x; acc.y ^= v[u].y; acc.z ^= v[u].z; acc.w ^= v[u].w;
    }
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc.x ^= a.x; acc.y ^= a.y; acc.z ^= a.z; acc.w ^= a.w;
  }
  out[size_t(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

// Every lane writes 16-byte vectors, grid-stride over the buffer (a plain HBM write
// stream).
__global__ __launch_bounds__(256) void write_stream(uint4* __restrict__ p, size_t n16) {
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  const uint4 v = make_uint4(t, t ^ 0x55555555u, t * 3u, ~t);
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride) p[i] = v;
}

__device__ __forceinline__ uint32_t mix(uint32_t v) {
  v ^= v >> 16; v *= 0x7feb352dU; v ^= v >> 15; v *= 0x846ca68bU; v ^= v >> 16;
  return v;
}

// Eight independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave on
// register operands (hashed lane-dependent bits, so the data toggles like real
// operands; bf16 values kept finite by clearing the top exponent bit).
__global__ __launch_bounds__(256) void mfma_loop_bf16(int iters, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  int ai[4], bi[4];
  for (int q = 0; q < 4; ++q) {
    ai[q] = int(mix(t * 8 + q) & 0xBFFFBFFFu);
    bi[q] = int(mix(t * 8 + 4 + q) & 0xBFFFBFFFu);
  }
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ai);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bi);
  f32x16_t acc[8];
  for (int c = 0; c < 8; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
  for (int c = 0; c < 8; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[t] = s;
}

// The same with the FP8 (e4m3) 32x32x64 block-scaled MFMA at unit scales.
__global__ __launch_bounds__(256) void mfma_loop_fp8(int iters, float* __restrict__ out) {
  const uint32_t t = blockIdx.x * blockDim.x + threadIdx.x;
  i32x8_t a, b;
  for (int q = 0; q < 8; ++q) {
    a[q] = int(mix(t * 16 + q) & 0x7E7E7E7Eu);      // finite e4m3 codes
    b[q] = int(mix(t * 16 + 8 + q) & 0x7E7E7E7Eu);
  }
  f32x16_t acc[8];
  for (int c = 0; c < 8; ++c)
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc[c] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, acc[c], 0, 0, 0, 127, 0, 127);
  }
  float s = 0.f;
  for (int c = 0; c < 8; ++c)
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  out[t] = s;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from the device buffer `buf` once (eight 16-byte
// loads in flight per lane); `out` is a device
// buffer of blocks * 256 * 16 bytes.  Returns a hipError_t.
int moe_calib_read(const void* buf, size_t bytes, void* out, int blocks, void* stream) {
  hipLaunchKernelGGL(read_stream, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), bytes / 16, static_cast<uint4*>(out));
  return int(hipGetLastError());
}

// Writes `bytes` (a multiple of 16) to the device buffer `buf` once.  Returns a
// hipError_t.
int moe_calib_write(void* buf, size_t bytes, int blocks, void* stream) {
  hipLaunchKernelGGL(write_stream, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(buf), bytes / 16);
  return int(hipGetLastError());
}

// blocks workgroups of four waves, each wave iters x 8 MFMAs: bf16 32x32x16 (fp8 == 0,
// 32768 flops each) or e4m3 32x32x64 (fp8 != 0, 131072 flops each).  `out` is a device
// buffer of blocks * 256 floats.  Returns a hipError_t.
int moe_calib_mfma(int fp8, int iters, float* out, int blocks, void* stream) {
  if (fp8)
    hipLaunchKernelGGL(mfma_loop_fp8, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       iters, out);
  else
    hipLaunchKernelGGL(mfma_loop_bf16, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                       iters, out);
  return int(hipGetLastError());
}

}  // extern "C"
