// Permute: group the (token, expert) pairs by expert, tokens ascending inside an
// expert, with no pair dropped ("DeepSeek-V3 Technical Report 深度解读报告",
// section 2.4: no token dropping; section 2.3: loads are counted over the whole
// batch).
//
// Deterministic, in three passes over 64-token chunks:
//   1. masks: every (token, k) entry of a chunk ORs its token's bit into its expert's
//      64-bit mask in LDS (an OR commutes: the masks do not depend on the order; no
//      counter is shared);
//   2. scan:  one workgroup: per expert, running popcounts over the chunks give each
//      chunk's base row and the expert load; an LDS scan over experts gives offsets;
//   3. scatter: pair (t, k) with expert e goes to row
//      offsets[e] + base[chunk][e] + popcount(mask[chunk][e] & bits below t).
#include "kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void permute_masks(const int32_t* __restrict__ idx, int T,
                                                     int K, int E, uint64_t* __restrict__ masks) {
  // each (token, k) entry of the chunk sets its token's bit in its expert's mask (an OR:
  // the same masks in any order); entries outside [0, E) set nothing
  __shared__ unsigned long long m[256];
  const int c = blockIdx.x;
  const int t0 = c * kTokChunk;
  const int ntok = min(kTokChunk, T - t0);
  if (threadIdx.x < E) m[threadIdx.x] = 0ull;
  __syncthreads();
  for (int i = threadIdx.x; i < ntok * K; i += 256) {
    const int e = idx[size_t(t0) * K + i];
    if (e >= 0 && e < E) atomicOr(&m[e], 1ull << (i / K));
  }
  __syncthreads();
  if (threadIdx.x < E) masks[size_t(c) * E + threadIdx.x] = m[threadIdx.x];
}

// One workgroup of 256 threads (E <= 256).
__global__ __launch_bounds__(256) void permute_scan(const uint64_t* __restrict__ masks,
                                                    int chunks, int E,
                                                    int32_t* __restrict__ base,
                                                    int32_t* __restrict__ load,
                                                    int32_t* __restrict__ offsets) {
  __shared__ int32_t scan[256];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    int c = 0;
    for (; c + 8 <= chunks; c += 8) {
      int cnt[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) cnt[u] = __popcll(masks[size_t(c + u) * E + e]);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        base[size_t(c + u) * E + e] = run;
        run += cnt[u];
      }
    }
    for (; c < chunks; ++c) {
      base[size_t(c) * E + e] = run;
      run += __popcll(masks[size_t(c) * E + e]);
    }
  }
  // inclusive Hillis-Steele scan of the loads over experts
  scan[e] = run;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    int add = e >= d ? scan[e - d] : 0;
    __syncthreads();
    scan[e] += add;
    __syncthreads();
  }
  if (e < E) {
    load[e] = run;
    offsets[e] = scan[e] - run;
  }
  if (e == E - 1) offsets[E] = scan[e];
}

__global__ __launch_bounds__(256) void permute_scatter(
    const int32_t* __restrict__ idx, const uint64_t* __restrict__ masks,
    const int32_t* __restrict__ base, const int32_t* __restrict__ offsets, int T, int K, int E,
    int32_t* __restrict__ row_token, int32_t* __restrict__ pair_row) {
  __shared__ uint64_t m_lds[256];
  __shared__ int32_t b_lds[256];
  const int c = blockIdx.x;
  const int t0 = c * kTokChunk;
  const int ntok = min(kTokChunk, T - t0);
  if (threadIdx.x < E) {
    m_lds[threadIdx.x] = masks[size_t(c) * E + threadIdx.x];
    b_lds[threadIdx.x] = base[size_t(c) * E + threadIdx.x] + offsets[threadIdx.x];
  }
  __syncthreads();
  for (int p = threadIdx.x; p < ntok * K; p += 256) {
    const int tl = p / K;
    const size_t pair = size_t(t0) * K + p;
    const int e = idx[pair];
    if (unsigned(e) >= unsigned(E)) {   // outside the contract: keep every write in bounds
      pair_row[pair] = -1;
      continue;
    }
    const uint64_t below = tl == 0 ? 0ull : (~0ull >> (64 - tl));
    const int row = b_lds[e] + __popcll(m_lds[e] & below);
    row_token[row] = t0 + tl;
    pair_row[pair] = row;
  }
}

hipError_t launch_permute(const moe_config& c, const int32_t* idx, int32_t* load,
                          int32_t* offsets, int32_t* row_token, int32_t* pair_row,
                          const Workspace& ws, hipStream_t s) {
  const int T = c.num_tokens, K = c.top_k, E = c.num_experts;
  const int chunks = ceil_div(T, kTokChunk);
  hipLaunchKernelGGL(permute_masks, dim3(chunks), dim3(256), 0, s, idx, T, K, E, ws.masks);
  hipLaunchKernelGGL(permute_scan, dim3(1), dim3(256), 0, s, ws.masks, chunks, E, ws.base, load,
                     offsets);
  hipLaunchKernelGGL(permute_scatter, dim3(chunks), dim3(256), 0, s, idx, ws.masks, ws.base,
                     offsets, T, K, E, row_token, pair_row);
  return hipGetLastError();
}

}  // namespace moe
