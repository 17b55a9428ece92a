// Router affinities and the sequence-wise balance loss.
//
// "DeepSeek-V3 Technical Report 深度解读报告", section 2.3: beside the selection
// bias, a sequence-level balance loss L_Bal with a very small coefficient alpha
// keeps a single sequence from routing all its tokens to a few experts; section
// 4.4 compares sequence-wise with batch-wise auxiliary losses.  The pages give no
// formula; the form used is the usual one (per sequence of L tokens):
//   s'_{t,e} = s_{t,e} / sum_j s_{t,j}
//   f_e = E / (K L) * (number of the sequence's tokens that selected e)
//   P_e = (1 / L) * sum_t s'_{t,e}
//   loss = alpha * sum_e f_e P_e
// and its gradient with respect to the router logits (f held fixed):
//   dz_{t,e} = alpha / L * (f_e - sum_i f_i s'_{t,i}) / sum_j s_{t,j} * s_{t,e} (1 - s_{t,e}).
//
// All three kernels are small and memory-bound ([T, E] fp32 in, [T, E] fp32 out for
// the gradient).  Every sum runs in a fixed order, so results are deterministic:
//  - balance_partials: one workgroup per chunk of kBalChunk tokens of one sequence;
//    its waves load their rows together, stage them in LDS and form each row's sum
//    (a fixed butterfly, identical in every lane); thread e then walks the chunk's
//    tokens in order, summing s'_{t,e}; selections are counted with integer LDS
//    atomics (one per thread).
//  - balance_reduce: one workgroup per sequence; four slices of threads add the
//    chunk partials in batches of 16 loads in flight, the slices are added in a
//    fixed order, and a fixed-shape LDS tree sums f_e P_e.
//  - balance_grad: one wave per token (4 experts per lane), the same row sum as
//    balance_partials, and a second butterfly for sum_i f_i s_{t,i}.
#include "kernels.h"

namespace moe {

constexpr int kBalChunk = 32;   // tokens per partial-sum chunk
constexpr int kGradWaves = 4;

// affinities = sigmoid(split-K logit partials summed in split order): the same
// additions and the same sigmoid expression as the selection kernel, so these are
// the values the router selected on
__global__ __launch_bounds__(256) void router_scores(const float* __restrict__ z, int splits,
                                                     int n, float* __restrict__ s) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float acc = z[i];
  for (int p = 1; p < splits; ++p) acc += z[size_t(p) * n + i];
  s[i] = 1.0f / (1.0f + expf(-acc));
}

// sum over a wave of the lane's four experts (fixed association; every lane ends
// with the same bits because each butterfly step adds the same two values)
__device__ __forceinline__ float wave_sum4(const float v[4]) {
  float x = ((v[0] + v[1]) + v[2]) + v[3];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ __launch_bounds__(256) void balance_partials(
    const float* __restrict__ s, const int32_t* __restrict__ idx, int E, int K, int L,
    int chunks_per_seq, float* __restrict__ part_p, int32_t* __restrict__ part_c) {
  constexpr int kRows = kBalChunk / 4;      // rows per wave
  __shared__ float tile[kBalChunk][256];
  __shared__ float row_sum[kBalChunk];
  __shared__ int32_t count[256];
  const int c = blockIdx.x;
  const int q = c / chunks_per_seq, j = c % chunks_per_seq;
  const int t0 = q * L + j * kBalChunk;
  const int rem = L - j * kBalChunk;
  const int nt = rem < kBalChunk ? rem : kBalChunk;
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  count[threadIdx.x] = 0;

  // all of the wave's rows in flight at once (and one selection per thread: nt*K
  // <= 256), then the row sums
  float v[kRows][4];
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr) {
    const int r = w + 4 * rr;
    const float* row = s + size_t(t0 + (r < nt ? r : 0)) * E;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int e = l + 64 * jj;
      v[rr][jj] = (r < nt && e < E) ? row[e] : 0.0f;
    }
  }
  const int my_sel = threadIdx.x < nt * K ? idx[size_t(t0) * K + threadIdx.x] : -1;
#pragma unroll
  for (int rr = 0; rr < kRows; ++rr) {
    const int r = w + 4 * rr;
    if (r < nt) {                           // uniform over the wave
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) tile[r][l + 64 * jj] = v[rr][jj];
      const float sum = wave_sum4(v[rr]);
      if (l == 0) row_sum[r] = sum;
    }
  }
  __syncthreads();
  // selections per expert: integer LDS atomics (exact in any order); entries
  // outside [0, E) are not counted
  if (my_sel >= 0 && my_sel < E) atomicAdd(&count[my_sel], 1);

  const int e = threadIdx.x;
  float acc = 0.0f;
  if (e < E) {
#pragma unroll 8
    for (int r = 0; r < nt; ++r) acc += tile[r][e] / row_sum[r];
  }
  __syncthreads();
  if (e >= E) return;
  part_p[size_t(c) * E + e] = acc;
  part_c[size_t(c) * E + e] = count[e];
}

// one workgroup per sequence: kRedSlices slices of 256 threads (thread = expert);
// slice k takes chunk batches k, k + kRedSlices, ... of kRedBatch chunks each, all
// of a batch's loads in flight at once; the slices' sums are then added in slice
// order, so the result does not depend on timing
constexpr int kRedSlices = 4;
constexpr int kRedBatch = 16;

__global__ __launch_bounds__(kRedSlices * 256) void balance_reduce(
    const float* __restrict__ part_p, const int32_t* __restrict__ part_c, int E, int K, int L,
    int chunks_per_seq, float alpha, float* __restrict__ loss, float* __restrict__ f_out,
    float* __restrict__ p_out) {
  __shared__ float ps[kRedSlices][256];
  __shared__ int32_t cs[kRedSlices][256];
  __shared__ float prod[256];
  const int q = blockIdx.x, e = threadIdx.x % 256, slice = threadIdx.x / 256;
  float psum = 0.0f;
  int cnt = 0;
  if (e < E) {
    const size_t base = size_t(q) * chunks_per_seq;
    for (int j0 = slice * kRedBatch; j0 < chunks_per_seq; j0 += kRedSlices * kRedBatch) {
      float pv[kRedBatch];
      int cv[kRedBatch];
#pragma unroll
      for (int i = 0; i < kRedBatch; ++i) {
        const bool ok = j0 + i < chunks_per_seq;
        const size_t at = (base + (ok ? j0 + i : 0)) * E + e;
        pv[i] = ok ? part_p[at] : 0.0f;
        cv[i] = ok ? part_c[at] : 0;
      }
#pragma unroll
      for (int i = 0; i < kRedBatch; ++i) {
        psum += pv[i];
        cnt += cv[i];
      }
    }
  }
  ps[slice][e] = psum;
  cs[slice][e] = cnt;
  __syncthreads();
  if (slice == 0) {
    float fe = 0.0f, pe = 0.0f;
    if (e < E) {
      float p = ps[0][e];
      int n = cs[0][e];
#pragma unroll
      for (int k = 1; k < kRedSlices; ++k) {
        p += ps[k][e];
        n += cs[k][e];
      }
      fe = float(double(n) * E / (double(K) * L));   // one rounding of the exact ratio
      pe = p / float(L);
      f_out[size_t(q) * E + e] = fe;
      if (p_out) p_out[size_t(q) * E + e] = pe;
    }
    prod[e] = fe * pe;
  }
  __syncthreads();
#pragma unroll
  for (int h = 128; h >= 1; h >>= 1) {
    if (threadIdx.x < h) prod[threadIdx.x] += prod[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[q] = alpha * prod[0];
}

__global__ __launch_bounds__(kGradWaves * 64) void balance_grad(
    const float* __restrict__ s, const float* __restrict__ f, int T, int E, int L, float alpha,
    float* __restrict__ grad) {
  const int w = threadIdx.x / 64, l = threadIdx.x % 64;
  const int t = blockIdx.x * kGradWaves + w;
  if (t >= T) return;                       // no barrier below: whole waves leave
  const float* row = s + size_t(t) * E;
  const float* fq = f + size_t(t / L) * E;
  float v[4], fv[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int e = l + 64 * jj;
    v[jj] = e < E ? row[e] : 0.0f;
    fv[jj] = e < E ? fq[e] * v[jj] : 0.0f;
  }
  const float sum = wave_sum4(v);
  const float weighted = wave_sum4(fv) / sum;        // sum_i f_i s'_{t,i}
  const float scale = alpha / float(L) / sum;
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int e = l + 64 * jj;
    if (e < E)
      grad[size_t(t) * E + e] = scale * (fq[e] - weighted) * (v[jj] * (1.0f - v[jj]));
  }
}

hipError_t launch_router_scores(const moe_config& c, const float* z, float* scores,
                                hipStream_t st) {
  const int n = c.num_tokens * c.num_experts;
  hipLaunchKernelGGL(router_scores, dim3(ceil_div(n, 256)), dim3(256), 0, st, z,
                     router_splits(c), n, scores);
  return hipGetLastError();
}

hipError_t launch_balance_loss(const moe_config& c, const float* scores, const int32_t* idx,
                               int L, float alpha, float* loss, float* frac, float* prob,
                               float* grad, const Workspace& w, hipStream_t st) {
  const int T = c.num_tokens, E = c.num_experts, K = c.top_k;
  const int S = T / L;
  const int cps = ceil_div(L, kBalChunk);
  float* f = frac ? frac : w.bal_f;
  hipLaunchKernelGGL(balance_partials, dim3(S * cps), dim3(256), 0, st, scores, idx, E, K, L,
                     cps, w.bal_p, w.bal_c);
  hipLaunchKernelGGL(balance_reduce, dim3(S), dim3(kRedSlices * 256), 0, st, w.bal_p, w.bal_c, E, K, L, cps,
                     alpha, loss, f, prob);
  if (grad)
    hipLaunchKernelGGL(balance_grad, dim3(ceil_div(T, kGradWaves)), dim3(kGradWaves * 64), 0, st,
                       scores, f, T, E, L, alpha, grad);
  return hipGetLastError();
}

}  // namespace moe
