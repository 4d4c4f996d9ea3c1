// score_norm.hip -- the sequence RMS normalisation of the scores and the
// softmax-over-S gate.
//
// TokenGate deep dive ("TokenGate: Learnable Token Pruning for Fast,
// Memory-Efficient LLM Prefill"):
//   section 3.1, Eq. 3 (second part): the raw scores of one request are divided
//     by their root mean square over the prunable positions P, and the
//     non-prunable positions N get 0:
//       b_j = b~_j / sqrt((1/|P|) sum_{j' in P} b~_{j'}^2 + eps)   (j in P)
//       b_j = 0                                                   (j in N)
//   section 3.2, Eq. 5: the gate of a kept token is the softmax of b over the
//     kept set S: g_j = exp(b_j) / sum_{j' in S} exp(b_j').  (Eq. 6's per-head
//     gain c multiplies b inside the softmax; softmax_S(c b) = softmax_S(b)^c / Z,
//     so the attention bias gamma_h ln g_j with gamma_h = c_h gives Eq. 6 up to a
//     per-head constant that the attention softmax removes.)
//
// Each is one work-group of 1024 threads per row (a row is a few thousand to a
// few hundred thousand values, streamed twice: once for the reduction, once
// for the output), with fixed-shape reductions (bitwise deterministic).  These
// are latency-bound passes; they keep the whole scoring definition on the
// device without a host round trip.  The normalisation may run in place.
#include "tg_common.h"

namespace tg {

constexpr int SN_T = 1024;  // threads per work-group

// Fixed-shape block reduction (sum or max) over the 1024 threads.
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float y = __shfl_xor(v, o);
    v = MAX ? fmaxf(v, y) : v + y;
  }
  __syncthreads();  // red is free (a previous reduction's readers are done)
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < SN_T / 64; ++w) r = MAX ? fmaxf(r, red[w]) : r + red[w];
  return r;
}

__global__ __launch_bounds__(SN_T) void score_normalize_kernel(const float *s, const uint8_t *__restrict__ forced,
                                                              int64_t N, float eps, float *out) {
  __shared__ float red[SN_T / 64];
  const int64_t b = blockIdx.x;
  const float *row = s + b * N;
  const uint8_t *f = forced ? forced + b * N : nullptr;
  float ss = 0.f, np = 0.f;  // np counts exactly in fp32 up to 2^24 positions per thread
  for (int64_t j = threadIdx.x; j < N; j += SN_T) {
    const bool p = !(f && f[j]);
    const float x = row[j];
    if (p) {
      ss = __builtin_fmaf(x, x, ss);
      np += 1.f;
    }
  }
  const float tot = block_reduce<false>(ss, red);
  const float cnt = block_reduce<false>(np, red);
  const float r = cnt > 0.f ? sqrtf(tot / cnt + eps) : 1.f;
  for (int64_t j = threadIdx.x; j < N; j += SN_T) {
    const bool p = !(f && f[j]);
    out[b * N + j] = p ? row[j] / r : 0.f;
  }
}

__global__ __launch_bounds__(SN_T) void gate_softmax_kernel(const float *__restrict__ x, const int32_t *__restrict__ kept,
                                                           int64_t M, float *__restrict__ g) {
  __shared__ float red[SN_T / 64];
  const int64_t b = blockIdx.x;
  const float *row = x + b * M;
  const int32_t *k = kept ? kept + b * M : nullptr;
  float mx = -INFINITY;
  for (int64_t j = threadIdx.x; j < M; j += SN_T)
    if (!(k && k[j] < 0)) mx = fmaxf(mx, row[j]);
  mx = block_reduce<true>(mx, red);
  float z = 0.f;
  for (int64_t j = threadIdx.x; j < M; j += SN_T)
    if (!(k && k[j] < 0)) z += expf(row[j] - mx);
  z = block_reduce<false>(z, red);
  const float inv = z > 0.f ? 1.f / z : 0.f;
  for (int64_t j = threadIdx.x; j < M; j += SN_T)
    g[b * M + j] = (k && k[j] < 0) ? 0.f : expf(row[j] - mx) * inv;
}

// db_j = g_j (dg_j - sum_k g_k dg_k)
__global__ __launch_bounds__(SN_T) void gate_softmax_bwd_kernel(const float *__restrict__ g, const float *__restrict__ dg,
                                                               int64_t M, float *__restrict__ db) {
  __shared__ float red[SN_T / 64];
  const int64_t b = blockIdx.x;
  float dot = 0.f;
  for (int64_t j = threadIdx.x; j < M; j += SN_T) dot = __builtin_fmaf(g[b * M + j], dg[b * M + j], dot);
  dot = block_reduce<false>(dot, red);
  for (int64_t j = threadIdx.x; j < M; j += SN_T) db[b * M + j] = g[b * M + j] * (dg[b * M + j] - dot);
}

hipError_t launch_score_normalize(const float *s, const uint8_t *forced, int64_t B, int64_t N, float eps, float *out,
                                  hipStream_t st) {
  if (B * N == 0) return hipSuccess;
  hipLaunchKernelGGL(score_normalize_kernel, dim3((unsigned)B), dim3(SN_T), 0, st, s, forced, N, eps, out);
  return hipGetLastError();
}

hipError_t launch_gate_softmax(const float *x, const int32_t *kept, int64_t B, int64_t M, float *g, hipStream_t st) {
  if (B * M == 0) return hipSuccess;
  hipLaunchKernelGGL(gate_softmax_kernel, dim3((unsigned)B), dim3(SN_T), 0, st, x, kept, M, g);
  return hipGetLastError();
}

hipError_t launch_gate_softmax_bwd(const float *g, const float *dg, int64_t B, int64_t M, float *db, hipStream_t st) {
  if (B * M == 0) return hipSuccess;
  hipLaunchKernelGGL(gate_softmax_bwd_kernel, dim3((unsigned)B), dim3(SN_T), 0, st, g, dg, M, db);
  return hipGetLastError();
}

}  // namespace tg
