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
// Each is one work-group of 1024 threads per row with fixed-shape reductions
// (bitwise deterministic).  These are latency-bound passes; they keep the
// whole scoring definition on the device without a host round trip.  The
// normalisation may run in place.
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

// Rows are read in chunks of SN_R values per thread (SN_T SN_R per chunk): all of
// a chunk's loads are issued before any is used, so a pass costs one memory
// latency per chunk rather than one per value.  A row of at most one chunk
// (32 K values) stays in registers between the passes.
constexpr int SN_R = 32;
constexpr int64_t SN_CHUNK = (int64_t)SN_T * SN_R;

// Element u of a thread's chunk is row index idx(u) = base + V (SN_T (u / V) + tid) + u % V:
// with V = 4 (rows whose length is a multiple of 4, so 16-byte aligned) a thread
// loads 4 consecutive values per instruction, with V = 1 one.  Group u / V is
// live for some thread iff base + V SN_T (u / V) < n, a work-group-uniform test,
// so empty groups cost a scalar branch.
template <int V>
__device__ __forceinline__ int64_t elem(int64_t base, int u) {
  return base + (int64_t)V * ((int64_t)SN_T * (u / V) + threadIdx.x) + u % V;
}
template <int V>
__device__ __forceinline__ bool slot_live(int64_t base, int u, int64_t n) {
  return base + (int64_t)V * SN_T * (u / V) < n;
}

template <int V, typename T>
__device__ __forceinline__ void load_chunk(const T *row, int64_t base, int64_t n, T fill, T (&x)[SN_R]) {
#pragma unroll
  for (int u = 0; u < SN_R; u += V) {
    const int64_t j = elem<V>(base, u);
#pragma unroll
    for (int e = 0; e < V; ++e) x[u + e] = fill;
    if (slot_live<V>(base, u, n) && j < n) {
      if constexpr (V == 4) {  // n % 4 == 0: the whole group is in range
        if constexpr (sizeof(T) == 4) {
          const uint4 w = *(const uint4 *)(row + j);
          x[u] = __builtin_bit_cast(T, w.x);
          x[u + 1] = __builtin_bit_cast(T, w.y);
          x[u + 2] = __builtin_bit_cast(T, w.z);
          x[u + 3] = __builtin_bit_cast(T, w.w);
        } else {
          const uint32_t w = *(const uint32_t *)(row + j);
#pragma unroll
          for (int e = 0; e < 4; ++e) x[u + e] = (T)((w >> (8 * e)) & 0xFFu);
        }
      } else {
        x[u] = row[j];
      }
    }
  }
}

// Row blockIdx.x of [rows, N]; with per-head scores [B, H, N] the rows are
// (b, h) and the forced mask is b's: row / heads.
template <int V>
__global__ __launch_bounds__(SN_T) void score_normalize_kernel(const float *s, const uint8_t *__restrict__ forced,
                                                              int64_t N, float eps, int heads, float *out) {
  __shared__ float red[SN_T / 64];
  const int64_t b = blockIdx.x;
  const float *row = s + b * N;
  const uint8_t *f = forced ? forced + (b / heads) * N : nullptr;
  float x[SN_R];
  uint8_t fx[SN_R];
  float ss = 0.f, np = 0.f;  // np: exact in fp32 (at most 2^24 positions per row)
  for (int64_t base = 0; base < N; base += SN_CHUNK) {
    load_chunk<V>(row, base, N, 0.f, x);
    if (f) load_chunk<V>(f, base, N, (uint8_t)1, fx);
#pragma unroll
    for (int u = 0; u < SN_R; ++u) {
      if (!slot_live<V>(base, u, N)) break;
      const bool p = f ? fx[u] == 0 : elem<V>(base, u) < N;
      if (p) {
        ss = __builtin_fmaf(x[u], x[u], ss);
        np += 1.f;
      }
    }
  }
  const float tot = block_reduce<false>(ss, red);
  const float cnt = block_reduce<false>(np, red);
  const float r = cnt > 0.f ? sqrtf(tot / cnt + eps) : 1.f;
  const float rinv = 1.f / r;  // x * (1 / r): within an ulp of x / r
  for (int64_t base = 0; base < N; base += SN_CHUNK) {
    if (N > SN_CHUNK) {  // the row did not stay in registers
      load_chunk<V>(row, base, N, 0.f, x);
      if (f) load_chunk<V>(f, base, N, (uint8_t)1, fx);
    }
#pragma unroll
    for (int u = 0; u < SN_R; u += V) {
      if (!slot_live<V>(base, u, N)) break;
      const int64_t j = elem<V>(base, u);
      if (j >= N) continue;
      float y[V];
#pragma unroll
      for (int e = 0; e < V; ++e) y[e] = (f && fx[u + e]) ? 0.f : x[u + e] * rinv;
      if constexpr (V == 4)
        *(float4 *)(out + b * N + j) = make_float4(y[0], y[1], y[2], y[3]);
      else
        out[b * N + j] = y[0];
    }
  }
}

template <int V>
__global__ __launch_bounds__(SN_T) void gate_softmax_kernel(const float *__restrict__ xin,
                                                           const int32_t *__restrict__ kept, int64_t M, int heads,
                                                           float *__restrict__ g) {
  __shared__ float red[SN_T / 64];
  const int64_t b = blockIdx.x;  // row (b, h) with per-head scores: kept row b / heads
  const float *row = xin + b * M;
  const int32_t *k = kept ? kept + (b / heads) * M : nullptr;
  float x[SN_R];
  int32_t kx[SN_R];
  auto load = [&](int64_t base) __attribute__((always_inline)) {
    load_chunk<V>(row, base, M, -INFINITY, x);
    if (k) {
      load_chunk<V>(k, base, M, (int32_t)-1, kx);
#pragma unroll
      for (int u = 0; u < SN_R; ++u)
        if (kx[u] < 0) x[u] = -INFINITY;  // padding: not in S
    }
  };
  float mx = -INFINITY;
  for (int64_t base = 0; base < M; base += SN_CHUNK) {
    load(base);
#pragma unroll
    for (int u = 0; u < SN_R; ++u) {
      if (!slot_live<V>(base, u, M)) break;
      mx = fmaxf(mx, x[u]);
    }
  }
  mx = block_reduce<true>(mx, red);
  float z = 0.f;
  for (int64_t base = 0; base < M; base += SN_CHUNK) {
    if (M > SN_CHUNK) load(base);
#pragma unroll
    for (int u = 0; u < SN_R; ++u) {
      if (!slot_live<V>(base, u, M)) break;
      z += x[u] == -INFINITY ? 0.f : expf(x[u] - mx);
    }
  }
  z = block_reduce<false>(z, red);
  const float inv = z > 0.f ? 1.f / z : 0.f;
  for (int64_t base = 0; base < M; base += SN_CHUNK) {
    if (M > SN_CHUNK) load(base);
#pragma unroll
    for (int u = 0; u < SN_R; ++u) {
      if (!slot_live<V>(base, u, M)) break;
      const int64_t j = elem<V>(base, u);
      if (j < M) g[b * M + j] = x[u] == -INFINITY ? 0.f : expf(x[u] - mx) * inv;
    }
  }
}

// db_j = g_j (dg_j - sum_k g_k dg_k)
template <int V>
__global__ __launch_bounds__(SN_T) void gate_softmax_bwd_kernel(const float *__restrict__ g, const float *__restrict__ dg,
                                                               int64_t M, float *__restrict__ db) {
  __shared__ float red[SN_T / 64];
  const int64_t b = blockIdx.x;
  float gx[SN_R], dx[SN_R];
  float dot = 0.f;
  for (int64_t base = 0; base < M; base += SN_CHUNK) {
    load_chunk<V>(g + b * M, base, M, 0.f, gx);
    load_chunk<V>(dg + b * M, base, M, 0.f, dx);
#pragma unroll
    for (int u = 0; u < SN_R; ++u) {
      if (!slot_live<V>(base, u, M)) break;
      dot = __builtin_fmaf(gx[u], dx[u], dot);
    }
  }
  dot = block_reduce<false>(dot, red);
  for (int64_t base = 0; base < M; base += SN_CHUNK) {
    if (M > SN_CHUNK) {
      load_chunk<V>(g + b * M, base, M, 0.f, gx);
      load_chunk<V>(dg + b * M, base, M, 0.f, dx);
    }
#pragma unroll
    for (int u = 0; u < SN_R; ++u) {
      if (!slot_live<V>(base, u, M)) break;
      const int64_t j = elem<V>(base, u);
      if (j < M) db[b * M + j] = gx[u] * (dx[u] - dot);
    }
  }
}

// Uniform aggregation over heads for selection: out[b][n] = (sum_h s[b][h][n]) / H,
// heads summed in order.
__global__ __launch_bounds__(256) void aggregate_heads_kernel(const float *__restrict__ s, int64_t B, int H, int64_t N,
                                                             float *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= B * N) return;
  const int64_t b = i / N, n = i - b * N;
  float acc = 0.f;
  for (int h = 0; h < H; ++h) acc += s[(b * H + h) * N + n];
  out[i] = acc / (float)H;
}

// out[b][h][m] = s[b][h][kept[b][m]] (0 for padding, kept < 0)
__global__ __launch_bounds__(256) void gather_heads_kernel(const float *__restrict__ s, const int32_t *__restrict__ kept,
                                                          int64_t B, int H, int64_t N, int64_t M,
                                                          float *__restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= B * H * M) return;
  const int64_t bh = i / M, m = i - bh * M, b = bh / H;
  const int32_t j = kept[b * M + m];
  out[i] = (j >= 0 && j < N) ? s[bh * N + j] : 0.f;
}

hipError_t launch_score_normalize(const float *s, const uint8_t *forced, int64_t B, int64_t N, float eps, float *out,
                                  hipStream_t st, int heads) {
  if (B * N == 0) return hipSuccess;
  if (N % 4 == 0)
    hipLaunchKernelGGL(score_normalize_kernel<4>, dim3((unsigned)B), dim3(SN_T), 0, st, s, forced, N, eps, heads, out);
  else
    hipLaunchKernelGGL(score_normalize_kernel<1>, dim3((unsigned)B), dim3(SN_T), 0, st, s, forced, N, eps, heads, out);
  return hipGetLastError();
}

hipError_t launch_gate_softmax(const float *x, const int32_t *kept, int64_t B, int64_t M, float *g, hipStream_t st,
                               int heads) {
  if (B * M == 0) return hipSuccess;
  if (M % 4 == 0)
    hipLaunchKernelGGL(gate_softmax_kernel<4>, dim3((unsigned)B), dim3(SN_T), 0, st, x, kept, M, heads, g);
  else
    hipLaunchKernelGGL(gate_softmax_kernel<1>, dim3((unsigned)B), dim3(SN_T), 0, st, x, kept, M, heads, g);
  return hipGetLastError();
}

hipError_t launch_aggregate_heads(const float *s, int64_t B, int H, int64_t N, float *out, hipStream_t st) {
  if (B * N == 0) return hipSuccess;
  hipLaunchKernelGGL(aggregate_heads_kernel, dim3((unsigned)((B * N + 255) / 256)), dim3(256), 0, st, s, B, H, N, out);
  return hipGetLastError();
}

hipError_t launch_gather_heads(const float *s, const int32_t *kept, int64_t B, int H, int64_t N, int64_t M, float *out,
                               hipStream_t st) {
  if (B * H * M == 0) return hipSuccess;
  hipLaunchKernelGGL(gather_heads_kernel, dim3((unsigned)((B * H * M + 255) / 256)), dim3(256), 0, st, s, kept, B, H,
                     N, M, out);
  return hipGetLastError();
}

hipError_t launch_gate_softmax_bwd(const float *g, const float *dg, int64_t B, int64_t M, float *db, hipStream_t st) {
  if (B * M == 0) return hipSuccess;
  if (M % 4 == 0)
    hipLaunchKernelGGL(gate_softmax_bwd_kernel<4>, dim3((unsigned)B), dim3(SN_T), 0, st, g, dg, M, db);
  else
    hipLaunchKernelGGL(gate_softmax_bwd_kernel<1>, dim3((unsigned)B), dim3(SN_T), 0, st, g, dg, M, db);
  return hipGetLastError();
}

}  // namespace tg
