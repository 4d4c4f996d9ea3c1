// gate_score.hip -- the scoring MLP of every token and its gate value.
//
// TokenGate deep dive ("TokenGate: Learnable Token Pruning for Fast,
// Memory-Efficient LLM Prefill"), section 3.1, Eq. 3 first part: a small MLP
// maps each token's normalised residual to one scalar score; here
//     s_t = sum_k w2[k] * SiLU(sum_i w1[k,i] h[t,i]),
//     g_t = 1 for a forced token, else sigmoid(s_t).
//
// bf16 path: a [d_ff x d] x [d x T] product on the matrix cores (32x32x16 bf16
// MFMA, fp32 accumulation).  The W1 rows are the MFMA "A" operand and the
// token rows the "B" operand, so each lane's accumulator holds 16 units of ONE
// token: the SiLU * w2 reduction over units is lane-local, then one cross-half
// shuffle and a 4-way LDS sum across the waves that split the units.  Nothing
// of the [T, d_ff] activation ever leaves registers.
//
// Work-group tile: 128 tokens x 512 units, 8 waves (2 along tokens x 4 along
// units), each wave 64 tokens x 128 units (8 accumulators of 32x32).  The d
// loop runs in 32-wide slices, double-buffered in LDS, with the next slice's
// global loads in flight during the current slice's MFMAs.  d_ff > 512 loops
// over 512-unit chunks.
#include "tg_common.h"

namespace tg {

constexpr int GS_BU = 512;   // units per work-group chunk
constexpr int GS_BK = 32;    // d slice per pipeline stage
constexpr int GS_ROW = 40;   // LDS row pitch in u16: 32 data + 8 pad (80 B: conflict-free b128 reads)
constexpr int GS_THREADS = 512;

template <int TB>  // 32-token blocks per wave: 2 -> 128-token tiles, 1 -> 64-token tiles
__global__ __launch_bounds__(GS_THREADS) void gate_score_bf16_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ w1,
    const uint16_t *__restrict__ w2, const uint8_t *__restrict__ forced, int64_t T, int d,
    int d_ff, float *__restrict__ scores, float *__restrict__ gates) {
  constexpr int BT = 64 * TB;             // tokens per work-group
  constexpr int A_CHUNKS = GS_BU * 4;     // 16-byte chunks of a W1 slice (512 rows x 64 B)
  constexpr int B_CHUNKS = BT * 4;        // 16-byte chunks of a hidden slice
  constexpr int A_PER_T = A_CHUNKS / GS_THREADS;
  constexpr int B_PER_T = (B_CHUNKS + GS_THREADS - 1) / GS_THREADS;

  __shared__ __attribute__((aligned(16))) uint16_t sA[2][GS_BU * GS_ROW];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][BT * GS_ROW];
  __shared__ float sRed[4][BT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wn = wave & 3;   // unit quarter
  const int wm = wave >> 2;  // token half
  const int l32 = lane & 31;
  const int hl = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * BT;
  const int nk = d / GS_BK;

  float run = 0.f;  // running score of token t0 + tid (tid < BT), across unit chunks

  for (int u0 = 0; u0 < d_ff; u0 += GS_BU) {
    f32x16 acc[4][TB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TB; ++j) acc[i][j] = f32x16{};

    u32x4 ra[A_PER_T], rb[B_PER_T];
    auto gload = [&](int kt) {
      const int k0 = kt * GS_BK;
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const int id = tid + i * GS_THREADS;
        const int row = id >> 2, c = id & 3;
        const int u = u0 + row;
        ra[i] = (u < d_ff) ? *(const u32x4 *)(w1 + (int64_t)u * d + k0 + c * 8) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const int id = tid + i * GS_THREADS;
        const int row = id >> 2, c = id & 3;
        const int64_t t = t0 + row;
        rb[i] = (id < B_CHUNKS && t < T) ? *(const u32x4 *)(hidden + t * d + k0 + c * 8)
                                         : u32x4{0, 0, 0, 0};
      }
    };
    auto lstore = [&](int buf) {
#pragma unroll
      for (int i = 0; i < A_PER_T; ++i) {
        const int id = tid + i * GS_THREADS;
        *(u32x4 *)(&sA[buf][(id >> 2) * GS_ROW + (id & 3) * 8]) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < B_PER_T; ++i) {
        const int id = tid + i * GS_THREADS;
        if (id < B_CHUNKS) *(u32x4 *)(&sB[buf][(id >> 2) * GS_ROW + (id & 3) * 8]) = rb[i];
      }
    };

    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        u32x4 a[4], b[TB];
#pragma unroll
        for (int ub = 0; ub < 4; ++ub)
          a[ub] = *(const u32x4 *)(&sA[buf][(wn * 128 + ub * 32 + l32) * GS_ROW + ks * 16 + hl * 8]);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
          b[tb] = *(const u32x4 *)(&sB[buf][(wm * 32 * TB + tb * 32 + l32) * GS_ROW + ks * 16 + hl * 8]);
#pragma unroll
        for (int ub = 0; ub < 4; ++ub)
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[ub][tb] = mfma32(a[ub], b[tb], acc[ub][tb]);
      }
      if (kt + 1 < nk) lstore(buf ^ 1);
      __syncthreads();
    }

    // Epilogue: SiLU, times w2, summed over this lane's units.
    float part[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) part[tb] = 0.f;
#pragma unroll
    for (int ub = 0; ub < 4; ++ub) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ubase = u0 + wn * 128 + ub * 32 + 8 * g4 + 4 * hl;  // 4 consecutive units
        float wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int u = ubase + e;
          wv[e] = (u < d_ff) ? __uint_as_float((uint32_t)w2[u] << 16) : 0.f;
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = acc[ub][tb][g4 * 4 + e];
            const float silu = x * fast_rcp(1.f + fast_exp2(-x * kLog2e));
            part[tb] += silu * wv[e];
          }
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      part[tb] += __shfl_xor(part[tb], 32);
      if (hl == 0) sRed[wn][wm * 32 * TB + tb * 32 + l32] = part[tb];
    }
    __syncthreads();
    if (tid < BT) run += (sRed[0][tid] + sRed[1][tid]) + (sRed[2][tid] + sRed[3][tid]);
    __syncthreads();
  }

  if (tid < BT) {
    const int64_t t = t0 + tid;
    if (t < T) {
      scores[t] = run;
      if (gates) {
        const bool f = forced && forced[t];
        gates[t] = f ? 1.f : fast_rcp(1.f + fast_exp2(-run * kLog2e));
      }
    }
  }
}

// fp32 path: one work-group (4 waves) per token; waves take units round-robin,
// lanes split d; fixed-order reductions (deterministic).
__global__ __launch_bounds__(256) void gate_score_f32_kernel(
    const float *__restrict__ hidden, const float *__restrict__ w1, const float *__restrict__ w2,
    const uint8_t *__restrict__ forced, int64_t T, int d, int d_ff, float *__restrict__ scores,
    float *__restrict__ gates) {
  extern __shared__ float sh[];  // d floats
  __shared__ float sPart[4];
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < d; i += 256) sh[i] = hidden[t * d + i];
  __syncthreads();
  float part = 0.f;
  for (int k = wave; k < d_ff; k += 4) {
    const float *row = w1 + (int64_t)k * d;
    float u = 0.f;
    for (int i = lane; i < d; i += 64) u += row[i] * sh[i];
    u = wave_sum(u);
    const float silu = u / (1.f + expf(-u));
    part += silu * w2[k];
  }
  if (lane == 0) sPart[wave] = part;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float s = (sPart[0] + sPart[1]) + (sPart[2] + sPart[3]);
    scores[t] = s;
    if (gates) gates[t] = (forced && forced[t]) ? 1.f : 1.f / (1.f + expf(-s));
  }
}

hipError_t launch_gate_score(const void *hidden, const void *w1, const void *w2,
                             const uint8_t *forced, int64_t T, int d, int d_ff, bool bf16,
                             float *scores, float *gates, hipStream_t s) {
  if (T == 0) return hipSuccess;
  if (bf16) {
    const int64_t tiles128 = (T + 127) / 128;
    if (tiles128 >= 256) {
      hipLaunchKernelGGL(gate_score_bf16_kernel<2>, dim3((unsigned)tiles128), dim3(GS_THREADS), 0, s,
                         (const uint16_t *)hidden, (const uint16_t *)w1, (const uint16_t *)w2, forced,
                         T, d, d_ff, scores, gates);
    } else {
      hipLaunchKernelGGL(gate_score_bf16_kernel<1>, dim3((unsigned)((T + 63) / 64)), dim3(GS_THREADS), 0,
                         s, (const uint16_t *)hidden, (const uint16_t *)w1, (const uint16_t *)w2, forced,
                         T, d, d_ff, scores, gates);
    }
  } else {
    hipLaunchKernelGGL(gate_score_f32_kernel, dim3((unsigned)T), dim3(256), (size_t)d * sizeof(float), s,
                       (const float *)hidden, (const float *)w1, (const float *)w2, forced, T, d, d_ff,
                       scores, gates);
  }
  return hipGetLastError();
}

}  // namespace tg
