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
// d_ff > 512 loops over 512-unit chunks (the hidden tile is re-read from L2).
#include "tg_common.h"

namespace tg {

constexpr int GS_BU = 512;   // units per work-group chunk
constexpr int GS_BK = 32;    // d slice per pipeline stage (64-byte rows)
constexpr int GS_THREADS = 512;
constexpr int GS_NA = 3;     // W1 slice ring depth (L2-resident operand)
constexpr int GS_NB = 6;     // hidden slice ring depth (HBM-streamed operand)

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t lds_u32;
__device__ void gs_buffer_load_lds(i32x4 rsrc, lds_u32 *lds, int size, int voffset, int soffset, int offset,
                                   int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
__device__ __forceinline__ i32x4 gs_rsrc(const void *base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}

// Work-group tile: 128 tokens x 512 units, 8 waves (2 along tokens x 4 along
// units), each wave 64 tokens x 128 units (8 accumulators of 32x32).  Slices
// of 32 d arrive by direct buffer->LDS loads into two rings (W1: 3 stages,
// hidden: 6 stages, so the HBM stream is prefetched 5 slices ahead).  LDS rows
// are 64 bytes with the 16-byte chunk XOR-swizzled by (row / 4) % 4, which
// keeps the 16-row MFMA fragment reads free of bank conflicts.  Out-of-range
// rows (the ragged token tail, units past d_ff) read as zero.
template <int TB>  // 32-token blocks per wave: 2 -> 128-token tiles, 1 -> 64-token tiles
__global__ __launch_bounds__(GS_THREADS) void gate_score_bf16_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ w1, const uint16_t *__restrict__ w2,
    const uint8_t *__restrict__ forced, int64_t T, int d, int d_ff, float *__restrict__ scores,
    float *__restrict__ gates) {
  constexpr int BT = 64 * TB;               // tokens per work-group
  constexpr int A_ST = GS_BU * GS_BK;       // u16 per W1 stage (32 KB)
  constexpr int B_ST = BT * GS_BK;          // u16 per hidden stage
  constexpr int NBI = BT / 16;               // hidden load instructions per slice (16 rows each): 8 or 4
  __shared__ __attribute__((aligned(1024))) uint16_t sA[GS_NA * A_ST];
  __shared__ __attribute__((aligned(1024))) uint16_t sB[GS_NB * B_ST];
  __shared__ __attribute__((aligned(1024))) uint16_t sDummy[512];  // target of the zero-fill loads of idle waves
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
  const uint32_t rowb = (uint32_t)d * 2u;  // bytes per row of hidden / W1
  // lane part of every direct load: row lane/4 of a 16-row instruction, chunk swizzled by (row / 4) % 4
  const uint32_t lsw = (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
  const int64_t trows = T - t0 < BT ? T - t0 : BT;
  const i32x4 rH = gs_rsrc(hidden + t0 * d, (uint32_t)(trows * rowb));
  // fragment reads: row r of a stage, logical chunk c -> physical c ^ ((r / 4) % 4); the row's low bits are l32
  const int fsw = (l32 >> 2) & 3;

  float run = 0.f;  // running score of token t0 + tid (tid < BT), across unit chunks

  for (int u0 = 0; u0 < d_ff; u0 += GS_BU) {
    const int urows = d_ff - u0 < GS_BU ? d_ff - u0 : GS_BU;
    const i32x4 rW = gs_rsrc(w1 + (int64_t)u0 * d, (uint32_t)urows * rowb);
    // W1 slice kt -> ring stage kt % NA: wave w fills rows 64w .. 64w+63 (4 instructions)
    auto issue_a = [&](int kt) {
      const bool live = kt < nk;
      const int stage = kt % GS_NA;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 64 * wave + 16 * i;
        const uint32_t vo = live ? (uint32_t)(r0 + (lane >> 2)) * rowb + lsw : 0xFFFFFFF0u;  // dead: zero fill
        gs_buffer_load_lds(rW, (lds_u32 *)(sA + stage * A_ST + r0 * GS_BK), 16, (int)vo, live ? kt * GS_BK * 2 : 0, 0, 0);
      }
    };
    // hidden slice kt -> ring stage kt % NB: wave w fills rows 16w .. 16w+15.  Every
    // wave issues exactly one load per slice (waves past the tile's rows load zeros
    // into sDummy), so each wave's count of loads in flight is the same.
    auto issue_b = [&](int kt) {
      const bool live = kt < nk && wave < NBI;
      const int r0 = 16 * wave;
      const uint32_t vo = live ? (uint32_t)(r0 + (lane >> 2)) * rowb + lsw : 0xFFFFFFF0u;
      uint16_t *dst = wave < NBI ? sB + (kt % GS_NB) * B_ST + r0 * GS_BK : sDummy;
      gs_buffer_load_lds(rH, (lds_u32 *)dst, 16, (int)vo, live ? kt * GS_BK * 2 : 0, 0, 0);
    };

    f32x16 acc[4][TB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < TB; ++j) acc[i][j] = f32x16{};

    // Prologue: hidden slices 0..2, then the batches of "iterations" -2 and -1.
    // Every iteration issues one batch {W1(kt+2), hidden(kt+5)} (dead slices load
    // zeros), so the number of loads issued after W1(kt) is constant.
    issue_b(0);
    issue_b(1);
    issue_b(2);
    issue_a(0);
    issue_b(3);
    issue_a(1);
    issue_b(4);
    for (int kt = 0; kt < nk; ++kt) {
      // outstanding after W1(kt): hidden(kt+3) and the 5 loads of iteration kt-1
      asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
      __syncthreads();  // slice kt landed for every wave; every wave is done with slice kt-1
      issue_a(kt + 2);
      issue_b(kt + 5);
      const uint16_t *A = sA + (kt % GS_NA) * A_ST;
      const uint16_t *Bt = sB + (kt % GS_NB) * B_ST;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int pc = ((2 * ks + hl) ^ fsw) << 3;
        u32x4 a[4], b[TB];
#pragma unroll
        for (int ub = 0; ub < 4; ++ub) a[ub] = *(const u32x4 *)(A + (wn * 128 + ub * 32 + l32) * GS_BK + pc);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) b[tb] = *(const u32x4 *)(Bt + (wm * 32 * TB + tb * 32 + l32) * GS_BK + pc);
#pragma unroll
        for (int ub = 0; ub < 4; ++ub)
#pragma unroll
          for (int tb = 0; tb < TB; ++tb) acc[ub][tb] = mfma32(a[ub], b[tb], acc[ub][tb]);
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // drain the dead tail loads

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
