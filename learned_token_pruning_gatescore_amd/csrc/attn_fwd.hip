// attn_fwd.hip -- token-gated causal attention, forward.
//
// TokenGate deep dive ("TokenGate: Learnable Token Pruning for Fast,
// Memory-Efficient LLM Prefill"): section 2, Eq. 2 (causal attention with
// z = q.k / sqrt(d)); section 3.2, Eq. 5 (each attention weight multiplied by
// its key's gate value, renormalised) and Eq. 6 (per-head gain); section 3.4
// (temperature folded into the query-side scale, the gate handed to the
// kernel as a per-key bias).  Summary page, Figure 1(c).  In log2 units:
//     S2_ij = (q^_i . k^_j) * c2 + gamma_h * log2 g_j,   c2 = log2(e) / (sqrt(D) tau)
//     o_i = sum_{j<=i} 2^(S2_ij - m_i) v_j / sum_{j<=i} 2^(S2_ij - m_i)
//
// bf16 kernel layout (gfx950, 32x32x16 bf16 MFMA, fp32 accumulate):
//   * one work-group = 4 waves = one (batch, kv head) and 128 "columns",
//     a column being a (query, head) pair of the GQA group: BQ = 128 / G query
//     positions x G heads share every K/V tile staged in LDS;
//   * each wave owns 32 columns; it computes S^T = K Q^T (keys on the MFMA
//     rows, its columns on the MFMA columns), so every lane holds 16 keys of a
//     single column: the softmax max / sum is lane-local plus one cross-half
//     shuffle, and P^T feeds the P.V product straight from registers;
//   * O^T = V^T P^T with V^T staged transposed in LDS; Q (rotated) lives in
//     registers for the whole key loop; K tiles are rotated while staged;
//   * 64-key tiles, online softmax in fp32, P rounded to bf16 for the MFMA.
#include "tg_common.h"

namespace tg {

// cos/sin table for the kept positions: cs[row][i] = (cos, sin)(pos[row] * theta^(-2i/D)),
// angle and trigonometry in fp64, stored as fp32.
__global__ void rope_table_kernel(const int32_t *__restrict__ pos, int64_t rows, int half, double theta,
                                  float2 *__restrict__ cs) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * half) return;
  const int64_t r = idx / half;
  const int i = (int)(idx % half);
  const double inv = pow(theta, -2.0 * (double)i / (double)(2 * half));
  const double phi = (double)pos[r] * inv;
  double s, c;
  sincos(phi, &s, &c);
  cs[idx] = make_float2((float)c, (float)s);
}

__device__ __forceinline__ float u16_elem(const u32x4 &x, int e) {
  const uint32_t w = x[e >> 1];
  return (e & 1) ? bf16_hi(w) : bf16_lo(w);
}

// Rotate the pair (x, y) = (first-half chunk, second-half chunk) in place.
__device__ __forceinline__ void rope_chunk(u32x4 &x, u32x4 &y, const float2 *__restrict__ t) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2 c0 = t[2 * w], c1 = t[2 * w + 1];
    const float x0 = bf16_lo(x[w]), x1 = bf16_hi(x[w]);
    const float y0 = bf16_lo(y[w]), y1 = bf16_hi(y[w]);
    x[w] = pack_bf16x2(x0 * c0.x - y0 * c0.y, x1 * c1.x - y1 * c1.y);
    y[w] = pack_bf16x2(y0 * c0.x + x0 * c0.y, y1 * c1.x + x1 * c1.y);
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ gamma, const float2 *__restrict__ cs, float c2,
    int B, int M, int Hq, int Hkv, int G, int BQ, int nqb, uint16_t *__restrict__ o, float *__restrict__ lse) {
  constexpr int NKS = D / 16;  // 16-wide k steps over the head dim
  constexpr int NDB = D / 32;  // 32-row blocks of O^T
  constexpr int KP = D + 8;    // sK row pitch (u16): conflict-free 16-byte reads
  constexpr int VP = 64 + 4;   // sVt row pitch (u16): conflict-free 8-byte reads
  constexpr int HALF = D / 2;
  __shared__ __attribute__((aligned(16))) uint16_t sK[64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * VP];
  __shared__ float sLg[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int nbh = B * Hkv;
  const int idx = blockIdx.x;
  const int qb = nqb - 1 - idx / nbh;  // longest causal rows first
  const int bh = idx % nbh;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int q0 = qb * BQ;
  const int col = wave * 32 + l32;
  const int hq = kvh * G + col / BQ;
  const int qi = q0 + col % BQ;
  const bool vq = qi < M;
  const int qmax = min(q0 + BQ, M) - 1;
  const int nt = qmax / 64 + 1;
  const int64_t bM = (int64_t)b * M;

  // Q fragments (MFMA B operand): lane holds q[qi, hq, 16ks + 8hl .. +8].
  u32x4 qf[NKS];
  const uint16_t *qrow = q + ((bM + qi) * Hq + hq) * D;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = vq ? *(const u32x4 *)(qrow + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
  if (cs && vq) {
#pragma unroll
    for (int ks = 0; ks < NKS / 2; ++ks) rope_chunk(qf[ks], qf[ks + NKS / 2], cs + (bM + qi) * HALF + 16 * ks + 8 * hl);
  }
  const float gam = gamma[hq];

  float m2 = -INFINITY, lsum = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};

  for (int t = 0; t < nt; ++t) {
    const int j0 = t * 64;
    __syncthreads();
    // K tile, rotated: 64 keys x (D/16) chunk pairs (d = 8c and 8c + D/2).
    for (int p = tid; p < 64 * (D / 16); p += 256) {
      const int key = p / (D / 16), c = p % (D / 16);
      const int j = j0 + key;
      u32x4 x0 = {0, 0, 0, 0}, x1 = {0, 0, 0, 0};
      if (j < M) {
        const uint16_t *kr = k + ((bM + j) * Hkv + kvh) * D;
        x0 = *(const u32x4 *)(kr + 8 * c);
        x1 = *(const u32x4 *)(kr + HALF + 8 * c);
        if (cs) rope_chunk(x0, x1, cs + (bM + j) * HALF + 8 * c);
      }
      *(u32x4 *)(&sK[key * KP + 8 * c]) = x0;
      *(u32x4 *)(&sK[key * KP + HALF + 8 * c]) = x1;
    }
    // V tile, transposed: thread = (4-key group, 8-wide d chunk).
    if (tid < 16 * (D / 8)) {
      const int kg = tid & 15, dc = tid >> 4;
      u32x4 w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 4 * kg + i;
        w[i] = (j < M) ? *(const u32x4 *)(v + ((bM + j) * Hkv + kvh) * D + 8 * dc) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        const uint32_t k0 = (w[0][e >> 1] >> sh) & 0xFFFFu, k1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
        const uint32_t k2 = (w[2][e >> 1] >> sh) & 0xFFFFu, k3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
        *(u32x2 *)(&sVt[(8 * dc + e) * VP + 4 * kg]) = u32x2{k0 | (k1 << 16), k2 | (k3 << 16)};
      }
    }
    if (tid < 64) {
      const int j = j0 + tid;
      const float gv = (j < M) ? g[bM + j] : 0.f;
      sLg[tid] = gv > 0.f ? fast_log2(gv) : -INFINITY;
    }
    __syncthreads();

    // S^T = K Q^T for 64 keys x 32 columns.
    f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *(const u32x4 *)(&sK[(kb * 32 + l32) * KP + 16 * ks + 8 * hl]);
        s[kb] = mfma32(a, qf[ks], s[kb]);
      }
    }
    const bool diag = j0 + 63 > q0;
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + acc_row(r, hl);
        const float lg = sLg[key];
        float x = (lg == -INFINITY) ? -INFINITY : s[kb][r] * c2 + gam * lg;
        if (diag && j0 + key > qi) x = -INFINITY;
        s[kb][r] = x;
        mloc = fmaxf(mloc, x);
      }
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mnew = fmaxf(m2, mloc);
    const float muse = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = fast_exp2(m2 - muse);
    m2 = mnew;
    float psum = 0.f;
    u32x4 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = fast_exp2(s[kb][8 * hf + 2 * w] - muse);
          const float p1 = fast_exp2(s[kb][8 * hf + 2 * w + 1] - muse);
          psum += p0 + p1;
          pf[kb][hf][w] = pack_bf16x2(p0, p1);
        }
      }
    }
    lsum = lsum * alpha + psum;
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    // O^T += V^T P^T; key slot 8*hl + e of step (kb, hf) is key kb*32 + 16hf + 8(e/4) + 4hl + e%4.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint16_t *vr = &sVt[(db * 32 + l32) * VP + kb * 32 + 16 * hf + 4 * hl];
          const u32x2 lo = *(const u32x2 *)vr, hi = *(const u32x2 *)(vr + 8);
          acc[db] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, pf[kb][hf], acc[db]);
        }
      }
    }
  }

  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (vq) {
    uint16_t *orow = o + ((bM + qi) * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hl;
        *(u32x2 *)(orow + d) = u32x2{pack_bf16x2(acc[db][4 * g4] * inv, acc[db][4 * g4 + 1] * inv),
                                     pack_bf16x2(acc[db][4 * g4 + 2] * inv, acc[db][4 * g4 + 3] * inv)};
      }
    }
    if (lse && hl == 0)
      lse[((int64_t)b * Hq + hq) * M + qi] = ltot > 0.f ? (m2 + __log2f(ltot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// fp32 path (plain arithmetic; small problems): one wave per (b, h, i) query
// row, lane = rotary pair index (D <= 128).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bias_of(float gam, float gv) {
  return gv > 0.f ? gam * logf(gv) : -INFINITY;
}

__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ gamma, const float2 *__restrict__ cs, float c,
    int B, int M, int Hq, int Hkv, int D, float *__restrict__ o, float *__restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, i, h) flattened
  if (row >= (int64_t)B * M * Hq) return;
  const int h = (int)(row % Hq);
  const int64_t bi = row / Hq;
  const int i = (int)(bi % M);
  const int64_t bM = bi - i;
  const int kv = h / (Hq / Hkv);
  const int half = D / 2;
  const bool act = lane < half;
  float qx = 0.f, qy = 0.f;
  if (act) {
    qx = q[row * D + lane];
    qy = q[row * D + half + lane];
    if (cs) {
      const float2 t = cs[bi * half + lane];
      const float x = qx * t.x - qy * t.y, y = qy * t.x + qx * t.y;
      qx = x;
      qy = y;
    }
  }
  const float gam = gamma[h];
  float m = -INFINITY, l = 0.f, ax = 0.f, ay = 0.f;
  for (int j = 0; j <= i; ++j) {
    const int64_t kr = ((bM + j) * Hkv + kv) * D;
    float kx = 0.f, ky = 0.f;
    if (act) {
      kx = k[kr + lane];
      ky = k[kr + half + lane];
      if (cs) {
        const float2 t = cs[(bM + j) * half + lane];
        const float x = kx * t.x - ky * t.y, y = ky * t.x + kx * t.y;
        kx = x;
        ky = y;
      }
    }
    const float sj = wave_sum(qx * kx + qy * ky) * c + bias_of(gam, g[bM + j]);
    if (sj == -INFINITY) continue;
    const float mn = fmaxf(m, sj);
    const float al = expf(m - mn), p = expf(sj - mn);
    l = l * al + p;
    float vx = 0.f, vy = 0.f;
    if (act) {
      vx = v[kr + lane];
      vy = v[kr + half + lane];
    }
    ax = ax * al + p * vx;
    ay = ay * al + p * vy;
    m = mn;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  if (act) {
    o[row * D + lane] = ax * inv;
    o[row * D + half + lane] = ay * inv;
  }
  if (lse && lane == 0) lse[((bM / M) * Hq + h) * M + i] = l > 0.f ? m + logf(l) : -INFINITY;
}

hipError_t launch_rope_table(const int32_t *pos, int64_t rows, int D, double theta, float2 *cs, hipStream_t s) {
  const int64_t n = rows * (D / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, pos, rows, D / 2,
                     theta, cs);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                           const float2 *cs, float tau, int B, int M, int Hq, int Hkv, int D, bool bf16, void *o,
                           float *lse, hipStream_t s) {
  if ((int64_t)B * M == 0) return hipSuccess;
  const double c = 1.0 / (sqrt((double)D) * (double)tau);
  if (bf16) {
    const int G = Hq / Hkv;
    const int BQ = 128 / G;
    const int nqb = (M + BQ - 1) / BQ;
    const dim3 grid((unsigned)(nqb * B * Hkv));
    const float c2 = (float)(c * 1.4426950408889634);
    if (D == 128)
      hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, dim3(256), 0, s, (const uint16_t *)q,
                         (const uint16_t *)k, (const uint16_t *)v, g, gamma, cs, c2, B, M, Hq, Hkv, G, BQ, nqb,
                         (uint16_t *)o, lse);
    else
      hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, dim3(256), 0, s, (const uint16_t *)q,
                         (const uint16_t *)k, (const uint16_t *)v, g, gamma, cs, c2, B, M, Hq, Hkv, G, BQ, nqb,
                         (uint16_t *)o, lse);
  } else {
    const int64_t rows = (int64_t)B * M * Hq;
    hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, (const float *)q,
                       (const float *)k, (const float *)v, g, gamma, cs, (float)c, B, M, Hq, Hkv, D, (float *)o,
                       lse);
  }
  return hipGetLastError();
}

}  // namespace tg
