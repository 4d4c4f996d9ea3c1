// attn_bwd.hip -- token-gated causal attention, backward.
//
// The task gradient reaches the scorer through the attention bias (TokenGate
// deep dive, "TokenGate: Learnable Token Pruning for Fast, Memory-Efficient
// LLM Prefill", section 3.1 last paragraph, section 3.2, and the flowchart's
// "task gradient through bias" edge).  With P the forward's softmax and
// S_ij = c q^_i.k^_j + gamma_h ln g_j:
//     dP_ij = dO_i . v_j,   D_i = sum_j P_ij dP_ij,   dS_ij = P_ij (dP_ij - D_i)
//     dq^_i = c sum_j dS_ij k^_j,  dk^_j = c sum_i dS_ij q^_i,  dv_j = sum_i P_ij dO_i
//     colsum_h(j) = sum_i dS_ij -> dg_j = sum_h gamma_h colsum_h(j) / g_j,
//                                   dgamma_h = sum_{b,j} colsum_h(j) ln g_j
// then dq, dk rotated back by -phi.
//
// bf16 path, three launches, no atomics (bitwise deterministic):
//   1. q-outer (same work-group shape as the forward: 4 waves x 32 (query,
//      head) columns sharing one kv head's tiles): pass A forms D_i from fp32
//      P and fp32 dP (not from the rounded output), pass B forms dS and
//      accumulates dQ^T = K^T dS^T on the matrix cores; writes dq and D.
//   2. kv-outer: each wave owns 32 keys (MFMA columns = keys, so the column
//      sum of dS over queries is lane-local); loops over the group's heads and
//      the query tiles at or after its keys; accumulates dV^T = dO^T P and
//      dK^T = Q^T dS; writes dk, dv and colsum per head.
//   3. dg (per token, fixed head order) and dgamma (one work-group per head,
//      fixed-shape tree).
#include "tg_common.h"
#include "tg_attn.h"

namespace tg {

__device__ __forceinline__ void rope_chunk2(u32x4 &x, u32x4 &y, const float2 *__restrict__ t) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2 c0 = t[2 * w], c1 = t[2 * w + 1];
    const float x0 = bf16_lo(x[w]), x1 = bf16_hi(x[w]);
    const float y0 = bf16_lo(y[w]), y1 = bf16_hi(y[w]);
    x[w] = pack_bf16x2(x0 * c0.x - y0 * c0.y, x1 * c1.x - y1 * c1.y);
    y[w] = pack_bf16x2(y0 * c0.x + x0 * c0.y, y1 * c1.x + x1 * c1.y);
  }
}

// Writes 4 rows (consecutive tokens) x 8 columns (chunk of d) of bf16 both as
// rows of sRow[token][d] (pitch RP) and transposed into sT[d][token] (pitch TP).
template <int RP, int TP>
__device__ __forceinline__ void store_rows_and_transpose(uint16_t *sRow, uint16_t *sT, int tok0, int d0,
                                                         const u32x4 (&w)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) *(u32x4 *)(&sRow[(tok0 + i) * RP + d0]) = w[i];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int sh = (e & 1) * 16;
    const uint32_t a0 = (w[0][e >> 1] >> sh) & 0xFFFFu, a1 = (w[1][e >> 1] >> sh) & 0xFFFFu;
    const uint32_t a2 = (w[2][e >> 1] >> sh) & 0xFFFFu, a3 = (w[3][e >> 1] >> sh) & 0xFFFFu;
    *(u32x2 *)(&sT[(d0 + e) * TP + tok0]) = u32x2{a0 | (a1 << 16), a2 | (a3 << 16)};
  }
}

// Stage a 64-token tile of a [*, H, D] bf16 tensor (row stride H*D, head offset
// applied by the caller) into sRow (and, if TRANS, transposed into sT), rotating
// by the rotary table when cs != nullptr.  All 256 threads call it.
template <int D, bool TRANS>
__device__ __forceinline__ void stage_tile(const uint16_t *__restrict__ base, int64_t rstride, int t0, int M,
                                           const float2 *__restrict__ cs_b, uint16_t *sRow, uint16_t *sT, int tid) {
  constexpr int RP = D + 8, TP = 64 + 4, HALF = D / 2, NC = D / 16;
  // thread -> (4-token group tg4 in 0..15, chunk pair c in 0..NC-1); 16*NC <= 128 threads busy
  for (int p = tid; p < 16 * NC; p += 256) {
    const int tg4 = p & 15, c = p >> 4;
    u32x4 x[4], y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * tg4 + i;
      if (t < M) {
        const uint16_t *r = base + (int64_t)t * rstride;
        x[i] = *(const u32x4 *)(r + 8 * c);
        y[i] = *(const u32x4 *)(r + HALF + 8 * c);
        if (cs_b) rope_chunk2(x[i], y[i], cs_b + (int64_t)t * HALF + 8 * c);
      } else {
        x[i] = u32x4{0, 0, 0, 0};
        y[i] = u32x4{0, 0, 0, 0};
      }
    }
    if (TRANS) {
      store_rows_and_transpose<RP, TP>(sRow, sT, 4 * tg4, 8 * c, x);
      store_rows_and_transpose<RP, TP>(sRow, sT, 4 * tg4, HALF + 8 * c, y);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        *(u32x4 *)(&sRow[(4 * tg4 + i) * RP + 8 * c]) = x[i];
        *(u32x4 *)(&sRow[(4 * tg4 + i) * RP + HALF + 8 * c]) = y[i];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 1. q-outer: D_i and dq.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ gamma, const float2 *__restrict__ cs,
    const float *__restrict__ lse, const uint16_t *__restrict__ dout, float c, float c2, int B, int M, int Hq,
    int Hkv, int G, int BQ, int nqb, float *__restrict__ dq, float *__restrict__ delta_out) {
  constexpr int NKS = D / 16, NDB = D / 32, KP = D + 8, VP = 64 + 4, HALF = D / 2;
  __shared__ __attribute__((aligned(16))) uint16_t sK[64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sKt[D * VP];
  __shared__ __attribute__((aligned(16))) uint16_t sV[64 * KP];
  __shared__ float sLg[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int nbh = B * Hkv;
  const int idx = blockIdx.x;
  const int qb = nqb - 1 - idx / nbh;
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
  const float2 *cs_b = cs ? cs + bM * HALF : nullptr;

  u32x4 qf[NKS], df[NKS];
  const int64_t roff = ((bM + qi) * Hq + hq) * D;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    qf[ks] = vq ? *(const u32x4 *)(q + roff + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
    df[ks] = vq ? *(const u32x4 *)(dout + roff + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
  }
  if (cs && vq) {
#pragma unroll
    for (int ks = 0; ks < NKS / 2; ++ks) rope_chunk2(qf[ks], qf[ks + NKS / 2], cs + (bM + qi) * HALF + 16 * ks + 8 * hl);
  }
  const float gam = gamma[hq];
  const float lrow = vq ? lse[((int64_t)b * Hq + hq) * M + qi] : -INFINITY;
  const bool live = lrow != -INFINITY;
  const float l2 = live ? lrow * kLog2e : 0.f;
  const uint16_t *kb_ = k + (int64_t)kvh * D;
  const uint16_t *vb_ = v + (int64_t)kvh * D;
  const int64_t kstride = (int64_t)Hkv * D;

  // logits -> P (fp32) for one 64-key tile held as S^T in s[2]
  auto probs = [&](f32x16(&s)[2], int j0) {
    const bool diag = j0 + 63 > q0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb * 32 + acc_row(r, hl);
        const float lg = sLg[key];
        float p = (lg == -INFINITY || !live) ? 0.f : fast_exp2(s[kb][r] * c2 + gam * lg - l2);
        if (diag && j0 + key > qi) p = 0.f;
        s[kb][r] = p;
      }
    }
  };

  // pass A: D_i = sum_j P_ij dP_ij
  float dsum = 0.f;
  for (int pass = 0; pass < 2; ++pass) {
    f32x16 acc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
    float dlt = 0.f;
    if (pass == 1) dlt = dsum;
    for (int t = 0; t < nt; ++t) {
      const int j0 = t * 64;
      __syncthreads();
      const int64_t kbase_off = bM * kstride;
      stage_tile<D, true>(kb_ + kbase_off, kstride, j0, M, cs_b, sK, sKt, tid);
      stage_tile<D, false>(vb_ + kbase_off, kstride, j0, M, nullptr, sV, nullptr, (tid + 128) & 255);
      if (tid < 64) {
        const int j = j0 + tid;
        const float gv = (j < M) ? g[bM + j] : 0.f;
        sLg[tid] = gv > 0.f ? fast_log2(gv) : -INFINITY;
      }
      __syncthreads();
      f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a = *(const u32x4 *)(&sK[(kb * 32 + l32) * KP + 16 * ks + 8 * hl]);
          s[kb] = mfma32(a, qf[ks], s[kb]);
          const u32x4 av = *(const u32x4 *)(&sV[(kb * 32 + l32) * KP + 16 * ks + 8 * hl]);
          dp[kb] = mfma32(av, df[ks], dp[kb]);
        }
      }
      probs(s, j0);
      if (pass == 0) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) dsum += s[kb][r] * dp[kb][r];
      } else {
        u32x4 dsf[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const int r0 = 8 * hf + 2 * w;
              dsf[kb][hf][w] = pack_bf16x2(s[kb][r0] * (dp[kb][r0] - dlt), s[kb][r0 + 1] * (dp[kb][r0 + 1] - dlt));
            }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const uint16_t *kr = &sKt[(db * 32 + l32) * VP + kb * 32 + 16 * hf + 4 * hl];
              const u32x2 lo = *(const u32x2 *)kr, hi = *(const u32x2 *)(kr + 8);
              acc[db] = mfma32(u32x4{lo[0], lo[1], hi[0], hi[1]}, dsf[kb][hf], acc[db]);
            }
      }
    }
    if (pass == 0) {
      dsum += __shfl_xor(dsum, 32);
      if (vq && hl == 0) delta_out[((int64_t)b * Hq + hq) * M + qi] = dsum;
    } else if (vq) {
      // dq = c * R(-phi) dq^ ; lane holds rows d = db*32 + acc_row(r, hl)
      float *drow = dq + ((bM + qi) * Hq + hq) * D;
#pragma unroll
      for (int db = 0; db < NDB / 2; ++db) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hl;
          float xo[4], yo[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = acc[db][4 * g4 + e] * c, y = acc[db + NDB / 2][4 * g4 + e] * c;
            if (cs) {
              const float2 t = cs[(bM + qi) * HALF + d + e];
              xo[e] = x * t.x + y * t.y;
              yo[e] = y * t.x - x * t.y;
            } else {
              xo[e] = x;
              yo[e] = y;
            }
          }
          *(f32x4 *)(drow + d) = f32x4{xo[0], xo[1], xo[2], xo[3]};
          *(f32x4 *)(drow + HALF + d) = f32x4{yo[0], yo[1], yo[2], yo[3]};
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 2. kv-outer: dk, dv, colsum.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k, const uint16_t *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ gamma, const float2 *__restrict__ cs,
    const float *__restrict__ lse, const uint16_t *__restrict__ dout, const float *__restrict__ delta, float c,
    float c2, int B, int M, int Hq, int Hkv, int G, int nkb, float *__restrict__ dk, float *__restrict__ dv,
    float *__restrict__ colsum) {
  constexpr int NKS = D / 16, NDB = D / 32, KP = D + 8, VP = 64 + 4, HALF = D / 2;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sQt[D * VP];
  __shared__ __attribute__((aligned(16))) uint16_t sO[64 * KP];
  __shared__ __attribute__((aligned(16))) uint16_t sOt[D * VP];
  __shared__ float sL2[64], sDl[64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int nbh = B * Hkv;
  const int idx = blockIdx.x;
  const int kblk = idx / nbh;  // low keys (most queries) first
  const int bh = idx % nbh;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int k0 = kblk * 128;
  const int kw0 = k0 + wave * 32;  // this wave's first key
  const int key = kw0 + l32;
  const bool vk = key < M;
  const int64_t bM = (int64_t)b * M;
  const float2 *cs_b = cs ? cs + bM * HALF : nullptr;

  // K^, V fragments of this lane's key (MFMA B operand).
  u32x4 kf[NKS], vf[NKS];
  const int64_t koff = ((bM + key) * Hkv + kvh) * D;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    kf[ks] = vk ? *(const u32x4 *)(k + koff + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
    vf[ks] = vk ? *(const u32x4 *)(v + koff + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
  }
  if (cs && vk) {
#pragma unroll
    for (int ks = 0; ks < NKS / 2; ++ks) rope_chunk2(kf[ks], kf[ks + NKS / 2], cs + (bM + key) * HALF + 16 * ks + 8 * hl);
  }
  const float gv = vk ? g[bM + key] : 0.f;
  const float lg = gv > 0.f ? fast_log2(gv) : -INFINITY;

  f32x16 aK[NDB], aV[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    aK[i] = f32x16{};
    aV[i] = f32x16{};
  }
  const int tq0 = k0 / 64;  // first query tile that can see these keys
  const int ntq = (M + 63) / 64;
  const int64_t qstride = (int64_t)Hq * D;

  for (int hh = 0; hh < G; ++hh) {
    const int h = kvh * G + hh;
    const float gam = gamma[h];
    float csum = 0.f;
    for (int tq = tq0; tq < ntq; ++tq) {
      const int i0 = tq * 64;
      __syncthreads();
      stage_tile<D, true>(q + bM * qstride + (int64_t)h * D, qstride, i0, M, cs_b, sQ, sQt, tid);
      stage_tile<D, true>(dout + bM * qstride + (int64_t)h * D, qstride, i0, M, nullptr, sO, sOt, (tid + 128) & 255);
      if (tid < 64) {
        const int i = i0 + tid;
        const float l = i < M ? lse[((int64_t)b * Hq + h) * M + i] : -INFINITY;
        sL2[tid] = l == -INFINITY ? INFINITY : l * kLog2e;  // +inf -> P = 0
        sDl[tid] = i < M ? delta[((int64_t)b * Hq + h) * M + i] : 0.f;
      }
      __syncthreads();
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {  // 32-query halves of the tile
        const int qa = i0 + 32 * qh;
        if (qa + 31 < kw0) continue;  // every query before every key of this wave
        f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const u32x4 a = *(const u32x4 *)(&sQ[(32 * qh + l32) * KP + 16 * ks + 8 * hl]);
          s = mfma32(a, kf[ks], s);
          const u32x4 ao = *(const u32x4 *)(&sO[(32 * qh + l32) * KP + 16 * ks + 8 * hl]);
          dp = mfma32(ao, vf[ks], dp);
        }
        u32x4 pf[2], dsf[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            float pp[2], dd[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 8 * hf + 2 * w + e;
              const int ql = 32 * qh + acc_row(r, hl);  // query within the tile
              const int qg = i0 + ql;
              float p = (lg == -INFINITY || qg < key) ? 0.f : fast_exp2(s[r] * c2 + gam * lg - sL2[ql]);
              const float ds = p * (dp[r] - sDl[ql]);
              csum += ds;
              pp[e] = p;
              dd[e] = ds;
            }
            pf[hf][w] = pack_bf16x2(pp[0], pp[1]);
            dsf[hf][w] = pack_bf16x2(dd[0], dd[1]);
          }
        }
        // dV^T += dO^T P, dK^T += Q^T dS ; query slot 8hl+e of step hf is row 16hf + 8(e/4) + 4hl + e%4
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const uint16_t *orr = &sOt[(db * 32 + l32) * VP + 32 * qh + 16 * hf + 4 * hl];
            const u32x2 olo = *(const u32x2 *)orr, ohi = *(const u32x2 *)(orr + 8);
            aV[db] = mfma32(u32x4{olo[0], olo[1], ohi[0], ohi[1]}, pf[hf], aV[db]);
            const uint16_t *qr = &sQt[(db * 32 + l32) * VP + 32 * qh + 16 * hf + 4 * hl];
            const u32x2 qlo = *(const u32x2 *)qr, qhi = *(const u32x2 *)(qr + 8);
            aK[db] = mfma32(u32x4{qlo[0], qlo[1], qhi[0], qhi[1]}, dsf[hf], aK[db]);
          }
        }
      }
    }
    csum += __shfl_xor(csum, 32);
    if (vk && hl == 0) colsum[((int64_t)b * Hq + h) * M + key] = csum;
  }

  if (vk) {
    float *dkr = dk + koff;
    float *dvr = dv + koff;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hl;
        *(f32x4 *)(dvr + d) = f32x4{aV[db][4 * g4], aV[db][4 * g4 + 1], aV[db][4 * g4 + 2], aV[db][4 * g4 + 3]};
      }
    }
#pragma unroll
    for (int db = 0; db < NDB / 2; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hl;
        float xo[4], yo[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = aK[db][4 * g4 + e] * c, y = aK[db + NDB / 2][4 * g4 + e] * c;
          if (cs) {
            const float2 t = cs[(bM + key) * HALF + d + e];
            xo[e] = x * t.x + y * t.y;
            yo[e] = y * t.x - x * t.y;
          } else {
            xo[e] = x;
            yo[e] = y;
          }
        }
        *(f32x4 *)(dkr + d) = f32x4{xo[0], xo[1], xo[2], xo[3]};
        *(f32x4 *)(dkr + HALF + d) = f32x4{yo[0], yo[1], yo[2], yo[3]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 path (plain arithmetic; small problems).  Lane = rotary pair index.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void rot(float &x, float &y, const float2 *cs, int64_t idx, float sgn) {
  if (!cs) return;
  const float2 t = cs[idx];
  const float s = sgn * t.y;
  const float a = x * t.x - y * s, b = y * t.x + x * s;
  x = a;
  y = b;
}

__device__ __forceinline__ float logit_bias(float gam, float gv) { return gv > 0.f ? gam * logf(gv) : -INFINITY; }

// one wave per (b, i, h): D_i and dq
__global__ __launch_bounds__(256) void attn_bwd_dq_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ gamma, const float2 *__restrict__ cs,
    const float *__restrict__ lse, const float *__restrict__ dout, float c, int B, int M, int Hq, int Hkv, int D,
    float *__restrict__ dq, float *__restrict__ delta) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)B * M * Hq) return;
  const int h = (int)(row % Hq);
  const int64_t bi = row / Hq;
  const int i = (int)(bi % M);
  const int64_t bM = bi - i;
  const int64_t b = bM / M;
  const int kv = h / (Hq / Hkv);
  const int half = D / 2;
  const bool act = lane < half;
  float qx = 0.f, qy = 0.f, ox = 0.f, oy = 0.f;
  if (act) {
    qx = q[row * D + lane];
    qy = q[row * D + half + lane];
    rot(qx, qy, cs, bi * half + lane, 1.f);
    ox = dout[row * D + lane];
    oy = dout[row * D + half + lane];
  }
  const float gam = gamma[h];
  const float l = lse[(b * Hq + h) * M + i];
  float Di = 0.f;
  if (l != -INFINITY) {
    for (int j = 0; j <= i; ++j) {
      const int64_t kr = ((bM + j) * Hkv + kv) * D;
      float kx = 0.f, ky = 0.f, vx = 0.f, vy = 0.f;
      if (act) {
        kx = k[kr + lane];
        ky = k[kr + half + lane];
        rot(kx, ky, cs, (bM + j) * half + lane, 1.f);
        vx = v[kr + lane];
        vy = v[kr + half + lane];
      }
      const float sj = wave_sum(qx * kx + qy * ky) * c + logit_bias(gam, g[bM + j]);
      const float p = sj == -INFINITY ? 0.f : expf(sj - l);
      Di += p * wave_sum(ox * vx + oy * vy);
    }
  }
  float ax = 0.f, ay = 0.f;
  if (l != -INFINITY) {
    for (int j = 0; j <= i; ++j) {
      const int64_t kr = ((bM + j) * Hkv + kv) * D;
      float kx = 0.f, ky = 0.f, vx = 0.f, vy = 0.f;
      if (act) {
        kx = k[kr + lane];
        ky = k[kr + half + lane];
        rot(kx, ky, cs, (bM + j) * half + lane, 1.f);
        vx = v[kr + lane];
        vy = v[kr + half + lane];
      }
      const float sj = wave_sum(qx * kx + qy * ky) * c + logit_bias(gam, g[bM + j]);
      const float p = sj == -INFINITY ? 0.f : expf(sj - l);
      const float ds = p * (wave_sum(ox * vx + oy * vy) - Di);
      ax += ds * kx;
      ay += ds * ky;
    }
  }
  ax *= c;
  ay *= c;
  if (act) {
    rot(ax, ay, cs, bi * half + lane, -1.f);
    dq[row * D + lane] = ax;
    dq[row * D + half + lane] = ay;
  }
  if (lane == 0) delta[(b * Hq + h) * M + i] = Di;
}

// one wave per (b, j, kv head): dk, dv, colsum of every head of the group
__global__ __launch_bounds__(256) void attn_bwd_dkdv_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ gamma, const float2 *__restrict__ cs,
    const float *__restrict__ lse, const float *__restrict__ dout, const float *__restrict__ delta, float c, int B,
    int M, int Hq, int Hkv, int D, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ colsum) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, j, kv)
  if (row >= (int64_t)B * M * Hkv) return;
  const int kv = (int)(row % Hkv);
  const int64_t bj = row / Hkv;
  const int j = (int)(bj % M);
  const int64_t bM = bj - j;
  const int64_t b = bM / M;
  const int G = Hq / Hkv;
  const int half = D / 2;
  const bool act = lane < half;
  float kx = 0.f, ky = 0.f, vx = 0.f, vy = 0.f;
  if (act) {
    kx = k[row * D + lane];
    ky = k[row * D + half + lane];
    rot(kx, ky, cs, bj * half + lane, 1.f);
    vx = v[row * D + lane];
    vy = v[row * D + half + lane];
  }
  const float gv = g[bj];
  float akx = 0.f, aky = 0.f, avx = 0.f, avy = 0.f;
  for (int hh = 0; hh < G; ++hh) {
    const int h = kv * G + hh;
    const float bias = logit_bias(gamma[h], gv);
    float cs_h = 0.f;
    if (bias != -INFINITY) {
      for (int i = j; i < M; ++i) {
        const int64_t qr = ((bM + i) * Hq + h) * D;
        const float l = lse[(b * Hq + h) * M + i];
        if (l == -INFINITY) continue;
        float qx = 0.f, qy = 0.f, ox = 0.f, oy = 0.f;
        if (act) {
          qx = q[qr + lane];
          qy = q[qr + half + lane];
          rot(qx, qy, cs, (bM + i) * half + lane, 1.f);
          ox = dout[qr + lane];
          oy = dout[qr + half + lane];
        }
        const float p = expf(wave_sum(qx * kx + qy * ky) * c + bias - l);
        const float ds = p * (wave_sum(ox * vx + oy * vy) - delta[(b * Hq + h) * M + i]);
        cs_h += ds;
        akx += ds * qx;
        aky += ds * qy;
        avx += p * ox;
        avy += p * oy;
      }
    }
    if (lane == 0) colsum[(b * Hq + h) * M + j] = cs_h;
  }
  akx *= c;
  aky *= c;
  if (act) {
    rot(akx, aky, cs, bj * half + lane, -1.f);
    dk[row * D + lane] = akx;
    dk[row * D + half + lane] = aky;
    dv[row * D + lane] = avx;
    dv[row * D + half + lane] = avy;
  }
}

// ---------------------------------------------------------------------------
// 3. gate gradients
// ---------------------------------------------------------------------------
__global__ void dg_kernel(const float *__restrict__ colsum, const float *__restrict__ g,
                          const float *__restrict__ gamma, int B, int M, int Hq, float *__restrict__ dg) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)B * M) return;
  const int64_t b = idx / M, j = idx % M;
  float acc = 0.f;
  for (int h = 0; h < Hq; ++h) acc += gamma[h] * colsum[(b * Hq + h) * M + j];
  const float gv = g[idx];
  dg[idx] = gv > 0.f ? acc / gv : 0.f;
}

__global__ __launch_bounds__(256) void dgamma_kernel(const float *__restrict__ colsum, const float *__restrict__ g,
                                                     int B, int M, int Hq, float *__restrict__ dgamma) {
  __shared__ float red[256];
  const int h = blockIdx.x;
  float acc = 0.f;
  for (int64_t idx = threadIdx.x; idx < (int64_t)B * M; idx += 256) {
    const int64_t b = idx / M, j = idx % M;
    const float gv = g[idx];
    if (gv > 0.f) acc += colsum[(b * Hq + h) * M + j] * logf(gv);
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) dgamma[h] = red[0];
}

hipError_t launch_attn_bwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                           const int32_t *pos, double theta, float tau, const float *lse, const void *dout, int B,
                           int M, int Hq, int Hkv, int D, bool bf16, float *dq, float *dk, float *dv, float *dg,
                           float *dgamma, const AttnWs &w, hipStream_t s) {
  float *ws_delta = w.delta, *ws_colsum = w.colsum;
  const float2 *cs = pos ? w.cs : nullptr;
  if ((int64_t)B * M > 0 && pos) {
    hipError_t e = launch_attn_prep(k, g, gamma, pos, theta, B, M, Hq, Hkv, D, false, false, w, s);
    if (e != hipSuccess) return e;
  }
  const double cd = 1.0 / (sqrt((double)D) * (double)tau);
  const float c = (float)cd, c2 = (float)(cd * 1.4426950408889634);
  if ((int64_t)B * M > 0) {
    if (bf16) {
      const int G = Hq / Hkv;
      const int BQ = 128 / G;
      const int nqb = (M + BQ - 1) / BQ;
      const int nkb = (M + 127) / 128;
      const dim3 g1((unsigned)(nqb * B * Hkv)), g2((unsigned)(nkb * B * Hkv));
      if (D == 128) {
        hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel<128>, g1, dim3(256), 0, s, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, g, gamma, cs, lse, (const uint16_t *)dout, c,
                           c2, B, M, Hq, Hkv, G, BQ, nqb, dq, ws_delta);
        hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel<128>, g2, dim3(256), 0, s, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, g, gamma, cs, lse, (const uint16_t *)dout,
                           ws_delta, c, c2, B, M, Hq, Hkv, G, nkb, dk, dv, ws_colsum);
      } else {
        hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel<64>, g1, dim3(256), 0, s, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, g, gamma, cs, lse, (const uint16_t *)dout, c,
                           c2, B, M, Hq, Hkv, G, BQ, nqb, dq, ws_delta);
        hipLaunchKernelGGL(attn_bwd_dkdv_bf16_kernel<64>, g2, dim3(256), 0, s, (const uint16_t *)q,
                           (const uint16_t *)k, (const uint16_t *)v, g, gamma, cs, lse, (const uint16_t *)dout,
                           ws_delta, c, c2, B, M, Hq, Hkv, G, nkb, dk, dv, ws_colsum);
      }
    } else {
      const int64_t rq = (int64_t)B * M * Hq, rk = (int64_t)B * M * Hkv;
      hipLaunchKernelGGL(attn_bwd_dq_f32_kernel, dim3((unsigned)((rq + 3) / 4)), dim3(256), 0, s,
                         (const float *)q, (const float *)k, (const float *)v, g, gamma, cs, lse,
                         (const float *)dout, c, B, M, Hq, Hkv, D, dq, ws_delta);
      hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel, dim3((unsigned)((rk + 3) / 4)), dim3(256), 0, s,
                         (const float *)q, (const float *)k, (const float *)v, g, gamma, cs, lse,
                         (const float *)dout, ws_delta, c, B, M, Hq, Hkv, D, dk, dv, ws_colsum);
    }
    const int64_t n = (int64_t)B * M;
    hipLaunchKernelGGL(dg_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ws_colsum, g, gamma, B, M, Hq,
                       dg);
  }
  hipLaunchKernelGGL(dgamma_kernel, dim3((unsigned)Hq), dim3(256), 0, s, ws_colsum, g, B, M, Hq, dgamma);
  return hipGetLastError();
}

}  // namespace tg
