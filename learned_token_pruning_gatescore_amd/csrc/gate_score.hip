// gate_score.hip -- the scoring MLP of every token and its gate value.
//
// TokenGate deep dive ("TokenGate: Learnable Token Pruning for Fast,
// Memory-Efficient LLM Prefill"), section 3.1, Eq. 3 first part: a small MLP
// maps each token's normalised residual to one scalar score; here
//     s_t = sum_k w2[k] * SiLU(sum_i w1[k,i] h[t,i]),
//     g_t = 1 for a forced token, else sigmoid(s_t).
// With the layer's second normalisation in front (section 2, Eq. 1; RMSNorm
// with weight w, the Qwen3 normaliser): h is the raw residual a and
//     sum_i w1[k,i] a~[t,i] = r_t sum_i (w1[k,i] w[i]) a[t,i],
//     r_t = 1 / sqrt(mean_i a[t,i]^2 + eps),
// so w is folded into the packed W1 (one bf16 rounding of the product) and
// r_t scales each token's pre-activations before SiLU.
//
// bf16 path: a [d_ff x d] x [d x T] product on the matrix cores (32x32x16 bf16
// MFMA, fp32 accumulation).  W1 is the MFMA "A" operand (rows = units) and the
// token rows the "B" operand, so each lane's accumulator holds 16 units of ONE
// token: the SiLU * w2 reduction over units is lane-local, then one cross-half
// shuffle and a 4-way LDS sum across the waves that split the units.  Nothing
// of the [T, d_ff] activation ever leaves registers.
//
// Data movement.  Every work-group needs all of W1 (2 MB at d = 2048,
// d_ff = 512) for its token tile, so W1 dominates the bytes a compute unit
// pulls from L2.  A natural-layout MFMA fragment (32 rows x 16 inputs) touches
// 32 cache lines; a pack pass therefore first rewrites W1 in fragment order
// (each fragment one contiguous 1 KB block), which each wave then loads
// straight into registers, 4 to 8 16-input steps ahead.  Token rows stream
// from HBM through a 4-stage LDS ring by direct buffer->LDS loads, one full
// 128-byte line per row per stage.  Two waves per SIMD, each holding a
// 64-unit x 128-token accumulator tile (128 registers): a wave alone on its
// SIMD stalls on its own load and direct-load instructions (measured: about a
// third of the product time with one 128-unit wave per SIMD), and the second
// wave's products fill those gaps.
#include "tg_common.h"

namespace tg {

constexpr int GS_W = 8;      // waves per work-group (two per SIMD)
constexpr int GS_UB = 2;     // 32-unit blocks per wave
constexpr int GS_U = GS_W * GS_UB * 32;  // units per work-group chunk (8 waves x 64)
constexpr int GS_HMAX = 16;  // most output heads of the per-head scorer
constexpr int GS_BK = 64;    // inputs per hidden stage (one 128-byte line per token row)
constexpr int GS_NB = 4;     // hidden ring stages
constexpr int GS_NA = 8;     // W1 fragment register ring: one slot per 16-input step of a trip

// Packed W1 geometry: unit groups of 32 (padded to whole 512-unit chunks) x
// 16-input steps (d padded to whole pairs of 64-input stages).
__host__ __device__ inline int gate_nkk(int d) { return (d + 2 * GS_BK - 1) / (2 * GS_BK) * (2 * GS_BK / 16); }
__host__ __device__ inline int gate_ngp(int d_ff) { return (d_ff + GS_U - 1) / GS_U * (GS_U / 32); }
size_t gate_packed_bytes(int d, int d_ff) { return (size_t)gate_ngp(d_ff) * gate_nkk(d) * 64 * 16; }

// Fragment order: block (ug, kk) is 64 lanes x 8 bf16, lane L holding
// w1[32 ug + L % 32][16 kk + 8 (L / 32) .. +8] (zero past d_ff or d) -- the
// A operand of one 32x32x16 MFMA, as one contiguous 1 KB block.  A work-group
// packs 32 rows x 128 inputs: coalesced row reads into LDS, then eight
// contiguous 1 KB blocks out.
// With w_up (the gated MLP of the clone scorer, d_ff = units per matrix):
// group ug holds rows 32 (ug / 2) .. + 31 of w1 (the gate product) for even ug
// and of w_up for odd ug, so one wave's two 32-row blocks are the gate and up
// rows of the same 32 units.
__global__ __launch_bounds__(256) void gate_pack_w1_kernel(const uint16_t *__restrict__ w1,
                                                           const uint16_t *__restrict__ w_up,
                                                           const uint16_t *__restrict__ ln_w, int d, int d_ff,
                                                           int nkk, uint16_t *__restrict__ out) {
  __shared__ u32x4 t[32][17];  // 32 rows x 16 chunks of 8 inputs (+1 chunk of padding)
  const int tid = threadIdx.x, kc = blockIdx.x, ug = blockIdx.y;
  const uint16_t *src = w_up && (ug & 1) ? w_up : w1;
  const int ubase = w_up ? 32 * (ug >> 1) : 32 * ug;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 256 * j, row = idx >> 4, c = idx & 15;
    const int u = ubase + row, k0 = 128 * kc + 8 * c;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (u < d_ff && k0 < d) {
      v = *(const u32x4 *)(src + (int64_t)u * d + k0);  // d % 8 == 0: all 8 in range
      if (ln_w) {  // w1[u, i] * w[i]: exact in fp32 (bf16 x bf16), rounded once to bf16
        const u32x4 lw = *(const u32x4 *)(ln_w + k0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          v[e] = pack_bf16x2(bf16_lo(v[e]) * bf16_lo(lw[e]), bf16_hi(v[e]) * bf16_hi(lw[e]));
      }
    }
    t[row][c] = v;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int idx = tid + 256 * j, b = idx >> 6, L = idx & 63;
    const int kk = 8 * kc + b;
    if (kk < nkk) *(u32x4 *)(out + (((int64_t)ug * nkk + kk) * 64 + L) * 8) = t[L & 31][2 * b + (L >> 5)];
  }
}

// Work-group: 8 waves x (64 units x TT tokens), TT = 32 NTB.  Hidden stage st
// (inputs 64 st .. 64 st + 63 of the tile's TT rows) lives in ring buffer
// st % 4, rows of 128 bytes with the 16-byte chunk XOR-swizzled by
// (row / 2) % 8, which keeps the 16-row MFMA fragment reads free of bank
// conflicts.  Out-of-range rows and inputs read as zero.
// LN: the rows are raw residuals; each token's sum of squares is gathered from
// the B fragments the waves read anyway (fragment tb, step j of a trip is
// squared by the one wave with wave % NTB == tb and wave / NTB == j % (8 / NTB)),
// then r_t scales the pre-activations.
// MH: H output heads (w2 [H, d_ff]); scores [B, H, Nrow] head-major, no gates
// (the per-head gates come from the per-head softmax over the kept set).
// GLU (with MH): the clone scorer.  w1p is the interleaved gate/up packing
// (d_ff = 2 d_i rows), so wave w's blocks in chunk c are the gate (ub = 0) and
// up (ub = 1) rows of units 32 (c / 64 + w) .. + 31; m = SiLU(gate) * up, and
// the head sums take ufold [H, d_i] (the head projection times the down
// projection, fp32) in place of w2.
template <int NTB, bool LN, bool MH, bool GLU = false>
__global__ __launch_bounds__(64 * GS_W, 1) void gate_score_bf16_kernel(
    const uint16_t *__restrict__ hidden, const uint16_t *__restrict__ w1p, const uint16_t *__restrict__ w2,
    const uint8_t *__restrict__ forced, int64_t T, int d, int d_ff, int nkk, float ln_eps, int H, int64_t Nrow,
    float *__restrict__ scores, float *__restrict__ gates, const float *__restrict__ ufold) {
  static_assert(!GLU || MH, "the clone scorer writes per-head scores");
  constexpr int TT = 32 * NTB;         // tokens per work-group
  constexpr int ST = TT * GS_BK;       // u16 per hidden stage
  constexpr int NI = TT / (8 * GS_W);  // direct-load instructions (8 rows each) per wave per stage
  static_assert(NI >= 1 && TT % (8 * GS_W) == 0, "tile rows must split evenly over the waves");
  __shared__ __attribute__((aligned(1024))) uint16_t sH[GS_NB * ST];
  __shared__ float sRed[GS_W][TT];
  __shared__ float sW2[GS_U];
  __shared__ float sSq[LN ? GS_W : 1][64];
  __shared__ float sR[LN ? TT : 1];
  constexpr int SQP = GS_W / NTB;  // waves sharing one fragment's squares (by step parity)
  static_assert(GS_NA % SQP == 0, "a trip's steps split evenly over those waves");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hl = lane >> 5;
  const int64_t t0 = (int64_t)blockIdx.x * TT;
  const int64_t trows = T - t0 < TT ? T - t0 : TT;
  const uint32_t rowb = 2u * (uint32_t)d;
  const i32x4 rH = buffer_rsrc(hidden + t0 * d, (uint32_t)(trows * rowb));
  const int nst = nkk / 4;

  // direct loads: instruction i of this wave covers rows 8 (NI wave + i) .. +7;
  // lane -> row + lane / 8, physical chunk lane % 8, logical chunk (lane % 8) ^ ((row / 2) % 8)
  uint32_t dvo[NI];
  int dlc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int row = 8 * (NI * wave + i) + (lane >> 3);
    dlc[i] = (lane & 7) ^ ((row >> 1) & 7);
    dvo[i] = (uint32_t)row * rowb + 16u * (uint32_t)dlc[i];
  }
  // hidden stage st -> ring buffer st % 4 (past the end: zero fill)
  auto issue_h = [&](int st) {
    const uint32_t lbase = lds_addr(sH) + 2u * (uint32_t)((st % GS_NB) * ST);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool ok = st < nst && GS_BK * st + 8 * dlc[i] < d;
      dma_b128(rH, lbase + 2u * (uint32_t)(8 * (NI * wave + i) * GS_BK), ok ? dvo[i] + 128u * (uint32_t)st : 0x80000000u,
               0u);
    }
  };
  // B fragment offsets (u16) within a stage: token row 32 tb + l32, logical chunk 2 s + hl
  int brow[NTB], bsw[NTB];
#pragma unroll
  for (int tb = 0; tb < NTB; ++tb) {
    const int row = 32 * tb + l32;
    brow[tb] = row * GS_BK;
    bsw[tb] = (row >> 1) & 7;
  }

  float run = 0.f;  // running score of token t0 + tid (tid < TT), across unit chunks
  // MH: running scores of the (head, token) pairs (tid / TT + k NPS, t0 + tid % TT), k < NPH
  constexpr int NPS = 64 * GS_W / TT, NPH = GS_HMAX / NPS;
  float runh[MH ? NPH : 1];
#pragma unroll
  for (int k = 0; k < (MH ? NPH : 1); ++k) runh[k] = 0.f;

  for (int c = 0; c < d_ff; c += GS_U) {
    if (!MH)
      for (int i = tid; i < GS_U; i += 64 * GS_W) sW2[i] = c + i < d_ff ? __uint_as_float((uint32_t)w2[c + i] << 16) : 0.f;
    // this wave's unit groups: c / 32 + GS_UB wave + ub, ub < GS_UB
    const uint16_t *ap = w1p + ((int64_t)(c / 32 + GS_UB * wave) * nkk) * 512 + lane * 8;
    auto load_a1 = [&](int kk, int ub) {
      const int kc = kk < nkk ? kk : nkk - 1;  // past the end: any valid block, never used
      return *(const u32x4 *)(ap + ((int64_t)ub * nkk + kc) * 512);
    };

    const int sq_tb = __builtin_amdgcn_readfirstlane(wave % NTB), sq_ph = __builtin_amdgcn_readfirstlane(wave / NTB);
    float sq = 0.f;  // LN: this lane's share of token 32 sq_tb + l32's sum of squares
    f32x16 acc[GS_UB][NTB];
#pragma unroll
    for (int i = 0; i < GS_UB; ++i)
#pragma unroll
      for (int j = 0; j < NTB; ++j) acc[i][j] = f32x16{};

    // The K loop runs in trips of 8 16-input steps (two hidden stages), with
    // the W1 fragments of trip step j in register slot j.  Right after step
    // j's products have used slot j, the slot is reloaded with the next trip's
    // step j: four loads per step, each eight steps ahead of its use.  The
    // compiler cannot follow loads across the loop edge; it would wait for
    // every load in flight at the first use of a slot in a new trip (stalling
    // on loads issued a step earlier).  So at the end of a trip slots 0..3
    // (loaded four or more steps earlier) are marked used -- the wait for
    // them happens there, exactly -- and the first use of slots 4..7 comes
    // only after 4 GS_UB newer loads, so that wait too covers old loads only.
    // One barrier per trip: the trip's two hidden stages landed for every
    // wave and every wave is done with the previous trip; then the direct
    // loads of the next trip's stages go out.
    u32x4 a[GS_NA][GS_UB];
    static_assert(GS_UB == 2, "touch03 lists two unit blocks per slot");
    auto touch03 = [&]() {
      asm volatile("" ::"v"(a[0][0]), "v"(a[0][1]), "v"(a[1][0]), "v"(a[1][1]), "v"(a[2][0]), "v"(a[2][1]),
                   "v"(a[3][0]), "v"(a[3][1]));
    };
    issue_h(0);
    issue_h(1);
#pragma unroll
    for (int j = 0; j < GS_NA; ++j)
#pragma unroll
      for (int ub = 0; ub < GS_UB; ++ub) a[j][ub] = load_a1(j, ub);
    touch03();
    for (int st = 0; st < nst; st += 2) {  // nst is even
      const int k0 = 4 * st;               // first 16-input step of the trip
      // at most the 4 GS_UB loads of steps 4..7 of the previous trip (or of
      // the prologue) may be in flight: the direct loads of this trip's
      // stages, issued before them, are done
      sync_vm<4 * GS_UB>();
      issue_h(st + 2);
      issue_h(st + 3);
      u32x4 b[2][NTB];
      auto read_b = [&](int j, u32x4(&dst)[NTB]) {  // B fragments of trip step j
        const uint16_t *H = sH + ((st + (j >> 2)) % GS_NB) * ST;
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
          dst[tb] = *(const u32x4 *)(H + brow[tb] + (((2 * (j & 3) + hl) ^ bsw[tb]) << 3));
      };
      read_b(0, b[0]);
#pragma unroll
      for (int j = 0; j < GS_NA; ++j) {
        if (j < GS_NA - 1) read_b(j + 1, b[(j + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ub = 0; ub < GS_UB; ++ub) {
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb) acc[ub][tb] = mfma32(a[j][ub], b[j & 1][tb], acc[ub][tb]);
          __builtin_amdgcn_sched_barrier(0);
          a[j][ub] = load_a1(k0 + GS_NA + j, ub);  // slot j, ub: used up; next trip's step j
          __builtin_amdgcn_sched_barrier(0);
        }
        if (LN && j % SQP == sq_ph) {  // wave-uniform
#pragma unroll
          for (int tb = 0; tb < NTB; ++tb)
            if (tb == sq_tb) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float lo = bf16_lo(b[j & 1][tb][e]), hi = bf16_hi(b[j & 1][tb][e]);
                sq = __builtin_fmaf(lo, lo, sq);
                sq = __builtin_fmaf(hi, hi, sq);
              }
            }
        }
      }
      touch03();
    }
    // drain the tail loads before the ring is reused
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // LN: r_t of every token of the tile (fixed-order sum of its 2 SQP shares)
    float rt[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) rt[tb] = 1.f;
    if (LN) {
      sSq[wave][lane] = sq;
      __syncthreads();
      if (tid < TT) {
        const int tb = tid / 32, l = tid % 32;
        float ss = 0.f;
        for (int ph = 0; ph < SQP; ++ph) ss += sSq[ph * NTB + tb][l] + sSq[ph * NTB + tb][l + 32];
        sR[tid] = 1.f / sqrtf(ss / (float)d + ln_eps);
      }
      __syncthreads();
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb) rt[tb] = sR[32 * tb + l32];
    }
    if (MH) {
      f32x16 c2[NTB];
      if (GLU) {
        // The head sums C2[h][t] = sum_u U[h][u] m[u][t] over this wave's 32 units, two
        // 16-unit steps, with the B operand laid out as in the MH branch below (step sh, element
        // e: register 8 sh + e, unit 16 sh + 8 (e / 4) + 4 q + e % 4 of the block).  U and m
        // enter as bf16 pairs hi + lo; three products (hi hi, hi lo, lo hi) leave out lo lo.
        const int dI = d_ff / 2, ub0 = 32 * (c / 64 + wave);
        u32x4 uh[2], ul[2];
#pragma unroll
        for (int sh = 0; sh < 2; ++sh) {
          float uv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int u = ub0 + 16 * sh + 8 * (e >> 2) + 4 * hl + (e & 3);
            uv[e] = (l32 < H && u < dI) ? ufold[(int64_t)l32 * dI + u] : 0.f;
          }
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            uh[sh][w] = pack_bf16x2(uv[2 * w], uv[2 * w + 1]);
            ul[sh][w] = pack_bf16x2(uv[2 * w] - bf16_lo(uh[sh][w]), uv[2 * w + 1] - bf16_hi(uh[sh][w]));
          }
        }
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          c2[tb] = f32x16{};
#pragma unroll
          for (int sh = 0; sh < 2; ++sh) {
            u32x4 bh, bl;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              float m[2];
#pragma unroll
              for (int e = 0; e < 2; ++e) {
                float xg = acc[0][tb][8 * sh + 2 * w + e], xu = acc[1][tb][8 * sh + 2 * w + e];
                if (LN) {
                  xg *= rt[tb];
                  xu *= rt[tb];
                }
                m[e] = xg * fast_rcp(1.f + fast_exp2(-xg * kLog2e)) * xu;
              }
              bh[w] = pack_bf16x2(m[0], m[1]);
              bl[w] = pack_bf16x2(m[0] - bf16_lo(bh[w]), m[1] - bf16_hi(bh[w]));
            }
            c2[tb] = mfma32(uh[sh], bh, c2[tb]);
            c2[tb] = mfma32(uh[sh], bl, c2[tb]);
            c2[tb] = mfma32(ul[sh], bh, c2[tb]);
          }
        }
      } else {
        // The head sums are a second matrix product, C2[h][t] = sum_u w2[h][u] SiLU(a[u][t]),
        // over this wave's 64 units, four 16-unit steps.  The accumulator layout already is
        // the B operand: in step (ub, s) the lane of token j and half q holds, as element e,
        // registers 8 s + e of acc[ub][tb], i.e. unit 32 ub + 16 s + 8 (e / 4) + 4 q + e % 4;
        // the A operand (rows = heads, H <= 16 of 32) takes w2 in that unit order.  SiLU
        // enters as two bf16 parts (fp32 accumulate).
        u32x4 a2[GS_UB][2];
#pragma unroll
        for (int ub = 0; ub < GS_UB; ++ub)
#pragma unroll
          for (int sh = 0; sh < 2; ++sh) {
            const int u0 = c + wave * 32 * GS_UB + 32 * ub + 16 * sh + 4 * hl;  // units u0 + {0..3}, u0 + 8 + {0..3}
            const uint16_t *wr = w2 + (int64_t)l32 * d_ff;
            uint32_t e16[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int u = u0 + 8 * (e >> 2) + (e & 3);
              e16[e] = (l32 < H && u < d_ff) ? (uint32_t)wr[u] : 0u;
            }
#pragma unroll
            for (int w = 0; w < 4; ++w) a2[ub][sh][w] = e16[2 * w] | (e16[2 * w + 1] << 16);
          }
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
          c2[tb] = f32x16{};
#pragma unroll
          for (int ub = 0; ub < GS_UB; ++ub)
#pragma unroll
            for (int sh = 0; sh < 2; ++sh) {
              // SiLU as a bf16 pair hi + lo (|SiLU - hi - lo| <= 2^-17 |SiLU|): two products
              u32x4 bh, bl;
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                float x0 = acc[ub][tb][8 * sh + 2 * w], x1 = acc[ub][tb][8 * sh + 2 * w + 1];
                if (LN) {
                  x0 *= rt[tb];
                  x1 *= rt[tb];
                }
                const float s0 = x0 * fast_rcp(1.f + fast_exp2(-x0 * kLog2e));
                const float s1 = x1 * fast_rcp(1.f + fast_exp2(-x1 * kLog2e));
                bh[w] = pack_bf16x2(s0, s1);
                bl[w] = pack_bf16x2(s0 - bf16_lo(bh[w]), s1 - bf16_hi(bh[w]));
              }
              c2[tb] = mfma32(a2[ub][sh], bh, c2[tb]);
              c2[tb] = mfma32(a2[ub][sh], bl, c2[tb]);
            }
        }
      }
      // Sum over the waves (fixed order) through the hidden ring, free after the loop:
      // red[wave][h][t], registers 0..7 of c2 hold heads 8 (r / 4) + 4 q + r % 4 < 16.
      float *red = reinterpret_cast<float *>(sH);
      static_assert(GS_W * GS_HMAX * TT <= GS_NB * ST / 2, "the head partials fit in the hidden ring");
      __syncthreads();  // every wave's loads landed (drained above) and its ring reads done
#pragma unroll
      for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
          const int h = 8 * (r >> 2) + 4 * hl + (r & 3);
          if (h < H) red[(wave * GS_HMAX + h) * TT + 32 * tb + l32] = c2[tb][r];
        }
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NPH; ++k) {
        const int h = tid / TT + k * NPS, t = tid % TT;
        if (h < H) {
          const float *q = red + h * TT + t;
          constexpr int WS = GS_HMAX * TT;  // stride between the waves' partials
          runh[k] += ((q[0] + q[WS]) + (q[2 * WS] + q[3 * WS])) + ((q[4 * WS] + q[5 * WS]) + (q[6 * WS] + q[7 * WS]));
        }
      }
      __syncthreads();  // the ring is refilled by the next chunk
      continue;
    }
    // Epilogue: SiLU, times w2, summed over this lane's units.
    float part[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) part[tb] = 0.f;
#pragma unroll
    for (int ub = 0; ub < GS_UB; ++ub) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        // registers 4 g4 .. 4 g4 + 3 hold units 32 ub + 8 g4 + 4 hl + e
        const f32x4 wv = *(const f32x4 *)&sW2[wave * 32 * GS_UB + ub * 32 + 8 * g4 + 4 * hl];
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = LN ? acc[ub][tb][g4 * 4 + e] * rt[tb] : acc[ub][tb][g4 * 4 + e];
            const float silu = x * fast_rcp(1.f + fast_exp2(-x * kLog2e));
            part[tb] += silu * wv[e];
          }
        }
      }
    }
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb) {
      part[tb] += __shfl_xor(part[tb], 32);
      if (hl == 0) sRed[wave][32 * tb + l32] = part[tb];
    }
    __syncthreads();
    if (tid < TT)  // fixed-order tree over the waves
      run += ((sRed[0][tid] + sRed[1][tid]) + (sRed[2][tid] + sRed[3][tid])) +
             ((sRed[4][tid] + sRed[5][tid]) + (sRed[6][tid] + sRed[7][tid]));
    __syncthreads();
  }

  if (MH) {
    const int64_t t = t0 + tid % TT;
    if (t < T) {
      const int64_t b = t / Nrow, n = t - b * Nrow;
#pragma unroll
      for (int k = 0; k < NPH; ++k) {
        const int h = tid / TT + k * NPS;
        if (h < H) scores[(b * H + h) * Nrow + n] = runh[k];
      }
    }
    return;
  }
  if (tid < TT) {
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
// ln_w (with ln_eps): the row is RMS-normalised first (fixed-order sum of squares).
__global__ __launch_bounds__(256) void gate_score_f32_kernel(
    const float *__restrict__ hidden, const float *__restrict__ w1, const float *__restrict__ w2,
    const uint8_t *__restrict__ forced, int64_t T, int d, int d_ff, const float *__restrict__ ln_w, float ln_eps,
    bool ln, int H, int64_t Nrow, float *__restrict__ scores, float *__restrict__ gates) {
  extern __shared__ float sh[];  // d floats (+ d_ff activations with H > 0)
  __shared__ float sPart[4];
  __shared__ float sR;
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) {
    sh[i] = hidden[t * d + i];
    ss += sh[i] * sh[i];
  }
  if (ln) {
    ss = wave_sum(ss);
    if (lane == 0) sPart[wave] = ss;
    __syncthreads();
    if (threadIdx.x == 0) sR = 1.f / sqrtf(((sPart[0] + sPart[1]) + (sPart[2] + sPart[3])) / (float)d + ln_eps);
    __syncthreads();
    const float r = sR;
    for (int i = threadIdx.x; i < d; i += 256) sh[i] = sh[i] * r * (ln_w ? ln_w[i] : 1.f);
  }
  __syncthreads();
  if (H > 0) {  // per-head scores: the activations first, then one dot product per head
    float *act = sh + d;
    for (int k = wave; k < d_ff; k += 4) {
      const float *row = w1 + (int64_t)k * d;
      float u = 0.f;
      for (int i = lane; i < d; i += 64) u += row[i] * sh[i];
      u = wave_sum(u);
      if (lane == 0) act[k] = u / (1.f + expf(-u));
    }
    __syncthreads();
    const int64_t b = t / Nrow, n = t - b * Nrow;
    for (int h = wave; h < H; h += 4) {
      float sv = 0.f;
      for (int k = lane; k < d_ff; k += 64) sv += w2[(int64_t)h * d_ff + k] * act[k];
      sv = wave_sum(sv);
      if (lane == 0) scores[(b * H + h) * Nrow + n] = sv;
    }
    return;
  }
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

// The clone scorer's down and head projections folded into one matrix,
// U[h][k] = sum_o P[h][o] Wd[o][k] (fp32), so that b~^h = sum_k U[h][k] m_k:
// the same value as P (Wd m) with the two sums taken in the other order.
// Pass 1, work-group (64 units k, 256 outputs o): P's 256 columns staged in LDS
// as fp32, each lane one unit, the 4 waves every 4th output, the waves' sums
// added in a fixed order into part[o block][h][k].  Pass 2: U = the o blocks'
// partial sums in block order.
constexpr int GF_O = 256;  // outputs o per fold work-group
__device__ __forceinline__ float wf(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
__device__ __forceinline__ float wf(float x) { return x; }

template <typename TW>
__global__ __launch_bounds__(256) void gate_fold_part_kernel(const TW *__restrict__ wd, const TW *__restrict__ wh,
                                                             int d, int d_i, int H, float *__restrict__ part) {
  __shared__ float sP[GF_O][GS_HMAX];       // P[h][o0 + j] at [j][h]
  __shared__ float sAcc[4][GS_HMAX][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int k = blockIdx.x * 64 + lane, o0 = blockIdx.y * GF_O;
  const int no = d - o0 < GF_O ? d - o0 : GF_O;
  for (int i = tid; i < GF_O * GS_HMAX; i += 256) {
    const int h = i / GF_O, j = i % GF_O;
    sP[j][h] = (h < H && j < no) ? wf(wh[(int64_t)h * d + o0 + j]) : 0.f;
  }
  __syncthreads();
  float acc[GS_HMAX];
#pragma unroll
  for (int h = 0; h < GS_HMAX; ++h) acc[h] = 0.f;
  if (k < d_i) {
    const TW *col = wd + (int64_t)o0 * d_i + k;
#pragma unroll 4
    for (int j = wave; j < no; j += 4) {
      const float x = wf(col[(int64_t)j * d_i]);
#pragma unroll
      for (int h = 0; h < GS_HMAX; ++h) acc[h] = __builtin_fmaf(sP[j][h], x, acc[h]);
    }
  }
#pragma unroll
  for (int h = 0; h < GS_HMAX; ++h) sAcc[wave][h][lane] = acc[h];
  __syncthreads();
  if (wave == 0 && k < d_i)
    for (int h = 0; h < H; ++h)
      part[((int64_t)blockIdx.y * H + h) * d_i + k] =
          (sAcc[0][h][lane] + sAcc[1][h][lane]) + (sAcc[2][h][lane] + sAcc[3][h][lane]);
}

__global__ __launch_bounds__(256) void gate_fold_sum_kernel(const float *__restrict__ part, int nob, int64_t n,
                                                            float *__restrict__ U) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int ob = 0; ob < nob; ++ob) s += part[ob * n + i];
  U[i] = s;
}

// fp32 clone scorer: one work-group per token.  The (normalised) row goes to
// LDS, then m_k = SiLU(gate_k) up_k for every unit (waves round-robin, lanes
// split d), then one dot product with U per head.  Fixed-order reductions.
__global__ __launch_bounds__(256) void gate_clone_f32_kernel(const float *__restrict__ hidden,
                                                             const float *__restrict__ wg,
                                                             const float *__restrict__ wu,
                                                             const float *__restrict__ U, int64_t T, int d, int d_i,
                                                             const float *__restrict__ ln_w, float ln_eps, bool ln,
                                                             int H, int64_t Nrow, float *__restrict__ scores) {
  extern __shared__ float sh[];  // d inputs, then d_i activations
  __shared__ float sPart[4];
  __shared__ float sR;
  const int64_t t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 256) {
    sh[i] = hidden[t * d + i];
    ss += sh[i] * sh[i];
  }
  if (ln) {
    ss = wave_sum(ss);
    if (lane == 0) sPart[wave] = ss;
    __syncthreads();
    if (threadIdx.x == 0) sR = 1.f / sqrtf(((sPart[0] + sPart[1]) + (sPart[2] + sPart[3])) / (float)d + ln_eps);
    __syncthreads();
    const float r = sR;
    for (int i = threadIdx.x; i < d; i += 256) sh[i] = sh[i] * r * (ln_w ? ln_w[i] : 1.f);
  }
  __syncthreads();
  float *m = sh + d;
  for (int k = wave; k < d_i; k += 4) {
    const float *rg = wg + (int64_t)k * d, *ru = wu + (int64_t)k * d;
    float g = 0.f, u = 0.f;
    for (int i = lane; i < d; i += 64) {
      g += rg[i] * sh[i];
      u += ru[i] * sh[i];
    }
    g = wave_sum(g);
    u = wave_sum(u);
    if (lane == 0) m[k] = g / (1.f + expf(-g)) * u;
  }
  __syncthreads();
  const int64_t b = t / Nrow, n = t - b * Nrow;
  for (int h = wave; h < H; h += 4) {
    float sv = 0.f;
    for (int k = lane; k < d_i; k += 64) sv += U[(int64_t)h * d_i + k] * m[k];
    sv = wave_sum(sv);
    if (lane == 0) scores[(b * H + h) * Nrow + n] = sv;
  }
}

hipError_t launch_gate_pack_w1(const void *w1, const void *ln_w, int d, int d_ff, void *packed, hipStream_t s,
                               const void *w_up) {
  const int nkk = gate_nkk(d);
  const int ngp = gate_ngp(w_up ? 2 * d_ff : d_ff);
  hipLaunchKernelGGL(gate_pack_w1_kernel, dim3((unsigned)((nkk + 7) / 8), (unsigned)ngp), dim3(256), 0, s,
                     (const uint16_t *)w1, (const uint16_t *)w_up, (const uint16_t *)ln_w, d, d_ff, nkk,
                     (uint16_t *)packed);
  return hipGetLastError();
}

// bf16: w1 is the packed copy (gate_pack_w1_kernel, with the RMSNorm weight
// folded in when ln); f32: natural layout, ln_w applied in the kernel.
// H > 0: the per-head scorer (w2 [H, d_ff], scores [B, H, Nrow], no gates).
hipError_t launch_gate_score(const void *hidden, const void *w1, const void *w2,
                             const uint8_t *forced, int64_t T, int d, int d_ff, bool bf16, bool ln,
                             const void *ln_w, float ln_eps, float *scores, float *gates, hipStream_t s, int H,
                             int64_t Nrow) {
  if (T == 0) return hipSuccess;
  const bool mh = H > 0;
  if (bf16) {
    const int nkk = gate_nkk(d);
    // 128-token tiles when they still fill the 256 compute units, else 64
    const bool big = (T + 127) / 128 >= 256;
    auto k = big ? (mh ? (ln ? gate_score_bf16_kernel<4, true, true> : gate_score_bf16_kernel<4, false, true>)
                       : (ln ? gate_score_bf16_kernel<4, true, false> : gate_score_bf16_kernel<4, false, false>))
                 : (mh ? (ln ? gate_score_bf16_kernel<2, true, true> : gate_score_bf16_kernel<2, false, true>)
                       : (ln ? gate_score_bf16_kernel<2, true, false> : gate_score_bf16_kernel<2, false, false>));
    const int tt = big ? 128 : 64;
    hipLaunchKernelGGL(k, dim3((unsigned)((T + tt - 1) / tt)), dim3(64 * GS_W), 0, s, (const uint16_t *)hidden,
                       (const uint16_t *)w1, (const uint16_t *)w2, forced, T, d, d_ff, nkk, ln_eps, H, Nrow, scores,
                       gates, (const float *)nullptr);
  } else {
    hipLaunchKernelGGL(gate_score_f32_kernel, dim3((unsigned)T), dim3(256), (size_t)(d + d_ff) * sizeof(float), s,
                       (const float *)hidden, (const float *)w1, (const float *)w2, forced, T, d, d_ff,
                       (const float *)ln_w, ln_eps, ln, H, Nrow, scores, gates);
  }
  return hipGetLastError();
}

// The clone scorer (gate/up of d_i units each, down, head projection P [H, d]):
// bf16: w_gate / w_up packed interleaved into ws, U = P Wd (fp32) after them,
// then the fold's partial sums; f32: U and the partial sums.  scores [B, H, Nrow].
// ws: [packed gate/up (bf16 only)] [U: H d_i fp32] [fold partials: ceil(d / 256) H d_i fp32]
static size_t clone_pack_bytes(int d, int d_i, bool bf16) {
  return bf16 ? (gate_packed_bytes(d, 2 * d_i) + 255) / 256 * 256 : 0;
}
static size_t clone_u_bytes(int d_i, int H) { return ((size_t)H * d_i * sizeof(float) + 255) / 256 * 256; }

size_t gate_clone_ws_bytes(int d, int d_i, int H, bool bf16) {
  const size_t nob = (size_t)(d + GF_O - 1) / GF_O;
  return clone_pack_bytes(d, d_i, bf16) + clone_u_bytes(d_i, H) + nob * H * d_i * sizeof(float);
}

hipError_t launch_gate_clone(const void *hidden, const void *w_gate, const void *w_up, const void *w_down,
                             const void *w_head, int64_t T, int d, int d_i, int H, bool bf16, bool ln,
                             const void *ln_w, float ln_eps, float *scores, int64_t Nrow, void *ws, hipStream_t s) {
  if (T == 0) return hipSuccess;
  float *U = (float *)((char *)ws + clone_pack_bytes(d, d_i, bf16));
  float *part = (float *)((char *)U + clone_u_bytes(d_i, H));
  const int nob = (d + GF_O - 1) / GF_O;
  const dim3 gf((unsigned)((d_i + 63) / 64), (unsigned)nob);
  const int64_t nu = (int64_t)H * d_i;
  if (bf16) {
    hipError_t e = launch_gate_pack_w1(w_gate, ln ? ln_w : nullptr, d, d_i, ws, s, w_up);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gate_fold_part_kernel<uint16_t>, gf, dim3(256), 0, s, (const uint16_t *)w_down,
                       (const uint16_t *)w_head, d, d_i, H, part);
    hipLaunchKernelGGL(gate_fold_sum_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, s,
                       (const float *)part, nob, nu, U);
    const int nkk = gate_nkk(d);
    const bool big = (T + 127) / 128 >= 256;
    auto k = big ? (ln ? gate_score_bf16_kernel<4, true, true, true> : gate_score_bf16_kernel<4, false, true, true>)
                 : (ln ? gate_score_bf16_kernel<2, true, true, true> : gate_score_bf16_kernel<2, false, true, true>);
    const int tt = big ? 128 : 64;
    hipLaunchKernelGGL(k, dim3((unsigned)((T + tt - 1) / tt)), dim3(64 * GS_W), 0, s, (const uint16_t *)hidden,
                       (const uint16_t *)ws, (const uint16_t *)nullptr, (const uint8_t *)nullptr, T, d, 2 * d_i, nkk,
                       ln_eps, H, Nrow, scores, (float *)nullptr, (const float *)U);
  } else {
    hipLaunchKernelGGL(gate_fold_part_kernel<float>, gf, dim3(256), 0, s, (const float *)w_down,
                       (const float *)w_head, d, d_i, H, part);
    hipLaunchKernelGGL(gate_fold_sum_kernel, dim3((unsigned)((nu + 255) / 256)), dim3(256), 0, s,
                       (const float *)part, nob, nu, U);
    hipLaunchKernelGGL(gate_clone_f32_kernel, dim3((unsigned)T), dim3(256), (size_t)(d + d_i) * sizeof(float), s,
                       (const float *)hidden, (const float *)w_gate, (const float *)w_up, (const float *)U, T, d, d_i,
                       (const float *)ln_w, ln_eps, ln, H, Nrow, scores);
  }
  return hipGetLastError();
}

}  // namespace tg
