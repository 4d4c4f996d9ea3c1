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
//   * a prep pass computes the cos/sin table of the kept positions (fp64
//     angles), the rotated keys and log2 g once per row;
//   * one work-group = 4 waves = one (batch, kv head) and 128 "columns",
//     a column being a (query, head) pair of the GQA group: BQ = 128 / G query
//     positions x G heads share every K/V tile staged in LDS;
//   * each wave owns 32 columns; it computes S^T = K Q^T (keys on the MFMA
//     rows, its columns on the MFMA columns), so every lane holds 16 keys of a
//     single column: the softmax max / sum is lane-local plus one cross-half
//     shuffle, and P^T feeds the P.V product straight from registers;
//   * O^T = V^T P^T reads V row-major through the transposing LDS read
//     ds_read_b64_tr_b16; Q (rotated) lives in registers for the whole loop;
//   * 64-key tiles are double-buffered in LDS and filled by direct
//     global->LDS loads issued one tile ahead (one barrier per tile);
//   * online softmax in fp32, P rounded to bf16 for the MFMA.
#include "tg_common.h"
#include "tg_attn.h"

namespace tg {

// Prep pass over the B*M kept rows (one thread per (row, rotary pair)):
//   cs[row][i]    = (cos, sin)(pos[row] * inv_freq[i]) with the angle and the
//                   trigonometry in fp64 (inv_freq[i] = theta^(-2i/D), computed
//                   on the host in fp64), stored as fp32;
//   khat[row]     = k[row] rotated (bf16, every kv head), when khat != nullptr;
//   bias[b][h][j] = gamma_h * log2 g_j (-inf where g_j <= 0), the per-key,
//                   per-head logit bias in log2 units, when bias != nullptr.
// Rotating K once here replaces a rotation per query block in the main loop.
struct InvFreq {
  double v[64];
};

__global__ __launch_bounds__(256) void attn_prep_kernel(const uint16_t *__restrict__ k, const float *__restrict__ g,
                                                        const float *__restrict__ gamma,
                                                        const int32_t *__restrict__ pos, InvFreq inv, int64_t rows,
                                                        int M, int Hq, int Hkv, int D, float2 *__restrict__ cs,
                                                        uint16_t *__restrict__ khat, float *__restrict__ bias,
                                                        int *__restrict__ cnt, int ncnt) {
  const int half = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, rotary pair)
  if (idx < ncnt) cnt[idx] = 0;  // the split-row arrival counters of the forward kernel
  if (idx >= rows * half) return;
  const int64_t r = idx / half;  // b * M + j
  const int i = (int)(idx % half);
  if (pos) {
    const double phi = (double)pos[r] * inv.v[i];
    double sn, cn;
    sincos(phi, &sn, &cn);
    const float c = (float)cn, s = (float)sn;
    cs[r * half + i] = make_float2(c, s);
    if (khat) {
      for (int h = 0; h < Hkv; ++h) {
        const int64_t o = (r * Hkv + h) * D;
        const float x = __uint_as_float((uint32_t)k[o + i] << 16);
        const float y = __uint_as_float((uint32_t)k[o + half + i] << 16);
        khat[o + i] = (uint16_t)f32_to_bf16_bits(x * c - y * s);
        khat[o + half + i] = (uint16_t)f32_to_bf16_bits(y * c + x * s);
      }
    }
  }
  if (bias) {
    const float gv = g[r];
    const float lg = gv > 0.f ? log2f(gv) : -INFINITY;
    const int64_t b = r / M, j = r % M;
    for (int h = i; h < Hq; h += half) bias[(b * Hq + h) * M + j] = gv > 0.f ? gamma[h] * lg : -INFINITY;
  }
}


typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

// LDS layout of a bf16 tile (row = key): rows of D elements, unpadded, with
// 16-byte chunks XOR-swizzled per row.  gfx950 LDS serves 64 banks (256 bytes)
// per cycle: 16 lanes of a 16-byte read, 32 lanes of an 8-byte read.
//   K tiles are read as 16-byte MFMA fragments, 16 consecutive rows at one
//   logical chunk per 16 lanes: the 16 rows must hit 16 distinct 16-byte slots
//   of the 256-byte bank window -> chunk ^ (row % 16) for D = 128 (one row per
//   window), chunk ^ ((row / 2) % 8) for D = 64 (two rows per window).
//   V tiles are read with ds_read_b64_tr_b16: per 32 lanes, 4 consecutive rows
//   x logical chunks {4db .. 4db+3} (8 bytes per lane): the XOR must move the
//   4 rows to distinct chunk groups -> chunk ^ 4 (row % 4) for D = 128,
//   chunk ^ 4 ((row / 2) % 2) for D = 64.
template <int D>
struct Tile {
  static constexpr int C = D / 8;               // 16-byte chunks per row
  static constexpr int RPI = 1024 / (2 * D);    // rows per 1 KB direct-load instruction
  static constexpr int NI = 64 / RPI;           // instructions per 64-row tile
  __device__ static int kswz(int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); }
  __device__ static int vswz(int row) { return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1); }
};


// ---------------------------------------------------------------------------
// bf16 forward.  Work-group = 4 waves (one per SIMD) = 256 columns, a column
// being a (query, head) pair of the GQA group: BQ = 256 / G queries x G
// heads.  Wave w owns columns 64w .. 64w+63 as two 32-column blocks (cb); a
// block lies in one head.  Keys come in 32-key tiles.
//
// Per tile a wave runs 16 products for S^T = K Q^T (each K fragment read
// from LDS feeds both column blocks) and 16 for O^T += V^T P^T, and the
// softmax of 32 logits per lane.  The loop is pipelined two deep: iteration
// t issues the products of S(t+1) and of P(t-1) V(t-1) and, in the same
// basic block, the softmax of S(t), so the matrix cores and the vector ALU of
// one wave overlap.  P(t) is computed with the running maximum before tile t;
// only when a logit exceeds it by more than 8 (log2 units) is the maximum
// raised, O and the sum rescaled and P(t) recomputed (rare branch).
//
// Long causal rows are split along the keys into pieces (at most C tiles
// each, the diagonal in the last piece) so that the work spreads over every
// compute unit.  Each piece of a split query block writes its unnormalised
// (O, max, sum) to the workspace and bumps a per-block counter; the last to
// arrive merges all pieces in piece order (deterministic) and writes o, lse.
// ---------------------------------------------------------------------------
constexpr int AF_TK = 32;  // keys per tile

template <int D>
struct FwdCfg {
  static constexpr int NDB = D / 32;           // 32-row blocks of O^T
  static constexpr int NKS = D / 16;           // 16-wide steps over the head dim
  static constexpr int TILE = AF_TK * D;       // u16 per K or V tile
  static constexpr int NIW = AF_TK / Tile<D>::RPI / 4;  // direct loads per wave per K (or V) tile
  static constexpr int NVM = 2 * NIW + 1;      // direct loads per wave per iteration (K, V, bias)
  static constexpr int NR = 2 * NDB * 16 + 4;  // floats per lane in a partial record
};

// Tiles of query block qb (keys 0 .. min((qb+1) BQ, M) - 1) and its pieces.
__host__ __device__ inline int fwd_ntiles(int qb, int BQ, int M) {
  const int qe = (qb + 1) * BQ < M ? (qb + 1) * BQ : M;
  return (qe + AF_TK - 1) / AF_TK;
}
__host__ __device__ inline int fwd_npieces(int n, int C) { return (n + C - 1) / C; }

template <int D>
__global__ __launch_bounds__(256, 1) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ khat, const uint16_t *__restrict__ v,
    const float *__restrict__ bias, const float2 *__restrict__ cs, float c2, int B, int M, int Hq, int Hkv, int G,
    int BQ, int nqb, int C, float *__restrict__ part, int *__restrict__ cnt, uint16_t *__restrict__ o,
    float *__restrict__ lse) {
  using T = Tile<D>;
  using F = FwdCfg<D>;
  constexpr int NDB = F::NDB, NKS = F::NKS, HALF = D / 2;
  __shared__ __attribute__((aligned(1024))) uint16_t sK[3 * F::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[3 * F::TILE];
  __shared__ __attribute__((aligned(1024))) float sBias[3][8][AF_TK];
  __shared__ __attribute__((aligned(1024))) float sDummy[256];  // target of the other waves' bias loads
  __shared__ int sLast;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int l32 = lane & 31, hl = lane >> 5;
  const int nbh = B * Hkv;
  // consecutive work-groups take consecutive (batch, kv head): with the
  // round-robin placement over the 8 XCDs one head's keys stay in one L2
  const int bh = blockIdx.x % nbh;
  const int b = bh / Hkv, kvh = bh % Hkv;

  // Piece -> (query block, piece index).  Pieces are listed by descending query
  // block (longest rows first); each wave scans 64 blocks at a time.
  int qb = 0, p = 0, np = 1, pfirst = 0;
  {
    int rem = blockIdx.x / nbh, base = 0;
    for (int c0 = 0; c0 < nqb; c0 += 64) {
      const int qq = nqb - 1 - (c0 + lane);
      const int mine = qq >= 0 ? fwd_npieces(fwd_ntiles(qq, BQ, M), C) : 0;
      int incl = mine;
      for (int o2 = 1; o2 < 64; o2 <<= 1) {
        const int y = __shfl_up(incl, o2);
        if (lane >= o2) incl += y;
      }
      const int tot = __shfl(incl, 63);
      if (rem < tot) {
        const int src = __ffsll((unsigned long long)__ballot(incl > rem)) - 1;
        const int excl = __shfl(incl - mine, src);
        qb = nqb - 1 - (c0 + src);
        np = __shfl(mine, src);
        p = rem - excl;
        pfirst = base + excl;
        break;
      }
      rem -= tot;
      base += tot;
    }
  }
  const int ntq = fwd_ntiles(qb, BQ, M);
  const int kt0 = p * ntq / np, nt = (p + 1) * ntq / np - kt0;  // this piece: tiles kt0 .. kt0+nt-1
  const int q0 = qb * BQ;
  // tiles from here on hold keys past some query of the block: causal mask
  const int tdiag = (q0 / AF_TK - kt0) > 0 ? q0 / AF_TK - kt0 : 0;

  int hloc[2], qi[2];
  bool vq[2];
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const int c0 = 64 * wave + 32 * cb;
    hloc[cb] = c0 / BQ;
    qi[cb] = q0 + c0 % BQ + l32;
    vq[cb] = qi[cb] < M;
  }
  const int64_t bM = (int64_t)b * M;
  const uint32_t rsb = (uint32_t)(Hkv * D * 2);  // bytes between consecutive keys
  const uint32_t kv_bytes = (uint32_t)(M - 1) * rsb + D * 2;
  const i32x4 rK = buffer_rsrc(khat + (bM * Hkv + kvh) * D, kv_bytes);
  const i32x4 rV = buffer_rsrc(v + (bM * Hkv + kvh) * D, kv_bytes);
  const i32x4 rB = buffer_rsrc(bias + (int64_t)b * Hq * M, (uint32_t)(Hq * M * 4));

  // Direct loads.  Tile t of the piece (key tile kt0 + t) lives in ring slot
  // t % 3.  Iteration i issues K(i+3), V(i+1) and bias(i+2) (slots freed by
  // iteration i-1); slots of tiles outside the piece are zero-filled.
  // per-lane byte offsets within a tile (row of instruction i, swizzled chunk)
  uint32_t kvo[F::NIW], vvo[F::NIW];
#pragma unroll
  for (int i = 0; i < F::NIW; ++i) {
    const int row = (wave * F::NIW + i) * T::RPI + lane / T::C;
    kvo[i] = (uint32_t)row * rsb + ((uint32_t)((lane % T::C) ^ T::kswz(row)) << 4);
    vvo[i] = (uint32_t)row * rsb + ((uint32_t)((lane % T::C) ^ T::vswz(row)) << 4);
  }
  // bias: wave 0 loads the G rows (8 lanes x 16 bytes per head); the other
  // waves issue one load too (zeros, into sDummy) so every wave's count is fixed
  const bool breal = wave == 0 && (lane >> 3) < G;
  const uint32_t bvo = (uint32_t)((((lane >> 3) * M) + 4 * (lane & 7)) * 4);
  auto slot = [](int t) __attribute__((always_inline)) { return ((t % 3) + 3) % 3; };
  auto issue_kv = [&](int t, bool is_v) __attribute__((always_inline)) {
    const bool live = t >= 0 && t < nt;
    const uint32_t toff = (uint32_t)((kt0 + t) * AF_TK) * rsb;  // uniform
    const uint32_t lb = lds_addr(is_v ? sV : sK) + 2u * (uint32_t)(slot(t) * F::TILE);
#pragma unroll
    for (int i = 0; i < F::NIW; ++i)
      dma_b128(is_v ? rV : rK, lb + 2u * (uint32_t)((wave * F::NIW + i) * T::RPI * D),
               live ? (is_v ? vvo[i] : kvo[i]) + toff : 0x80000000u, 0u);
  };
  auto issue_bias = [&](int t) __attribute__((always_inline)) {
    const bool live = t >= 0 && t < nt;
    const uint32_t toff = (uint32_t)((kvh * G * M + (kt0 + t) * AF_TK) * 4);  // uniform
    dma_b128(rB, wave == 0 ? lds_addr(&sBias[slot(t)][0][0]) : lds_addr(sDummy),
             live && breal ? bvo + toff : 0x80000000u, 0u);
  };
  auto issue_group = [&](int i) __attribute__((always_inline)) {
    issue_kv(i + 3, false);
    issue_kv(i + 1, true);
    issue_bias(i + 2);
  };
  // The first pass's direct loads go out first; the Q and rotation loads
  // below (all issued before any use) overlap with them.
  issue_group(-3);
  issue_group(-2);
  issue_group(-1);

  // Q fragments (MFMA B operand): lane holds q^[qi, h, 16 ks + 8 hl .. +8] of each column block
  u32x4 qf[2][NKS];
  f32x4 csv[2][NKS / 2][4];  // (cos, sin) of the 8 rotary pairs of (ks, hl), two pairs per vector
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const uint16_t *qrow = q + ((bM + qi[cb]) * Hq + kvh * G + hloc[cb]) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      qf[cb][ks] = vq[cb] ? *(const u32x4 *)(qrow + 16 * ks + 8 * hl) : u32x4{0u, 0u, 0u, 0u};
    const f32x4 *crow = (const f32x4 *)(cs + (bM + (vq[cb] ? qi[cb] : 0)) * HALF);
#pragma unroll
    for (int ks = 0; ks < NKS / 2; ++ks)
#pragma unroll
      for (int w = 0; w < 4; ++w) csv[cb][ks][w] = cs ? crow[(16 * ks + 8 * hl) / 2 + w] : f32x4{1.f, 0.f, 1.f, 0.f};
  }
  if (cs) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int ks = 0; ks < NKS / 2; ++ks) {
        u32x4 &x = qf[cb][ks], &y = qf[cb][ks + NKS / 2];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x4 c = csv[cb][ks][w];  // pairs 2w, 2w+1: (cos, sin, cos, sin)
          const float x0 = bf16_lo(x[w]), x1 = bf16_hi(x[w]);
          const float y0 = bf16_lo(y[w]), y1 = bf16_hi(y[w]);
          x[w] = pack_bf16x2(x0 * c[0] - y0 * c[1], x1 * c[2] - y1 * c[3]);
          y[w] = pack_bf16x2(y0 * c[0] + x0 * c[1], y1 * c[2] + x1 * c[3]);
        }
      }
  }

  // fragment-read offsets: K row l32, logical chunk 2ks + hl; V transposing
  // reads as in the tile layout notes above
  const int krow = l32 * D;
  const int kx = T::kswz(l32);
  const int gi = lane >> 4, li = lane & 15, kq = li >> 2, cc = li & 3;
  int vlo[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int dd = 32 * db + 16 * (gi & 1) + 4 * cc;
    vlo[db] = (4 * hl + kq) * D + (((dd >> 3) ^ T::vswz(kq)) << 3) + (dd & 7);
  }

  f32x16 acc[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db][0] = acc[db][1] = f32x16{};
  // m2: reference maximum of each column (the probabilities are 2^(x - m2)).
  // The S^T products subtract it themselves: one more 16-wide product step
  // with a constant A fragment (1, 1 in k = 0, 1) and a per-column B fragment
  // (-m2 / c2 as a bf16 pair hi + lo) adds -m2 / c2 to every raw dot product.
  float m2[2] = {0.f, 0.f}, lsum[2] = {0.f, 0.f};
  auto mref = [&](int cb) __attribute__((always_inline)) { return m2[cb]; };
  const u32x4 kaug = hl == 0 ? u32x4{0x3F803F80u, 0u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
  u32x4 qaug[2];
  const float inv_c2 = 1.f / c2;
  auto set_ref = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      const float r = -m2[cb] * inv_c2;
      const uint32_t hi = f32_to_bf16_bits(r);
      const uint32_t lo = f32_to_bf16_bits(r - bf16_lo(hi));
      qaug[cb] = hl == 0 ? u32x4{hi | (lo << 16), 0u, 0u, 0u} : u32x4{0u, 0u, 0u, 0u};
    }
  };

  auto qk = [&](int t, f32x16(&s)[2]) __attribute__((always_inline)) {  // S(t)^T - m2 / c2
    const uint16_t *K = sK + slot(t) * F::TILE;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) s[cb] = mfma32(kaug, qaug[cb], f32x16{});
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const u32x4 a = *(const u32x4 *)(K + krow + (((2 * ks + hl) ^ kx) << 3));
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) s[cb] = mfma32(a, qf[cb][ks], s[cb]);
    }
  };
  // O^T += V(t)^T P(t)^T.  P slot 8hl + e of step hf is key 16hf + 8(e/4) + 4hl + e%4,
  // which is register 8hf + e of the S accumulator.
  auto pv = [&](int t, const u32x4(&pp)[2][2]) __attribute__((always_inline)) {
    const uint16_t *V = sV + slot(t) * F::TILE;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x2 pr[2];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr)
          pr[rr] = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(V + (16 * hf + 8 * rr) * D + vlo[db])));
        const u32x4 a = {pr[0][0], pr[0][1], pr[1][0], pr[1][1]};
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[db][cb] = mfma32(a, pp[cb][hf], acc[db][cb]);
      }
  };
  // One iteration: wait for group t-2, issue group t, then, interleaved by hand
  // in 16 slots (sched_barrier keeps the order): the products of S(t+1) and of
  // P(t-1) V(t-1), one of each per slot, and the softmax of S(t), one logit
  // pair per slot, against the fixed reference maximum m2 (no rescaling).
  auto body = [&](int t, f32x16(&sc)[2], f32x16(&sn)[2], u32x4(&pc)[2][2], const u32x4(&pp)[2][2],
                  bool masked) __attribute__((always_inline)) {
    sync_vm<F::NVM>();
    issue_group(t);
    const uint16_t *K = sK + slot(t + 1) * F::TILE;
    const uint16_t *V = sV + slot(t - 1) * F::TILE;
    const float(*bi)[AF_TK] = sBias[slot(t)];
    auto kread = [&](int ks) __attribute__((always_inline)) { return *(const u32x4 *)(K + krow + (((2 * ks + hl) ^ kx) << 3)); };
    auto vread = [&](int j) __attribute__((always_inline)) {  // A fragment of P.V step j = (hf, db)
      const int hf = j / NDB, db = j % NDB;
      u32x2 pr[2];
#pragma unroll
      for (int rr = 0; rr < 2; ++rr)
        pr[rr] = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(V + (16 * hf + 8 * rr) * D + vlo[db])));
      return u32x4{pr[0][0], pr[0][1], pr[1][0], pr[1][1]};
    };
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) sn[cb] = mfma32(kaug, qaug[cb], f32x16{});
    u32x4 kf[NKS], vf[2 * NDB];
    kf[0] = kread(0);
    kf[1] = kread(1);
    vf[0] = vread(0);
    vf[1] = vread(1);
    // bias pair of slot i: keys 8(r0/4) + 4hl + r0%4 (+1) of column block i / 8, r0 = 2 (i % 8);
    // read two slots ahead into a ring of 3
    auto bread = [&](int i) __attribute__((always_inline)) {
      const int r0 = 2 * (i & 7);
      return *(const float2 *)(bi[hloc[i >> 3]] + 8 * (r0 >> 2) + 4 * hl + (r0 & 3));
    };
    float2 bq[3];
    bq[0] = bread(0);
    bq[1] = bread(1);
    float ps[2] = {0.f, 0.f};
    const int lim[2] = {qi[0] - (kt0 + t) * AF_TK, qi[1] - (kt0 + t) * AF_TK};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if ((i & 1) == 0 && i / 2 + 2 < NKS) kf[i / 2 + 2] = kread(i / 2 + 2);
      if ((i & 1) == 0 && i / 2 + 2 < 2 * NDB) vf[i / 2 + 2] = vread(i / 2 + 2);
      if (i + 2 < 16) bq[(i + 2) % 3] = bread(i + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (i / 2 < NKS) sn[i & 1] = mfma32(kf[i / 2], qf[i & 1][i / 2], sn[i & 1]);
      if (i / 2 < 2 * NDB) {
        const int j = i / 2;
        acc[j % NDB][i & 1] = mfma32(vf[j], pp[i & 1][j / NDB], acc[j % NDB][i & 1]);
      }
      {
        const int cb = i >> 3, r0 = 2 * (i & 7);
        const int key = 8 * (r0 >> 2) + 4 * hl + (r0 & 3);  // keys key, key + 1
        const float2 bv = bq[i % 3];
        float x0 = __builtin_fmaf(sc[cb][r0], c2, bv.x);
        float x1 = __builtin_fmaf(sc[cb][r0 + 1], c2, bv.y);
        if (masked) {
          x0 = key > lim[cb] ? -INFINITY : x0;
          x1 = key + 1 > lim[cb] ? -INFINITY : x1;
        }
        const float p0 = fast_exp2(x0), p1 = fast_exp2(x1);
        pc[cb][r0 >> 3][(r0 & 7) >> 1] = pack_bf16x2(p0, p1);
        ps[cb] += p0 + p1;  // fp32 sums: the row statistics (lse) stay exact to fp32
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    lsum[0] += ps[0];
    lsum[1] += ps[1];
  };

  f32x16 sA[2], sB[2];
  u32x4 pA[2][2], pB[2][2];
  // One pass over the piece.  The probabilities use a fixed reference maximum
  // per column: the maximum of the first tile on the first pass.  Later logits
  // may exceed it: while the row sum stays below 2^64, O and the sums are far
  // from fp32 overflow and the result is exact up to rounding.  A piece whose
  // sum does not (or is not finite) is run again with the reference raised by
  // log2 of that sum (which bounds every probability by 1 on the next pass).
  auto run = [&](bool first) __attribute__((always_inline)) {
    if (!first) {  // a repeated pass refills the ring (the first pass's loads went out above)
      issue_group(-3);
      issue_group(-2);
      issue_group(-1);
    }
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) pB[cb][hf] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db][0] = acc[db][1] = f32x16{};
    lsum[0] = lsum[1] = 0.f;
    sync_vm<F::NVM>();  // K(0) and bias(0) landed
    qk(0, sA);
    if (first) {  // reference = maximum logit of tile 0 (S(0) was computed with reference 0)
      const float(*bi)[AF_TK] = sBias[slot(0)];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const int lim = qi[cb] - kt0 * AF_TK;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 8 * (r >> 2) + 4 * hl + (r & 3);
          const float x = __builtin_fmaf(sA[cb][r], c2, bi[hloc[cb]][key]);
          mx = fmaxf(mx, (tdiag == 0 && key > lim) ? -INFINITY : x);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        m2[cb] = mx == -INFINITY ? 0.f : mx;
        const float sh = m2[cb] * inv_c2;
#pragma unroll
        for (int r = 0; r < 16; ++r) sA[cb][r] -= sh;
      }
      set_ref();
    }
    for (int t = 0; t < nt; t += 2) {
      if (t >= tdiag) body(t, sA, sB, pA, pB, true);
      else body(t, sA, sB, pA, pB, false);
      if (t + 1 >= nt) break;
      if (t + 1 >= tdiag) body(t + 1, sB, sA, pB, pA, true);
      else body(t + 1, sB, sA, pB, pA, false);
    }
    sync_vm<F::NVM>();  // V(nt-1) landed
    if (nt & 1) pv(nt - 1, pA);
    else pv(nt - 1, pB);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the tail's zero-fill loads
  };
  set_ref();
  for (int pass = 0; pass < 4; ++pass) {
    run(pass == 0);
    float lt[2];
    bool bad = false;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      lt[cb] = lsum[cb] + __shfl_xor(lsum[cb], 32);
      bad = bad || !(lt[cb] < 0x1p64f);
    }
    if (!__syncthreads_or(bad) || pass == 3) break;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb)
      if (!(lt[cb] < 0x1p64f)) m2[cb] = mref(cb) + (lt[cb] < INFINITY ? __log2f(lt[cb]) : 120.f);
    set_ref();
  }

  // Split block: publish this piece, the last one to finish merges.  Records
  // are written and read with device-scope relaxed atomic accesses (coherent
  // across the XCDs' L2s without flushing them); the counter bump follows the
  // completed stores, the merger's loads follow the counter.
  auto st_dev = [](float *a, float x) __attribute__((always_inline)) {
    __hip_atomic_store(a, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto ld_dev = [](const float *a) __attribute__((always_inline)) {
    return __hip_atomic_load(a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  int npm = 1;
  if (np > 1) {
    float *rec = part + ((int64_t)(pfirst + p) * nbh + bh) * (4 * F::NR * 64) + wave * F::NR * 64 + lane;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb)
#pragma unroll
        for (int r = 0; r < 16; ++r) st_dev(rec + ((db * 2 + cb) * 16 + r) * 64, acc[db][cb][r]);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      st_dev(rec + (F::NR - 4 + cb) * 64, mref(cb));  // the reference O and the sum are relative to
      st_dev(rec + (F::NR - 2 + cb) * 64, lsum[cb]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      sLast = __hip_atomic_fetch_add(&cnt[bh * nqb + qb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == np - 1;
    __syncthreads();
    if (!sLast) return;
    npm = np;
  }
  // merge pieces 0 .. npm-1 in order, all from their records (this one's too)
  float mm[2], lt[2];
  if (npm == 1) {
    mm[0] = mref(0), mm[1] = mref(1);
    lt[0] = lsum[0], lt[1] = lsum[1];
  } else {
    const float *rec0 = part + ((int64_t)pfirst * nbh + bh) * (4 * F::NR * 64) + wave * F::NR * 64 + lane;
    const int64_t pstride = (int64_t)nbh * (4 * F::NR * 64);
    mm[0] = mm[1] = -INFINITY;
    for (int pp2 = 0; pp2 < npm; ++pp2)
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) mm[cb] = fmaxf(mm[cb], ld_dev(rec0 + pp2 * pstride + (F::NR - 4 + cb) * 64));
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db][0] = acc[db][1] = f32x16{};
    lt[0] = lt[1] = 0.f;
    for (int pp2 = 0; pp2 < npm; ++pp2) {
      const float *rec = rec0 + pp2 * pstride;
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        const float sc = mm[cb] == -INFINITY ? 0.f : fast_exp2(ld_dev(rec + (F::NR - 4 + cb) * 64) - mm[cb]);
        lt[cb] += ld_dev(rec + (F::NR - 2 + cb) * 64) * sc;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][cb][r] += ld_dev(rec + ((db * 2 + cb) * 16 + r) * 64) * sc;
      }
    }
  }
#pragma unroll
  for (int cb = 0; cb < 2; ++cb) {
    const float ltot = lt[cb] + __shfl_xor(lt[cb], 32);
    const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
    if (!vq[cb]) continue;
    const int hq = kvh * G + hloc[cb];
    uint16_t *orow = o + ((bM + qi[cb]) * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = db * 32 + 8 * g4 + 4 * hl;
        *(u32x2 *)(orow + d) = u32x2{pack_bf16x2(acc[db][cb][4 * g4] * inv, acc[db][cb][4 * g4 + 1] * inv),
                                     pack_bf16x2(acc[db][cb][4 * g4 + 2] * inv, acc[db][cb][4 * g4 + 3] * inv)};
      }
    if (lse && hl == 0)
      lse[((int64_t)b * Hq + hq) * M + qi[cb]] = ltot > 0.f ? (mm[cb] + __log2f(ltot)) * kLn2 : -INFINITY;
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

// Split schedule of the bf16 forward: query blocks of BQ = 256 / G queries,
// pieces of at most C 32-key tiles, one work-group per piece and (batch, kv
// head), one work-group per compute unit at a time (256 of them).  When the
// unsplit blocks already fill the compute units, C is the average work per
// unit (blocks longer than that are split).  Otherwise C is the smallest piece
// length (at least 8 tiles) that keeps every piece in a single wave of 256
// work-groups.  Pieces of split blocks get a partial record each; split
// blocks form a prefix of the piece list.
FwdSched fwd_sched(int64_t B, int64_t M, int64_t Hq, int64_t Hkv) {
  FwdSched f{};
  const int64_t G = Hkv > 0 ? Hq / Hkv : 0;
  if (M <= 0 || G < 1 || G > 8 || (G & (G - 1)) != 0) return f;
  f.BQ = (int)(256 / G);
  f.nqb = (int)((M + f.BQ - 1) / f.BQ);
  const int64_t nbh = B * Hkv;
  int64_t tiles = 0;
  int nmax = 0;
  for (int qb = 0; qb < f.nqb; ++qb) {
    const int n = fwd_ntiles(qb, f.BQ, (int)M);
    tiles += n;
    nmax = n > nmax ? n : nmax;
  }
  auto pieces = [&](int C) {
    int64_t np = 0;
    for (int qb = 0; qb < f.nqb; ++qb) np += fwd_npieces(fwd_ntiles(qb, f.BQ, (int)M), C);
    return np;
  };
  if (nbh * f.nqb >= 256) {
    const int64_t avg = (nbh * tiles + 255) / 256;
    f.C = (int)(avg > 8 ? avg : 8);
  } else {
    f.C = 8;
    while (f.C < nmax && nbh * pieces(f.C) > 256) ++f.C;
  }
  for (int qb = 0; qb < f.nqb; ++qb) {
    const int np = fwd_npieces(fwd_ntiles(qb, f.BQ, (int)M), f.C);
    f.npieces += np;
    if (np > 1) f.nmulti += np;
  }
  return f;
}

// Workspace of the attention calls (256-byte aligned regions):
//   cs [B*M*D/2] float2 | khat [B*M*Hkv*D] bf16 | bias [B*Hq*M] f32 |
//   part [nmulti*B*Hkv * 4 waves * NR * 64] f32 | cnt [B*Hkv*nqb] i32 |
//   (backward) qhat [B*M*Hq*D] bf16 | rowstat [B*Hq*M] float2 | colsum [B*Hq*M] f32
static size_t rup(size_t x) { return (x + 255) / 256 * 256; }

static size_t part_floats(int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D) {
  const FwdSched f = fwd_sched(B, M, Hq, Hkv);
  const int64_t nr = 2 * (D / 32) * 16 + 4;
  return (size_t)(f.nmulti * B * Hkv * 4 * nr * 64);
}

static size_t cnt_ints(int64_t B, int64_t M, int64_t Hq, int64_t Hkv) {
  return (size_t)(B * Hkv * fwd_sched(B, M, Hq, Hkv).nqb);
}

size_t attn_workspace_bytes(int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D, bool bwd) {
  size_t n = rup((size_t)(B * M * (D / 2)) * sizeof(float2)) + rup((size_t)(B * M * Hkv * D) * 2) +
             rup((size_t)(B * Hq * M) * sizeof(float)) + rup(part_floats(B, M, Hq, Hkv, D) * sizeof(float)) +
             rup(cnt_ints(B, M, Hq, Hkv) * sizeof(int));
  if (bwd)
    n += rup((size_t)(B * M * Hq * D) * 2) + rup((size_t)(B * Hq * M) * sizeof(float2)) +
         rup((size_t)(B * Hq * M) * sizeof(float));
  return n;
}

AttnWs carve_attn_ws(void *ws, int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D) {
  AttnWs w;
  char *p = (char *)ws;
  w.cs = (float2 *)p;
  p += rup((size_t)(B * M * (D / 2)) * sizeof(float2));
  w.khat = (uint16_t *)p;
  p += rup((size_t)(B * M * Hkv * D) * 2);
  w.bias = (float *)p;
  p += rup((size_t)(B * Hq * M) * sizeof(float));
  w.part = (float *)p;
  p += rup(part_floats(B, M, Hq, Hkv, D) * sizeof(float));
  w.cnt = (int *)p;
  w.ncnt = (int)cnt_ints(B, M, Hq, Hkv);
  p += rup((size_t)w.ncnt * sizeof(int));
  w.qhat = (uint16_t *)p;
  p += rup((size_t)(B * M * Hq * D) * 2);
  w.rowstat = (float2 *)p;
  p += rup((size_t)(B * Hq * M) * sizeof(float2));
  w.colsum = (float *)p;
  return w;
}

hipError_t launch_attn_prep(const void *k, const float *g, const float *gamma, const int32_t *pos, double theta,
                            int B, int M, int Hq, int Hkv, int D, bool rot_k, bool with_bias, const AttnWs &w,
                            hipStream_t s) {
  if ((int64_t)B * M == 0) return hipSuccess;
  InvFreq inv;
  for (int i = 0; i < 64; ++i) inv.v[i] = i < D / 2 ? pow(theta, -2.0 * (double)i / (double)D) : 0.0;
  const int64_t rows = (int64_t)B * M;
  hipLaunchKernelGGL(attn_prep_kernel, dim3((unsigned)((rows * (D / 2) + 255) / 256)), dim3(256), 0, s,
                     (rot_k && pos) ? (const uint16_t *)k : nullptr, g, gamma, pos, inv, rows, M, Hq, Hkv, D, w.cs,
                     (rot_k && pos) ? w.khat : nullptr, with_bias ? w.bias : nullptr, w.cnt, with_bias ? w.ncnt : 0);
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                           const int32_t *pos, double theta, float tau, int B, int M, int Hq, int Hkv, int D,
                           bool bf16, void *o, float *lse, const AttnWs &w, hipStream_t s) {
  if ((int64_t)B * M == 0) return hipSuccess;
  hipError_t e = launch_attn_prep(k, g, gamma, pos, theta, B, M, Hq, Hkv, D, bf16, bf16, w, s);
  if (e != hipSuccess) return e;
  const float2 *cs = pos ? w.cs : nullptr;
  const double c = 1.0 / (sqrt((double)D) * (double)tau);
  if (bf16) {
    const FwdSched f = fwd_sched(B, M, Hq, Hkv);
    const dim3 grid((unsigned)(f.npieces * B * Hkv));
    const float c2 = (float)(c * 1.4426950408889634);
    const uint16_t *kh = pos ? w.khat : (const uint16_t *)k;
    if (D == 128)
      hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, dim3(256), 0, s, (const uint16_t *)q, kh,
                         (const uint16_t *)v, w.bias, cs, c2, B, M, Hq, Hkv, Hq / Hkv, f.BQ, f.nqb, f.C, w.part,
                         w.cnt, (uint16_t *)o, lse);
    else
      hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, dim3(256), 0, s, (const uint16_t *)q, kh,
                         (const uint16_t *)v, w.bias, cs, c2, B, M, Hq, Hkv, Hq / Hkv, f.BQ, f.nqb, f.C, w.part,
                         w.cnt, (uint16_t *)o, lse);
  } else {
    const int64_t rows = (int64_t)B * M * Hq;
    hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, (const float *)q,
                       (const float *)k, (const float *)v, g, gamma, cs, (float)c, B, M, Hq, Hkv, D, (float *)o,
                       lse);
  }
  return hipGetLastError();
}

}  // namespace tg
