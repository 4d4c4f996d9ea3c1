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
//     angles), the rotated keys and the per-head bias gamma_h log2 g_j;
//   * one work-group = 8 waves (two per SIMD) = one (batch, kv head) and 256
//     "columns", a column being a (query, head) pair of the GQA group:
//     BQ = 256 / G query positions x G heads share every K/V tile in LDS;
//   * each wave owns 32 columns; it computes S^T = K Q^T (keys on the MFMA
//     rows, its columns on the MFMA columns), so every lane holds 16 keys of a
//     single column: the row statistics are lane-local plus one cross-half
//     shuffle, and P^T feeds the P.V product straight from registers;
//   * O^T = V^T P^T reads V through the transposing LDS read
//     ds_read_b64_tr_b16; Q (rotated) lives in registers for the whole loop;
//   * 32-key tiles in chunk-major LDS layout (tg_tile.h), filled by direct
//     global->LDS loads AF_NS - 1 tiles ahead into a ring of AF_NS slots (one barrier
//     per tile), issued by one wave per SIMD;
//   * software pipeline per wave: S^T of tile t+1 on the matrix cores while the
//     softmax of tile t runs on the vector units; the per-key bias enters the
//     S^T products through their extra 16-deep step;
//   * softmax in fp32 against a fixed per-column reference, P rounded to
//     bf16 for the MFMA, row sums in fp32.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "tg_common.h"
#include "tg_attn.h"
#include "tg_tile.h"

namespace tg {

// Prep pass over the B*M kept rows (R = 256 / (D/2) rows per work-group, one
// thread per (row, rotary pair); the rotations by the work-group's threads in
// 16-byte pieces):
//   cs[row][i]    = (cos, sin)(pos[row] * inv_freq[i]) with the angle and the
//                   trigonometry in fp64 (inv_freq[i] = theta^(-2i/D), computed
//                   on the host in fp64), stored as fp32;
//   khat[row]     = k[row] rotated (bf16, every kv head), when khat != nullptr;
//   qfr           = q (rotated when positions are given), bf16, in the order
//                   of the forward's MFMA B fragments, when qfr != nullptr:
//                   block (b, head, 32-row block, 16-element step) is 64
//                   lanes x 16 bytes, lane l32 + 32 hl holding elements
//                   16 step + 8 hl .. +8 of row 32 block + l32, so the forward
//                   loads each of its fragments as one contiguous 1 KB block
//                   (consecutive threads here write consecutive rows' slots);
//   bias[b][h][j] = gamma_h * log2 g_j (-inf where g_j <= 0), the per-key,
//                   per-head logit bias in log2 units, when bias != nullptr
//                   (g_hj with per-head gates);
//   ratio[row]    = ln m_i / ln max(2, p_i), the row factor of the attention
//                   temperature (m_i = i + 1, p_i = pos + 1, or i + 1 without
//                   positions), when ratio != nullptr.
// Rotating K and Q once here replaces a rotation per query block in the main
// loop.
struct InvFreq {
  double v[64];
};

// rotate-half of one 16-byte piece x (elements i..i+7) with its partner y
// (elements i + D/2 ..), angles of pairs i..i+7 in cp
__device__ __forceinline__ void rot8(u32x4 &x, u32x4 &y, const float2 *cp) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float2 a0 = cp[2 * w], a1 = cp[2 * w + 1];
    const float x0 = bf16_lo(x[w]), x1 = bf16_hi(x[w]);
    const float y0 = bf16_lo(y[w]), y1 = bf16_hi(y[w]);
    x[w] = pack_bf16x2(x0 * a0.x - y0 * a0.y, x1 * a1.x - y1 * a1.y);
    y[w] = pack_bf16x2(y0 * a0.x + x0 * a0.y, y1 * a1.x + x1 * a1.y);
  }
}

// The runs of a packed group for the prep pass: run i starts at row off[i]
// (off[0] = 0, rows counted from the group's first token) and at padded row
// poff[i]; its sequences have M[i] tokens.
struct PrepRuns {
  int nr;
  int off[kMaxRuns], poff[kMaxRuns], M[kMaxRuns];
};
// Row r of a group: its run's length M, the row's sequence bb within the run
// and index j within the sequence, and the run's first row and padded row.
struct PrepRow {
  int M, bb, j, off, poff;
};
__device__ __forceinline__ PrepRow prep_row(const PrepRuns &pr, int64_t r) {
  PrepRow x{pr.M[0], 0, 0, 0, 0};
#pragma unroll
  for (int i = 1; i < kMaxRuns; ++i)
    if (i < pr.nr && r >= pr.off[i]) {
      x.M = pr.M[i];
      x.off = pr.off[i];
      x.poff = pr.poff[i];
    }
  const int loc = (int)(r - x.off);
  x.bb = loc / x.M;
  x.j = loc - x.bb * x.M;
  return x;
}

// MR: the rows are a packed group of runs (pr); bias and the query
// fragments are placed per run, M and nq32 are unused.
template <bool MR>
__global__ __launch_bounds__(256) void attn_prep_kernel(const uint16_t *__restrict__ k, const float *__restrict__ g,
                                                        const float *__restrict__ gamma,
                                                        const int32_t *__restrict__ pos, InvFreq inv, int64_t rows,
                                                        int M, int Hq, int Hkv, int D, float2 *__restrict__ cs,
                                                        uint16_t *__restrict__ khat, float *__restrict__ bias,
                                                        float *__restrict__ ratio, int *__restrict__ cnt, int ncnt,
                                                        int gph, const uint16_t *__restrict__ q,
                                                        uint16_t *__restrict__ qfr, int nq32, const PrepRuns pr) {
  __shared__ float2 scs[256];
  __shared__ PrepRow srow[8];  // MR: the placement of the work-group's rows, found once
  const int half = D / 2, R = 256 / half;  // R rows per work-group, one thread per (row, rotary pair)
  const int t = threadIdx.x;
  const int64_t idx = (int64_t)blockIdx.x * 256 + t;
  if (idx < ncnt) cnt[idx] = 0;  // the split-row arrival counters of the forward kernel
  const int lr = t / half, i = t - lr * half;
  const int64_t r0 = (int64_t)blockIdx.x * R, r = r0 + lr;
  const bool vr = lr < R && r < rows;
  if constexpr (MR) {
    if (t < R && r0 + t < rows) srow[t] = prep_row(pr, r0 + t);
    __syncthreads();
  }
  if (pos && vr) {
    double sn, cn;
    sincos((double)pos[r] * inv.v[i], &sn, &cn);
    const float2 v = make_float2((float)cn, (float)sn);
    cs[r * half + i] = v;
    scs[t] = v;
  }
  if (pos && (khat || qfr)) __syncthreads();
  if (pos && khat) {
    // the work-group's R rows x Hkv heads x (half / 8) piece pairs: 16-byte loads and stores
    const int nch = half / 8, per_row = Hkv * nch;
    for (int it = t; it < R * per_row; it += 256) {
      const int lr2 = it / per_row, rem = it - lr2 * per_row, h = rem / nch, ch = rem - h * nch;
      if (r0 + lr2 >= rows) break;
      const int64_t o = ((r0 + lr2) * Hkv + h) * D + 8 * ch;
      u32x4 x = *(const u32x4 *)(k + o), y = *(const u32x4 *)(k + o + half);
      rot8(x, y, scs + lr2 * half + 8 * ch);
      *(u32x4 *)(khat + o) = x;
      *(u32x4 *)(khat + o + half) = y;
    }
  }
  if (qfr) {
    // items (head, step pair kp, half hl, row lr2), the row fastest: row j's piece of elements
    // e = 16 kp + 8 hl goes to slot (j % 32) + 32 hl of block (b, head, j / 32, kp), its rotary
    // partner e + D/2 to the same slot of step kp + D/32
    const int nks = D / 16, npair = nks / 2;
    for (int it = t; it < R * 2 * Hq * npair; it += 256) {
      const int lr2 = it % R, rest = it / R, hl = rest & 1, rest2 = rest >> 1, kp = rest2 % npair,
                h = rest2 / npair;
      const int64_t row = r0 + lr2;
      if (row >= rows) continue;
      const int e = 16 * kp + 8 * hl;
      const int64_t o = (row * Hq + h) * D + e;
      u32x4 x = *(const u32x4 *)(q + o), y = *(const u32x4 *)(q + o + half);
      if (pos) rot8(x, y, scs + lr2 * half + e);
      uint16_t *blk;
      if constexpr (MR) {
        const PrepRow x = srow[lr2];
        blk = qfr + (int64_t)x.poff * Hq * D +
              ((((int64_t)x.bb * Hq + h) * ((x.M + 31) / 32) + x.j / 32) * nks) * 512 + ((x.j & 31) + 32 * hl) * 8;
      } else {
        const int bb = (int)(row / M), j = (int)(row - (int64_t)bb * M);
        blk = qfr + ((((int64_t)bb * Hq + h) * nq32 + j / 32) * nks) * 512 + ((j & 31) + 32 * hl) * 8;
      }
      *(u32x4 *)(blk + kp * 512) = x;
      *(u32x4 *)(blk + (kp + npair) * 512) = y;
    }
  }
  if constexpr (MR) {  // one gate per key, g [rows]; each run's bias [n, Hq, M] from its first row's Hq-fold
    if (bias && vr) {
      const PrepRow x = srow[lr];
      float *bq = bias + (int64_t)x.off * Hq + ((int64_t)x.bb * Hq) * x.M + x.j;
      const float gv = g[r];
      for (int h = i; h < Hq; h += half) bq[(int64_t)h * x.M] = gv > 0.f ? gamma[h] * log2f(gv) : -INFINITY;
    }
  } else if (bias && vr) {  // gph: one gate per (head, key), g [B, Hq, M]; else one per key, g [B, M]
    const int64_t bb = r / M, j = r - bb * M;
    for (int h = i; h < Hq; h += half) {
      const float gv = g[gph ? (bb * Hq + h) * M + j : r];
      bias[(bb * Hq + h) * M + j] = gv > 0.f ? gamma[h] * log2f(gv) : -INFINITY;
    }
  }
  if (ratio && vr && i == 0) {  // the temperature's row factor ln m_i / ln max(2, p_i) (fp64 logs)
    int64_t j;
    if constexpr (MR) j = srow[lr].j;
    else j = r - (r / M) * M;
    const double m = (double)j + 1.0, pp = pos ? (double)pos[r] + 1.0 : m;
    ratio[r] = (float)(log(m) / log(pp > 2.0 ? pp : 2.0));
  }
}


// ---------------------------------------------------------------------------
// bf16 forward.  Work-group = 8 waves (two per SIMD) = 256 columns, a column
// being a (query, head) pair of the GQA group: BQ = 256 / G queries x G
// heads.  Wave w owns columns 32w .. 32w+31 (one head).  Keys come in 32-key
// tiles, shared by the 8 waves through LDS (direct loads AF_NS - 1 tiles
// ahead, issued by one wave per SIMD; one barrier per tile).  Per tile a wave
// runs S^T = K Q^T (keys on the MFMA rows: each lane holds 16 keys of one
// column, so the row statistics are lane-local plus one cross-half shuffle),
// the softmax of its 16 logits per lane, and O^T += V^T P^T with V^T from the
// transposing LDS read.  Software pipeline: the S^T products of tile t+1 run
// while the softmax of tile t is on the vector units; the other wave of the
// SIMD fills remaining gaps.
//
// The probabilities use a fixed reference maximum per column (the maximum of
// the piece's first tile), subtracted inside the S^T products by one more
// 16-deep step; no rescaling in the loop.  While the row sum stays below 2^64,
// O and the sums are far from fp32 overflow and the result is exact up to
// rounding; a piece whose sum does not is run again with the reference
// raised by log2 of that sum (which bounds every probability by 1).  The
// causal split puts a visible key in every piece's first tile; only keys with
// bias -inf (g = 0) can leave that tile without a live key for a column.  Such
// a column takes instead the logit of the first key of the piece whose bias
// is finite (if it sees one): any live logit is a valid reference, since
// every probability of the column is then 2^(x - m2) with m2 <= max x, and
// the guard above bounds the sum.
//
// Long causal rows are split along the keys into pieces (at most C tiles
// each, the diagonal in the last piece) so that the work spreads over every
// compute unit.  Each piece of a split query block writes its unnormalised
// (O, reference, sum) to the workspace and bumps a per-block counter; the last
// to arrive merges all pieces in piece order (deterministic) and writes o, lse.
// ---------------------------------------------------------------------------
constexpr int AF_TK = AB_T;  // keys per tile
constexpr int AF_NS = 4;     // slots of the LDS tile ring (loads go out AF_NS - 1 tiles ahead)

template <int D>
struct FwdCfg {
  static constexpr int NDB = D / 32;    // 32-row blocks of O^T
  static constexpr int NR = NDB * 16 + 2;  // floats per lane in a partial record (O^T, reference, sum)
};

// Tiles of query block qb (keys 0 .. min((qb+1) BQ, M) - 1) and its pieces.
__host__ __device__ inline int fwd_ntiles(int qb, int BQ, int M) {
  const int qe = (qb + 1) * BQ < M ? (qb + 1) * BQ : M;
  return (qe + AF_TK - 1) / AF_TK;
}
__host__ __device__ inline int fwd_npieces(int n, int C) { return (n + C - 1) / C; }

// x as three bf16 parts (hi, mid, lo; their sum is x to about 2^-24 relative).
__device__ __forceinline__ void split3(float x, uint32_t &h, uint32_t &m, uint32_t &l) {
  h = pack_bf16x2(x, 0.f) & 0xFFFFu;
  const float r1 = x - bf16_lo(h);
  m = pack_bf16x2(r1, 0.f) & 0xFFFFu;
  l = pack_bf16x2(r1 - bf16_lo(m), 0.f) & 0xFFFFu;
}
// Operands of the extra 16-deep step of an S^T = K Q^T product (32x32x16
// layout: element k of row i in lane i + 32 (k / 8)).  Key side (A, one row
// per key): ones at k = 0..2, the key's x in three parts at k = 3..5.  Query
// side (B, one column per query): the column's x in three parts at k = 0..2,
// ones at k = 3..5.  The step adds key value + query value to every product.
__device__ __forceinline__ u32x4 aug_key(float x, int hl) {
  uint32_t h, m, l;
  split3(x, h, m, l);
  return hl == 0 ? u32x4{0x3F803F80u, 0x3F80u | (h << 16), m | (l << 16), 0u} : u32x4{0u, 0u, 0u, 0u};
}
__device__ __forceinline__ u32x4 aug_query(float x, int hl) {
  uint32_t h, m, l;
  split3(x, h, m, l);
  return hl == 0 ? u32x4{h | (m << 16), l | (0x3F80u << 16), 0x3F803F80u, 0u} : u32x4{0u, 0u, 0u, 0u};
}

// The work-group table argument: a RunTable over packed runs, nothing for
// one batch.
struct NoTable {
  int unused;
};
template <bool MR>
using FwdTab = std::conditional_t<MR, RunTable, NoTable>;

// MR: the work-groups cover the runs of a packed group through the table rt;
// the pointers are those of the whole packed batch and workspace, and B, M,
// nq32, nqb and C are taken from the work-group's run.
template <int D, bool TEMP, bool MR>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ qfr, int nq32, const uint16_t *__restrict__ khat, const uint16_t *__restrict__ v,
    const float *__restrict__ bias, float c2, const float *__restrict__ sigma,
    const float *__restrict__ ratio, int B, int M, int Hq, int Hkv, int G, int BQ, int nqb, int C,
    float *__restrict__ part, int *__restrict__ cnt, uint16_t *__restrict__ o, float *__restrict__ lse,
    uint16_t *__restrict__ o_lo, const FwdTab<MR> rt) {
  using T = BTile<D>;
  using F = FwdCfg<D>;
  constexpr int NKS = T::NKS, NDB = T::NDB;
  // The tiles' direct loads are issued by the first wave of each SIMD only
  // (waves 0..3): issuing them takes the vector-memory path a few hundred
  // clocks per tile, and those waves reach the barrier first.
  constexpr int NLW = 4;                  // loader waves
  constexpr int NIW = 2 * T::NI / NLW;    // K and V direct loads per loader wave per tile
  constexpr int NVM = NIW + 1;            // + the bias load (wave 0 only)
  __shared__ __attribute__((aligned(1024))) uint16_t sK[AF_NS * T::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[AF_NS * T::TILE];
  __shared__ __attribute__((aligned(1024))) float sBias[AF_NS][8][AF_TK];
  __shared__ int sLast;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  const int l32 = lane & 31, hl = lane >> 5;
  constexpr int RW = AB_NW * F::NR * 64;  // floats per work-group record
  unsigned wg = blockIdx.x;  // the work-group within its range of the table (all of them for one batch)
  int top = nqb - 1;         // the piece listing: blocks top, top - 1, ...
  bool across = false;       // one block of consecutive runs, one piece each
  int ri = 0;                // the run (MR)
  if constexpr (MR) {
    // the range: the last e with start[e] <= wg (binary search, uniform)
    int e = 0;
#pragma unroll
    for (int step = kMaxEnt / 2; step >= 1; step >>= 1)
      if ((int)wg >= rt.start[e + step]) e += step;
    const int code = rt.code[e];
    ri = code & 0xFF;
    wg -= rt.start[e];
    top = (code >> 8) & 0x3FFFFF;
    across = (code >> 30) & 1;
    if (across)
      for (int i = 0; i < kMaxRuns - 1; ++i) {
        const unsigned nb = rt.run[ri].n * Hkv;
        if (wg < nb) break;
        wg -= nb;
        ++ri;
      }
    const RunRow &r = rt.run[ri];
    B = r.n;
    M = r.M;
    C = r.C;
    nqb = (M + BQ - 1) / BQ;
    nq32 = (M + 31) / 32;
    const int64_t off = r.off;
    qfr += (int64_t)r.poff * Hq * D;
    khat += off * Hkv * D;
    v += off * Hkv * D;
    bias += off * Hq;
    if (TEMP) ratio += off;
  }
  const int nbh = B * Hkv;
  // consecutive work-groups take consecutive (batch, kv head): with the
  // round-robin placement over the 8 XCDs one head's keys stay in one L2
  const int bh = wg % nbh;
  const int b = bh / Hkv, kvh = bh % Hkv;

  // Piece -> (query block, piece index).  Pieces are listed by descending query
  // block (longest rows first); each wave scans 64 blocks at a time.
  int qb = across ? top : 0, p = 0, np = 1, pfirst = 0;
  if (!across) {
    int rem = wg / nbh, base = 0;
    for (int c0 = 0; c0 <= top; c0 += 64) {
      const int qq = top - (c0 + lane);
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
        qb = top - (c0 + src);
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
  const int tu = tdiag < nt ? tdiag : nt;

  const int hloc = (AF_TK * wave) / BQ;
  const int qi = q0 + (AF_TK * wave) % BQ + l32;
  const bool vq = qi < M;
  const int64_t bM = (int64_t)b * M;
  const uint32_t rsb = (uint32_t)(Hkv * D * 2);  // bytes between consecutive keys
  const uint32_t kv_bytes = (uint32_t)(M - 1) * rsb + D * 2;
  const i32x4 rK = buffer_rsrc(khat + (bM * Hkv + kvh) * D, kv_bytes);
  const i32x4 rV = buffer_rsrc(v + (bM * Hkv + kvh) * D, kv_bytes);
  const i32x4 rB = buffer_rsrc(bias + (int64_t)b * Hq * M, (uint32_t)(Hq * M * 4));

  BFrag<D> fr;
  fr.init(lane);
  // loader wave w issues direct load j = w + 4 n of the tile's 2 NI (K for
  // n < NIW / 2, then V)
  const bool loader = wave < NLW;
  uint32_t dgo[NIW], dlo[NIW];
#pragma unroll
  for (int n = 0; n < NIW; ++n) {
    const int j = (wave % NLW + NLW * n) % T::NI;
    dgo[n] = T::goff(j, lane, rsb);
    dlo[n] = 1024u * (uint32_t)j;
  }
  // bias: wave 0 loads the G rows of the tile (8 lanes x 16 bytes per head)
  const bool breal = wave == 0 && (lane >> 3) < G;
  const uint32_t bvo = (uint32_t)((((lane >> 3) * M) + 4 * (lane & 7)) * 4);
  auto slot = [](int t) __attribute__((always_inline)) { return t & (AF_NS - 1); };
  auto issue = [&](int t) __attribute__((always_inline)) {
    if (!loader) return;
    const bool live = t < nt;
    const uint32_t toff = (uint32_t)((kt0 + t) * AF_TK) * rsb;  // uniform
    const uint32_t so = 2u * (uint32_t)(slot(t) * T::TILE);
#pragma unroll
    for (int n = 0; n < NIW; ++n)
      dma_b128(n >= NIW / 2 ? rV : rK, (n >= NIW / 2 ? lds_addr(sV) : lds_addr(sK)) + so + dlo[n],
               live ? dgo[n] + toff : 0x80000000u, 0u);
    const uint32_t boff = (uint32_t)((kvh * G * M + (kt0 + t) * AF_TK) * 4);  // uniform
    if (wave == 0) dma_b128(rB, lds_addr(&sBias[slot(t)][0][0]), live && breal ? bvo + boff : 0x80000000u, 0u);
  };
  // wait for this wave's loads of the oldest tile in flight, then the barrier
  auto sync_tile = [&]() __attribute__((always_inline)) {
    if (wave == 0) sync_vm<(AF_NS - 3) * NVM>();
    else if (loader) sync_vm<(AF_NS - 3) * (NVM - 1)>();
    else sync_vm<0>();
  };
  auto issue_first = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < AF_NS - 1; ++t) issue(t);
  };
  // The first pass's direct loads go out first; the Q and rotation loads
  // below (all issued before any use) overlap with them.
  issue_first();

  // Q fragments (MFMA B operand): lane holds q^[qi, h, 16 ks + 8 hl .. +8],
  // from the prep pass's fragment-ordered copy (one contiguous 1 KB block
  // per wave and 16-element step)
  u32x4 qf[NKS];
  {
    const int qb32 = (q0 + (AF_TK * wave) % BQ) / AF_TK;
    const u32x4 *src = (const u32x4 *)(qfr + (((int64_t)b * Hq + kvh * G + hloc) * nq32 + qb32) * NKS * 512) + lane;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const u32x4 x = src[64 * ks];
      qf[ks] = vq ? x : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) settle(qf[ks]);
  }

  // Temperature of the column's row (1 without it): x = t (c2 s + bias).  t is
  // kept >= 1e-30 (t = 0 at the first row, where every live logit is 0 either
  // way).
  float tq = 1.f;
  if (TEMP && vq) tq = fmaxf(softplus_f(sigma[kvh * G + hloc]) * ratio[bM + qi], 1e-30f);
  settle(tq);
  const float tc2 = c2 * tq;           // logit = tc2 * (S^T entry)
  const float inv_c2 = 1.f / tc2;      // reference -> S units
  const float inv_c2k = 1.f / c2;      // bias -> S units
  // m2: reference maximum of the column (probabilities are 2^(x - m2)).  The
  // extra 16-deep step of every S^T product adds bias_j / c2 (key side) and
  // -m2 / (t c2) (query side), each as three bf16 parts against ones, so the
  // logit is one multiply.  A key with bias -inf enters with bias / c2
  // clamped to -2^127: its logit is then about -2^127 t c2 (below -1e7 for any
  // t >= 1e-30) and its probability 0.
  float m2 = 0.f, lsum = 0.f;
  u32x4 qaug = aug_query(0.f, hl);
  f32x16 acc[NDB];

  // S^T = K Q^T + extra step for tile t (K fragments read three steps ahead)
  auto key_aug = [&](float bv) __attribute__((always_inline)) {
    return aug_key(fmaxf(bv * inv_c2k, -0x1p127f), hl);
  };
  // Logit x = t (c2 q^.k^_j0 + bias_j0) of the first key j0 of tiles 1 .. nt-1
  // of the piece whose bias (this wave's head) is finite, for each column that
  // sees it; -inf for the others, or when there is no such key.  Wave-uniform
  // search over the bias row in global memory, then q^.k^_j0 for the wave's 32
  // columns as one S^T product whose 32 key rows all hold k^_j0.
  auto first_live_logit = [&]() __attribute__((always_inline)) -> float {
    const float *brow = bias + ((int64_t)b * Hq + kvh * G + hloc) * M;
    const int jend = (kt0 + nt) * AF_TK < M ? (kt0 + nt) * AF_TK : M;
    int j0 = jend;
    for (int j = (kt0 + 1) * AF_TK; j < jend; j += 64) {
      const uint64_t live = __ballot(j + lane < jend && brow[j + lane] != -INFINITY);
      if (live) {
        j0 = j + __ffsll((unsigned long long)live) - 1;
        break;
      }
    }
    if (j0 >= jend) return -INFINITY;
    const uint16_t *krow = khat + ((bM + j0) * Hkv + kvh) * D + 8 * hl;
    f32x16 s0 = f32x16{};
    for (int ks = 0; ks < NKS; ++ks) s0 = mfma32(*(const u32x4 *)(krow + 16 * ks), qf[ks], s0);
    return qi >= j0 ? tc2 * (s0[0] + brow[j0] * inv_c2k) : -INFINITY;
  };
  // softmax of 2 of the 16 logits per lane (registers 2c, 2c+1) of a tile
  auto soft2 = [&](const f32x16 &s, int c, float msub, bool masked, int lim, float &ps, u32x4(&pf)[2])
      __attribute__((always_inline)) {
    float x0 = __builtin_fmaf(s[2 * c], tc2, -msub), x1 = __builtin_fmaf(s[2 * c + 1], tc2, -msub);
    if (masked) {
      if (acc_row(2 * c, hl) > lim) x0 = -INFINITY;
      if (acc_row(2 * c + 1, hl) > lim) x1 = -INFINITY;
    }
    const float p0 = fast_exp2(x0), p1 = fast_exp2(x1);
    const uint32_t pk = pack_bf16x2(p0, p1);
    ps += p0 + p1;  // fp32 sums: the row statistics (lse) stay exact to fp32
    // an empty volatile statement on the results keeps this work where it is
    // written (between the products it overlaps) instead of sunk to its uses
    asm volatile("" : "+v"(ps) : "v"(pk));
    pf[c >> 2][c & 3] = pk;
  };
  // One step of the software pipeline: wait for tile t+1;
  // S^T of tile t+1 on the matrix cores while the first half of the softmax
  // of tile t (S^T in sc, msub the reference it was computed without) runs on
  // the vector units; then O^T += V^T P^T of tile t, its first 16 keys while
  // the second half of the softmax runs; then the loads of tile t+AF_NS-1.
  // After the barrier every wave is done with tile t-1, whose ring slot that
  // tile takes.
  // (masked_c: std::true_type on the tiles that reach the diagonal, std::false_type before:
  // two instantiations, so the tiles before the diagonal carry no mask work)
  auto step = [&](int t, f32x16 &sc, auto masked_c, float msub) __attribute__((always_inline)) {
    constexpr bool masked = decltype(masked_c)::value;
    sync_tile();
    const uint16_t *K = sK + slot(t + 1) * T::TILE, *V = sV + slot(t) * T::TILE;
    const float bnext = sBias[slot(t + 1)][hloc][l32];
    const int lim = qi - (kt0 + t) * AF_TK;  // keys (within the tile) past the query are masked
    f32x16 sn = f32x16{};
    float ps = 0.f;
    u32x4 pf[2];
    {
      u32x4 f[NKS];
#pragma unroll
      for (int i = 0; i < 3; ++i) f[i] = fr.rows(K, i);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 3 < NKS) f[ks + 3] = fr.rows(K, ks + 3);
        __builtin_amdgcn_sched_barrier(0);
        sn = mfma32(f[ks], qf[ks], sn);
#pragma unroll
        for (int c = 0; c < 4; ++c)  // chunk c after the last product of its quarter of the k-steps
          if ((c + 1) * NKS / 4 - 1 == ks) soft2(sc, c, msub, masked, lim, ps, pf);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    sn = mfma32(key_aug(bnext), qaug, sn);
    {
      u32x4 f[2 * NDB];
#pragma unroll
      for (int i = 0; i < 3; ++i) f[i] = fr.tr(V, i / NDB, i % NDB);
#pragma unroll
      for (int i = 0; i < 2 * NDB; ++i) {
        if (i + 3 < 2 * NDB) f[i + 3] = fr.tr(V, (i + 3) / NDB, (i + 3) % NDB);
        __builtin_amdgcn_sched_barrier(0);
        acc[i % NDB] = mfma32(f[i], pf[i / NDB], acc[i % NDB]);
#pragma unroll
        for (int c = 0; c < 4; ++c)  // chunks 4..7 spread over the products of the first 16 keys
          if (i < NDB && c * NDB / 4 == i) soft2(sc, 4 + c, msub, masked, lim, ps, pf);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    lsum += ps;
    sc = sn;
    issue(t + AF_NS - 1);  // the loader waves, after their work: into tile t-1's slot
  };
  auto run = [&](bool first) __attribute__((always_inline)) {
    if (!first) issue_first();  // a repeated pass refills the ring (the first pass's loads went out above)
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    lsum = 0.f;
    // prologue: S^T of tile 0 (tiles 1 .. AF_NS - 2 may still be in flight)
    if (wave == 0) sync_vm<(AF_NS - 2) * NVM>();
    else if (loader) sync_vm<(AF_NS - 2) * (NVM - 1)>();
    else sync_vm<0>();
    f32x16 sc = f32x16{};
    float msub = 0.f;
    {
      const uint16_t *K = sK + slot(0) * T::TILE;
      const float b0 = sBias[slot(0)][hloc][l32];
      u32x4 f[NKS];
#pragma unroll
      for (int i = 0; i < 3; ++i) f[i] = fr.rows(K, i);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 3 < NKS) f[ks + 3] = fr.rows(K, ks + 3);
        __builtin_amdgcn_sched_barrier(0);
        sc = mfma32(f[ks], qf[ks], sc);
        __builtin_amdgcn_sched_barrier(0);
      }
      sc = mfma32(key_aug(b0), qaug, sc);
      if (first) {  // tile 0 sets the reference: the maximum over its live keys
        const uint64_t dead = __ballot(b0 == -INFINITY);  // bit j (j < 32): key j of the tile
        const int lim = qi - kt0 * AF_TK;
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = acc_row(r, hl);
          const bool live = !((dead >> row) & 1u) && !(tu == 0 && row > lim);
          if (live) mx = fmaxf(mx, sc[r] * tc2);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        // a column that sees no live key in tile 0 (g = 0 on all of them) but
        // one later in the piece: the logit of the piece's first live key
        if (nt > 1 && __ballot(vq && mx == -INFINITY)) mx = fmaxf(mx, first_live_logit());
        m2 = mx == -INFINITY ? 0.f : mx;
        msub = m2;  // tile 0's products ran without it
        qaug = aug_query(-m2 * inv_c2, hl);
      }
    }
    int t = 0;
    for (; t < tu; ++t) {
      step(t, sc, std::false_type{}, msub);
      msub = 0.f;
    }
    for (; t < nt; ++t) {
      step(t, sc, std::true_type{}, msub);
      msub = 0.f;
    }
    sync_vm<0>();  // the tail's zero-fill loads landed, every wave done with the ring
  };
  for (int pass = 0; pass < 4; ++pass) {
    run(pass == 0);
    const float lt = lsum + __shfl_xor(lsum, 32);
    const bool bad = !(lt < 0x1p64f);
    if (!__syncthreads_or(bad) || pass == 3) break;
    if (bad) m2 += lt < INFINITY ? __log2f(lt) : 120.f;
    qaug = aug_query(-m2 * inv_c2, hl);
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
  if constexpr (MR) {
    // the outputs of the work-group's run, placed only now (the run read from
    // the table again instead of holding its pointers through the loop)
    int rj = ri;
    asm volatile("" : "+s"(rj));
    const RunRow &r = rt.run[rj];
    const int64_t off = r.off;
    part += (int64_t)r.rec0 * RW;
    cnt += r.cnt0;
    o += off * Hq * D;
    if (lse) lse += off * Hq;
    if (o_lo) o_lo += off * Hq * D;
  }
  int npm = 1;
  if (np > 1) {
    float *rec = part + ((int64_t)(pfirst + p) * nbh + bh) * RW + wave * F::NR * 64 + lane;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st_dev(rec + (db * 16 + r) * 64, acc[db][r]);
    // the reference O and the sum are relative to; -inf for a column with no
    // live key in this piece (every key it sees has bias -inf), which the merge
    // then skips instead of letting its placeholder reference 0 set the scale
    const float lcol = lsum + __shfl_xor(lsum, 32);
    st_dev(rec + (F::NR - 2) * 64, lcol > 0.f ? m2 : -INFINITY);
    st_dev(rec + (F::NR - 1) * 64, lsum);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0)
      sLast = __hip_atomic_fetch_add(&cnt[bh * nqb + qb], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == np - 1;
    __syncthreads();
    if (!sLast) return;
    npm = np;
  }
  // merge pieces 0 .. npm-1 in piece order: the other pieces from their
  // records, this one from its registers (the same values its record holds,
  // so the sums do not depend on which piece arrives last)
  float mm = m2, lt = lsum;
  if (npm > 1) {
    const float *rec0 = part + ((int64_t)pfirst * nbh + bh) * RW + wave * F::NR * 64 + lane;
    const int64_t pstride = (int64_t)nbh * RW;
    const float ref_own = lsum + __shfl_xor(lsum, 32) > 0.f ? m2 : -INFINITY, l_own = lsum;
    f32x16 own[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) own[db] = acc[db];
    mm = -INFINITY;
    for (int pp2 = 0; pp2 < npm; ++pp2)
      mm = fmaxf(mm, pp2 == p ? ref_own : ld_dev(rec0 + pp2 * pstride + (F::NR - 2) * 64));
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    lt = 0.f;
    for (int pp2 = 0; pp2 < npm; ++pp2) {
      const float *rec = rec0 + pp2 * pstride;
      const bool mine = pp2 == p;  // work-group uniform
      const float rf = mine ? ref_own : ld_dev(rec + (F::NR - 2) * 64);
      const float sc = mm == -INFINITY ? 0.f : fast_exp2(rf - mm);
      lt += (mine ? l_own : ld_dev(rec + (F::NR - 1) * 64)) * sc;
      if (mine) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] += own[db][r] * sc;
      } else {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[db][r] += ld_dev(rec + (db * 16 + r) * 64) * sc;
      }
    }
  }
  const float ltot = lt + __shfl_xor(lt, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  const int hq = kvh * G + hloc;
  if (lse && hl == 0 && vq)
    lse[((int64_t)b * Hq + hq) * M + qi] = ltot > 0.f ? (mm + __log2f(ltot)) * kLn2 : -INFINITY;
  // The normalised O^T tile goes out through LDS (the K/V ring, idle now):
  // wave w stages its 32 columns x D as rows of D bf16 (16-byte pieces
  // XOR-swizzled by the column), then writes each column's row of o as D/8
  // contiguous 16-byte pieces.
  // With o_lo, the same tile again as the residual of the bf16 rounding
  // (o + o_lo is the fp32 output to about 2^-18 relative).
  constexpr int CPR = D / 8;  // 16-byte pieces per row
  __syncthreads();            // every wave is done with the ring
  uint8_t *stg = (uint8_t *)(wave < 4 ? sK : sV) + (wave & 3) * (AF_TK * D * 2);
  const int qcol0 = q0 + (AF_TK * wave) % BQ;  // query of column 0 of this wave
  auto emit = [&](uint16_t *dst, bool lo) __attribute__((always_inline)) {
    auto pk = [&](float a, float c) __attribute__((always_inline)) {
      const uint32_t h = pack_bf16x2(a, c);
      return lo ? pack_bf16x2(a - bf16_lo(h), c - bf16_hi(h)) : h;
    };
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int pc = (4 * db + g4) ^ (l32 & (CPR - 1));  // piece of elements 32 db + 8 g4 ..
        *(u32x2 *)(stg + l32 * (2 * D) + pc * 16 + 8 * hl) =
            u32x2{pk(acc[db][4 * g4] * inv, acc[db][4 * g4 + 1] * inv),
                  pk(acc[db][4 * g4 + 2] * inv, acc[db][4 * g4 + 3] * inv)};
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the wave reads back only what it wrote
#pragma unroll
    for (int it = 0; it < AF_TK * CPR / 64; ++it) {
      const int c = lane + 64 * it, col = c / CPR, ch = c % CPR;
      const u32x4 x = *(const u32x4 *)(stg + col * (2 * D) + ((ch ^ (col & (CPR - 1))) * 16));
      if (qcol0 + col < M) *(u32x4 *)(dst + ((bM + qcol0 + col) * Hq + hq) * D + 8 * ch) = x;
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the reads done before the area is written again
  };
  emit(o, false);
  if (o_lo) emit(o_lo, true);
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
    const float *__restrict__ sigma, const float *__restrict__ ratio, int B, int M, int Hq, int Hkv, int D,
    int gph, float *__restrict__ o, float *__restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, i, h) flattened
  if (row >= (int64_t)B * M * Hq) return;
  const int h = (int)(row % Hq);
  const int64_t bi = row / Hq;
  const int i = (int)(bi % M);
  const int64_t bM = bi - i;
  const int kv = h / (Hq / Hkv);
  const int half = D / 2;
  const float t = sigma ? fmaxf(softplus_f(sigma[h]) * ratio[bi], 1e-30f) : 1.f;
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
  const float *gh = gph ? g + ((bM / M) * Hq + h) * M : g + bM;  // this head's gates of the row
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
    const float sj = t * (wave_sum(qx * kx + qy * ky) * c + bias_of(gam, gh[j]));
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
// blocks form a prefix of the piece list.  Runs launched together share one
// C, chosen the same way over all their blocks.
static int fwd_group_c(const RunRow *runs, int nruns, int64_t Hq, int64_t Hkv) {
  const int64_t G = Hkv > 0 ? Hq / Hkv : 0;
  if (G < 1 || G > 8 || (G & (G - 1)) != 0) return 0;
  const int BQ = (int)(256 / G);
  int64_t blocks = 0, tiles = 0;
  int nmax = 0;
  for (int i = 0; i < nruns; ++i) {
    const int64_t nbh = (int64_t)runs[i].n * Hkv;
    const int M = runs[i].M, nqb = (M + BQ - 1) / BQ;
    blocks += nbh * nqb;
    for (int qb = 0; qb < nqb; ++qb) {
      const int n = fwd_ntiles(qb, BQ, M);
      tiles += nbh * n;
      nmax = n > nmax ? n : nmax;
    }
  }
  if (blocks >= 256) {
    const int64_t avg = (tiles + 255) / 256;
    return (int)(avg > 8 ? avg : 8);
  }
  auto pieces = [&](int C) {
    int64_t np = 0;
    for (int i = 0; i < nruns; ++i) {
      const int M = runs[i].M, nqb = (M + BQ - 1) / BQ;
      for (int qb = 0; qb < nqb; ++qb) np += (int64_t)runs[i].n * Hkv * fwd_npieces(fwd_ntiles(qb, BQ, M), C);
    }
    return np;
  };
  int C = 8;
  while (C < nmax && pieces(C) > 256) ++C;
  return C;
}

FwdSched fwd_sched_c(int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int C) {
  FwdSched f{};
  const int64_t G = Hkv > 0 ? Hq / Hkv : 0;
  if (M <= 0 || G < 1 || G > 8 || (G & (G - 1)) != 0 || C < 1) return f;
  (void)B;
  f.BQ = (int)(256 / G);
  f.nqb = (int)((M + f.BQ - 1) / f.BQ);
  f.C = C;
  for (int qb = 0; qb < f.nqb; ++qb) {
    const int np = fwd_npieces(fwd_ntiles(qb, f.BQ, (int)M), f.C);
    f.npieces += np;
    if (np > 1) f.nmulti += np;
  }
  return f;
}

FwdSched fwd_sched(int64_t B, int64_t M, int64_t Hq, int64_t Hkv) {
  const RunRow r{0, 0, (int)B, (int)M, 0, 0, 0};
  return fwd_sched_c(B, M, Hq, Hkv, M > 0 && B > 0 ? fwd_group_c(&r, 1, Hq, Hkv) : 0);
}

// Workspace of the attention calls (256-byte aligned regions):
//   cs [B*M*D/2] float2 | khat [B*M*Hkv*D] bf16 | bias [B*Hq*M] f32 |
//   part [nmulti*B*Hkv * 4 waves * NR * 64] f32 | cnt [B*Hkv*nqb] i32 |
//   ratio [B*M] f32 |
//   (backward) qhat [B*M*Hq*D] bf16 | rowstat [B*Hq*M] float2 | colsum [B*Hq*M] f32 |
//   tau [B*Hq*Mp] f32 (Mp = M rounded up to 32) | tstat [B*Hq*M] f32
static size_t rup(size_t x) { return (x + 255) / 256 * 256; }

static size_t cnt_ints(int64_t B, int64_t M, int64_t Hq, int64_t Hkv) {
  return (size_t)(B * Hkv * fwd_sched(B, M, Hq, Hkv).nqb);
}

// rotated queries: the backward's [B, M, Hq, D] or the forward's fragment
// order over 32-query blocks [B, Hq, ceil(M / 32) * 32, D] (the larger)
static size_t qhat_bytes(int64_t B, int64_t M, int64_t Hq, int64_t D) {
  return (size_t)(B * Hq * ((M + 31) / 32 * 32) * D) * 2;
}

// floats of one partial record (8 waves x 64 lanes x NR)
static int64_t rec_floats(int64_t D) { return 8 * ((D / 32) * 16 + 2) * 64; }

void plan_runs(RunRow *runs, int nruns, int64_t Hq, int64_t Hkv, int64_t D) {
  (void)D;
  for (int g0 = 0; g0 < nruns; g0 += kMaxRuns) {
    const int ng = nruns - g0 < kMaxRuns ? nruns - g0 : kMaxRuns;
    const int C = fwd_group_c(runs + g0, ng, Hq, Hkv);
    for (int i = g0; i < g0 + ng; ++i) runs[i].C = C;
  }
  int64_t poff = 0, rec = 0, cnt = 0;
  for (int i = 0; i < nruns; ++i) {
    RunRow &r = runs[i];
    r.poff = (int)poff;
    r.rec0 = (int)rec;
    r.cnt0 = (int)cnt;
    const FwdSched f = fwd_sched_c(r.n, r.M, Hq, Hkv, r.C);
    poff += (int64_t)r.n * ((r.M + 31) / 32 * 32);
    rec += (int64_t)f.nmulti * r.n * Hkv;
    cnt += (int64_t)r.n * Hkv * f.nqb;
  }
}

namespace {
struct RunTotals {
  int64_t T = 0, PT = 0, recs = 0, cnts = 0;
};
// totals over the runs as plan_runs places them
RunTotals run_totals(const RunRow *runs_in, int nruns, int64_t Hq, int64_t Hkv) {
  std::vector<RunRow> runs(runs_in, runs_in + nruns);
  plan_runs(runs.data(), nruns, Hq, Hkv, 0);
  RunTotals t;
  for (const RunRow &r : runs) {
    const FwdSched f = fwd_sched_c(r.n, r.M, Hq, Hkv, r.C);
    t.T += (int64_t)r.n * r.M;
    t.PT += (int64_t)r.n * ((r.M + 31) / 32 * 32);
    t.recs += (int64_t)f.nmulti * r.n * Hkv;
    t.cnts += (int64_t)r.n * Hkv * f.nqb;
  }
  return t;
}
}  // namespace

size_t attn_workspace_bytes_runs(const RunRow *runs, int nruns, int64_t Hq, int64_t Hkv, int64_t D, bool bwd) {
  const RunTotals t = run_totals(runs, nruns, Hq, Hkv);
  size_t n = rup((size_t)(t.T * (D / 2)) * sizeof(float2)) + rup((size_t)(t.T * Hkv * D) * 2) +
             rup((size_t)(Hq * t.T) * sizeof(float)) + rup((size_t)(t.recs * rec_floats(D)) * sizeof(float)) +
             rup((size_t)t.cnts * sizeof(int)) + rup((size_t)t.T * sizeof(float)) +
             rup((size_t)(t.PT * Hq * D) * 2);
  if (bwd)
    n += rup((size_t)(Hq * t.T) * sizeof(float2)) + 2 * rup((size_t)(Hq * t.T) * sizeof(float)) +
         rup((size_t)(t.PT * Hq) * sizeof(float));
  return n;
}

AttnWs carve_attn_ws_runs(void *ws, const RunRow *runs, int nruns, int64_t Hq, int64_t Hkv, int64_t D) {
  const RunTotals t = run_totals(runs, nruns, Hq, Hkv);
  AttnWs w;
  char *p = (char *)ws;
  w.cs = (float2 *)p;
  p += rup((size_t)(t.T * (D / 2)) * sizeof(float2));
  w.khat = (uint16_t *)p;
  p += rup((size_t)(t.T * Hkv * D) * 2);
  w.bias = (float *)p;
  p += rup((size_t)(Hq * t.T) * sizeof(float));
  w.part = (float *)p;
  p += rup((size_t)(t.recs * rec_floats(D)) * sizeof(float));
  w.cnt = (int *)p;
  w.ncnt = (int)t.cnts;
  p += rup((size_t)t.cnts * sizeof(int));
  w.ratio = (float *)p;
  p += rup((size_t)t.T * sizeof(float));
  w.qhat = (uint16_t *)p;
  p += rup((size_t)(t.PT * Hq * D) * 2);
  w.rowstat = (float2 *)p;
  p += rup((size_t)(Hq * t.T) * sizeof(float2));
  w.colsum = (float *)p;
  p += rup((size_t)(Hq * t.T) * sizeof(float));
  w.tau = (float *)p;
  p += rup((size_t)(t.PT * Hq) * sizeof(float));
  w.tstat = (float *)p;
  return w;
}

AttnWs run_view(const AttnWs &w, const RunRow &r, int64_t Hq, int64_t Hkv, int64_t D) {
  AttnWs v = w;
  const int64_t off = r.off, poff = r.poff;
  v.cs = w.cs + off * (D / 2);
  v.khat = w.khat + off * Hkv * D;
  v.bias = w.bias + off * Hq;
  v.part = w.part + (int64_t)r.rec0 * rec_floats(D);
  v.cnt = w.cnt + r.cnt0;
  v.ncnt = (int)cnt_ints(r.n, r.M, Hq, Hkv);
  v.ratio = w.ratio + off;
  v.qhat = w.qhat + poff * Hq * D;
  v.rowstat = w.rowstat + off * Hq;
  v.colsum = w.colsum + off * Hq;
  v.tau = w.tau + poff * Hq;
  v.tstat = w.tstat + off * Hq;
  return v;
}

size_t attn_workspace_bytes(int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D, bool bwd) {
  const RunRow r{0, 0, (int)B, (int)M, 0, 0, 0};
  return attn_workspace_bytes_runs(&r, 1, Hq, Hkv, D, bwd);
}

AttnWs carve_attn_ws(void *ws, int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D) {
  const RunRow r{0, 0, (int)B, (int)M, 0, 0, 0};
  return carve_attn_ws_runs(ws, &r, 1, Hq, Hkv, D);
}

void make_tables(std::vector<Level> &lv, const RunRow *runs, int nruns, int Hkv, std::vector<RunTable> &tabs,
                 std::vector<unsigned> &grids) {
  std::stable_sort(lv.begin(), lv.end(), [](const Level &a, const Level &b) {
    return a.cost != b.cost ? a.cost > b.cost : a.run < b.run;
  });
  tabs.clear();
  grids.clear();
  RunTable t;
  int ne = 0, cur_run = -1, blk0 = 0, last = 0, len = 0;
  bool desc = false;
  unsigned wg = 0;
  auto flush = [&]() {
    for (int i = ne; i < kMaxEnt; ++i) {
      t.start[i] = INT_MAX;
      t.code[i] = 0;
    }
    for (int i = 0; i < kMaxRuns; ++i) t.run[i] = i < nruns ? runs[i] : RunRow{0, 0, 0, 0, 0, 0, 0};
    tabs.push_back(t);
    grids.push_back(wg);
    ne = 0;
    wg = 0;
    cur_run = -1;
  };
  for (const Level &L : lv) {
    const unsigned nbh = (unsigned)(runs[L.run].n * Hkv);
    bool merge = ne > 0 && L.run == cur_run;
    if (merge) {
      if (len == 1 && (L.blk == last + 1 || L.blk == last - 1)) desc = L.blk < last;
      else merge = len > 1 && L.blk == last + (desc ? -1 : 1);
    }
    if (!merge) {
      if (ne == kMaxEnt) flush();
      t.start[ne++] = (int)wg;
      cur_run = L.run;
      blk0 = L.blk;
      len = 0;
      desc = false;
    }
    last = L.blk;
    ++len;
    t.code[ne - 1] = L.run | blk0 << 8 | (desc ? 1 : 0) << 30;
    wg += nbh;
  }
  if (ne) flush();
}

bool make_fwd_tables(const RunRow *runs, int nruns, int64_t Hq, int64_t Hkv, std::vector<RunTable> &tabs,
                     std::vector<unsigned> &grids) {
  struct FL {
    int run, blk, cost;
    bool split, top;
    unsigned wgs;
  };
  std::vector<FL> lv;
  for (int i = 0; i < nruns; ++i) {
    const RunRow &r = runs[i];
    const FwdSched f = fwd_sched_c(r.n, r.M, Hq, Hkv, r.C);
    if (f.nqb == 0 || r.n <= 0) return false;
    for (int qb = f.nqb - 1; qb >= 0; --qb) {
      const int nt = fwd_ntiles(qb, f.BQ, r.M), np = fwd_npieces(nt, f.C);
      lv.push_back(FL{i, qb, np > 1 ? f.C : nt, np > 1, qb == f.nqb - 1, (unsigned)(np * r.n * Hkv)});
    }
  }
  // split blocks first, each run's from the top; then the unsplit blocks
  // longest first, equal lengths by block (down), then run
  std::stable_sort(lv.begin(), lv.end(), [](const FL &a, const FL &b) {
    if (a.split != b.split) return a.split;
    if (a.split) return a.run != b.run ? a.run < b.run : a.blk > b.blk;
    if (a.cost != b.cost) return a.cost > b.cost;
    return a.blk != b.blk ? a.blk > b.blk : a.run < b.run;
  });
  tabs.clear();
  grids.clear();
  RunTable t;
  int ne = 0, run0 = 0, blk0 = 0, last_run = -1, last_blk = 0, len = 0;
  bool across = false, unsplit = false;
  uint64_t wg = 0;
  auto flush = [&]() {
    for (int i = ne; i < kMaxEnt; ++i) {
      t.start[i] = INT_MAX;
      t.code[i] = 0;
    }
    for (int i = 0; i < kMaxRuns; ++i) t.run[i] = i < nruns ? runs[i] : RunRow{0, 0, 0, 0, 0, 0, 0};
    tabs.push_back(t);
    grids.push_back((unsigned)wg);
    ne = 0;
    wg = 0;
    last_run = -1;
  };
  for (const FL &L : lv) {
    const bool down = L.run == last_run && L.blk == last_blk - 1;
    const bool side = unsplit && !L.split && L.blk == last_blk && L.run == last_run + 1;
    bool merge = ne > 0 && last_run >= 0 && (len == 1 ? down || side : across ? side : down);
    if (merge && len == 1) across = side;
    if (!merge) {
      if (L.split && !L.top) return false;  // a run's split blocks are numbered from its top block
      if (ne == kMaxEnt) flush();
      t.start[ne++] = (int)wg;
      run0 = L.run;
      blk0 = L.blk;
      len = 0;
      across = false;
      unsplit = true;
    }
    unsplit = unsplit && !L.split;
    last_run = L.run;
    last_blk = L.blk;
    ++len;
    t.code[ne - 1] = run0 | blk0 << 8 | (across ? 1 : 0) << 30;
    wg += L.wgs;
    if (wg > (uint64_t)INT_MAX) return false;
  }
  if (ne) flush();
  return true;
}

hipError_t launch_attn_prep(const void *k, const float *g, const float *gamma, const int32_t *pos, double theta,
                            int B, int M, int Hq, int Hkv, int D, bool rot_k, bool with_bias, bool with_ratio,
                            bool g_per_head, const AttnWs &w, hipStream_t s, const void *q) {
  if ((int64_t)B * M == 0) return hipSuccess;
  InvFreq inv;
  for (int i = 0; i < 64; ++i) inv.v[i] = i < D / 2 ? pow(theta, -2.0 * (double)i / (double)D) : 0.0;
  const int64_t rows = (int64_t)B * M;
  const int64_t R = 256 / (D / 2), nwg_rows = (rows + R - 1) / R, nwg_cnt = ((int64_t)w.ncnt + 255) / 256;
  hipLaunchKernelGGL(attn_prep_kernel<false>, dim3((unsigned)(nwg_rows > nwg_cnt ? nwg_rows : nwg_cnt)), dim3(256), 0,
                     s, (rot_k && pos) ? (const uint16_t *)k : nullptr, g, gamma, pos, inv, rows, M, Hq, Hkv, D, w.cs,
                     (rot_k && pos) ? w.khat : nullptr, with_bias ? w.bias : nullptr, with_ratio ? w.ratio : nullptr,
                     w.cnt, with_bias ? w.ncnt : 0, (int)g_per_head, (const uint16_t *)q, q ? w.qhat : nullptr,
                     (M + 31) / 32, PrepRuns{});
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                           const int32_t *pos, double theta, float tau, const float *sigma, int B, int M, int Hq,
                           int Hkv, int D, bool bf16, bool g_per_head, void *o, float *lse, void *o_lo,
                           const AttnWs &w, hipStream_t s) {
  if ((int64_t)B * M == 0) return hipSuccess;
  hipError_t e = launch_attn_prep(k, g, gamma, pos, theta, B, M, Hq, Hkv, D, bf16, bf16, sigma != nullptr, g_per_head,
                                  w, s, bf16 ? q : nullptr);
  if (e != hipSuccess) return e;
  const float2 *cs = pos ? w.cs : nullptr;
  const double c = 1.0 / (sqrt((double)D) * (double)tau);
  if (bf16) {
    const FwdSched f = fwd_sched(B, M, Hq, Hkv);
    const dim3 grid((unsigned)(f.npieces * B * Hkv));
    const float c2 = (float)(c * 1.4426950408889634);
    const uint16_t *kh = pos ? w.khat : (const uint16_t *)k;
    auto kern = D == 128 ? (sigma ? attn_fwd_bf16_kernel<128, true, false> : attn_fwd_bf16_kernel<128, false, false>)
                         : (sigma ? attn_fwd_bf16_kernel<64, true, false> : attn_fwd_bf16_kernel<64, false, false>);
    hipLaunchKernelGGL(kern, grid, dim3(512), 0, s, (const uint16_t *)w.qhat, (M + 31) / 32, kh, (const uint16_t *)v,
                       w.bias, c2, sigma, w.ratio, B, M, Hq, Hkv, Hq / Hkv, f.BQ, f.nqb, f.C, w.part, w.cnt,
                       (uint16_t *)o, lse, (uint16_t *)o_lo, NoTable{});
  } else {
    const int64_t rows = (int64_t)B * M * Hq;
    hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, (const float *)q,
                       (const float *)k, (const float *)v, g, gamma, cs, (float)c, sigma, w.ratio, B, M, Hq, Hkv,
                       D, (int)g_per_head, (float *)o, lse);
  }
  return hipGetLastError();
}

hipError_t launch_attn_prep_runs(const void *k, const float *g, const float *gamma, const int32_t *pos, double theta,
                                 const RunRow *runs, int nruns, int Hq, int Hkv, int D, bool with_ratio,
                                 const AttnWs &w, hipStream_t s, const void *q) {
  if (nruns < 1 || nruns > kMaxRuns) return hipErrorInvalidValue;
  InvFreq inv;
  for (int i = 0; i < 64; ++i) inv.v[i] = i < D / 2 ? pow(theta, -2.0 * (double)i / (double)D) : 0.0;
  const int BQ = 256 / (Hq / Hkv);
  PrepRuns pr{};
  pr.nr = nruns;
  int64_t rows = 0, ncnt = 0;
  for (int i = 0; i < nruns; ++i) {
    pr.off[i] = runs[i].off - runs[0].off;
    pr.poff[i] = runs[i].poff - runs[0].poff;
    pr.M[i] = runs[i].M;
    rows += (int64_t)runs[i].n * runs[i].M;
    ncnt += (int64_t)runs[i].n * Hkv * ((runs[i].M + BQ - 1) / BQ);
  }
  if (rows == 0) return hipSuccess;
  const int64_t off0 = runs[0].off, R = 256 / (D / 2), nwg_rows = (rows + R - 1) / R, nwg_cnt = (ncnt + 255) / 256;
  hipLaunchKernelGGL(attn_prep_kernel<true>, dim3((unsigned)(nwg_rows > nwg_cnt ? nwg_rows : nwg_cnt)), dim3(256), 0,
                     s, pos ? (const uint16_t *)k + off0 * Hkv * D : nullptr, g + off0, gamma,
                     pos ? pos + off0 : nullptr, inv, rows, 0, Hq, Hkv, D, w.cs + off0 * (D / 2),
                     pos ? w.khat + off0 * Hkv * D : nullptr, w.bias + off0 * Hq, with_ratio ? w.ratio + off0 : nullptr,
                     w.cnt + runs[0].cnt0, (int)ncnt, 0, q ? (const uint16_t *)q + off0 * Hq * D : nullptr,
                     q ? w.qhat + (int64_t)runs[0].poff * Hq * D : nullptr, 0, pr);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_runs(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                                const int32_t *pos, double theta, float tau, const float *sigma, const RunRow *runs,
                                int nruns, int Hq, int Hkv, int D, void *o, float *lse, void *o_lo, const AttnWs &w,
                                hipStream_t s) {
  if (D != 64 && D != 128) return hipErrorInvalidValue;
  const double c = 1.0 / (sqrt((double)D) * (double)tau);
  const float c2 = (float)(c * 1.4426950408889634);
  const int G = Hq / Hkv, BQ = 256 / G;
  auto kern = D == 128 ? (sigma ? attn_fwd_bf16_kernel<128, true, true> : attn_fwd_bf16_kernel<128, false, true>)
                       : (sigma ? attn_fwd_bf16_kernel<64, true, true> : attn_fwd_bf16_kernel<64, false, true>);
  std::vector<RunTable> tabs;
  std::vector<unsigned> grids;
  for (int g0 = 0; g0 < nruns; g0 += kMaxRuns) {
    const int ng = nruns - g0 < kMaxRuns ? nruns - g0 : kMaxRuns;
    const RunRow *gr = runs + g0;
    hipError_t e = launch_attn_prep_runs(k, g, gamma, pos, theta, gr, ng, Hq, Hkv, D, sigma != nullptr, w, s, q);
    if (e != hipSuccess) return e;
    if (!make_fwd_tables(gr, ng, Hq, Hkv, tabs, grids)) return hipErrorInvalidValue;
    const uint16_t *kh = pos ? w.khat : (const uint16_t *)k;
    for (size_t t = 0; t < tabs.size(); ++t) {
      hipLaunchKernelGGL(kern, dim3(grids[t]), dim3(512), 0, s, (const uint16_t *)w.qhat, 0, kh, (const uint16_t *)v,
                         w.bias, c2, sigma, w.ratio, 0, 0, Hq, Hkv, G, BQ, 0, 0, w.part, w.cnt, (uint16_t *)o, lse,
                         (uint16_t *)o_lo, tabs[t]);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace tg
