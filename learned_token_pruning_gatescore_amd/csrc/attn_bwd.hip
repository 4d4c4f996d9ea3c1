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
// bf16 path: prep (rotated keys, log2-gate bias), then two matrix-core
// kernels and two small reductions, no atomics (bitwise deterministic):
//   1. query-outer: per (query, head) column, pass A forms D_i from fp32 P and
//      fp32 dP (not from the rounded output), pass B forms dS and accumulates
//      dQ^T = K^T dS^T; writes dq, D_i and the rotated queries;
//   2. key-outer: per key, dV^T = dO^T P and dK^T = Q^T dS over every head of
//      the group and every query at or after the key; writes dk, dv and the
//      column sums of dS per head;
//   3. dg (per token, fixed head order) and dgamma (one work-group per head,
//      fixed-shape tree).
//
// Both matrix-core kernels run 8 waves per work-group, two per SIMD, so that
// one wave's products overlap the other's vector work.  32-row tiles of the
// streamed operand (keys for kernel 1, queries for kernel 2) are shared by
// all 8 waves: direct global->LDS loads, two tiles ahead, one barrier per
// tile.  The per-row terms of the exponent and of dS (-lse / c and -D_i)
// enter the products as one extra 16-deep step whose operand holds the value
// split into three bf16 parts, so the vector work per logit is one fma, one
// exp2 and the product with dP.
#include "tg_common.h"
#include "tg_attn.h"
#include "tg_tile.h"

namespace tg {

// ---------------------------------------------------------------------------
// 1. query-outer: D_i, dq and the rotated queries.
//
// Work-group = 8 waves = 256 columns, a column being a (query, head) pair of
// the GQA group (BQ = 256 / G queries x G heads); wave w owns columns
// 32w .. 32w+31 (one head).  It computes S^T = K Q^T and dP^T = V dO^T (keys
// on the MFMA rows: 16 keys of one column per lane), P and dS in registers,
// and dQ^T += K^T dS^T with K^T read through the transposing LDS read.  A
// work-group takes one query block of one run (RunTable): the blocks go out
// longest first, so the dispatcher balances them over the compute units.
// ---------------------------------------------------------------------------
template <int D, bool TEMP>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kh, const uint16_t *__restrict__ v,
    const float *__restrict__ bias, const float2 *__restrict__ cs, const float *__restrict__ lse,
    const uint16_t *__restrict__ dout, float c, float c2, const float *__restrict__ sigma,
    const float *__restrict__ ratio, int Hq, int Hkv, int G, int BQ, float *__restrict__ dq,
    uint16_t *__restrict__ qhat, float2 *__restrict__ rowstat, float *__restrict__ tau, float *__restrict__ tstat,
    const uint16_t *__restrict__ o, const uint16_t *__restrict__ o_lo, const RunTable rt) {
  using T = BTile<D>;
  constexpr int NKS = T::NKS, NDB = T::NDB, HALF = D / 2;
  constexpr int NIW = 2 * T::NI / AB_NW;  // K and V direct loads per wave per tile (+ wave 0's bias load)
  __shared__ __attribute__((aligned(1024))) uint16_t sK[4 * T::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[4 * T::TILE];
  __shared__ __attribute__((aligned(1024))) float sBias[4][8][AB_T];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hl = lane >> 5;
  const Unit u = unit_of(rt, blockIdx.x, Hkv);
  const int M = rt.run[u.run].M;
  {  // the run's tensors and workspace
    const int64_t t0 = rt.run[u.run].off, p0 = rt.run[u.run].poff;
    q += t0 * Hq * D;
    kh += t0 * Hkv * D;
    v += t0 * Hkv * D;
    bias += t0 * Hq;
    if (cs) cs += t0 * HALF;
    lse += t0 * Hq;
    dout += t0 * Hq * D;
    if (o) {
      o += t0 * Hq * D;
      o_lo += t0 * Hq * D;
    }
    if (TEMP) ratio += t0;
    dq += t0 * Hq * D;
    qhat += p0 * Hq * D;
    rowstat += t0 * Hq;
    tau += p0 * Hq;
    tstat += t0 * Hq;
  }
  const int bh = u.bh;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int64_t bM = (int64_t)b * M;
  const uint32_t rsb = (uint32_t)(Hkv * D * 2);  // bytes between consecutive keys
  const uint32_t kv_bytes = (uint32_t)(M - 1) * rsb + D * 2;
  const i32x4 rK = buffer_rsrc(kh + (bM * Hkv + kvh) * D, kv_bytes);
  const i32x4 rV = buffer_rsrc(v + (bM * Hkv + kvh) * D, kv_bytes);
  const i32x4 rB = buffer_rsrc(bias + ((int64_t)b * Hq + (int64_t)kvh * G) * M, (uint32_t)(G * M * 4));

  BFrag<D> fr;
  fr.init(lane);
  // direct load j = wave + 8 n of the tile's 2 NI (K first, then V)
  uint32_t dgo[NIW], dlo[NIW];
  bool isv[NIW];
#pragma unroll
  for (int n = 0; n < NIW; ++n) {
    const int j = wave + AB_NW * n;
    isv[n] = j >= T::NI;
    dgo[n] = T::goff(j % T::NI, lane, rsb);
    dlo[n] = 1024u * (uint32_t)(j % T::NI);
  }
  // bias: wave 0 loads the G rows of the tile (8 lanes x 16 bytes per head)
  const bool breal = wave == 0 && (lane >> 3) < G;
  const uint32_t bvo = (uint32_t)((((lane >> 3) * M) + 4 * (lane & 7)) * 4);
  const u32x4 kones = ones3(hl);

  auto slot = [](int t) __attribute__((always_inline)) { return t & 3; };
  auto issue = [&](int t, int nt) __attribute__((always_inline)) {
    const bool live = t < nt;
    const uint32_t toff = (uint32_t)(t * AB_T) * rsb;
    const uint32_t so = 2u * (uint32_t)(slot(t) * T::TILE);
#pragma unroll
    for (int n = 0; n < NIW; ++n)
      dma_b128(isv[n] ? rV : rK, (isv[n] ? lds_addr(sV) : lds_addr(sK)) + so + dlo[n],
               live ? dgo[n] + toff : 0x80000000u, 0u);
    if (wave == 0)
      dma_b128(rB, lds_addr(&sBias[slot(t)][0][0]), live && breal ? bvo + (uint32_t)(t * AB_T * 4) : 0x80000000u,
               0u);
  };
  // barrier of tile t: its loads landed (this wave's loads of tile t + 1 may still be in flight)
  auto sync_tile = [&]() __attribute__((always_inline)) {
    if (wave == 0) sync_vm<NIW + 1>();
    else sync_vm<NIW>();
  };

  {
    const int qb = u.blk;
    const int q0 = qb * BQ;
    const int qe = q0 + BQ < M ? q0 + BQ : M;
    const int nt = (qe + AB_T - 1) / AB_T;
    const int tdiag = q0 / AB_T;  // tiles from here on hold keys past some query of the block
    const int hloc = (AB_T * wave) / BQ;
    const int h = kvh * G + hloc;
    const int qi = q0 + (AB_T * wave) % BQ + l32;
    const bool vq = qi < M;

    issue(0, nt);
    issue(1, nt);

    // temperature of the column (1 without it, and past M): logits t Z, with
    // t >= 1e-30 so that a key with bias -inf stays at -inf
    float tq = 1.f, rq = 0.f;
    if (TEMP && vq) {
      rq = ratio[bM + qi];
      tq = fmaxf(softplus_f(sigma[h]) * rq, 1e-30f);
    }

    // Q and dO fragments (MFMA B operands): lane holds [qi, h, 16 ks + 8 hl .. +8]
    u32x4 qf[NKS], of[NKS];
    const int64_t roff = ((bM + (vq ? qi : 0)) * Hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[ks] = vq ? *(const u32x4 *)(q + roff + 16 * ks + 8 * hl) : u32x4{0u, 0u, 0u, 0u};
      of[ks] = vq ? *(const u32x4 *)(dout + roff + 16 * ks + 8 * hl) : u32x4{0u, 0u, 0u, 0u};
    }
    const float lrow = vq ? lse[((int64_t)b * Hq + h) * M + qi] : -INFINITY;
    // With the forward's output o and its rounding residual o_lo: D_o = dO_i . (o_i + o_lo_i)
    // stands for D_i = sum_j P_ij dP_ij (= dO_i . O_i) in pass B's dS, without pass A.  The
    // forward's O carries P's bf16 rounding, so D_o is off by about 2^-9 relative; pass B also
    // sums the row of its dS, sum_j P_ij (dP_ij - D_o) = D_i - D_o (sum_j P_ij = 1), so the
    // exact D_i goes to the key-outer kernel (dk, dv, the column sums, dg) and to the
    // temperature's term; only dq keeps D_o (an error of c (D_i - D_o) sum_j P_ij k_j).
    // (every load issued before the first use: roff names a valid row for every lane, and a
    // column past M contributes 0)
    float dso = 0.f;
    if (o) {
      u32x4 oh[NKS], ol[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        oh[ks] = *(const u32x4 *)(o + roff + 16 * ks + 8 * hl);
        ol[ks] = *(const u32x4 *)(o_lo + roff + 16 * ks + 8 * hl);
      }
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          dso += bf16_lo(of[ks][w]) * (bf16_lo(oh[ks][w]) + bf16_lo(ol[ks][w])) +
                 bf16_hi(of[ks][w]) * (bf16_hi(oh[ks][w]) + bf16_hi(ol[ks][w]));
      if (!vq) dso = 0.f;
      dso += __shfl_xor(dso, 32);
    }
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      settle(qf[ks]);
      settle(of[ks]);
    }
    settle(lrow);
    settle(tq);
    settle(rq);
    if (cs) {
      // the row's angles in one batch of loads (in four, one per step pair, they cost a memory
      // round trip each)
      const f32x4 *crow = (const f32x4 *)(cs + (bM + (vq ? qi : 0)) * HALF);
      f32x4 ang[NKS / 2][4];
#pragma unroll
      for (int ks = 0; ks < NKS / 2; ++ks)
#pragma unroll
        for (int w = 0; w < 4; ++w) ang[ks][w] = crow[(16 * ks + 8 * hl) / 2 + w];
#pragma unroll
      for (int ks = 0; ks < NKS / 2; ++ks) {
        u32x4 &x = qf[ks], &y = qf[ks + NKS / 2];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x4 t = ang[ks][w];  // pairs 2w, 2w+1: (cos, sin, cos, sin)
          const float x0 = bf16_lo(x[w]), x1 = bf16_hi(x[w]);
          const float y0 = bf16_lo(y[w]), y1 = bf16_hi(y[w]);
          x[w] = pack_bf16x2(x0 * t[0] - y0 * t[1], x1 * t[2] - y1 * t[3]);
          y[w] = pack_bf16x2(y0 * t[0] + x0 * t[1], y1 * t[2] + x1 * t[3]);
        }
      }
      if (vq) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) *(u32x4 *)(qhat + roff + 16 * ks + 8 * hl) = qf[ks];
      }
    }
    // exponent of P in log2 units: t ((S + la) c2 + bias) with la = -lse / (c t)
    // (dead rows and columns past M: -1e30, P = 0)
    const float la = lrow == -INFINITY ? -1e30f : -lrow / (TEMP ? c * tq : c);
    const u32x4 laug = aug3(la, hl);

    // S^T and dP^T products over the head dim, fragments read two steps ahead
    // (sched_barrier keeps the reads from being hoisted all at once)
    auto sdp = [&](const uint16_t *K, const uint16_t *V, f32x16 &s, f32x16 &dp) __attribute__((always_inline)) {
      u32x4 ka[NKS], va[NKS];
      ka[0] = fr.rows(K, 0);
      va[0] = fr.rows(V, 0);
      ka[1] = fr.rows(K, 1);
      va[1] = fr.rows(V, 1);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (ks + 2 < NKS) {
          ka[ks + 2] = fr.rows(K, ks + 2);
          va[ks + 2] = fr.rows(V, ks + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        s = mfma32(ka[ks], qf[ks], s);
        dp = mfma32(va[ks], of[ks], dp);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // acc[db] += (tile^T)[db] . x over the tile rows, transposing reads two steps ahead
    auto trprod = [&](const uint16_t *X, const u32x4(&x)[2], f32x16(&a)[NDB]) __attribute__((always_inline)) {
      u32x4 f[2 * NDB];
      f[0] = fr.tr(X, 0, 0);
      f[1] = fr.tr(X, 0, 1);
#pragma unroll
      for (int i = 0; i < 2 * NDB; ++i) {
        if (i + 2 < 2 * NDB) f[i + 2] = fr.tr(X, (i + 2) / NDB, (i + 2) % NDB);
        __builtin_amdgcn_sched_barrier(0);
        a[i % NDB] = mfma32(f[i], x[i / NDB], a[i % NDB]);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    const int tu = tdiag < nt ? tdiag : nt;  // unmasked tiles first, then the masked ones
    auto tile = [&](int t, f32x16 &s, f32x16 &dp, const u32x4 &dinit, bool with_d) __attribute__((always_inline)) {
      s = mfma32(kones, laug, f32x16{});
      dp = with_d ? mfma32(kones, dinit, f32x16{}) : f32x16{};
      sdp(sK + slot(t) * T::TILE, sV + slot(t) * T::TILE, s, dp);
    };

    // pass A (without o): D_i = sum_j P_ij dP_ij
    float dsa[4] = {0.f, 0.f, 0.f, 0.f};
    auto valu_a = [&](int t, const f32x16 &s, const f32x16 &dp, bool masked) __attribute__((always_inline)) {
      const float *bi = &sBias[slot(t)][hloc][4 * hl];
      const int lim = qi - t * AB_T;  // keys (within the tile) past the query are masked
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float2 bv = *(const float2 *)(bi + 8 * (j >> 1) + 2 * (j & 1));
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * j + e;
          float x = __builtin_fmaf(s[r], c2, e ? bv.y : bv.x);
          if (TEMP) x *= tq;
          if (masked && acc_row(r, hl) > lim) x = -INFINITY;
          dsa[r & 3] = __builtin_fmaf(fast_exp2(x), dp[r], dsa[r & 3]);
        }
      }
    };
    float dsum = dso;  // the D_i of pass B's dS
    if (!o) {
      f32x16 s, dp;
      for (int t = 0; t < tu; ++t) {
        sync_tile();
        issue(t + 2, nt);
        tile(t, s, dp, kones, false);
        valu_a(t, s, dp, false);
      }
      for (int t = tu; t < nt; ++t) {
        sync_tile();
        issue(t + 2, nt);
        tile(t, s, dp, kones, false);
        valu_a(t, s, dp, true);
      }
      sync_vm<0>();  // the tail's zero-fill loads landed, every wave done with the ring
      dsum = (dsa[0] + dsa[1]) + (dsa[2] + dsa[3]);
      dsum += __shfl_xor(dsum, 32);
      // pass B's first tiles (with o, the ones issued above serve it)
      issue(0, nt);
      issue(1, nt);
    }
    const u32x4 daug = aug3(-dsum, hl);

    // pass B: dS and dQ^T
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    // dS of tile t as the B operand of the dQ^T product: step hf, slot e = register 8 hf + e.
    // With the temperature, dt = sum_j dS_ij Z_ij: Z_ij is y / log2(e) plus a
    // per-row constant (the exponent's shift), and sum_j dS_ij = 0, so the
    // shifted y = (S + la) c2 + bias serves (-inf clamped: there dS = 0).
    float dty[4] = {0.f, 0.f, 0.f, 0.f};
    float drs = 0.f, dpy = 0.f;  // with o: sum_j dS_ij and (temperature) sum_j P_ij y_ij
    auto valu_b = [&](int t, const f32x16 &s, const f32x16 &dp, bool masked, u32x4(&dsf)[2]) __attribute__((always_inline)) {
      const float *bi = &sBias[slot(t)][hloc][4 * hl];
      const int lim = qi - t * AB_T;
      float ds[16];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float2 bv = *(const float2 *)(bi + 8 * (j >> 1) + 2 * (j & 1));
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * j + e;
          const float y = __builtin_fmaf(s[r], c2, e ? bv.y : bv.x);
          float x = TEMP ? y * tq : y;
          if (masked && acc_row(r, hl) > lim) x = -INFINITY;
          const float pr = fast_exp2(x);
          ds[r] = pr * dp[r];
          if (TEMP) dty[r & 3] = __builtin_fmaf(ds[r], fmaxf(y, -1e30f), dty[r & 3]);
          if (o) {
            drs += ds[r];
            if (TEMP) dpy = __builtin_fmaf(pr, fmaxf(y, -1e30f), dpy);
          }
        }
      }
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int w = 0; w < 4; ++w) dsf[hf][w] = pack_bf16x2(ds[8 * hf + 2 * w], ds[8 * hf + 2 * w + 1]);
    };
    {
      f32x16 s, dp;
      u32x4 dsf[2];
      for (int t = 0; t < tu; ++t) {
        sync_tile();
        issue(t + 2, nt);
        tile(t, s, dp, daug, true);
        valu_b(t, s, dp, false, dsf);
        trprod(sK + slot(t) * T::TILE, dsf, acc);
      }
      for (int t = tu; t < nt; ++t) {
        sync_tile();
        issue(t + 2, nt);
        tile(t, s, dp, daug, true);
        valu_b(t, s, dp, true, dsf);
        trprod(sK + slot(t) * T::TILE, dsf, acc);
      }
    }
    sync_vm<0>();
    float dex = dsum;  // the exact D_i
    if (o) {
      dex += drs + __shfl_xor(drs, 32);
      dpy += __shfl_xor(dpy, 32);
    }
    if (vq && hl == 0) rowstat[((int64_t)b * Hq + h) * M + qi] = make_float2(la, dex);
    if (TEMP) {  // the temperature for the key-outer kernel, and ratio_i dL/dt_ih
      float dts = (dty[0] + dty[1]) + (dty[2] + dty[3]);
      dts += __shfl_xor(dts, 32);
      // with D_o in dS: sum_j dS_ij y_ij with the exact D_i (the shift of y cancels only then)
      if (o) dts -= (dex - dsum) * dpy;
      const int64_t Mp = (M + AB_T - 1) / AB_T * AB_T;
      if (hl == 0 && qi < Mp) tau[((int64_t)b * Hq + h) * Mp + qi] = tq;
      if (hl == 0 && vq) tstat[((int64_t)b * Hq + h) * M + qi] = rq * dts * kLn2;
    }

    // dq = c t R(-phi) dq^ ; lane holds rows d = 32 db + acc_row(r, hl) of its column
    // (the angles of all its rows loaded at once, then the products)
    const float cq = TEMP ? c * tq : c;
    if (vq) {
      float *drow = dq + ((bM + qi) * Hq + h) * D;
      f32x4 ca[NDB / 2][4][2];
#pragma unroll
      for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          ca[db][g4][0] = ca[db][g4][1] = f32x4{1.f, 0.f, 1.f, 0.f};
          if (cs) {
            const f32x4 *cp = (const f32x4 *)(cs + (bM + qi) * HALF + db * 32 + 8 * g4 + 4 * hl);
            ca[db][g4][0] = cp[0];
            ca[db][g4][1] = cp[1];
          }
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = db * 32 + 8 * g4 + 4 * hl;
          float xo[4], yo[4];
          const f32x4 t0 = ca[db][g4][0], t1 = ca[db][g4][1];
          const float cv[4] = {t0[0], t0[2], t1[0], t1[2]}, sv[4] = {t0[1], t0[3], t1[1], t1[3]};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = acc[db][4 * g4 + e] * cq, y = acc[db + NDB / 2][4 * g4 + e] * cq;
            xo[e] = x * cv[e] + y * sv[e];
            yo[e] = y * cv[e] - x * sv[e];
          }
          *(f32x4 *)(drow + d) = f32x4{xo[0], xo[1], xo[2], xo[3]};
          *(f32x4 *)(drow + HALF + d) = f32x4{yo[0], yo[1], yo[2], yo[3]};
        }
    }
  }
}

// ---------------------------------------------------------------------------
// 2. key-outer: dk, dv and the column sums of dS.
//
// Work-group = 8 waves over a block of 128 keys (32 per wave) and every
// (head of the group, 32-query tile at or after the block) item, the items
// streamed through LDS in order.  The waves split the work by role, so that
// each fits in the registers of two waves per SIMD:
//   role 0 (waves 0-3, K^ of its keys in registers): S = Q K^T (queries on
//     the MFMA rows, keys on the columns: one key per lane), P, dV^T += dO^T P;
//     hands P (fp32) to its partner through LDS;
//   role 1 (waves 4-7, V of the same keys): one item behind, dP = dO V^T,
//     dS = P (dP - D) and the column sums; the product dK^T += Q^T dS of an
//     item runs one iteration later still, first in the iteration, so that
//     the two waves of a SIMD are not both in their products at once.
// Items live in a ring of 5 LDS slots (two in flight, three in use).  A
// work-group takes one key block of one run (RunTable), longest first.
// ---------------------------------------------------------------------------
template <int D, bool TEMP>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_bf16_kernel(
    const uint16_t *__restrict__ qh, const uint16_t *__restrict__ dout, const float2 *__restrict__ rowstat,
    const float *__restrict__ tau, const uint16_t *__restrict__ kh, const uint16_t *__restrict__ v,
    const float *__restrict__ bias, const float2 *__restrict__ cs, float c, float c2, int Hq, int Hkv, int G,
    int qh_padded, float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ colsum, const RunTable rt) {
  using T = BTile<D>;
  constexpr int NKS = T::NKS, NDB = T::NDB, HALF = D / 2;
  constexpr int NIW = 2 * T::NI / 4;  // Q and dO direct loads per role-0 wave per item
  constexpr int KB = 4 * AB_T;            // keys per block
  __shared__ __attribute__((aligned(1024))) uint16_t sQ[5 * T::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sO[5 * T::TILE];
  __shared__ __attribute__((aligned(1024))) float2 sRS[5][AB_T];
  __shared__ __attribute__((aligned(256))) float sT[TEMP ? 5 : 1][64];  // [slot][row] t (rows 32..63: fill)
  __shared__ __attribute__((aligned(1024))) f32x4 sP[2][4][4][64];  // [item parity][wave][r / 4][lane]
  __shared__ __attribute__((aligned(1024))) float sCol[8][KB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int role = wave >> 2, sub = wave & 3;
  const int l32 = lane & 31, hl = lane >> 5;
  const Unit u = unit_of(rt, blockIdx.x, Hkv);
  const int M = rt.run[u.run].M;
  {  // the run's tensors and workspace (qh: the rotated queries of the workspace,
     // placed by padded tokens, or the caller's q)
    const int64_t t0 = rt.run[u.run].off, p0 = rt.run[u.run].poff;
    qh += (qh_padded ? p0 : t0) * Hq * D;
    dout += t0 * Hq * D;
    rowstat += t0 * Hq;
    tau += p0 * Hq;
    kh += t0 * Hkv * D;
    v += t0 * Hkv * D;
    bias += t0 * Hq;
    if (cs) cs += t0 * HALF;
    dk += t0 * Hkv * D;
    dv += t0 * Hkv * D;
    colsum += t0 * Hq;
  }
  const int bh = u.bh;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int64_t bM = (int64_t)b * M;
  const uint32_t rsq = (uint32_t)(Hq * D * 2);  // bytes between consecutive queries of one head
  const uint32_t q_bytes = (uint32_t)(M - 1) * rsq + D * 2;
  const int ntq = (M + AB_T - 1) / AB_T;
  const int64_t Mp = (int64_t)ntq * AB_T;  // row stride of the temperatures

  BFrag<D> fr;
  fr.init(lane);
  uint32_t dgo[NIW], dlo[NIW];
  bool iso[NIW];
#pragma unroll
  for (int n = 0; n < NIW; ++n) {
    const int j = sub + 4 * n;
    iso[n] = j >= T::NI;
    dgo[n] = T::goff(j % T::NI, lane, rsq);
    dlo[n] = 1024u * (uint32_t)(j % T::NI);
  }
  const u32x4 kones = ones3(hl);
  // acc[db] += (tile^T)[db] . x over the tile rows, transposing reads two steps ahead
  auto trprod = [&](const uint16_t *X, const u32x4(&x)[2], f32x16(&a)[NDB]) __attribute__((always_inline)) {
    u32x4 f[2 * NDB];
    f[0] = fr.tr(X, 0, 0);
    f[1] = fr.tr(X, 0, 1);
#pragma unroll
    for (int i = 0; i < 2 * NDB; ++i) {
      if (i + 2 < 2 * NDB) f[i + 2] = fr.tr(X, (i + 2) / NDB, (i + 2) % NDB);
      __builtin_amdgcn_sched_barrier(0);
      a[i % NDB] = mfma32(f[i], x[i / NDB], a[i % NDB]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  {
    const int kb = u.blk;
    const int k0 = kb * KB;
    const int tq0 = k0 / AB_T;
    const int ntl = ntq - tq0;  // query tiles per head
    const int nit = G * ntl;    // items
    const int kw0 = k0 + AB_T * sub;
    const int key = kw0 + l32;
    const bool vk = key < M;

    // item it: head it / ntl of the group, query tile tq0 + it % ntl; ring slot it % 5.
    // Only the role-0 waves load (role 1, on the critical path, never queues behind
    // the direct loads): the Q and dO tiles split over the four of them, the row
    // statistics from wave 0, the temperatures from wave 1.  A load past the end
    // (an item >= nit) reads zeros, so every item has the same loads per wave.
    auto issue = [&](int it) __attribute__((always_inline)) {
      const bool live = it < nit;
      const int hh = live ? it / ntl : 0;
      const int tq = live ? tq0 + it - hh * ntl : 0;
      const int64_t h = (int64_t)kvh * G + hh;
      const i32x4 rQ = buffer_rsrc(qh + (bM * Hq + h) * D, q_bytes);
      const i32x4 rO = buffer_rsrc(dout + (bM * Hq + h) * D, q_bytes);
      const i32x4 rR = buffer_rsrc(rowstat + ((int64_t)b * Hq + h) * M, (uint32_t)M * 8u);
      const uint32_t toff = (uint32_t)(tq * AB_T) * rsq;
      const uint32_t so = 2u * (uint32_t)((it % 5) * T::TILE);
#pragma unroll
      for (int n = 0; n < NIW; ++n)
        dma_b128(iso[n] ? rO : rQ, (iso[n] ? lds_addr(sO) : lds_addr(sQ)) + so + dlo[n],
                 live ? dgo[n] + toff : 0x80000000u, 0u);
      if (wave == 0) dma_b32(rR, lds_addr(&sRS[it % 5][0]), live ? (uint32_t)(tq * AB_T * 8 + 4 * lane) : 0x80000000u, 0u);
      if (TEMP && wave == 1) {
        const i32x4 rT = buffer_rsrc(tau + ((int64_t)b * Hq + h) * Mp, (uint32_t)Mp * 4u);
        dma_b32(rT, lds_addr(&sT[it % 5][0]), live && lane < AB_T ? (uint32_t)(tq * AB_T * 4 + 4 * lane) : 0x80000000u,
                0u);
      }
    };
    // Barrier of an item: the loads of item it landed (this wave's loads of item
    // it + 1 may still be in flight).  Role 1 has none of its own.
    auto sync_item = [&]() __attribute__((always_inline)) {
      if (role == 1) sync_vm<0>();
      else if (wave == 0 || (TEMP && wave == 1)) sync_vm<NIW + 1>();
      else sync_vm<NIW>();
    };
    if (role == 0) {
      issue(0);
      issue(1);
    }

    const int64_t koff = ((bM + (vk ? key : 0)) * Hkv + kvh) * D;
    // Per head the items of this wave are: tiles before its keys (nothing to
    // do), the diagonal tile (causal mask), then unmasked tiles.
    const int nskip = sub < ntl ? sub : ntl;
    if (role == 0) {
      // ---- role 0: S, P, dV ----
      u32x4 kf[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        kf[ks] = vk ? *(const u32x4 *)(kh + koff + 16 * ks + 8 * hl) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) settle(kf[ks]);
      f32x16 aV[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) aV[db] = f32x16{};
      float blane = -INFINITY;
      auto item = [&](int it, bool masked) __attribute__((always_inline)) {
        const int i0 = (tq0 + it % ntl) * AB_T;
        const uint16_t *Qt = sQ + (it % 5) * T::TILE, *Ot = sO + (it % 5) * T::TILE;
        const float2 rs = sRS[it % 5][l32];
        f32x16 s = mfma32(aug3(i0 + l32 < M ? rs.x : -1e30f, hl), kones, f32x16{});
        {
          u32x4 f[NKS];
          f[0] = fr.rows(Qt, 0);
          f[1] = fr.rows(Qt, 1);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            if (ks + 2 < NKS) f[ks + 2] = fr.rows(Qt, ks + 2);
            __builtin_amdgcn_sched_barrier(0);
            s = mfma32(f[ks], kf[ks], s);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // temperatures of the item's rows (lane rows acc_row(4 j .. 4 j + 3, hl))
        f32x4 tv[4];
        if (TEMP) {
#pragma unroll
          for (int j = 0; j < 4; ++j) tv[j] = *(const f32x4 *)&sT[TEMP ? it % 5 : 0][8 * j + 4 * hl];
        }
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = __builtin_fmaf(s[r], c2, blane);
          if (TEMP) x *= tv[r >> 2][r & 3];
          if (masked && key > i0 + acc_row(r, hl)) x = -INFINITY;
          p[r] = fast_exp2(x);
        }
        // the partner's dS takes t P (dL/dZ = t dL/dS)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 pj = f32x4{p[4 * j], p[4 * j + 1], p[4 * j + 2], p[4 * j + 3]};
          if (TEMP) pj *= tv[j];
          sP[it & 1][sub][j][lane] = pj;
        }
        u32x4 pf[2];
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int w = 0; w < 4; ++w) pf[hf][w] = pack_bf16x2(p[8 * hf + 2 * w], p[8 * hf + 2 * w + 1]);
        trprod(Ot, pf, aV);
      };
      for (int hh = 0; hh < G; ++hh) {
        const int it0 = hh * ntl;
        blane = vk ? bias[((int64_t)b * Hq + kvh * G + hh) * M + key] : -INFINITY;
        settle(blane);
        for (int n = 0; n < nskip; ++n) {
          sync_item();
          issue(it0 + n + 2);
        }
        if (nskip < ntl) {
          sync_item();
          issue(it0 + nskip + 2);
          item(it0 + nskip, true);
        }
        for (int n = nskip + 1; n < ntl; ++n) {
          sync_item();
          issue(it0 + n + 2);
          item(it0 + n, false);
        }
      }
      // the barriers of role 1's last two iterations
      sync_vm<0>();
      sync_vm<0>();
      sync_vm<0>();
      if (vk) {
        float *dvr = dv + koff;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d = db * 32 + 8 * g4 + 4 * hl;
            *(f32x4 *)(dvr + d) = f32x4{aV[db][4 * g4], aV[db][4 * g4 + 1], aV[db][4 * g4 + 2], aV[db][4 * g4 + 3]};
          }
      }
    } else {
      // ---- role 1: dP, dS and the column sums one item behind role 0, the
      // dK product of an item one iteration later still (before the next dP) ----
      u32x4 vf[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        vf[ks] = vk ? *(const u32x4 *)(v + koff + 16 * ks + 8 * hl) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) settle(vf[ks]);
      f32x16 aK[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) aK[db] = f32x16{};
      float csum = 0.f;
      u32x4 dsf[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
      int pit = -1;  // item whose dS waits for its dK product
      auto dstep = [&](int jt) __attribute__((always_inline)) {
        const uint16_t *Ot = sO + (jt % 5) * T::TILE;
        const float2 rs = sRS[jt % 5][l32];
        f32x16 dp = mfma32(aug3(-rs.y, hl), kones, f32x16{});
        {
          u32x4 f[NKS];
          f[0] = fr.rows(Ot, 0);
          f[1] = fr.rows(Ot, 1);
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            if (ks + 2 < NKS) f[ks + 2] = fr.rows(Ot, ks + 2);
            __builtin_amdgcn_sched_barrier(0);
            dp = mfma32(f[ks], vf[ks], dp);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        float ds[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 pv = sP[jt & 1][sub][j][lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            ds[4 * j + e] = pv[e] * dp[4 * j + e];
            csum += ds[4 * j + e];
          }
        }
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int w = 0; w < 4; ++w) dsf[hf][w] = pack_bf16x2(ds[8 * hf + 2 * w], ds[8 * hf + 2 * w + 1]);
      };
      sync_item();
      for (int hh = 0; hh < G; ++hh) {
        const int it0 = hh * ntl;
        for (int n = 0; n < ntl; ++n) {
          sync_item();
          if (pit >= 0) trprod(sQ + (pit % 5) * T::TILE, dsf, aK);
          pit = -1;
          if (n >= nskip) {
            dstep(it0 + n);
            pit = it0 + n;
          }
        }
        const float tot = csum + __shfl_xor(csum, 32);
        if (hl == 0) sCol[hh][AB_T * sub + l32] = tot;
        csum = 0.f;
      }
      sync_item();
      if (pit >= 0) trprod(sQ + (pit % 5) * T::TILE, dsf, aK);
      sync_vm<0>();
      if (vk) {
        float *dkr = dk + koff;
        f32x4 ca[NDB / 2][4][2];  // the key's angles, all loaded before the products
#pragma unroll
        for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            ca[db][g4][0] = ca[db][g4][1] = f32x4{1.f, 0.f, 1.f, 0.f};
            if (cs) {
              const f32x4 *cp = (const f32x4 *)(cs + (bM + key) * HALF + db * 32 + 8 * g4 + 4 * hl);
              ca[db][g4][0] = cp[0];
              ca[db][g4][1] = cp[1];
            }
          }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < NDB / 2; ++db)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d = db * 32 + 8 * g4 + 4 * hl;
            const f32x4 t0 = ca[db][g4][0], t1 = ca[db][g4][1];
            const float cv[4] = {t0[0], t0[2], t1[0], t1[2]}, sv[4] = {t0[1], t0[3], t1[1], t1[3]};
            float xo[4], yo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float x = aK[db][4 * g4 + e] * c, y = aK[db + NDB / 2][4 * g4 + e] * c;
              xo[e] = x * cv[e] + y * sv[e];
              yo[e] = y * cv[e] - x * sv[e];
            }
            *(f32x4 *)(dkr + d) = f32x4{xo[0], xo[1], xo[2], xo[3]};
            *(f32x4 *)(dkr + HALF + d) = f32x4{yo[0], yo[1], yo[2], yo[3]};
          }
      }
    }
    sync_vm<0>();  // sCol complete
    for (int i = tid; i < G * KB; i += AB_NW * 64) {
      const int hh = i / KB, kk = i % KB;
      if (k0 + kk < M) colsum[((int64_t)b * Hq + kvh * G + hh) * M + k0 + kk] = sCol[hh][kk];
    }
    sync_vm<0>();  // sCol read before the next block writes it
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
    const float *__restrict__ lse, const float *__restrict__ dout, float c, const float *__restrict__ sigma,
    const float *__restrict__ ratio, int B, int M, int Hq, int Hkv, int D, int gph, float *__restrict__ dq,
    float *__restrict__ delta, float *__restrict__ tstat) {
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
  const float *gh = gph ? g + (b * Hq + h) * M : g + bM;  // this head's gates of the row
  const float l = lse[(b * Hq + h) * M + i];
  const float t = sigma ? fmaxf(softplus_f(sigma[h]) * ratio[bi], 1e-30f) : 1.f;  // logits t Z
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
      const float zj = wave_sum(qx * kx + qy * ky) * c + logit_bias(gam, gh[j]);
      const float p = zj == -INFINITY ? 0.f : expf(t * zj - l);
      Di += p * wave_sum(ox * vx + oy * vy);
    }
  }
  float ax = 0.f, ay = 0.f, dt = 0.f;
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
      const float zj = wave_sum(qx * kx + qy * ky) * c + logit_bias(gam, gh[j]);
      if (zj == -INFINITY) continue;
      const float p = expf(t * zj - l);
      const float ds = p * (wave_sum(ox * vx + oy * vy) - Di);
      dt += ds * zj;
      ax += ds * kx;
      ay += ds * ky;
    }
  }
  ax *= c * t;
  ay *= c * t;
  if (act) {
    rot(ax, ay, cs, bi * half + lane, -1.f);
    dq[row * D + lane] = ax;
    dq[row * D + half + lane] = ay;
  }
  if (lane == 0) delta[(b * Hq + h) * M + i] = Di;
  if (sigma && lane == 0) tstat[(b * Hq + h) * M + i] = ratio[bi] * dt;
}

// one wave per (b, j, kv head): dk, dv, colsum of every head of the group
__global__ __launch_bounds__(256) void attn_bwd_dkdv_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ gamma, const float2 *__restrict__ cs,
    const float *__restrict__ lse, const float *__restrict__ dout, const float *__restrict__ delta, float c,
    const float *__restrict__ sigma, const float *__restrict__ ratio, int B, int M, int Hq, int Hkv, int D, int gph,
    float *__restrict__ dk, float *__restrict__ dv, float *__restrict__ colsum) {
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
  float akx = 0.f, aky = 0.f, avx = 0.f, avy = 0.f;
  for (int hh = 0; hh < G; ++hh) {
    const int h = kv * G + hh;
    const float bias = logit_bias(gamma[h], g[gph ? (b * Hq + h) * M + j : bj]);
    const float sp = sigma ? softplus_f(sigma[h]) : 1.f;
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
        const float t = sigma ? fmaxf(sp * ratio[bM + i], 1e-30f) : 1.f;
        const float p = expf(t * (wave_sum(qx * kx + qy * ky) * c + bias) - l);
        const float ds = t * p * (wave_sum(ox * vx + oy * vy) - delta[(b * Hq + h) * M + i]);  // dL/dZ
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
// dg_j = sum_h gamma_h colsum_h(j) / g_j, one thread per token in fixed head
// order.  Each work-group also leaves, per head, its tokens' share of dgamma,
// sum_j colsum_h(j) ln g_j, and (with the temperature) of the dsigma sum,
// sum_j tstat_h(j), in part[b][bx][h] and part[n + (b][bx][h)] (n = the
// number of shares): butterfly sums within each wave, then the four waves in
// order, so the shares are fixed-shape (bitwise deterministic).  Heads go in
// chunks of 64 per barrier.
// With per-head gates (gph) g and dg are [B, Hq, M]: dg_hj = gamma_h colsum_h(j) / g_hj and the
// dgamma share uses ln g_hj.
// One sequence's 256-token block: token j of row pointers colsum_b, tstat_b
// ([Hq, M] each), g_b, dg_b; the block's shares go to share[h] (dgamma) and
// share_t[h] (dsigma, with the temperature).
__device__ __forceinline__ void dg_tile(const float *__restrict__ colsum_b, const float *__restrict__ tstat_b,
                                        const float *__restrict__ g_b, const float *__restrict__ gamma, int M, int Hq,
                                        int gph, int j, float *__restrict__ dg_b, float *__restrict__ share,
                                        float *__restrict__ share_t, float (*red)[64][4]) {
  const bool vj = j < M;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float *cr = colsum_b + j;
  const float *tr = tstat_b ? tstat_b + j : nullptr;
  const float gv = vj && !gph ? g_b[j] : 0.f;
  const float lg = gv > 0.f ? logf(gv) : 0.f;
  float acc = 0.f;
  for (int h0 = 0; h0 < Hq; h0 += 64) {
    const int nh = Hq - h0 < 64 ? Hq - h0 : 64;
    for (int hh = 0; hh < nh; hh += 8) {
      float v[8], ts[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // eight independent loads in flight
        const bool ok = vj && hh + e < nh;
        v[e] = ok ? cr[(int64_t)(h0 + hh + e) * M] : 0.f;
        ts[e] = ok && tr ? tr[(int64_t)(h0 + hh + e) * M] : 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (hh + e >= nh) break;
        acc += gamma[h0 + hh + e] * v[e];
        float t = gv > 0.f ? v[e] * lg : 0.f;
        if (gph) {  // this head's own gate
          const int64_t o = (int64_t)(h0 + hh + e) * M + j;
          const float gh = vj ? g_b[o] : 0.f;
          t = gh > 0.f ? v[e] * logf(gh) : 0.f;
          if (vj) dg_b[o] = gh > 0.f ? gamma[h0 + hh + e] * v[e] / gh : 0.f;
        }
        float u = ts[e];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          t += __shfl_xor(t, o);
          u += __shfl_xor(u, o);
        }
        if (lane == 0) {
          red[0][hh + e][wave] = t;
          red[1][hh + e][wave] = u;
        }
      }
    }
    __syncthreads();
    if ((int)threadIdx.x < nh) {
      const int h = h0 + threadIdx.x;
      const float(*r0)[4] = red[0], (*r1)[4] = red[1];
      share[h] = (r0[threadIdx.x][0] + r0[threadIdx.x][1]) + (r0[threadIdx.x][2] + r0[threadIdx.x][3]);
      if (tstat_b) share_t[h] = (r1[threadIdx.x][0] + r1[threadIdx.x][1]) + (r1[threadIdx.x][2] + r1[threadIdx.x][3]);
    }
    __syncthreads();
  }
  if (vj && !gph) dg_b[j] = gv > 0.f ? acc / gv : 0.f;
}

__global__ __launch_bounds__(256) void dg_kernel(const float *__restrict__ colsum, const float *__restrict__ g,
                                                 const float *__restrict__ gamma, const float *__restrict__ tstat,
                                                 int B, int M, int Hq, int gph, float *__restrict__ dg,
                                                 float *__restrict__ part) {
  __shared__ float red[2][64][4];
  const int j = blockIdx.x * 256 + threadIdx.x;  // grid (ceil(M / 256), min(B, 65535))
  const int64_t nshare = (int64_t)B * gridDim.x * Hq;
  for (int b = blockIdx.y; b < B; b += gridDim.y) {
    const int64_t o = ((int64_t)b * gridDim.x + blockIdx.x) * Hq;
    const int64_t gb = gph ? (int64_t)b * Hq * M : (int64_t)b * M;
    dg_tile(colsum + (int64_t)b * Hq * M, tstat ? tstat + (int64_t)b * Hq * M : nullptr, g + gb, gamma, M, Hq, gph,
            j, dg + gb, part + o, tstat ? part + nshare + o : nullptr, red);
  }
}

// The same over a packed group of runs (one gate per key): work-group w takes
// block x of sequence b of run i, where w = wg0[i] + b ceil(M_i / 256) + x;
// its shares go to slot sh0 + w of a share array that lists every run's
// blocks in order (nshare slots in all, dsigma shares after them).
struct DgRuns {
  int nr, sh0;
  int wg0[kMaxRuns + 1];
  int off[kMaxRuns], M[kMaxRuns];
};

__global__ __launch_bounds__(256) void dg_runs_kernel(const float *__restrict__ colsum, const float *__restrict__ g,
                                                      const float *__restrict__ gamma,
                                                      const float *__restrict__ tstat, int Hq, int64_t nshare,
                                                      float *__restrict__ dg, float *__restrict__ part,
                                                      const DgRuns dr) {
  __shared__ float red[2][64][4];
  const int w = blockIdx.x;
  int ri = 0;
  for (int i = 1; i < dr.nr; ++i) ri = w >= dr.wg0[i] ? i : ri;  // uniform
  const int M = dr.M[ri], nbx = (M + 255) / 256, loc = w - dr.wg0[ri], b = loc / nbx, x = loc - b * nbx;
  const int64_t off = dr.off[ri];
  const int64_t rb = off * Hq + (int64_t)b * Hq * M;  // [Hq, M] block of sequence b in a run's [n, Hq, M] array
  const int64_t o = ((int64_t)dr.sh0 + w) * Hq;
  dg_tile(colsum + rb, tstat ? tstat + rb : nullptr, g + off + (int64_t)b * M, gamma, M, Hq, 0, x * 256 + threadIdx.x,
          dg + off + (int64_t)b * M, part + o, tstat ? part + nshare * Hq + o : nullptr, red);
}

// Block h < Hq: dgamma_h = sum over the n = B * ceil(M / 256) shares of head h;
// block Hq + h (with the temperature): dsigma_h = sigmoid(sigma_h) times the
// sum of head h's dsigma shares (softplus' = sigmoid).  Fixed-shape tree.
__global__ __launch_bounds__(256) void dgamma_kernel(const float *__restrict__ part, int n, int Hq,
                                                     const float *__restrict__ sigma, float *__restrict__ dgamma,
                                                     float *__restrict__ dsigma) {
  __shared__ float red[256];
  const bool sig = (int)blockIdx.x >= Hq;
  const int h = sig ? blockIdx.x - Hq : blockIdx.x;
  const float *p = part + (sig ? (int64_t)n * Hq : 0);
  float acc = 0.f;
  for (int i = threadIdx.x; i < n; i += 256) acc += p[(int64_t)i * Hq + h];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (sig) dsigma[h] = red[0] / (1.f + expf(-sigma[h]));
    else dgamma[h] = red[0];
  }
}

// Packed variable-length calls run one backward per run of equal-length
// sequences, each leaving its dgamma (and dsigma) in part[r][0 .. Hq) (and
// part[r][Hq .. 2 Hq)); this sums them in run order (deterministic).  With no
// run at all it writes zeros.
__global__ __launch_bounds__(256) void sum_runs_kernel(const float *__restrict__ part, int nruns, int Hq,
                                                       float *__restrict__ dgamma, float *__restrict__ dsigma) {
  const int h = blockIdx.x * 256 + threadIdx.x;
  if (h >= Hq) return;
  float a = 0.f, b = 0.f;
  for (int r = 0; r < nruns; ++r) {
    a += part[(int64_t)r * 2 * Hq + h];
    b += part[(int64_t)r * 2 * Hq + Hq + h];
  }
  dgamma[h] = a;
  if (dsigma) dsigma[h] = b;
}

hipError_t launch_sum_runs(const float *part, int nruns, int Hq, float *dgamma, float *dsigma, hipStream_t s) {
  hipLaunchKernelGGL(sum_runs_kernel, dim3((unsigned)((Hq + 255) / 256)), dim3(256), 0, s, part, nruns, Hq, dgamma,
                     dsigma);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                           const int32_t *pos, double theta, float tau, const float *sigma, const float *lse,
                           const void *dout, const void *o, const void *o_lo, const RunRow *runs, int nruns, int Hq,
                           int Hkv, int D, bool bf16, bool g_per_head, float *dq, float *dk, float *dv, float *dg,
                           float *dgamma, float *dsigma, float *part, const AttnWs &w, hipStream_t s) {
  const int gph = (int)g_per_head;
  const int64_t esz = bf16 ? 2 : 4;
  auto live = [](const RunRow &r) { return (int64_t)r.n * r.M > 0; };
  // Packed bf16 runs with one gate per key: the prep and dg passes take a
  // group of runs per launch, and one reduction gives dgamma (dsigma).
  const bool grouped = bf16 && nruns > 1 && !g_per_head;
  if (grouped) {
    for (int g0 = 0; g0 < nruns; g0 += kMaxRuns) {
      const int ng = nruns - g0 < kMaxRuns ? nruns - g0 : kMaxRuns;
      const hipError_t e =
          launch_attn_prep_runs(k, g, gamma, pos, theta, runs + g0, ng, Hq, Hkv, D, sigma != nullptr, w, s, nullptr);
      if (e != hipSuccess) return e;
    }
  }
  // rotated keys, biases, temperature ratios of every run
  for (int i = 0; i < nruns && !grouped; ++i) {
    const RunRow &r = runs[i];
    if (!live(r) || !(pos || bf16 || sigma)) continue;
    const int64_t t0 = r.off;
    const hipError_t e = launch_attn_prep((const char *)k + t0 * Hkv * D * esz, g + (gph ? t0 * Hq : t0), gamma,
                                          pos ? pos + t0 : nullptr, theta, r.n, r.M, Hq, Hkv, D, bf16, bf16,
                                          sigma != nullptr, g_per_head, run_view(w, r, Hq, Hkv, D), s);
    if (e != hipSuccess) return e;
  }
  const double cd = 1.0 / (sqrt((double)D) * (double)tau);
  const float c = (float)cd, c2 = (float)(cd * 1.4426950408889634);
  if (bf16) {
    // one launch per kernel over all runs (kMaxRuns at a time): query
    // blocks cost their key tiles plus about six tiles of fixed work, key
    // blocks their items plus about two
    const int G = Hq / Hkv;
    const int BQ = 256 / G;
    const uint16_t *kh = pos ? w.khat : (const uint16_t *)k;
    const uint16_t *qh = pos ? w.qhat : (const uint16_t *)q;
    const bool t = sigma != nullptr;
    auto k1 = D == 128 ? (t ? attn_bwd_dq_bf16_kernel<128, true> : attn_bwd_dq_bf16_kernel<128, false>)
                       : (t ? attn_bwd_dq_bf16_kernel<64, true> : attn_bwd_dq_bf16_kernel<64, false>);
    auto k2 = D == 128 ? (t ? attn_bwd_dkdv_bf16_kernel<128, true> : attn_bwd_dkdv_bf16_kernel<128, false>)
                       : (t ? attn_bwd_dkdv_bf16_kernel<64, true> : attn_bwd_dkdv_bf16_kernel<64, false>);
    std::vector<Level> l1, l2;
    std::vector<RunTable> t1, t2;
    std::vector<unsigned> g1, g2;
    for (int r0 = 0; r0 < nruns; r0 += kMaxRuns) {
      const int nr = nruns - r0 < kMaxRuns ? nruns - r0 : kMaxRuns;
      const RunRow *rr = runs + r0;
      l1.clear();
      l2.clear();
      for (int i = 0; i < nr; ++i) {
        if (!live(rr[i])) continue;
        const int M = rr[i].M, nqb = (M + BQ - 1) / BQ, nkb = (M + 127) / 128, ntq = (M + AB_T - 1) / AB_T;
        for (int qb = 0; qb < nqb; ++qb) {
          const int qe = (qb + 1) * BQ < M ? (qb + 1) * BQ : M;
          l1.push_back(Level{i, qb, (int64_t)((qe + AB_T - 1) / AB_T) + 6});
        }
        for (int kb = 0; kb < nkb; ++kb) l2.push_back(Level{i, kb, (int64_t)G * (ntq - 4 * kb) + 2});
      }
      if (l1.empty()) continue;
      make_tables(l1, rr, nr, Hkv, t1, g1);
      make_tables(l2, rr, nr, Hkv, t2, g2);
      for (size_t j = 0; j < t1.size(); ++j)
        hipLaunchKernelGGL(k1, dim3(g1[j]), dim3(512), 0, s, (const uint16_t *)q, kh, (const uint16_t *)v, w.bias,
                           pos ? w.cs : nullptr, lse, (const uint16_t *)dout, c, c2, sigma, w.ratio, Hq, Hkv, G, BQ,
                           dq, w.qhat, w.rowstat, w.tau, w.tstat, (const uint16_t *)o, (const uint16_t *)o_lo,
                           t1[j]);
      for (size_t j = 0; j < t2.size(); ++j)
        hipLaunchKernelGGL(k2, dim3(g2[j]), dim3(512), 0, s, qh, (const uint16_t *)dout, w.rowstat,
                           (const float *)w.tau, kh, (const uint16_t *)v, w.bias, pos ? w.cs : nullptr, c, c2, Hq,
                           Hkv, G, pos ? 1 : 0, dk, dv, w.colsum, t2[j]);
    }
  } else {
    for (int i = 0; i < nruns; ++i) {
      const RunRow &r = runs[i];
      if (!live(r)) continue;
      const AttnWs wv = run_view(w, r, Hq, Hkv, D);
      const int64_t t0 = r.off;
      const float *qr = (const float *)q + t0 * Hq * D, *kr = (const float *)k + t0 * Hkv * D,
                  *vr = (const float *)v + t0 * Hkv * D, *gr = g + (gph ? t0 * Hq : t0), *lr = lse + t0 * Hq,
                  *dr = (const float *)dout + t0 * Hq * D;
      float *delta = (float *)wv.rowstat;
      const float2 *cs = pos ? wv.cs : nullptr;
      const int64_t rq = (int64_t)r.n * r.M * Hq, rk = (int64_t)r.n * r.M * Hkv;
      hipLaunchKernelGGL(attn_bwd_dq_f32_kernel, dim3((unsigned)((rq + 3) / 4)), dim3(256), 0, s, qr, kr, vr, gr,
                         gamma, cs, lr, dr, c, sigma, wv.ratio, r.n, r.M, Hq, Hkv, D, gph, dq + t0 * Hq * D, delta,
                         wv.tstat);
      hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel, dim3((unsigned)((rk + 3) / 4)), dim3(256), 0, s, qr, kr, vr, gr,
                         gamma, cs, lr, dr, delta, c, sigma, wv.ratio, r.n, r.M, Hq, Hkv, D, gph, dk + t0 * Hkv * D,
                         dv + t0 * Hkv * D, wv.colsum);
    }
  }
  if (grouped) {
    // every run's 256-token blocks in order, one share slot each; the row
    // statistics of all runs are dead by now and hold the shares (2 nshare Hq
    // floats of their 2 Hq T)
    int64_t nshare = 0;
    for (int i = 0; i < nruns; ++i) nshare += (int64_t)runs[i].n * ((runs[i].M + 255) / 256);
    float *shares = (float *)w.rowstat;
    int64_t sh = 0;
    for (int g0 = 0; g0 < nruns; g0 += kMaxRuns) {
      const int ng = nruns - g0 < kMaxRuns ? nruns - g0 : kMaxRuns;
      DgRuns dr{};
      dr.nr = ng;
      dr.sh0 = (int)sh;
      int64_t wg = 0;
      for (int i = 0; i < ng; ++i) {
        const RunRow &r = runs[g0 + i];
        dr.wg0[i] = (int)wg;
        dr.off[i] = r.off;
        dr.M[i] = r.M;
        wg += (int64_t)r.n * ((r.M + 255) / 256);
      }
      dr.wg0[ng] = (int)wg;
      if (wg > 0)
        hipLaunchKernelGGL(dg_runs_kernel, dim3((unsigned)wg), dim3(256), 0, s, w.colsum, g, gamma,
                           sigma ? (const float *)w.tstat : nullptr, Hq, nshare, dg, shares, dr);
      sh += wg;
    }
    hipLaunchKernelGGL(dgamma_kernel, dim3((unsigned)(sigma ? 2 * Hq : Hq)), dim3(256), 0, s, (const float *)shares,
                       (int)nshare, Hq, sigma, dgamma, dsigma);
    return hipGetLastError();
  }
  // dg per token, and per run the dgamma (dsigma) sums; a run's row
  // statistics are dead by now: their space (2 n Hq M floats) takes its
  // shares (2 n ceil(M / 256) Hq floats)
  for (int i = 0; i < nruns; ++i) {
    const RunRow &r = runs[i];
    const AttnWs wv = run_view(w, r, Hq, Hkv, D);
    const int64_t t0 = r.off;
    if (live(r))
      hipLaunchKernelGGL(dg_kernel, dim3((unsigned)((r.M + 255) / 256), (unsigned)(r.n < 65535 ? r.n : 65535)),
                         dim3(256), 0, s, wv.colsum, g + (gph ? t0 * Hq : t0), gamma,
                         sigma ? (const float *)wv.tstat : nullptr, r.n, r.M, Hq, gph, dg + (gph ? t0 * Hq : t0),
                         (float *)wv.rowstat);
    float *dgo = part ? part + (int64_t)i * 2 * Hq : dgamma;
    float *dso = part ? (sigma ? part + (int64_t)i * 2 * Hq + Hq : nullptr) : dsigma;
    hipLaunchKernelGGL(dgamma_kernel, dim3((unsigned)(sigma ? 2 * Hq : Hq)), dim3(256), 0, s,
                       (const float *)wv.rowstat, live(r) ? r.n * ((r.M + 255) / 256) : 0, Hq, sigma, dgo, dso);
  }
  if (part) return launch_sum_runs(part, nruns, Hq, dgamma, dsigma, s);
  return hipGetLastError();
}

}  // namespace tg
