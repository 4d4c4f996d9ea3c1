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
                                                        uint16_t *__restrict__ khat, float *__restrict__ bias) {
  const int half = D / 2;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (row, rotary pair)
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


// Work-group: 8 waves = two teams of 4.  The 4 waves of a team own the 128
// columns; each 128-key super-tile is split between the teams (team t takes
// keys 64t..64t+63), so a query block's key chain is walked in half the steps
// and each SIMD holds one wave of each team.  The teams merge (max, sum, O)
// through LDS at the end.  Tiles arrive by direct buffer->LDS loads issued one
// super-tile ahead; every per-lane address is computed once before the loop.
template <int D>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ khat, const uint16_t *__restrict__ v,
    const float *__restrict__ bias, const float2 *__restrict__ cs, float c2, int B, int M, int Hq, int Hkv, int G,
    int BQ, int nqb, uint16_t *__restrict__ o, float *__restrict__ lse) {
  using T = Tile<D>;
  constexpr int NKS = D / 16;        // 16-wide k steps over the head dim
  constexpr int NDB = D / 32;        // 32-row blocks of O^T
  constexpr int HALF = D / 2;
  constexpr int TK = 128;            // keys per super-tile
  constexpr int GMAX = 8;            // query heads per kv head handled here
  constexpr int TILE = TK * D;       // u16 elements per K (or V) super-tile
  constexpr int NIW = TK / T::RPI / 8;  // direct-load instructions per wave per K (or V) super-tile
  // K tiles (2 buffers) then V tiles (2 buffers); reused for the team merge
  __shared__ __attribute__((aligned(1024))) uint16_t sKV[4 * TILE];
  __shared__ __attribute__((aligned(16))) float sB[2][GMAX][TK];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int team = wave >> 2, wt = wave & 3;
  const int l32 = lane & 31, hl = lane >> 5;
  const int nbh = B * Hkv;
  const int idx = blockIdx.x;
  const int qb = nqb - 1 - idx / nbh;  // longest causal rows first
  const int bh = idx % nbh;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int q0 = qb * BQ;
  const int col = wt * 32 + l32;
  const int hloc = col / BQ;
  const int hq = kvh * G + hloc;
  const int qi = q0 + col % BQ;
  const bool vq = qi < M;
  const int qmax = min(q0 + BQ, M) - 1;
  const int nst = qmax / TK + 1;
  const int64_t bM = (int64_t)b * M;
  const uint32_t rsb = (uint32_t)(Hkv * D * 2);  // bytes between consecutive keys
  const uint32_t kv_bytes = (uint32_t)(M - 1) * rsb + D * 2;
  const i32x4 rK = buffer_rsrc(khat + (bM * Hkv + kvh) * D, kv_bytes);
  const i32x4 rV = buffer_rsrc(v + (bM * Hkv + kvh) * D, kv_bytes);
  const i32x4 rB = buffer_rsrc(bias + ((int64_t)b * Hq + (int64_t)kvh * G) * M, (uint32_t)(G * M * 4));
  // per-lane byte offset of this wave's direct-load instruction i: row * rsb +
  // swizzled chunk; row = (wave * NIW + i) * RPI + lane / C
  const uint32_t lrow = (uint32_t)(wave * NIW * T::RPI + lane / T::C) * rsb;
  const int lpc = lane % T::C;
  auto kofs = [&](int i) {
    const int row = (wave * NIW + i) * T::RPI + lane / T::C;
    return lrow + (uint32_t)(i * T::RPI) * rsb + ((lpc ^ T::kswz(row)) << 4);
  };
  auto vofs = [&](int i) {
    const int row = (wave * NIW + i) * T::RPI + lane / T::C;
    return lrow + (uint32_t)(i * T::RPI) * rsb + ((lpc ^ T::vswz(row)) << 4);
  };
  // highest query among this wave's columns (the causal limit of its keys)
  int wq = vq ? qi : -1;
  for (int o2 = 32; o2 > 0; o2 >>= 1) wq = max(wq, __shfl_xor(wq, o2));

  // Buffers: K super-tile t lives in K buffer t % 2, V super-tile t (with its
  // bias rows) in V buffer t % 2.  The K stream runs one super-tile ahead of V:
  // iteration t computes S(t+1) from K(t+1) while it turns S(t) into P(t) and
  // multiplies P(t) by V(t).
  auto issue_k = [&](int t) {
    const int soff = t * TK * (int)rsb;
#pragma unroll
    for (int i = 0; i < NIW; ++i)
      dma_b128(rK, lds_addr(sKV) + 2u * (uint32_t)((t & 1) * TILE + (wave * NIW + i) * 512), kofs(i), (uint32_t)soff);
  };
  auto issue_v = [&](int t) {
    const int j0 = t * TK;
    const int soff = j0 * (int)rsb;
#pragma unroll
    for (int i = 0; i < NIW; ++i)
      dma_b128(rV, lds_addr(sKV) + 2u * (uint32_t)((2 + (t & 1)) * TILE + (wave * NIW + i) * 512), vofs(i),
               (uint32_t)soff);
    // bias rows: G x 128 floats, 64 floats per 4-byte direct-load instruction
    for (int ii = wave; ii < 2 * G; ii += 8)
      dma_b32(rB, lds_addr(&sB[t & 1][ii >> 1][(ii & 1) * 64]), (uint32_t)(((ii >> 1) * M + (ii & 1) * 64 + lane) * 4),
              (uint32_t)(j0 * 4));
  };
  issue_k(0);
  issue_v(0);
  if (nst > 1) issue_k(1);

  // Q fragments (MFMA B operand): lane holds q^[qi, hq, 16ks + 8hl .. +8].
  u32x4 qf[NKS];
  const uint16_t *qrow = q + ((bM + qi) * Hq + hq) * D;
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) qf[ks] = vq ? *(const u32x4 *)(qrow + 16 * ks + 8 * hl) : u32x4{0, 0, 0, 0};
  if (cs && vq) {
#pragma unroll
    for (int ks = 0; ks < NKS / 2; ++ks) rope_chunk(qf[ks], qf[ks + NKS / 2], cs + (bM + qi) * HALF + 16 * ks + 8 * hl);
  }

  // LDS element offsets of this lane's fragment reads (within a team's 64-row half tile)
  // K: row kb*32 + l32 (swizzle depends on l32 only), logical chunk 2ks + hl.
  const int krow = l32 * D;
  const int kx = T::kswz(l32);
  // V (transposing read): source lane li = 4kq + cc of 16-lane group gi reads key
  // kb*32 + 16hf + 8rr + 4hl + kq, d = 32db + 16(gi%2) + 4cc; swizzle depends on kq only.
  const int gi = lane >> 4, li = lane & 15, kq = li >> 2, cc = li & 3;
  int vlo[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int dd = 32 * db + 16 * (gi & 1) + 4 * cc;
    vlo[db] = (4 * hl + kq) * D + (((dd >> 3) ^ T::vswz(kq)) << 3) + (dd & 7);
  }

  // S^T = K Q^T for this team's 64 keys of super-tile t (raw dot products).
  auto qk = [&](int t, f32x16(&s)[2]) {
    const uint16_t *K = sKV + (t & 1) * TILE + 64 * team * D;
    s[0] = f32x16{};
    s[1] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = *(const u32x4 *)(K + kb * 32 * D + krow + (((2 * ks + hl) ^ kx) << 3));
        s[kb] = mfma32(a, qf[ks], s[kb]);
      }
    }
  };

  float m2 = -INFINITY, lsum = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};

  // softmax of S(t) in `s` and O^T += V(t)^T P(t)^T
  auto attend = [&](int t, f32x16(&s)[2]) {
    const int j0 = t * TK + 64 * team;  // this team's first key
    if (j0 > wq) return;                // every key after every query of this wave
    const uint16_t *V = sKV + (2 + (t & 1)) * TILE + 64 * team * D;
    const float *bi = &sB[t & 1][hloc][64 * team];
    // logits: x = s * c2 + bias (bias is -inf for g = 0); causal mask on the diagonal
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 bv = *(const f32x4 *)(bi + kb * 32 + 8 * g4 + 4 * hl);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[kb][4 * g4 + e] = __builtin_fmaf(s[kb][4 * g4 + e], c2, bv[e]);
      }
    }
    if (j0 + 63 > q0) {  // diagonal tile: keys after the query get -inf
      const int lim = qi - j0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = (kb * 32 + acc_row(r, hl) > lim) ? -INFINITY : s[kb][r];
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kb][r]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    // Lazy rescaling: keep the running max unless a logit exceeds it by more
    // than 8 (log2 units), so probabilities stay <= 256 and O is rescaled rarely.
    if (__any(mloc > m2 + 8.f)) {
      const float mnew = fmaxf(m2, mloc);
      const float alpha = fast_exp2(m2 - ((mnew == -INFINITY) ? 0.f : mnew));
      m2 = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    const float muse = (m2 == -INFINITY) ? 0.f : m2;
    float psum = 0.f;
    u32x4 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float p0 = fast_exp2(s[kb][8 * hf + 2 * w] - muse);
          const float p1 = fast_exp2(s[kb][8 * hf + 2 * w + 1] - muse);
          psum += p0 + p1;
          pf[kb][hf][w] = pack_bf16x2(p0, p1);
        }
    lsum += psum;
    // O^T += V^T P^T.  Key slot 8hl + e of step (kb, hf) is key kb*32 + 16hf + 8(e/4) + 4hl + e%4.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf)
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          u32x2 part[2];
#pragma unroll
          for (int rr = 0; rr < 2; ++rr)
            part[rr] = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                    (lds_i16x4 *)(V + (kb * 32 + 16 * hf + 8 * rr) * D + vlo[db])));
          acc[db] = mfma32(u32x4{part[0][0], part[0][1], part[1][0], part[1][1]}, pf[kb][hf], acc[db]);
        }
  };

  f32x16 sA[2], sB2[2];
  sync_vm<0>();
  qk(0, sA);
  // Two iterations per trip so the current / next S accumulators swap roles without copies.
  for (int t = 0; t < nst; t += 2) {
    // iteration t: S(t) in sA, computes S(t+1) into sB2
    sync_vm<0>();  // K(t+1), V(t) landed; every wave is done with iteration t-1
    if (t + 2 < nst) issue_k(t + 2);
    if (t + 1 < nst) issue_v(t + 1);
    // ping-pong: team 0 multiplies the next tile first, team 1 softmaxes first,
    // so each SIMD overlaps one wave's matrix work with the other's vector work
    if (team == 0) {
      if (t + 1 < nst) qk(t + 1, sB2);
      attend(t, sA);
    } else {
      attend(t, sA);
      if (t + 1 < nst) qk(t + 1, sB2);
    }
    if (t + 1 >= nst) break;
    // iteration t+1: S(t+1) in sB2, computes S(t+2) into sA
    sync_vm<0>();
    if (t + 3 < nst) issue_k(t + 3);
    if (t + 2 < nst) issue_v(t + 2);
    if (team == 0) {
      if (t + 2 < nst) qk(t + 2, sA);
      attend(t + 1, sB2);
    } else {
      attend(t + 1, sB2);
      if (t + 2 < nst) qk(t + 2, sA);
    }
  }

  // Merge team 1 into team 0 through LDS (the tile buffers are free now).
  sync_vm<0>();
  constexpr int NR = NDB * 16 + 2;
  static_assert(4 * NR * 64 * 4 <= 4 * TILE * 2, "team exchange must fit in the tile buffers");
  float *xch = reinterpret_cast<float *>(sKV) + wt * NR * 64;
  if (team == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) xch[(db * 16 + r) * 64 + lane] = acc[db][r];
    xch[(NR - 2) * 64 + lane] = m2;
    xch[(NR - 1) * 64 + lane] = lsum;
  }
  __syncthreads();
  if (team == 1) return;
  const float m1 = xch[(NR - 2) * 64 + lane], l1 = xch[(NR - 1) * 64 + lane];
  const float mm = fmaxf(m2, m1);
  const float mu = (mm == -INFINITY) ? 0.f : mm;
  const float a0 = fast_exp2(m2 - mu), a1 = fast_exp2(m1 - mu);
  const float lpart = lsum * a0 + l1 * a1;
  const float ltot = lpart + __shfl_xor(lpart, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (vq) {
    uint16_t *orow = o + ((bM + qi) * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float ov[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          ov[e] = (acc[db][4 * g4 + e] * a0 + xch[(db * 16 + 4 * g4 + e) * 64 + lane] * a1) * inv;
        const int d = db * 32 + 8 * g4 + 4 * hl;
        *(u32x2 *)(orow + d) = u32x2{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
      }
    }
    if (lse && hl == 0) lse[((int64_t)b * Hq + hq) * M + qi] = ltot > 0.f ? (mm + __log2f(ltot)) * kLn2 : -INFINITY;
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

// Workspace of the attention calls (256-byte aligned regions):
//   cs [B*M*D/2] float2 | khat [B*M*Hkv*D] bf16 | lg2 [B*M] f32 | delta [B*Hq*M] f32 | colsum [B*Hq*M] f32
static size_t rup(size_t x) { return (x + 255) / 256 * 256; }

size_t attn_workspace_bytes(int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D, bool bwd) {
  size_t n = rup((size_t)(B * M * (D / 2)) * sizeof(float2)) + rup((size_t)(B * M * Hkv * D) * 2) +
             rup((size_t)(B * Hq * M) * sizeof(float));
  if (bwd) n += 2 * rup((size_t)(B * Hq * M) * sizeof(float));
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
  w.delta = (float *)p;
  p += rup((size_t)(B * Hq * M) * sizeof(float));
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
                     (rot_k && pos) ? w.khat : nullptr, with_bias ? w.bias : nullptr);
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
    const int G = Hq / Hkv;
    const int BQ = 128 / G;
    const int nqb = (M + BQ - 1) / BQ;
    const dim3 grid((unsigned)(nqb * B * Hkv));
    const float c2 = (float)(c * 1.4426950408889634);
    const uint16_t *kh = pos ? w.khat : (const uint16_t *)k;
    if (D == 128)
      hipLaunchKernelGGL(attn_fwd_bf16_kernel<128>, grid, dim3(512), 0, s, (const uint16_t *)q, kh,
                         (const uint16_t *)v, w.bias, cs, c2, B, M, Hq, Hkv, G, BQ, nqb, (uint16_t *)o, lse);
    else
      hipLaunchKernelGGL(attn_fwd_bf16_kernel<64>, grid, dim3(512), 0, s, (const uint16_t *)q, kh,
                         (const uint16_t *)v, w.bias, cs, c2, B, M, Hq, Hkv, G, BQ, nqb, (uint16_t *)o, lse);
  } else {
    const int64_t rows = (int64_t)B * M * Hq;
    hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, (const float *)q,
                       (const float *)k, (const float *)v, g, gamma, cs, (float)c, B, M, Hq, Hkv, D, (float *)o,
                       lse);
  }
  return hipGetLastError();
}

}  // namespace tg
