// tg_attn.h -- attention workspace layout shared by the forward and backward launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tg {

struct AttnWs {
  float2 *cs;        // [B*M, D/2] (cos, sin) of the kept positions
  uint16_t *khat;    // [B, M, Hkv, D] rotated keys (bf16)
  float *bias;       // [B, Hq, M] gamma_h * log2 g_j (-inf where g_j <= 0)
  float *part;       // partial (O, max, sum) records of the forward's split query blocks
  int *cnt;          // [B*Hkv, nqb] arrival counters of the split query blocks
  int ncnt;
  float *ratio;      // [B, M] ln m_i / ln max(2, p_i), the temperature's row factor
  uint16_t *qhat;    // rotated queries (bf16): the backward's [B, M, Hq, D], or the forward's
                     // MFMA-fragment order [B, Hq, ceil(M / 32), D / 16, 64 lanes, 8]
  float2 *rowstat;   // [B, Hq, M] (-lse / c, D_i) of the backward (fp32 path: D_i alone)
  float *colsum;     // [B, Hq, M] column sums of dS per head
  float *tau;        // [B, Hq, Mp] temperature of each (row, head) of the backward, Mp = M rounded up
                     // to 32 (1 past M)
  float *tstat;      // [B, Hq, M] ratio_i * dL/dtau_ih, reduced into dsigma
};

// Split schedule of the bf16 forward (query block size, blocks, tiles per
// piece, pieces, pieces of split blocks).
struct FwdSched {
  int BQ, nqb, C, npieces, nmulti;
};
FwdSched fwd_sched(int64_t B, int64_t M, int64_t Hq, int64_t Hkv);

size_t attn_workspace_bytes(int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D, bool bwd);
AttnWs carve_attn_ws(void *ws, int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D);
hipError_t launch_attn_prep(const void *k, const float *g, const float *gamma, const int32_t *pos, double theta,
                            int B, int M, int Hq, int Hkv, int D, bool rot_k, bool with_bias, bool with_ratio,
                            bool g_per_head, const AttnWs &w, hipStream_t s, const void *q = nullptr);
hipError_t launch_attn_fwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                           const int32_t *pos, double theta, float tau, const float *sigma, int B, int M, int Hq,
                           int Hkv, int D, bool bf16, bool g_per_head, void *o, float *lse, const AttnWs &w,
                           hipStream_t s);
hipError_t launch_attn_bwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                           const int32_t *pos, double theta, float tau, const float *sigma, const float *lse,
                           const void *dout, int B, int M, int Hq, int Hkv, int D, bool bf16, bool g_per_head,
                           float *dq, float *dk, float *dv, float *dg, float *dgamma, float *dsigma, const AttnWs &w,
                           hipStream_t s);

hipError_t launch_sum_runs(const float *part, int nruns, int Hq, float *dgamma, float *dsigma, hipStream_t s);

// softplus in fp32 (the temperature's positive scale)
__device__ __forceinline__ float softplus_f(float x) { return x > 20.f ? x : log1pf(__expf(x)); }

}  // namespace tg
