// tg_attn.h -- attention workspace layout shared by the forward and backward launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

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

// Packed batches.  A run is n sequences of M tokens each, stored one after
// another from token off of the packed tensors; poff counts the padded tokens
// before it (each sequence's length rounded up to 32), which place the
// padded workspace arrays.  rec0 and cnt0 are the run's first partial record
// and first arrival counter of the forward's split query blocks, C the key
// tiles per piece of its forward (one value for all runs of a launch).
struct RunRow {
  int off, poff, n, M, rec0, cnt0, C;
};
constexpr int kMaxRuns = 16;  // runs per launch
constexpr int kMaxEnt = 256;  // work-group ranges per launch

// Work-group table of one launch over runs.  The launch's work-groups are
// cut into ranges; range e starts at work-group start[e] (start[0] = 0,
// INT_MAX past the last range) and holds whole blocks of one run, each block
// as n Hkv consecutive work-groups (batch row, kv head), the blocks numbered
// from blk0 upwards or downwards.  code[e] = run | blk0 << 8 | descending << 30.
struct RunTable {
  int start[kMaxEnt];
  int code[kMaxEnt];
  RunRow run[kMaxRuns];
};

struct Unit {
  int run, blk, bh;
};
// The run, block and (batch row * Hkv + kv head) of work-group w.
__host__ __device__ __forceinline__ Unit unit_of(const RunTable &rt, int w, int Hkv) {
  // the range: the last e with start[e] <= w (start rises from start[0] = 0,
  // INT_MAX past the last range); a binary search, uniform on the device
  int e = 0;
#pragma unroll
  for (int step = kMaxEnt / 2; step >= 1; step >>= 1)
    if (w >= rt.start[e + step]) e += step;
  const int code = rt.code[e];
  Unit u;
  u.run = code & 0xFF;
  const int nbh = rt.run[u.run].n * Hkv, loc = w - rt.start[e], blk0 = (code >> 8) & 0x3FFFFF;
  u.bh = loc % nbh;
  u.blk = (code >> 30) & 1 ? blk0 - loc / nbh : blk0 + loc / nbh;
  return u;
}

// One (run, block) group of n Hkv work-groups of equal cost.
struct Level {
  int run, blk;
  int64_t cost;
};
// Tables and grids of the launches over runs[0 .. nruns) (nruns <= kMaxRuns):
// the levels longest first (the dispatcher places work-groups in order on the
// first free compute unit, so this is a longest-processing-time schedule
// across the runs), consecutive blocks of one run merged into one range, at
// most kMaxEnt ranges per launch.
void make_tables(std::vector<Level> &lv, const RunRow *runs, int nruns, int Hkv, std::vector<RunTable> &tabs,
                 std::vector<unsigned> &grids);

// Runs of a packed batch and the workspace that holds all of them: the
// arrays of every run side by side (the layout of one run's workspace with
// B M tokens replaced by the runs' total, and the padded arrays by the
// padded total).  run_view gives one run's part of it as a workspace of its
// own.  plan_runs sets each run's placement and its forward's C, one per
// group of kMaxRuns consecutive runs (the runs one forward launch takes).
void plan_runs(RunRow *runs, int nruns, int64_t Hq, int64_t Hkv, int64_t D);
size_t attn_workspace_bytes_runs(const RunRow *runs, int nruns, int64_t Hq, int64_t Hkv, int64_t D, bool bwd);
AttnWs carve_attn_ws_runs(void *ws, const RunRow *runs, int nruns, int64_t Hq, int64_t Hkv, int64_t D);
AttnWs run_view(const AttnWs &w, const RunRow &r, int64_t Hq, int64_t Hkv, int64_t D);

// Split schedule of the bf16 forward (query block size, blocks, tiles per
// piece, pieces, pieces of split blocks).  fwd_sched_c: the schedule with C
// tiles per piece; fwd_sched: with the C chosen for the batch alone.
struct FwdSched {
  int BQ, nqb, C, npieces, nmulti;
};
FwdSched fwd_sched(int64_t B, int64_t M, int64_t Hq, int64_t Hkv);
FwdSched fwd_sched_c(int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int C);

// Work-group tables of the bf16 forward over runs[0 .. nruns) (one group of
// at most kMaxRuns runs, planned by plan_runs, so every run has the same C).
// A level is one query block of one run with all its pieces (n Hkv
// work-groups per piece, the pieces outer).  Levels of split blocks come
// first, each run's from its top block down (their records are numbered from
// the top); then the unsplit blocks longest first.  A range holds the blocks
// blk0, blk0 - 1, ... of one run (code bit 30 clear), or block blk0 of the
// runs run, run + 1, ... (bit 30 set; unsplit blocks only).
// code[e] = run | blk0 << 8 | across_runs << 30.  Returns false when a table
// cannot hold the schedule (never for the shapes the planner admits).
bool make_fwd_tables(const RunRow *runs, int nruns, int64_t Hq, int64_t Hkv, std::vector<RunTable> &tabs,
                     std::vector<unsigned> &grids);

size_t attn_workspace_bytes(int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D, bool bwd);
AttnWs carve_attn_ws(void *ws, int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D);
hipError_t launch_attn_prep(const void *k, const float *g, const float *gamma, const int32_t *pos, double theta,
                            int B, int M, int Hq, int Hkv, int D, bool rot_k, bool with_bias, bool with_ratio,
                            bool g_per_head, const AttnWs &w, hipStream_t s, const void *q = nullptr);
hipError_t launch_attn_fwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                           const int32_t *pos, double theta, float tau, const float *sigma, int B, int M, int Hq,
                           int Hkv, int D, bool bf16, bool g_per_head, void *o, float *lse, void *o_lo,
                           const AttnWs &w, hipStream_t s);
// The prep pass over one group of at most kMaxRuns consecutive runs of a
// packed batch, in one launch: the angles, rotated keys (bf16, with positions),
// biases (one gate per key), temperature ratios (with_ratio), and with q the
// forward's query fragments; the group's arrival counters cleared.
hipError_t launch_attn_prep_runs(const void *k, const float *g, const float *gamma, const int32_t *pos, double theta,
                                 const RunRow *runs, int nruns, int Hq, int Hkv, int D, bool with_ratio,
                                 const AttnWs &w, hipStream_t s, const void *q);
// bf16 forward over the runs of a packed batch (planned by plan_runs; w is
// the workspace of all runs): per group of kMaxRuns runs one prep launch and
// one forward launch per work-group table.  The tensors are the packed ones.
hipError_t launch_attn_fwd_runs(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                                const int32_t *pos, double theta, float tau, const float *sigma, const RunRow *runs,
                                int nruns, int Hq, int Hkv, int D, void *o, float *lse, void *o_lo, const AttnWs &w,
                                hipStream_t s);
// Backward over the runs of a packed batch (one run: an ordinary batch).
// The tensors are the packed ones; w is the workspace of all runs.  With o
// and o_lo (bf16) the row terms D_i come from dO . (o + o_lo).  With
// one run dgamma / dsigma receive the sums; with several, part holds 2 Hq
// floats per run (its dgamma, then its dsigma shares) and one fixed-order
// pass sums them into dgamma / dsigma.
hipError_t launch_attn_bwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                           const int32_t *pos, double theta, float tau, const float *sigma, const float *lse,
                           const void *dout, const void *o, const void *o_lo, const RunRow *runs, int nruns, int Hq,
                           int Hkv, int D, bool bf16, bool g_per_head, float *dq, float *dk, float *dv, float *dg,
                           float *dgamma, float *dsigma, float *part, const AttnWs &w, hipStream_t s);

hipError_t launch_sum_runs(const float *part, int nruns, int Hq, float *dgamma, float *dsigma, hipStream_t s);

// softplus in fp32 (the temperature's positive scale)
__device__ __forceinline__ float softplus_f(float x) { return x > 20.f ? x : log1pf(__expf(x)); }

}  // namespace tg
