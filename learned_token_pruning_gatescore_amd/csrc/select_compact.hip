// select_compact.hip -- scaffold-aware top-K selection and the gather of the
// kept tokens.
//
// TokenGate deep dive ("TokenGate: Learnable Token Pruning for Fast,
// Memory-Efficient LLM Prefill"): section 3.1, Eq. 4 (S = top-K of the
// prunable set by score, united with the non-prunable set) and section 3.4
// (budget clamped, full-sequence keep mask, hidden states and position ids
// sliced with the keep indices).
//
// Selection is an exact radix select over a 32-bit order key of the fp32
// score.  Rows of up to 32768 tokens take one work-group each (described with
// its kernel below); longer rows are spread over many work-groups per row
// (4096 tokens each) in three launches:
//   1. histogram: each work-group histograms the top 12 key bits of its
//      prunable tokens in LDS and writes the 4096 counts (and their 256
//      coarse sums, and its forced count) to its own slot of the workspace;
//   2. refine: every work-group finds, from the slots, the 12-bit bin d0 that
//      holds the K'-th best prunable key (coarse bins first), writes its own
//      tokens of that bin as (key, index) candidates at a fixed offset, and
//      its count of surely kept tokens (forced, or a bin above d0); the last
//      work-group of the row to arrive resolves the exact threshold key T and
//      the tie quota from the candidates (two 10-bit LDS passes) and turns
//      the per-work-group counts into output offsets;
//   3. emit: each work-group writes its kept indices, ascending, at its offset
//      (forced tokens, keys above T, and the first quota keys equal to T in
//      index order across the row).
// Every count is an integer and every position comes from a prefix sum, so
// the output is deterministic; the workspace needs no initial contents (each
// launch writes what the next one reads).
#include <mutex>

#include "tg_common.h"

namespace tg {

// Monotone map of fp32 onto uint32 for the ranking: NaN -> 0 (lowest),
// -0 -> +0, then sign-magnitude to unsigned order.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}


constexpr int SEL_T = 1024;              // threads per batch row
constexpr int SEL_I = 32;                // tokens per thread per chunk (a contiguous segment)
constexpr int SEL_CHUNK = SEL_T * SEL_I; // 32768 tokens per chunk
constexpr int SEL_W = SEL_T / 64;        // waves per work-group

// Block-wide exclusive scans of two uint32 values over the SEL_W waves.
__device__ __forceinline__ void block_exscan2(uint32_t a, uint32_t b, uint32_t &ea, uint32_t &eb, uint32_t &ta,
                                              uint32_t &tb, uint32_t *sw, int tid) {
  const int lane = tid & 63, wave = tid >> 6;
  uint32_t xa = a, xb = b;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t ya = __shfl_up(xa, o), yb = __shfl_up(xb, o);
    if (lane >= o) {
      xa += ya;
      xb += yb;
    }
  }
  if (lane == 63) {
    sw[wave] = xa;
    sw[SEL_W + wave] = xb;
  }
  __syncthreads();
  if (wave == 0) {
    uint32_t wa = lane < SEL_W ? sw[lane] : 0u, wb = lane < SEL_W ? sw[SEL_W + lane] : 0u;
    for (int o = 1; o < SEL_W; o <<= 1) {
      const uint32_t ya = __shfl_up(wa, o), yb = __shfl_up(wb, o);
      if (lane >= o) {
        wa += ya;
        wb += yb;
      }
    }
    if (lane < SEL_W) {
      sw[lane] = wa;
      sw[SEL_W + lane] = wb;
    }
  }
  __syncthreads();
  ea = (wave ? sw[wave - 1] : 0u) + xa - a;
  eb = (wave ? sw[SEL_W + wave - 1] : 0u) + xb - b;
  ta = sw[SEL_W - 1];
  tb = sw[2 * SEL_W - 1];
  __syncthreads();
}

// Finds the bin holding the need-th largest candidate.  Bins are scanned from
// the top; thread t owns BPT consecutive bins of group (SEL_T - 1 - t).  Writes
// the bin and the remaining need (rank inside the bin) to res[0], res[1].
template <int BPT>
__device__ __forceinline__ void find_bin(const uint32_t *hist, uint32_t need, uint32_t *res, uint32_t *sw, int tid) {
  const int g = SEL_T - 1 - tid;
  uint32_t h[BPT], loc = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    h[j] = hist[g * BPT + (BPT - 1 - j)];  // descending bins
    loc += h[j];
  }
  uint32_t above, dummy, tot, tot2;
  block_exscan2(loc, 0u, above, dummy, tot, tot2, sw, tid);
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    if (above < need && need <= above + h[j]) {
      res[0] = (uint32_t)(g * BPT + (BPT - 1 - j));
      res[1] = need - above;
    }
    above += h[j];
  }
  __syncthreads();
}

// Rows of up to 32768 tokens: one work-group per batch row, thread t owning
// the contiguous segment [t*32, t*32+32), whose 32 keys stay in registers for
// every pass (three digit passes, 12/10/10 bits, over an LDS histogram).
// Forced / valid / candidate flags are 32-bit masks, so the output positions
// of a segment come from popcounts of masks rather than from a dependent
// counter chain.  (A single work-group has no global synchronisation: at
// this size that is faster than spreading the rows, where every exchange
// between work-groups costs a few microseconds.)
template <bool RES>
__global__ __launch_bounds__(SEL_T) void select_topk_kernel(
    const float *__restrict__ scores, const uint8_t *__restrict__ forced, int64_t N, int64_t K,
    int64_t M_alloc, int32_t *__restrict__ kept, int32_t *__restrict__ kept_count) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t sw[2 * SEL_W];
  __shared__ uint32_t res[4];

  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t b = blockIdx.x;
  const float *sc = scores + b * N;
  const uint8_t *fo = forced ? forced + b * N : nullptr;
  int32_t *out = kept + b * M_alloc;
  // one chunk (N <= 32768): a compile-time single trip, so the keys die after their last use
  const int nchunks = RES ? 1 : (int)((N + SEL_CHUNK - 1) / SEL_CHUNK);
  const bool vec_s = ((uintptr_t)sc & 15) == 0;
  const bool vec_f = fo && ((uintptr_t)fo & 15) == 0;

  uint32_t key[SEL_I];
  uint32_t fbits = 0, vbits = 0;  // forced / valid (n < N) bit per item of this thread's segment
  auto load = [&](int c) {
    const int64_t n0 = (int64_t)c * SEL_CHUNK + (int64_t)tid * SEL_I;
    const int64_t cnt64 = N - n0;
    const int cnt = cnt64 <= 0 ? 0 : (cnt64 >= SEL_I ? SEL_I : (int)cnt64);
    vbits = cnt >= 32 ? 0xFFFFFFFFu : ((1u << cnt) - 1u);
    if (cnt == SEL_I && vec_s && (!fo || vec_f)) {
      // every load of the segment in flight before the first use
      f32x4 x[SEL_I / 4];
      u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int v = 0; v < SEL_I / 4; ++v) x[v] = *(const f32x4 *)(sc + n0 + 4 * v);
      if (fo) {
        x0 = *(const u32x4 *)(fo + n0);
        x1 = *(const u32x4 *)(fo + n0 + 16);
      }
#pragma unroll
      for (int v = 0; v < SEL_I / 4; ++v)
#pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * v + e] = order_key(x[v][e]);
      fbits = 0;
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          fbits |= (((x0[w] >> (8 * e)) & 0xFFu) ? 1u : 0u) << (4 * w + e);
          fbits |= (((x1[w] >> (8 * e)) & 0xFFu) ? 1u : 0u) << (16 + 4 * w + e);
        }
      return;
    }
    if (cnt == SEL_I && vec_s) {
#pragma unroll
      for (int v = 0; v < SEL_I / 4; ++v) {
        const f32x4 x = *(const f32x4 *)(sc + n0 + 4 * v);
#pragma unroll
        for (int e = 0; e < 4; ++e) key[4 * v + e] = order_key(x[e]);
      }
    } else {
#pragma unroll
      for (int i = 0; i < SEL_I; ++i) key[i] = i < cnt ? order_key(sc[n0 + i]) : 0u;
    }
    fbits = 0;
    if (fo) {
      if (cnt == SEL_I && vec_f) {
        const u32x4 x0 = *(const u32x4 *)(fo + n0), x1 = *(const u32x4 *)(fo + n0 + 16);
#pragma unroll
        for (int w = 0; w < 4; ++w)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            fbits |= (((x0[w] >> (8 * e)) & 0xFFu) ? 1u : 0u) << (4 * w + e);
            fbits |= (((x1[w] >> (8 * e)) & 0xFFu) ? 1u : 0u) << (16 + 4 * w + e);
          }
      } else {
        for (int i = 0; i < cnt; ++i) fbits |= (fo[n0 + i] ? 1u : 0u) << i;
      }
    }
  };

  for (int i = tid; i < 4096; i += SEL_T) hist[i] = 0;
  if (tid == 0) res[2] = 0;
  if (RES) load(0);
  __syncthreads();

  // Pass 0: forced count and the histogram of the top 12 key bits of prunable tokens.
  uint32_t nf = 0;
  for (int c = 0; c < nchunks; ++c) {
    if (!RES) load(c);
    nf += (uint32_t)__popc(fbits & vbits);
    const uint32_t cbits = vbits & ~fbits;
    // One LDS atomic per candidate.  A wave whose 2048 candidates all share one
    // key (a constant score vector) adds its count with a single atomic instead
    // of 2048 serialised ones.
    bool same = cbits == 0xFFFFFFFFu;
#pragma unroll
    for (int i = 1; i < SEL_I; ++i) same = same && key[i] == key[0];
    const uint32_t k0 = __shfl(key[0], 0);
    if (__all(same && key[0] == k0)) {
      if (lane == 0) atomicAdd(&hist[k0 >> 20], 64u * SEL_I);
    } else {
#pragma unroll
      for (int i = 0; i < SEL_I; ++i)
        if ((cbits >> i) & 1u) atomicAdd(&hist[key[i] >> 20], 1u);
    }
  }
  for (int o = 32; o > 0; o >>= 1) nf += __shfl_xor(nf, o);
  if (lane == 0 && nf) atomicAdd(&res[2], nf);
  __syncthreads();
  const int64_t nF = res[2];
  const int64_t nP = N - nF;
  const int64_t Kc = K < nP ? K : nP;
  const int64_t M_true = nF + Kc;

  // Threshold key and tie quota.  Kc == nP: keep all (thr 0 is the lowest key,
  // unlimited quota); Kc == 0: keep none (no key equals 0xFFFFFFFF).
  uint32_t thr;
  int64_t quota;
  if (Kc >= nP) {
    thr = 0u;
    quota = INT64_MAX;
  } else if (Kc <= 0) {
    thr = 0xFFFFFFFFu;
    quota = 0;
  } else {
    find_bin<4096 / SEL_T>(hist, (uint32_t)Kc, res, sw, tid);
    const uint32_t d0 = res[0];
    uint32_t need = res[1];
    for (int i = tid; i < 1024; i += SEL_T) hist[i] = 0;
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {  // few candidates remain: plain predicated atomics
      if (!RES) load(c);
      const uint32_t cbits = vbits & ~fbits;
#pragma unroll
      for (int i = 0; i < SEL_I; ++i)
        if (((cbits >> i) & 1u) && (key[i] >> 20) == d0) atomicAdd(&hist[(key[i] >> 10) & 1023u], 1u);
    }
    __syncthreads();
    find_bin<1024 / SEL_T>(hist, need, res, sw, tid);
    const uint32_t p1 = (d0 << 10) | res[0];
    need = res[1];
    for (int i = tid; i < 1024; i += SEL_T) hist[i] = 0;
    __syncthreads();
    for (int c = 0; c < nchunks; ++c) {
      if (!RES) load(c);
      const uint32_t cbits = vbits & ~fbits;
#pragma unroll
      for (int i = 0; i < SEL_I; ++i)
        if (((cbits >> i) & 1u) && (key[i] >> 10) == p1) atomicAdd(&hist[key[i] & 1023u], 1u);
    }
    __syncthreads();
    find_bin<1024 / SEL_T>(hist, need, res, sw, tid);
    thr = (p1 << 10) | res[0];
    quota = res[1];
  }

  // Output: ascending kept indices.  Per segment: mask of tokens kept without a
  // tie (forced, or key > thr) and mask of tied tokens (key == thr); one block
  // scan of their popcounts gives each segment its offsets, and the first
  // `quota` ties in index order are kept.
  int64_t runK = 0, runT = 0;
  for (int c = 0; c < nchunks; ++c) {
    if (!RES) load(c);
    uint32_t km = fbits & vbits, tm = 0;
#pragma unroll
    for (int i = 0; i < SEL_I; ++i) {
      const uint32_t bit = 1u << i;
      const bool cand = (vbits & ~fbits & bit) != 0;
      km |= (cand && key[i] > thr) ? bit : 0u;
      tm |= (cand && key[i] == thr) ? bit : 0u;
    }
    uint32_t ek, et, tk, tt;
    block_exscan2((uint32_t)__popc(km), (uint32_t)__popc(tm), ek, et, tk, tt, sw, tid);
    const int64_t kb = runK + ek, tb = runT + et;
    const int64_t n0 = (int64_t)c * SEL_CHUNK + (int64_t)tid * SEL_I;
    // a tie at item i is kept when tb + (ties before i in the segment) < quota
    const int64_t tq = quota - tb;  // ties of this segment that can still be kept
    uint32_t tkeep = tm;
    if (tq <= 0) {
      tkeep = 0u;
    } else if (tq < 32) {
      // keep the first tq set bits of tm
      uint32_t m = tm;
      for (int64_t r = 0; r < tq && m; ++r) m &= m - 1u;  // clear the lowest tq bits
      tkeep = tm & ~m;
    }
    const uint32_t all = km | tkeep;
    const int64_t p = kb + (tb < quota ? tb : quota);
    // this segment's kept tokens in ascending order: item i goes to p + (kept items before i)
    if (all) {
      int32_t *op = out + p;
      const int64_t room = M_alloc - p;
#pragma unroll
      for (int i = 0; i < SEL_I; ++i) {
        const int r = __popc(all & ((1u << i) - 1u));
        if (((all >> i) & 1u) && r < room) op[r] = (int32_t)(n0 + i);
      }
    }
    runK += tk;
    runT += tt;
  }
  const int64_t written = M_true < M_alloc ? M_true : M_alloc;
  for (int64_t m = written + tid; m < M_alloc; m += SEL_T) out[m] = -1;
  if (tid == 0 && kept_count) kept_count[b] = (int32_t)M_true;
}

constexpr int SEL_TPB = 256;               // threads per work-group
constexpr int SEL_IPT = 16;                // tokens per thread (a contiguous segment)
constexpr int SEL_TW = SEL_TPB * SEL_IPT;  // 4096 tokens per work-group
constexpr int SEL_NF = 4096;               // bins of the first digit (top 12 key bits)
constexpr int SEL_NC = 256;                // coarse bins (top 8 key bits)
constexpr int SEL_GMAX = 1024;             // work-groups per row (N <= 4 Mi tokens)
constexpr int SEL_CCAP = 4096;             // candidates the resolve keeps in LDS
constexpr int SEL_NW = SEL_TPB / 64;

enum : uint32_t { SEL_NORMAL = 0, SEL_ALL = 1, SEL_NONE = 2 };

// Workspace (see select_ws_bytes): per row b and work-group w of the row
//   coarse [B][G][256], fine [B][G][4096], nf [B][G] (forced tokens),
//   sure [B][G] (forced + keys in a bin above d0), wgp [B][G][2] (output
//   offset, tie quota), rowp [B][8] (arrival counter, mode, T, kept count),
//   cand [B][N] u64 ((key << 32) | token index).
struct SelWs {
  uint32_t *coarse, *fine, *nf, *sure, *wgp, *rowp;
  uint64_t *cand;
};

__host__ __device__ inline int sel_groups(int64_t N) { return N <= SEL_TW ? 1 : (int)((N + SEL_TW - 1) / SEL_TW); }

// This thread's 16 tokens n0 .. n0+15 of a row: order keys, forced bits,
// valid bits (n < N).  16-byte loads where the whole segment is aligned.
__device__ __forceinline__ void sel_load(const float *sc, const uint8_t *fo, int64_t N, int64_t n0,
                                         uint32_t (&key)[SEL_IPT], uint32_t &fbits, uint32_t &vbits) {
  const int64_t c64 = N - n0;
  const int cnt = c64 <= 0 ? 0 : (c64 >= SEL_IPT ? SEL_IPT : (int)c64);
  vbits = cnt >= SEL_IPT ? 0xFFFFu : ((1u << cnt) - 1u);
  fbits = 0;
  if (cnt == SEL_IPT && ((uintptr_t)(sc + n0) & 15) == 0) {
    f32x4 x[SEL_IPT / 4];
#pragma unroll
    for (int v = 0; v < SEL_IPT / 4; ++v) x[v] = *(const f32x4 *)(sc + n0 + 4 * v);
    u32x4 m = {0u, 0u, 0u, 0u};
    const bool vf = fo && ((uintptr_t)(fo + n0) & 15) == 0;
    if (vf) m = *(const u32x4 *)(fo + n0);
#pragma unroll
    for (int v = 0; v < SEL_IPT / 4; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) key[4 * v + e] = order_key(x[v][e]);
    if (vf) {
#pragma unroll
      for (int wd = 0; wd < 4; ++wd)
#pragma unroll
        for (int e = 0; e < 4; ++e) fbits |= (((m[wd] >> (8 * e)) & 0xFFu) ? 1u : 0u) << (4 * wd + e);
    } else if (fo) {
#pragma unroll
      for (int i = 0; i < SEL_IPT; ++i) fbits |= (fo[n0 + i] ? 1u : 0u) << i;
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < SEL_IPT; ++i) key[i] = i < cnt ? order_key(sc[n0 + i]) : 0u;
  if (fo)
    for (int i = 0; i < cnt; ++i) fbits |= (fo[n0 + i] ? 1u : 0u) << i;
}

// Block-wide sum and exclusive scan of one uint32 per thread (256 threads).
__device__ __forceinline__ uint32_t sel_block_sum(uint32_t v, uint32_t *red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  uint32_t t = 0;
#pragma unroll
  for (int i = 0; i < SEL_NW; ++i) t += red[i];
  __syncthreads();
  return t;
}
__device__ __forceinline__ uint32_t sel_block_exscan(uint32_t v, uint32_t *red, uint32_t &total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) red[wave] = x;
  __syncthreads();
  uint32_t before = 0;
  total = 0;
#pragma unroll
  for (int i = 0; i < SEL_NW; ++i) {
    before += i < wave ? red[i] : 0u;
    total += red[i];
  }
  __syncthreads();
  return before + x - v;
}

// Finds, over the 256 bins held one per thread in descending order (thread t
// holds the bin ranked t from the top), the bin where the running count from
// the top first reaches need; the owner writes (t, need left inside the bin)
// to res.
__device__ __forceinline__ void sel_find_desc(uint32_t cnt, uint32_t need, uint32_t *red, uint32_t *res) {
  uint32_t tot;
  const uint32_t above = sel_block_exscan(cnt, red, tot);
  if (above < need && need <= above + cnt) {
    res[0] = threadIdx.x;
    res[1] = need - above;
  }
  __syncthreads();
}

// Pass 1 (grid G x B): per work-group histogram of the top 12 key bits of its
// prunable tokens, written with its coarse sums and forced count to its slot.
__global__ __launch_bounds__(SEL_TPB) void select_hist_kernel(const float *__restrict__ scores,
                                                              const uint8_t *__restrict__ forced, int64_t N, int G,
                                                              SelWs ws) {
  __shared__ __attribute__((aligned(16))) uint32_t hist[SEL_NF];
  __shared__ uint32_t red[SEL_NW];
  const int tid = threadIdx.x, w = blockIdx.x;
  const int64_t b = blockIdx.y;
  const float *sc = scores + b * N;
  const uint8_t *fo = forced ? forced + b * N : nullptr;
  uint32_t key[SEL_IPT], fbits, vbits;
  sel_load(sc, fo, N, (int64_t)w * SEL_TW + (int64_t)tid * SEL_IPT, key, fbits, vbits);
#pragma unroll
  for (int i = 0; i < SEL_NF / SEL_TPB; ++i) hist[tid + SEL_TPB * i] = 0u;
  __syncthreads();
  // runs of equal digits inside the segment go in with one atomic (a constant
  // score vector costs one atomic per thread, not sixteen)
  const uint32_t cb = vbits & ~fbits;
  uint32_t run_d = 0u, run_n = 0u;
#pragma unroll
  for (int i = 0; i < SEL_IPT; ++i) {
    if ((cb >> i) & 1u) {
      const uint32_t d = key[i] >> 20;
      if (run_n && d == run_d) {
        ++run_n;
      } else {
        if (run_n) atomicAdd(&hist[run_d], run_n);
        run_d = d;
        run_n = 1u;
      }
    }
  }
  if (run_n) atomicAdd(&hist[run_d], run_n);
  const uint32_t nf = sel_block_sum((uint32_t)__popc(fbits & vbits), red);  // (its barrier also orders the LDS atomics)
  const int64_t slot = b * G + w;
  const u32x4 *hv = (const u32x4 *)(hist + SEL_IPT * tid);
  u32x4 *fs = (u32x4 *)(ws.fine + slot * SEL_NF + SEL_IPT * tid);
  uint32_t csum = 0u;
#pragma unroll
  for (int v = 0; v < SEL_IPT / 4; ++v) {
    const u32x4 x = hv[v];
    fs[v] = x;
    csum += x[0] + x[1] + x[2] + x[3];
  }
  ws.coarse[slot * SEL_NC + tid] = csum;
  if (tid == 0) {
    ws.nf[slot] = nf;
    if (w == 0) ws.rowp[b * 8] = 0u;  // the arrival counter of pass 2
  }
}

// Pass 2 (grid G x B): the bin d0 of the threshold from every slot, this
// work-group's candidates (keys in d0) at their fixed offset and its surely
// kept count; the last work-group of the row resolves T, the tie quota and
// every work-group's output offset.
__global__ __launch_bounds__(SEL_TPB) void select_refine_kernel(const float *__restrict__ scores,
                                                                const uint8_t *__restrict__ forced, int64_t N,
                                                                int64_t K, int G, SelWs ws,
                                                                int32_t *__restrict__ kept_count) {
  __shared__ uint32_t red[SEL_NW];
  __shared__ uint32_t res[4];
  __shared__ uint32_t sF[16];
  __shared__ uint32_t hA[1024];
  __shared__ uint32_t s_above[SEL_GMAX], s_ties[SEL_GMAX];
  __shared__ uint64_t scand[SEL_CCAP];
  __shared__ uint32_t s_last;
  const int tid = threadIdx.x, w = blockIdx.x;
  const int64_t b = blockIdx.y;
  const float *sc = scores + b * N;
  const uint8_t *fo = forced ? forced + b * N : nullptr;
  const int64_t n0 = (int64_t)w * SEL_TW + (int64_t)tid * SEL_IPT;
  uint32_t key[SEL_IPT], fbits, vbits;
  sel_load(sc, fo, N, n0, key, fbits, vbits);  // issued first: it does not depend on the slots
  const int64_t slot0 = b * G;
  if (tid == 0) {  // in-range bins even if a search below found nothing
    res[0] = res[2] = 0u;
    res[1] = res[3] = 1u;
  }

  // global coarse histogram (thread t: coarse bin 255 - t, descending) and forced count; the
  // slots' loads go out eight at a time (one at a time, each waited for, they cost a memory
  // round trip per work-group of the row)
  uint32_t c = 0u;
  {
    const uint32_t *cp = ws.coarse + slot0 * SEL_NC + (SEL_NC - 1 - tid);
    int g = 0;
    for (; g + 8 <= G; g += 8) {
      uint32_t x[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = cp[(g + j) * SEL_NC];
#pragma unroll
      for (int j = 0; j < 8; ++j) c += x[j];
    }
    for (; g < G; ++g) c += cp[g * SEL_NC];
  }
  uint32_t nfp = 0u;
  for (int g = tid; g < G; g += SEL_TPB) nfp += ws.nf[slot0 + g];
  const int64_t nF = sel_block_sum(nfp, red);
  const int64_t nP = N - nF;
  const int64_t Kc = K < nP ? K : nP;
  const uint32_t mode = Kc >= nP ? SEL_ALL : (Kc <= 0 ? SEL_NONE : SEL_NORMAL);
  int d0 = mode == SEL_ALL ? -1 : SEL_NF;  // keys in bins above d0 are kept for sure
  uint32_t need = 0u, ctot = 0u, coff = 0u;
  if (mode == SEL_NORMAL) {
    sel_find_desc(c, (uint32_t)Kc, red, res);
    const int c0 = SEL_NC - 1 - (int)res[0];
    const uint32_t need0 = res[1];
    if (tid < 16) sF[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < 16 * G; i += SEL_TPB) atomicAdd(&sF[i & 15], ws.fine[(slot0 + (i >> 4)) * SEL_NF + 16 * c0 + (i & 15)]);
    __syncthreads();
    if (tid == 0) {  // 16 fine bins from the top
      uint32_t above = 0u;
      for (int j = 15; j >= 0; --j) {
        if (above < need0 && need0 <= above + sF[j]) {
          res[2] = (uint32_t)j;
          res[3] = need0 - above;
          break;
        }
        above += sF[j];
      }
    }
    __syncthreads();
    d0 = 16 * c0 + (int)res[2];
    need = res[3];
    ctot = sF[res[2]];
    // this work-group's candidate offset: the d0 counts of the work-groups before it
    uint32_t part = 0u;
    for (int g = tid; g < w; g += SEL_TPB) part += ws.fine[(slot0 + g) * SEL_NF + d0];
    coff = sel_block_sum(part, red);
  }

  // own tokens: surely kept (forced, or a bin above d0) and candidates (bin d0)
  const uint32_t cb = vbits & ~fbits;
  uint32_t cm = 0u, sure = (uint32_t)__popc(fbits & vbits);
#pragma unroll
  for (int i = 0; i < SEL_IPT; ++i) {
    const int dg = (int)(key[i] >> 20);
    if ((cb >> i) & 1u) {
      sure += dg > d0 ? 1u : 0u;
      cm |= dg == d0 ? (1u << i) : 0u;
    }
  }
  uint32_t ncw;
  const uint32_t cpos = sel_block_exscan((uint32_t)__popc(cm), red, ncw);
  // Candidates and the count of surely kept tokens go out as agent-scope
  // relaxed atomic stores (written where every XCD reads them, not left in
  // this XCD's L2), and the row's last work-group reads them back with
  // agent-scope loads; s_waitcnt vmcnt(0) and the barrier put every store of
  // the work-group before its arrival.  A device-scope fence instead writes
  // back and invalidates the whole L2 on this chip (on both sides).
  {
    uint64_t *dst = ws.cand + b * N + coff + cpos;
    int r = 0;
#pragma unroll
    for (int i = 0; i < SEL_IPT; ++i)
      if ((cm >> i) & 1u)
        __hip_atomic_store(dst + r++, ((uint64_t)key[i] << 32) | (uint64_t)(n0 + i), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
  }
  const uint32_t sure_w = sel_block_sum(sure, red);
  if (tid == 0) __hip_atomic_store(&ws.sure[slot0 + w], sure_w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // publish, count arrivals; the last work-group of the row goes on
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(&ws.rowp[b * 8], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             (uint32_t)(G - 1);
  __syncthreads();
  if (!s_last) return;
  auto ld_cand = [&](const uint64_t *p) { return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };

  for (int g = tid; g < G; g += SEL_TPB) s_above[g] = s_ties[g] = 0u;
  uint32_t T = mode == SEL_ALL ? 0u : 0xFFFFFFFFu, quota = 0u;
  if (mode == SEL_NORMAL) {
    // exact threshold inside bin d0: two 10-bit passes over the candidates
    const uint64_t *cg = ws.cand + b * N;
    const bool in_lds = ctot <= (uint32_t)SEL_CCAP;
    if (in_lds) {  // eight loads in flight per thread
      uint32_t i0 = 0;
      for (; i0 + 8 * SEL_TPB <= ctot; i0 += 8 * SEL_TPB) {
        uint64_t x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = ld_cand(cg + i0 + j * SEL_TPB + tid);
#pragma unroll
        for (int j = 0; j < 8; ++j) scand[i0 + j * SEL_TPB + tid] = x[j];
      }
      for (uint32_t i = i0 + tid; i < ctot; i += SEL_TPB) scand[i] = ld_cand(cg + i);
    }
    auto cand = [&](uint32_t i) -> uint64_t { return in_lds ? scand[i] : ld_cand(cg + i); };
    uint32_t pre = (uint32_t)d0 << 10;  // key >> 10 of the keys still in play
    for (int pass = 0; pass < 2; ++pass) {
      const int sh = pass == 0 ? 10 : 0;
      for (int i = tid; i < 1024; i += SEL_TPB) hA[i] = 0u;
      __syncthreads();
      for (uint32_t i = tid; i < ctot; i += SEL_TPB) {
        const uint32_t k = (uint32_t)(cand(i) >> 32);
        if (pass == 0 || (k >> 10) == pre) atomicAdd(&hA[(k >> sh) & 1023u], 1u);
      }
      __syncthreads();
      // 1024 bins from the top, four per thread
      uint32_t h4[4], loc = 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        h4[j] = hA[1023 - (4 * tid + j)];
        loc += h4[j];
      }
      uint32_t tot;
      uint32_t above = sel_block_exscan(loc, red, tot);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (above < need && need <= above + h4[j]) {
          res[0] = 1023u - (uint32_t)(4 * tid + j);
          res[1] = need - above;
        }
        above += h4[j];
      }
      __syncthreads();
      if (pass == 0) pre = ((uint32_t)d0 << 10) | res[0];
      else T = (pre << 10) | res[0];
      need = res[1];
      __syncthreads();
    }
    quota = need;
    for (uint32_t i = tid; i < ctot; i += SEL_TPB) {
      const uint64_t x = cand(i);
      const uint32_t k = (uint32_t)(x >> 32);
      const int g = (int)((uint32_t)x / (uint32_t)SEL_TW);
      if (k > T) atomicAdd(&s_above[g], 1u);
      else if (k == T) atomicAdd(&s_ties[g], 1u);
    }
  }
  __syncthreads();
  // output offsets: thread t owns work-groups 4t .. 4t+3 (G <= 1024)
  uint32_t sv[4], tv[4], lt = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = 4 * tid + j;
    tv[j] = g < G ? s_ties[g] : 0u;
    lt += tv[j];
  }
  uint32_t tt;
  uint32_t tb = sel_block_exscan(lt, red, tt);  // ties of the work-groups before
  uint32_t lk = 0u, qv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = 4 * tid + j;
    qv[j] = tb >= quota ? 0u : (quota - tb < tv[j] ? quota - tb : tv[j]);  // ties this work-group keeps
    sv[j] = g < G ? __hip_atomic_load(&ws.sure[slot0 + g], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + s_above[g] +
                        qv[j]
                  : 0u;
    tb += tv[j];
    lk += sv[j];
  }
  uint32_t mtot;
  uint32_t ob = sel_block_exscan(lk, red, mtot);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int g = 4 * tid + j;
    if (g < G) {
      ws.wgp[(slot0 + g) * 2] = ob;
      ws.wgp[(slot0 + g) * 2 + 1] = qv[j];
    }
    ob += sv[j];
  }
  if (tid == 0) {
    ws.rowp[b * 8 + 1] = mode;
    ws.rowp[b * 8 + 2] = T;
    ws.rowp[b * 8 + 3] = mtot;
    if (kept_count) kept_count[b] = (int32_t)mtot;
  }
}

// Pass 3 (grid G x B): each work-group writes its kept indices, ascending, at
// its offset; the row's last work-group pads the rest of the row with -1.
__global__ __launch_bounds__(SEL_TPB) void select_emit_kernel(const float *__restrict__ scores,
                                                              const uint8_t *__restrict__ forced, int64_t N,
                                                              int64_t M_alloc, int G, SelWs ws,
                                                              int32_t *__restrict__ kept) {
  __shared__ uint32_t red[SEL_NW];
  const int tid = threadIdx.x, w = blockIdx.x;
  const int64_t b = blockIdx.y;
  const int64_t n0 = (int64_t)w * SEL_TW + (int64_t)tid * SEL_IPT;
  uint32_t key[SEL_IPT], fbits, vbits;
  sel_load(scores + b * N, forced ? forced + b * N : nullptr, N, n0, key, fbits, vbits);
  const uint32_t mode = ws.rowp[b * 8 + 1], T = ws.rowp[b * 8 + 2], mtrue = ws.rowp[b * 8 + 3];
  const uint32_t off = ws.wgp[(b * G + w) * 2], tq = ws.wgp[(b * G + w) * 2 + 1];
  const uint32_t cb = vbits & ~fbits;
  uint32_t km = fbits & vbits, tm = 0u;
  if (mode == SEL_ALL) {
    km |= cb;
  } else if (mode == SEL_NORMAL) {
#pragma unroll
    for (int i = 0; i < SEL_IPT; ++i) {
      km |= ((cb >> i) & 1u) && key[i] > T ? (1u << i) : 0u;
      tm |= ((cb >> i) & 1u) && key[i] == T ? (1u << i) : 0u;
    }
  }
  uint32_t tt;
  const uint32_t tbefore = sel_block_exscan((uint32_t)__popc(tm), red, tt);
  // the first (tq - tbefore) ties of this segment in index order are kept
  uint32_t tkeep = 0u;
  if (tbefore < tq) {
    uint32_t m = tm, left = tq - tbefore;
    while (m && left) {
      const uint32_t lo = m & (0u - m);
      tkeep |= lo;
      m ^= lo;
      --left;
    }
  }
  const uint32_t all = km | tkeep;
  uint32_t kt;
  const uint32_t pos = off + sel_block_exscan((uint32_t)__popc(all), red, kt);
  int32_t *out = kept + b * M_alloc;
#pragma unroll
  for (int i = 0; i < SEL_IPT; ++i) {
    const int64_t p = (int64_t)pos + __popc(all & ((1u << i) - 1u));
    if (((all >> i) & 1u) && p < M_alloc) out[p] = (int32_t)(n0 + i);
  }
  if (w == G - 1) {
    const int64_t written = (int64_t)mtrue < M_alloc ? (int64_t)mtrue : M_alloc;
    for (int64_t m = written + tid; m < M_alloc; m += SEL_TPB) out[m] = -1;
  }
}

size_t select_ws_bytes(int64_t B, int64_t N) {
  if (N <= SEL_CHUNK) return 256;  // the single-work-group path uses none
  const int64_t G = sel_groups(N);
  const int64_t words = B * G * (SEL_NC + SEL_NF + 1 + 1 + 2) + B * 8;
  return (size_t)((words * 4 + 255) / 256 * 256 + B * (N > 0 ? N : 1) * 8);
}

static SelWs carve_select_ws(void *ws, int64_t B, int64_t N) {
  const int64_t G = sel_groups(N);
  SelWs s;
  uint32_t *p = (uint32_t *)ws;
  s.coarse = p;
  p += B * G * SEL_NC;
  s.fine = p;
  p += B * G * SEL_NF;
  s.nf = p;
  p += B * G;
  s.sure = p;
  p += B * G;
  s.wgp = p;
  p += B * G * 2;
  s.rowp = p;
  p += B * 8;
  const int64_t words = B * G * (SEL_NC + SEL_NF + 1 + 1 + 2) + B * 8;
  s.cand = (uint64_t *)((char *)ws + (words * 4 + 255) / 256 * 256);
  return s;
}

// Gather: one wave per kept row; 16-byte chunks.  row_bytes % 16 == 0.
__global__ __launch_bounds__(256) void compact_kernel(
    const uint8_t *__restrict__ hidden, const int32_t *__restrict__ pos,
    const float *__restrict__ gates, const int32_t *__restrict__ kept, int64_t B, int64_t N,
    int64_t M, int64_t row_bytes, uint8_t *__restrict__ hidden_out, int32_t *__restrict__ pos_out,
    float *__restrict__ gates_out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= B * M) return;
  const int64_t b = row / M;
  const int64_t n = kept[row];
  const bool valid = n >= 0 && n < N;
  if (hidden_out) {
    const int64_t chunks = row_bytes >> 4;
    u32x4 *dst = (u32x4 *)(hidden_out + row * row_bytes);
    if (valid) {
      const u32x4 *src = (const u32x4 *)(hidden + (b * N + n) * row_bytes);
      for (int64_t c = lane; c < chunks; c += 64) dst[c] = src[c];
    } else {
      for (int64_t c = lane; c < chunks; c += 64) dst[c] = u32x4{0, 0, 0, 0};
    }
  }
  if (lane == 0) {
    if (pos_out) pos_out[row] = valid ? (pos ? pos[b * N + n] : (int32_t)n) : -1;
    if (gates_out) gates_out[row] = valid ? gates[b * N + n] : 0.f;
  }
}

hipError_t launch_select_topk(const float *scores, const uint8_t *forced, int64_t B, int64_t N,
                              int64_t K, int64_t M_alloc, int32_t *kept, int32_t *kept_count, void *ws,
                              hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (N <= SEL_CHUNK) {
    hipLaunchKernelGGL(select_topk_kernel<true>, dim3((unsigned)B), dim3(SEL_T), 0, s, scores, forced, N, K, M_alloc,
                       kept, kept_count);
    return hipGetLastError();
  }
  const int G = sel_groups(N);
  const dim3 grid((unsigned)G, (unsigned)B);
  const SelWs w = carve_select_ws(ws, B, N);
  hipLaunchKernelGGL(select_hist_kernel, grid, dim3(SEL_TPB), 0, s, scores, forced, N, G, w);
  hipLaunchKernelGGL(select_refine_kernel, grid, dim3(SEL_TPB), 0, s, scores, forced, N, K, G, w, kept_count);
  hipLaunchKernelGGL(select_emit_kernel, grid, dim3(SEL_TPB), 0, s, scores, forced, N, M_alloc, G, w, kept);
  return hipGetLastError();
}

// Allocation-free selection: the workspace lives in a device array of this
// library, one per GPU (each GPU holds its own copy at its own address, taken
// once per device with hipGetSymbolAddress; host code uses only that address,
// never the array's name).  Calls on one GPU share it, so calls that overlap
// on that GPU race; every launch of a call writes what the next one reads, so
// nothing needs clearing between calls.
constexpr size_t kSelScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kSelScratchBytes];

size_t select_scratch_bytes() { return kSelScratchBytes; }

// The device address of this GPU's scratch array (nullptr on failure, with
// the HIP error in *err).  The first call on a device, with that device
// current, takes the address; later calls reuse it.
void *select_scratch(hipError_t *err) {
  static std::mutex mu;
  static void *ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= 64)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) {
      *err = e;
      return nullptr;
    }
    ptr[dev] = p;
  }
  *err = hipSuccess;
  return ptr[dev];
}

hipError_t launch_compact(const void *hidden, const int32_t *pos, const float *gates,
                          const int32_t *kept, int64_t B, int64_t N, int64_t M, int64_t row_bytes,
                          void *hidden_out, int32_t *pos_out, float *gates_out, hipStream_t s) {
  if (B * M == 0) return hipSuccess;
  const int64_t blocks = (B * M + 3) / 4;
  hipLaunchKernelGGL(compact_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t *)hidden, pos,
                     gates, kept, B, N, M, row_bytes, (uint8_t *)hidden_out, pos_out, gates_out);
  return hipGetLastError();
}

}  // namespace tg
