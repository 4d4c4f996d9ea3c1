// select_compact.hip -- scaffold-aware top-K selection and the gather of the
// kept tokens.
//
// TokenGate deep dive ("TokenGate: Learnable Token Pruning for Fast,
// Memory-Efficient LLM Prefill"): section 3.1, Eq. 4 (S = top-K of the
// prunable set by score, united with the non-prunable set) and section 3.4
// (budget clamped, full-sequence keep mask, hidden states and position ids
// sliced with the keep indices).
//
// Selection is a radix select over a 32-bit order key of the fp32 score, one
// work-group per batch row: three digit passes (12, 10, 10 bits) over an LDS
// histogram (a wavefront vote collapses a wave whose keys are all equal into a
// single atomic) find the exact key T of
// the K'-th best prunable token and how many tokens with key == T to take
// (lowest index first).  Each thread owns contiguous 32-token segments whose
// keys stay in registers; a final pass emits the kept indices in ascending
// order from one block-wide scan of per-segment counts.  No host
// synchronisation and no global atomics: the output is deterministic.
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

// One work-group per batch row.  Tokens are processed in 32768-token chunks;
// thread t owns the contiguous segment [t*32, t*32+32) of a chunk.  With one
// chunk (N <= 32768) its 32 keys stay in registers for every pass, otherwise
// each pass reloads the chunk (L2-resident).  Forced / valid / candidate flags
// are 32-bit masks, so the output positions of a segment come from popcounts
// of masks rather than from a dependent counter chain.
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
                              int64_t K, int64_t M_alloc, int32_t *kept, int32_t *kept_count,
                              hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (N <= SEL_CHUNK)
    hipLaunchKernelGGL(select_topk_kernel<true>, dim3((unsigned)B), dim3(SEL_T), 0, s, scores, forced, N, K, M_alloc,
                       kept, kept_count);
  else
    hipLaunchKernelGGL(select_topk_kernel<false>, dim3((unsigned)B), dim3(SEL_T), 0, s, scores, forced, N, K,
                       M_alloc, kept, kept_count);
  return hipGetLastError();
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
