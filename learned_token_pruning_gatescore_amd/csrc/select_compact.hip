// select_compact.hip -- scaffold-aware top-K selection and the gather of the
// kept tokens.
//
// TokenGate deep dive ("TokenGate: Learnable Token Pruning for Fast,
// Memory-Efficient LLM Prefill"): section 3.1, Eq. 4 (S = top-K of the
// prunable set by score, united with the non-prunable set) and section 3.4
// (budget clamped, full-sequence keep mask, hidden states and position ids
// sliced with the keep indices).
//
// Selection is a radix select over a 32-bit order key of the fp32 score:
// four 8-bit digit passes, each a 256-bin LDS histogram fed by wavefront
// ballots (lanes holding the same digit are counted with one ballot and one
// atomic), find the exact key T of the K'-th best prunable token and how many
// tokens with key == T to take (lowest index first).  A final pass emits the
// kept indices in ascending order: per 64-token wave slice, ballots of
// "kept, not tied" and "tied" plus mbcnt give each lane its rank, a
// single-wave scan over the wave totals gives the slice offsets.  There is no
// host synchronisation and no global atomics, so the output is deterministic.
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

__device__ __forceinline__ uint32_t lane_rank(uint64_t mask) {
  // number of set bits of mask below this lane
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_ITEMS = 4;  // sub-slices of 1024 tokens per output round

// Adds one to hist[digit] for every lane with `active`, one atomic per
// distinct digit in the wave (up to 8 rounds, then one atomic per lane).
__device__ __forceinline__ void ballot_hist_add(uint32_t *hist, bool active, uint32_t digit, int lane) {
  uint64_t act = __ballot(active);
  for (int it = 0; act != 0; ++it) {
    if (it == 8) {
      if (active) atomicAdd(&hist[digit], 1u);
      break;
    }
    const int leader = __ffsll((unsigned long long)act) - 1;
    const uint32_t dl = __shfl(digit, leader);
    const uint64_t same = __ballot(active && digit == dl);
    if (lane == leader) atomicAdd(&hist[dl], (uint32_t)__popcll(same));
    if (active && digit == dl) active = false;
    act &= ~same;
  }
}

__global__ __launch_bounds__(SEL_THREADS) void select_topk_kernel(
    const float *__restrict__ scores, const uint8_t *__restrict__ forced, int64_t N, int64_t K,
    int64_t M_alloc, int32_t *__restrict__ kept, int32_t *__restrict__ kept_count) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t sSuffix[256];
  __shared__ uint32_t sCnt[SEL_ITEMS * SEL_WAVES];   // packed (keep_nt | tie << 16) per wave slice
  __shared__ uint32_t sOffK[SEL_ITEMS * SEL_WAVES];
  __shared__ uint32_t sOffT[SEL_ITEMS * SEL_WAVES];
  __shared__ int64_t sForced;
  __shared__ uint32_t sState[4];  // prefix, mask, need, digit
  __shared__ int64_t sRun[2];     // running kept-not-tied, running tied

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.x;
  const float *sc = scores + b * N;
  const uint8_t *fo = forced ? forced + b * N : nullptr;
  int32_t *out = kept + b * M_alloc;

  if (tid < 256) hist[tid] = 0;
  if (tid == 0) sForced = 0;
  __syncthreads();

  // Pass 0: forced count and the top-digit histogram of the prunable keys.
  uint32_t prefix = 0, pmask = 0;
  int64_t nF_local = 0;
  for (int64_t base = 0; base < N; base += SEL_THREADS) {
    const int64_t n = base + tid;
    bool cand = false;
    uint32_t digit = 0;
    if (n < N) {
      const bool f = fo && fo[n];
      nF_local += f ? 1 : 0;
      if (!f) {
        cand = true;
        digit = order_key(sc[n]) >> 24;
      }
    }
    ballot_hist_add(hist, cand, digit, lane);
  }
  {
    // block sum of nF_local
    int64_t v = nF_local;
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if (lane == 0 && v) atomicAdd((unsigned long long *)&sForced, (unsigned long long)v);
  }
  __syncthreads();
  const int64_t nF = sForced;
  const int64_t nP = N - nF;
  const int64_t Kc = K < nP ? K : nP;
  const int64_t M_true = nF + Kc;

  // Threshold key and tie quota.  Kc == nP: keep all (thr 0, unlimited quota);
  // Kc == 0: keep none (no key equals 0xFFFFFFFF).
  uint32_t thr;
  int64_t quota;
  if (Kc >= nP) {
    thr = 0u;
    quota = INT64_MAX;
  } else if (Kc <= 0) {
    thr = 0xFFFFFFFFu;
    quota = 0;
  } else {
    uint32_t need = (uint32_t)Kc;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      if (pass > 0) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        for (int64_t base = 0; base < N; base += SEL_THREADS) {
          const int64_t n = base + tid;
          bool cand = false;
          uint32_t digit = 0;
          if (n < N && !(fo && fo[n])) {
            const uint32_t key = order_key(sc[n]);
            if ((key & pmask) == prefix) {
              cand = true;
              digit = (key >> shift) & 255u;
            }
          }
          ballot_hist_add(hist, cand, digit, lane);
        }
        __syncthreads();
      }
      // suffix sums: sSuffix[d] = sum_{d' >= d} hist[d']  (wave 0, 4 bins per lane)
      if (wave == 0) {
        const int d0 = 252 - 4 * lane;  // lane 0 holds bins 252..255
        uint32_t h[4], loc = 0;
#pragma unroll
        for (int e = 3; e >= 0; --e) {
          h[e] = hist[d0 + e];
          loc += h[e];
        }
        uint32_t inc = loc;  // inclusive scan over lanes (lane 0 = top bins)
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t t = __shfl_up(inc, o);
          if (lane >= o) inc += t;
        }
        uint32_t run = inc - loc;  // count above bin d0+3
#pragma unroll
        for (int e = 3; e >= 0; --e) {
          run += h[e];
          sSuffix[d0 + e] = run;
        }
      }
      __syncthreads();
      // digit d* with suffix(d*+1) < need <= suffix(d*)
      if (tid < 256) {
        const uint32_t here = sSuffix[tid];
        const uint32_t above = tid < 255 ? sSuffix[tid + 1] : 0u;
        if (above < need && need <= here) {
          sState[2] = need - above;
          sState[3] = (uint32_t)tid;
        }
      }
      __syncthreads();
      need = sState[2];
      prefix |= sState[3] << shift;
      pmask |= 255u << shift;
      __syncthreads();
    }
    thr = prefix;
    quota = need;
  }

  // Output pass: ascending kept indices.
  if (tid == 0) {
    sRun[0] = 0;
    sRun[1] = 0;
  }
  __syncthreads();
  for (int64_t base = 0; base < N; base += (int64_t)SEL_THREADS * SEL_ITEMS) {
    bool knt[SEL_ITEMS], tie[SEL_ITEMS];
    uint32_t rk[SEL_ITEMS], rt[SEL_ITEMS];
#pragma unroll
    for (int it = 0; it < SEL_ITEMS; ++it) {
      const int64_t n = base + (int64_t)it * SEL_THREADS + tid;
      knt[it] = false;
      tie[it] = false;
      if (n < N) {
        if (fo && fo[n]) {
          knt[it] = true;
        } else {
          const uint32_t key = order_key(sc[n]);
          knt[it] = key > thr;
          tie[it] = key == thr;
        }
      }
      const uint64_t bk = __ballot(knt[it]);
      const uint64_t bt = __ballot(tie[it]);
      rk[it] = lane_rank(bk);
      rt[it] = lane_rank(bt);
      if (lane == 0) sCnt[it * SEL_WAVES + wave] = (uint32_t)__popcll(bk) | ((uint32_t)__popcll(bt) << 16);
    }
    __syncthreads();
    if (wave == 0) {
      const uint32_t c = sCnt[lane];  // 64 = SEL_ITEMS * SEL_WAVES entries, in token order
      uint32_t ck = c & 0xFFFFu, ct = c >> 16;
      uint32_t ik = ck, itt = ct;
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t a = __shfl_up(ik, o), bb = __shfl_up(itt, o);
        if (lane >= o) {
          ik += a;
          itt += bb;
        }
      }
      sOffK[lane] = ik - ck;
      sOffT[lane] = itt - ct;
      if (lane == 63) {
        sState[0] = ik;
        sState[1] = itt;
      }
    }
    __syncthreads();
    const int64_t runK = sRun[0], runT = sRun[1];
#pragma unroll
    for (int it = 0; it < SEL_ITEMS; ++it) {
      const int64_t n = base + (int64_t)it * SEL_THREADS + tid;
      const int slot = it * SEL_WAVES + wave;
      const int64_t kb = runK + sOffK[slot] + rk[it];  // kept-not-tied tokens before n
      const int64_t tb = runT + sOffT[slot] + rt[it];  // tied tokens before n
      const int64_t tk = tb < quota ? tb : quota;      // tied tokens kept before n
      if (knt[it] || (tie[it] && tb < quota)) {
        const int64_t p = kb + tk;
        if (p < M_alloc) out[p] = (int32_t)n;
      }
    }
    __syncthreads();
    if (tid == 0) {
      sRun[0] = runK + sState[0];
      sRun[1] = runT + sState[1];
    }
    __syncthreads();
  }
  // pad and report
  const int64_t written = M_true < M_alloc ? M_true : M_alloc;
  for (int64_t m = written + tid; m < M_alloc; m += SEL_THREADS) out[m] = -1;
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
  hipLaunchKernelGGL(select_topk_kernel, dim3((unsigned)B), dim3(SEL_THREADS), 0, s, scores, forced, N, K,
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
