// api.hip -- the C ABI of libtokengate: argument validation, workspace
// carving and kernel launches.  Every check that the host can make happens
// before the first HIP call, so invalid calls never touch the device.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/tokengate.h"
#include "tg_attn.h"

namespace tg {
size_t gate_packed_bytes(int d, int d_ff);
hipError_t launch_gate_pack_w1(const void *w1, const void *ln_w, int d, int d_ff, void *packed, hipStream_t s,
                               const void *w_up = nullptr);
size_t gate_clone_ws_bytes(int d, int d_i, int H, bool bf16);
hipError_t launch_gate_clone(const void *hidden, const void *w_gate, const void *w_up, const void *w_down,
                             const void *w_head, int64_t T, int d, int d_i, int H, bool bf16, bool ln,
                             const void *ln_w, float ln_eps, float *scores, int64_t Nrow, void *ws, hipStream_t s);
hipError_t launch_gate_score(const void *hidden, const void *w1, const void *w2, const uint8_t *forced, int64_t T,
                             int d, int d_ff, bool bf16, bool ln, const void *ln_w, float ln_eps, float *scores,
                             float *gates, hipStream_t s, int H = 0, int64_t Nrow = 0);
hipError_t launch_score_normalize(const float *s, const uint8_t *forced, int64_t B, int64_t N, float eps, float *out,
                                  hipStream_t st, int heads = 1);
hipError_t launch_gate_softmax(const float *x, const int32_t *kept, int64_t B, int64_t M, float *g, hipStream_t st,
                               int heads = 1);
hipError_t launch_aggregate_heads(const float *s, int64_t B, int H, int64_t N, float *out, hipStream_t st);
hipError_t launch_gather_heads(const float *s, const int32_t *kept, int64_t B, int H, int64_t N, int64_t M, float *out,
                               hipStream_t st);
hipError_t launch_gate_softmax_bwd(const float *g, const float *dg, int64_t B, int64_t M, float *db, hipStream_t st);
hipError_t launch_select_topk(const float *scores, const uint8_t *forced, int64_t B, int64_t N, int64_t K,
                              int64_t M_alloc, int32_t *kept, int32_t *kept_count, void *ws, hipStream_t s);
size_t select_ws_bytes(int64_t B, int64_t N);
size_t select_scratch_bytes();
void *select_scratch(hipError_t *err);
hipError_t launch_compact(const void *hidden, const int32_t *pos, const float *gates, const int32_t *kept,
                          int64_t B, int64_t N, int64_t M, int64_t row_bytes, void *hidden_out, int32_t *pos_out,
                          float *gates_out, hipStream_t s);
}  // namespace tg

namespace {

thread_local char g_err[512] = "";

tg_status fail(tg_status st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

tg_status ok() {
  g_err[0] = '\0';
  return TG_OK;
}

tg_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return ok();
  return fail(TG_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr int64_t kMaxInt = 0x7FFFFFFF;
constexpr int64_t kSelMaxN = (int64_t)1 << 22;  // selection: 1024 work-groups of 4096 tokens per row
constexpr size_t kAlign = 256;

#define REQUIRE(cond, st, ...) \
  do {                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

tg_status check_attn(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                     float tau, int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D, tg_dtype dt) {
  REQUIRE(q && k && v && g && gamma, TG_ERR_INVALID_ARG, "q, k, v, g and gamma are required");
  REQUIRE(B >= 0 && M >= 0, TG_ERR_INVALID_ARG, "B and M must be >= 0 (B=%lld M=%lld)", (long long)B, (long long)M);
  REQUIRE(Hq > 0 && Hkv > 0 && Hq % Hkv == 0, TG_ERR_INVALID_ARG, "Hq (%lld) must be a positive multiple of Hkv (%lld)",
          (long long)Hq, (long long)Hkv);
  REQUIRE(dt == TG_F32 || dt == TG_BF16, TG_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  REQUIRE(std::isfinite(tau) && tau > 0.f, TG_ERR_INVALID_ARG, "tau must be finite and > 0");
  REQUIRE(B * M <= kMaxInt && B * M * Hq <= kMaxInt / 4, TG_ERR_UNSUPPORTED, "problem too large");
  if (dt == TG_BF16) {
    REQUIRE(D == 64 || D == 128, TG_ERR_UNSUPPORTED, "bf16 attention needs D in {64, 128} (got %lld)", (long long)D);
    const int64_t G = Hq / Hkv;
    REQUIRE(G <= 8 && (G & (G - 1)) == 0, TG_ERR_UNSUPPORTED, "bf16 attention needs Hq/Hkv in {1, 2, 4, 8}");
    // the bf16 kernels address one row's q, k, v (and the per-head bias and
    // row statistics, which are smaller) through buffer resources with 32-bit
    // byte ranges, and park dead loads at offset 2^31: every range stays below it
    REQUIRE(M * (Hq > Hkv ? Hq : Hkv) * D * 2 < ((int64_t)1 << 31), TG_ERR_UNSUPPORTED,
            "bf16 attention needs M * max(Hq, Hkv) * D * 2 < 2^31 bytes (M=%lld)", (long long)M);
  } else {
    REQUIRE(D >= 2 && D <= 128 && D % 2 == 0, TG_ERR_UNSUPPORTED, "f32 attention needs even D <= 128");
  }
  REQUIRE(aligned16(q) && aligned16(k) && aligned16(v) && aligned16(g) && aligned16(gamma), TG_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  return TG_OK;
}

}  // namespace

extern "C" {

int tg_version(void) { return 100; }

const char *tg_status_string(tg_status s) {
  switch (s) {
    case TG_OK: return "ok";
    case TG_ERR_INVALID_ARG: return "invalid argument";
    case TG_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case TG_ERR_WORKSPACE: return "workspace missing or too small";
    case TG_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *tg_last_error(void) { return g_err; }

int64_t tg_kept_count(int64_t N, int64_t n_forced, int64_t K) {
  if (N < 0 || K < 0 || n_forced < 0 || n_forced > N) return -1;
  const int64_t nP = N - n_forced;
  return n_forced + (K < nP ? K : nP);
}

}  // extern "C"

namespace {

tg_status check_gate(const void *hidden, const void *w1, const void *w2, int64_t B, int64_t N, int64_t d,
                     int64_t d_ff, tg_dtype dt, const float *scores, const float *gates) {
  REQUIRE(hidden && w1 && w2 && scores, TG_ERR_INVALID_ARG, "hidden, w1, w2 and scores are required");
  REQUIRE(B >= 0 && N >= 0, TG_ERR_INVALID_ARG, "B and N must be >= 0");
  REQUIRE(d > 0 && d_ff > 0, TG_ERR_INVALID_ARG, "d and d_ff must be > 0 (d=%lld d_ff=%lld)", (long long)d,
          (long long)d_ff);
  REQUIRE(dt == TG_F32 || dt == TG_BF16, TG_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  REQUIRE(d <= 65536 && d_ff <= 65536 && B * N <= kMaxInt * 16, TG_ERR_UNSUPPORTED, "problem too large");
  if (dt == TG_BF16)
    REQUIRE(d % 32 == 0, TG_ERR_UNSUPPORTED, "bf16 scoring needs d %% 32 == 0 (d=%lld)", (long long)d);
  else
    REQUIRE(d % 4 == 0 && d <= 8192, TG_ERR_UNSUPPORTED, "f32 scoring needs d %% 4 == 0 and d <= 8192");
  REQUIRE(aligned16(hidden) && aligned16(w1) && aligned16(w2) && aligned16(scores) && aligned16(gates),
          TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  return TG_OK;
}

// Packed variable-length attention: maximal runs of adjacent sequences of
// equal length (empty sequences skipped, which keeps a run's tokens
// contiguous).  The workspace holds every run's arrays side by side, and the
// per-dgamma-run partial sums after them (backward).
tg_status varlen_runs(const int64_t *cu, int64_t nseq, int64_t Hq, int64_t Hkv, int64_t D,
                      std::vector<tg::RunRow> &runs) {
  REQUIRE(cu, TG_ERR_INVALID_ARG, "cu_seqlens (host array of nseq + 1 offsets) is required");
  REQUIRE(nseq >= 0, TG_ERR_INVALID_ARG, "nseq must be >= 0");
  REQUIRE(cu[0] == 0, TG_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  for (int64_t s = 0; s < nseq; ++s)
    REQUIRE(cu[s + 1] >= cu[s], TG_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing (at %lld)", (long long)s);
  REQUIRE(cu[nseq] <= kMaxInt, TG_ERR_UNSUPPORTED, "problem too large");
  runs.clear();
  int64_t padded = 0;
  for (int64_t s = 0; s < nseq; ++s) {
    const int64_t M = cu[s + 1] - cu[s];
    if (M == 0) continue;
    padded += (M + 31) / 32 * 32;
    if (!runs.empty() && runs.back().M == M) ++runs.back().n;
    else runs.push_back(tg::RunRow{(int)cu[s], 0, 1, (int)M, 0, 0});
  }
  REQUIRE(padded <= kMaxInt, TG_ERR_UNSUPPORTED, "problem too large");
  tg::plan_runs(runs.data(), (int)runs.size(), Hq, Hkv, D);
  return TG_OK;
}

size_t rup256(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t varlen_ws_bytes(const std::vector<tg::RunRow> &runs, int64_t Hq, int64_t Hkv, int64_t D, bool bwd,
                       size_t *part_off) {
  const size_t n = rup256(tg::attn_workspace_bytes_runs(runs.data(), (int)runs.size(), Hq, Hkv, D, bwd));
  if (part_off) *part_off = n;
  return n + (bwd ? rup256(runs.size() * 2 * (size_t)Hq * sizeof(float)) : 0);
}

}  // namespace

extern "C" {

size_t tg_gate_score_workspace_size(int64_t d, int64_t d_ff, tg_dtype dt) {
  if (dt != TG_BF16 || d <= 0 || d_ff <= 0 || d > 65536 || d_ff > 65536) return 0;
  return tg::gate_packed_bytes((int)d, (int)d_ff);
}

tg_status tg_gate_pack_w1(const void *w1, int64_t d, int64_t d_ff, tg_dtype dt, void *w1_packed, size_t bytes,
                          void *stream) {
  REQUIRE(w1 && w1_packed, TG_ERR_INVALID_ARG, "w1 and w1_packed are required");
  REQUIRE(dt == TG_BF16, TG_ERR_UNSUPPORTED, "only bf16 weights are packed");
  REQUIRE(d > 0 && d_ff > 0 && d <= 65536 && d_ff <= 65536, TG_ERR_INVALID_ARG, "bad d / d_ff");
  REQUIRE(d % 32 == 0, TG_ERR_UNSUPPORTED, "bf16 scoring needs d %% 32 == 0 (d=%lld)", (long long)d);
  REQUIRE(aligned16(w1) && aligned16(w1_packed), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  const size_t need = tg::gate_packed_bytes((int)d, (int)d_ff);
  REQUIRE(bytes >= need, TG_ERR_WORKSPACE, "w1_packed holds %zu bytes, needs %zu", bytes, need);
  return hip_status(tg::launch_gate_pack_w1(w1, nullptr, (int)d, (int)d_ff, w1_packed, (hipStream_t)stream),
                    "tg_gate_pack_w1 launch");
}

tg_status tg_gate_score_packed(const void *hidden, const void *w1_packed, const void *w2,
                               const uint8_t *forced_keep, int64_t B, int64_t N, int64_t d, int64_t d_ff,
                               tg_dtype dt, float *scores, float *gates, void *stream) {
  REQUIRE(dt == TG_BF16, TG_ERR_UNSUPPORTED, "packed weights exist for bf16 only");
  const tg_status st = check_gate(hidden, w1_packed, w2, B, N, d, d_ff, dt, scores, gates);
  if (st != TG_OK) return st;
  return hip_status(tg::launch_gate_score(hidden, w1_packed, w2, forced_keep, B * N, (int)d, (int)d_ff, true, false,
                                          nullptr, 0.f, scores, gates, (hipStream_t)stream),
                    "tg_gate_score_packed launch");
}

tg_status tg_gate_score(const void *hidden, const void *w1, const void *w2, const uint8_t *forced_keep, int64_t B,
                        int64_t N, int64_t d, int64_t d_ff, tg_dtype dt, float *scores, float *gates, void *ws,
                        size_t ws_bytes, void *stream) {
  const tg_status st = check_gate(hidden, w1, w2, B, N, d, d_ff, dt, scores, gates);
  if (st != TG_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  if (dt == TG_BF16) {
    const size_t need = tg::gate_packed_bytes((int)d, (int)d_ff);
    REQUIRE(ws && ws_bytes >= need, TG_ERR_WORKSPACE, "bf16 scoring needs a %zu-byte workspace (got %zu)", need,
            ws ? ws_bytes : (size_t)0);
    REQUIRE(aligned16(ws), TG_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (B * N == 0) return ok();
    const tg_status pst =
        hip_status(tg::launch_gate_pack_w1(w1, nullptr, (int)d, (int)d_ff, ws, s), "tg_gate_score pack");
    if (pst != TG_OK) return pst;
    return hip_status(tg::launch_gate_score(hidden, ws, w2, forced_keep, B * N, (int)d, (int)d_ff, true, false,
                                            nullptr, 0.f, scores, gates, s),
                      "tg_gate_score launch");
  }
  return hip_status(tg::launch_gate_score(hidden, w1, w2, forced_keep, B * N, (int)d, (int)d_ff, false, false,
                                          nullptr, 0.f, scores, gates, s),
                    "tg_gate_score launch");
}

tg_status tg_gate_score_ln(const void *hidden, const void *ln_w, float ln_eps, const void *w1, const void *w2,
                           const uint8_t *forced_keep, int64_t B, int64_t N, int64_t d, int64_t d_ff, tg_dtype dt,
                           float *scores, float *gates, void *ws, size_t ws_bytes, void *stream) {
  const tg_status st = check_gate(hidden, w1, w2, B, N, d, d_ff, dt, scores, gates);
  if (st != TG_OK) return st;
  REQUIRE(std::isfinite(ln_eps) && ln_eps >= 0.f, TG_ERR_INVALID_ARG, "ln_eps must be finite and >= 0");
  REQUIRE(aligned16(ln_w), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  hipStream_t s = (hipStream_t)stream;
  if (dt == TG_BF16) {
    const size_t need = tg::gate_packed_bytes((int)d, (int)d_ff);
    REQUIRE(ws && ws_bytes >= need, TG_ERR_WORKSPACE, "bf16 scoring needs a %zu-byte workspace (got %zu)", need,
            ws ? ws_bytes : (size_t)0);
    REQUIRE(aligned16(ws), TG_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (B * N == 0) return ok();
    const tg_status pst =
        hip_status(tg::launch_gate_pack_w1(w1, ln_w, (int)d, (int)d_ff, ws, s), "tg_gate_score_ln pack");
    if (pst != TG_OK) return pst;
    return hip_status(tg::launch_gate_score(hidden, ws, w2, forced_keep, B * N, (int)d, (int)d_ff, true, true,
                                            nullptr, ln_eps, scores, gates, s),
                      "tg_gate_score_ln launch");
  }
  return hip_status(tg::launch_gate_score(hidden, w1, w2, forced_keep, B * N, (int)d, (int)d_ff, false, true, ln_w,
                                          ln_eps, scores, gates, s),
                    "tg_gate_score_ln launch");
}

tg_status tg_gate_score_heads(const void *hidden, int ln, const void *ln_w, float ln_eps, const void *w1,
                              const void *w2, int64_t B, int64_t N, int64_t d, int64_t d_ff, int64_t H, tg_dtype dt,
                              float *scores, void *ws, size_t ws_bytes, void *stream) {
  const tg_status st = check_gate(hidden, w1, w2, B, N, d, d_ff, dt, scores, nullptr);
  if (st != TG_OK) return st;
  REQUIRE(H >= 1 && H <= 16, TG_ERR_UNSUPPORTED, "1 <= H <= 16 heads (got %lld)", (long long)H);
  if (ln) {
    REQUIRE(std::isfinite(ln_eps) && ln_eps >= 0.f, TG_ERR_INVALID_ARG, "ln_eps must be finite and >= 0");
    REQUIRE(aligned16(ln_w), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  }
  hipStream_t s = (hipStream_t)stream;
  if (dt == TG_BF16) {
    const size_t need = tg::gate_packed_bytes((int)d, (int)d_ff);
    REQUIRE(ws && ws_bytes >= need, TG_ERR_WORKSPACE, "bf16 scoring needs a %zu-byte workspace (got %zu)", need,
            ws ? ws_bytes : (size_t)0);
    REQUIRE(aligned16(ws), TG_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    if (B * N == 0) return ok();
    const tg_status pst = hip_status(
        tg::launch_gate_pack_w1(w1, ln ? ln_w : nullptr, (int)d, (int)d_ff, ws, s), "tg_gate_score_heads pack");
    if (pst != TG_OK) return pst;
    return hip_status(tg::launch_gate_score(hidden, ws, w2, nullptr, B * N, (int)d, (int)d_ff, true, ln != 0, nullptr,
                                            ln_eps, scores, nullptr, s, (int)H, N),
                      "tg_gate_score_heads launch");
  }
  if (B * N == 0) return ok();
  return hip_status(tg::launch_gate_score(hidden, w1, w2, nullptr, B * N, (int)d, (int)d_ff, false, ln != 0, ln_w,
                                          ln_eps, scores, nullptr, s, (int)H, N),
                    "tg_gate_score_heads launch");
}

size_t tg_gate_score_clone_workspace_size(int64_t d, int64_t d_i, int64_t H, tg_dtype dt) {
  if ((dt != TG_BF16 && dt != TG_F32) || d <= 0 || d_i <= 0 || H < 1 || H > 16 || d > 65536 || d_i > 32768) return 0;
  return tg::gate_clone_ws_bytes((int)d, (int)d_i, (int)H, dt == TG_BF16);
}

tg_status tg_gate_score_clone(const void *hidden, int ln, const void *ln_w, float ln_eps, const void *w_gate,
                              const void *w_up, const void *w_down, const void *w_head, int64_t B, int64_t N,
                              int64_t d, int64_t d_i, int64_t H, tg_dtype dt, float *scores, void *ws,
                              size_t ws_bytes, void *stream) {
  const tg_status st = check_gate(hidden, w_gate, w_up, B, N, d, d_i, dt, scores, nullptr);
  if (st != TG_OK) return st;
  REQUIRE(w_down && w_head, TG_ERR_INVALID_ARG, "w_down and w_head are required");
  REQUIRE(aligned16(w_down) && aligned16(w_head), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  REQUIRE(H >= 1 && H <= 16, TG_ERR_UNSUPPORTED, "1 <= H <= 16 heads (got %lld)", (long long)H);
  REQUIRE(d_i <= 32768, TG_ERR_UNSUPPORTED, "d_i <= 32768 (got %lld)", (long long)d_i);
  if (dt == TG_F32)
    REQUIRE(d + d_i <= 16000, TG_ERR_UNSUPPORTED, "f32 clone scoring needs d + d_i <= 16000 (one row in LDS)");
  if (ln) {
    REQUIRE(std::isfinite(ln_eps) && ln_eps >= 0.f, TG_ERR_INVALID_ARG, "ln_eps must be finite and >= 0");
    REQUIRE(aligned16(ln_w), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  }
  const size_t need = tg::gate_clone_ws_bytes((int)d, (int)d_i, (int)H, dt == TG_BF16);
  REQUIRE(ws && ws_bytes >= need, TG_ERR_WORKSPACE, "clone scoring needs a %zu-byte workspace (got %zu)", need,
          ws ? ws_bytes : (size_t)0);
  REQUIRE(aligned16(ws), TG_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  if (B * N == 0) return ok();
  return hip_status(tg::launch_gate_clone(hidden, w_gate, w_up, w_down, w_head, B * N, (int)d, (int)d_i, (int)H,
                                          dt == TG_BF16, ln != 0, ln_w, ln_eps, scores, N, ws, (hipStream_t)stream),
                    "tg_gate_score_clone launch");
}

tg_status tg_score_normalize(const float *scores, const uint8_t *forced_keep, int64_t B, int64_t N, float eps,
                             float *out, void *stream) {
  REQUIRE(scores && out, TG_ERR_INVALID_ARG, "scores and out are required");
  REQUIRE(B >= 0 && N >= 0, TG_ERR_INVALID_ARG, "B and N must be >= 0");
  REQUIRE(B <= 0x7FFFFFFF && N <= (int64_t)1 << 24, TG_ERR_UNSUPPORTED, "problem too large");
  REQUIRE(std::isfinite(eps) && eps >= 0.f, TG_ERR_INVALID_ARG, "eps must be finite and >= 0");
  REQUIRE(aligned16(scores) && aligned16(out), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  return hip_status(tg::launch_score_normalize(scores, forced_keep, B, N, eps, out, (hipStream_t)stream),
                    "tg_score_normalize launch");
}

tg_status tg_gate_softmax(const float *b, const int32_t *kept_idx, int64_t B, int64_t M, float *g, void *stream) {
  REQUIRE(b && g, TG_ERR_INVALID_ARG, "b and g are required");
  REQUIRE(B >= 0 && M >= 0, TG_ERR_INVALID_ARG, "B and M must be >= 0");
  REQUIRE(B <= 0x7FFFFFFF, TG_ERR_UNSUPPORTED, "problem too large");
  REQUIRE(aligned16(b) && aligned16(kept_idx) && aligned16(g), TG_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  return hip_status(tg::launch_gate_softmax(b, kept_idx, B, M, g, (hipStream_t)stream), "tg_gate_softmax launch");
}

tg_status tg_score_normalize_heads(const float *scores, const uint8_t *forced_keep, int64_t B, int64_t H, int64_t N,
                                   float eps, float *out, void *stream) {
  REQUIRE(scores && out, TG_ERR_INVALID_ARG, "scores and out are required");
  REQUIRE(B >= 0 && N >= 0 && H >= 1, TG_ERR_INVALID_ARG, "B, N >= 0 and H >= 1");
  REQUIRE(B * H <= 0x7FFFFFFF && H <= 0x7FFFFFFF && N <= (int64_t)1 << 24, TG_ERR_UNSUPPORTED, "problem too large");
  REQUIRE(std::isfinite(eps) && eps >= 0.f, TG_ERR_INVALID_ARG, "eps must be finite and >= 0");
  REQUIRE(aligned16(scores) && aligned16(out), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  return hip_status(tg::launch_score_normalize(scores, forced_keep, B * H, N, eps, out, (hipStream_t)stream, (int)H),
                    "tg_score_normalize_heads launch");
}

tg_status tg_aggregate_heads(const float *b, int64_t B, int64_t H, int64_t N, float *out, void *stream) {
  REQUIRE(b && out, TG_ERR_INVALID_ARG, "b and out are required");
  REQUIRE(B >= 0 && N >= 0 && H >= 1, TG_ERR_INVALID_ARG, "B, N >= 0 and H >= 1");
  REQUIRE(B * N <= kMaxInt * 16 && H <= 0x7FFFFFFF, TG_ERR_UNSUPPORTED, "problem too large");
  REQUIRE(aligned16(b) && aligned16(out), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  return hip_status(tg::launch_aggregate_heads(b, B, (int)H, N, out, (hipStream_t)stream),
                    "tg_aggregate_heads launch");
}

tg_status tg_gather_heads(const float *b, const int32_t *kept_idx, int64_t B, int64_t H, int64_t N, int64_t M,
                          float *out, void *stream) {
  REQUIRE(b && kept_idx && out, TG_ERR_INVALID_ARG, "b, kept_idx and out are required");
  REQUIRE(B >= 0 && N >= 0 && M >= 0 && H >= 1, TG_ERR_INVALID_ARG, "B, N, M >= 0 and H >= 1");
  REQUIRE(B * H * M <= kMaxInt * 16 && H <= 0x7FFFFFFF && N <= kMaxInt, TG_ERR_UNSUPPORTED, "problem too large");
  REQUIRE(aligned16(b) && aligned16(kept_idx) && aligned16(out), TG_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  return hip_status(tg::launch_gather_heads(b, kept_idx, B, (int)H, N, M, out, (hipStream_t)stream),
                    "tg_gather_heads launch");
}

tg_status tg_gate_softmax_heads(const float *b, const int32_t *kept_idx, int64_t B, int64_t H, int64_t M, float *g,
                                void *stream) {
  REQUIRE(b && g, TG_ERR_INVALID_ARG, "b and g are required");
  REQUIRE(B >= 0 && M >= 0 && H >= 1, TG_ERR_INVALID_ARG, "B, M >= 0 and H >= 1");
  REQUIRE(B * H <= 0x7FFFFFFF, TG_ERR_UNSUPPORTED, "problem too large");
  REQUIRE(aligned16(b) && aligned16(kept_idx) && aligned16(g), TG_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  return hip_status(tg::launch_gate_softmax(b, kept_idx, B * H, M, g, (hipStream_t)stream, (int)H),
                    "tg_gate_softmax_heads launch");
}

tg_status tg_gate_softmax_bwd(const float *g, const float *dg, int64_t B, int64_t M, float *db, void *stream) {
  REQUIRE(g && dg && db, TG_ERR_INVALID_ARG, "g, dg and db are required");
  REQUIRE(B >= 0 && M >= 0, TG_ERR_INVALID_ARG, "B and M must be >= 0");
  REQUIRE(B <= 0x7FFFFFFF, TG_ERR_UNSUPPORTED, "problem too large");
  REQUIRE(aligned16(g) && aligned16(dg) && aligned16(db), TG_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  return hip_status(tg::launch_gate_softmax_bwd(g, dg, B, M, db, (hipStream_t)stream),
                    "tg_gate_softmax_bwd launch");
}

size_t tg_select_topk_workspace_size(int64_t B, int64_t N) {
  if (B < 0 || N < 0 || N > kSelMaxN) return 0;
  return tg::select_ws_bytes(B, N);
}

tg_status tg_select_topk(const float *scores, const uint8_t *forced_keep, int64_t B, int64_t N, int64_t K,
                         int64_t n_forced, int32_t *kept_idx, int32_t *kept_count, void *ws, size_t ws_bytes,
                         void *stream) {
  REQUIRE(B >= 0 && N >= 0, TG_ERR_INVALID_ARG, "B and N must be >= 0");
  REQUIRE(K >= 0, TG_ERR_INVALID_ARG, "K must be >= 0 (got %lld)", (long long)K);
  REQUIRE(n_forced >= 0 && n_forced <= N, TG_ERR_INVALID_ARG, "need 0 <= n_forced <= N (n_forced=%lld N=%lld)",
          (long long)n_forced, (long long)N);
  REQUIRE(forced_keep || n_forced == 0, TG_ERR_INVALID_ARG, "forced_keep is NULL but n_forced > 0");
  REQUIRE(N <= kSelMaxN && B <= 65535, TG_ERR_UNSUPPORTED, "selection needs N <= 2^22 and B <= 65535");
  const int64_t M = tg_kept_count(N, n_forced, K);
  if (B * N > 0) REQUIRE(scores && kept_idx, TG_ERR_INVALID_ARG, "scores and kept_idx are required");
  REQUIRE(aligned16(scores) && aligned16(kept_idx), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (B == 0) return ok();
  const size_t need = tg::select_ws_bytes(B, N);
  REQUIRE(ws && ws_bytes >= need, TG_ERR_WORKSPACE, "selection needs a %zu-byte workspace (got %zu)", need,
          ws ? ws_bytes : (size_t)0);
  REQUIRE(reinterpret_cast<uintptr_t>(ws) % kAlign == 0, TG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return hip_status(tg::launch_select_topk(scores, forced_keep, B, N, K, M, kept_idx, kept_count, ws,
                                           (hipStream_t)stream),
                    "tg_select_topk launch");
}

tg_status tg_select_topk_noalloc(const float *scores, const uint8_t *forced_keep, int64_t B, int64_t N, int64_t K,
                                 int64_t n_forced, int32_t *kept_idx, int32_t *kept_count, void *stream) {
  REQUIRE(B >= 0 && N >= 0, TG_ERR_INVALID_ARG, "B and N must be >= 0");
  REQUIRE(K >= 0, TG_ERR_INVALID_ARG, "K must be >= 0 (got %lld)", (long long)K);
  REQUIRE(n_forced >= 0 && n_forced <= N, TG_ERR_INVALID_ARG, "need 0 <= n_forced <= N (n_forced=%lld N=%lld)",
          (long long)n_forced, (long long)N);
  REQUIRE(forced_keep || n_forced == 0, TG_ERR_INVALID_ARG, "forced_keep is NULL but n_forced > 0");
  REQUIRE(N <= kSelMaxN && B <= 65535, TG_ERR_UNSUPPORTED, "selection needs N <= 2^22 and B <= 65535");
  const size_t need = tg::select_ws_bytes(B, N), cap = tg::select_scratch_bytes();
  REQUIRE(need <= cap, TG_ERR_UNSUPPORTED,
          "tg_select_topk_noalloc: B=%lld, N=%lld needs %zu bytes of scratch, more than its %zu (use tg_select_topk "
          "with a workspace)", (long long)B, (long long)N, need, cap);
  const int64_t M = tg_kept_count(N, n_forced, K);
  if (B * N > 0) REQUIRE(scores && kept_idx, TG_ERR_INVALID_ARG, "scores and kept_idx are required");
  REQUIRE(aligned16(scores) && aligned16(kept_idx), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  if (B == 0) return ok();
  hipError_t e = hipSuccess;
  void *ws = tg::select_scratch(&e);
  if (!ws) return hip_status(e, "tg_select_topk_noalloc scratch address");
  return hip_status(tg::launch_select_topk(scores, forced_keep, B, N, K, M, kept_idx, kept_count, ws,
                                           (hipStream_t)stream),
                    "tg_select_topk_noalloc launch");
}

tg_status tg_compact(const void *hidden, const int32_t *pos, const float *gates, const int32_t *kept_idx,
                     int64_t B, int64_t N, int64_t M, int64_t d, tg_dtype dt, void *hidden_out, int32_t *pos_out,
                     float *gates_out, void *stream) {
  REQUIRE(B >= 0 && N >= 0 && M >= 0, TG_ERR_INVALID_ARG, "B, N and M must be >= 0");
  REQUIRE(dt == TG_F32 || dt == TG_BF16, TG_ERR_INVALID_ARG, "unknown dtype %d", (int)dt);
  REQUIRE(B * M == 0 || kept_idx, TG_ERR_INVALID_ARG, "kept_idx is required");
  REQUIRE(!hidden_out || (hidden && d > 0), TG_ERR_INVALID_ARG, "hidden_out needs hidden and d > 0");
  REQUIRE(!gates_out || gates, TG_ERR_INVALID_ARG, "gates_out needs gates");
  const int64_t esz = dt == TG_BF16 ? 2 : 4;
  const int64_t row_bytes = hidden_out ? d * esz : 0;
  REQUIRE(!hidden_out || row_bytes % 16 == 0, TG_ERR_UNSUPPORTED, "rows must be a multiple of 16 bytes");
  REQUIRE(B * M <= kMaxInt * 4, TG_ERR_UNSUPPORTED, "problem too large");
  REQUIRE(aligned16(hidden) && aligned16(hidden_out) && aligned16(kept_idx), TG_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  if (B * M == 0) return ok();
  return hip_status(tg::launch_compact(hidden, pos, gates, kept_idx, B, N, M, row_bytes, hidden_out, pos_out,
                                       gates_out, (hipStream_t)stream),
                    "tg_compact launch");
}

size_t tg_gated_attn_workspace_size(int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D, int bwd) {
  if (B < 0 || M < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return 0;
  return tg::attn_workspace_bytes(B, M, Hq, Hkv, D, bwd != 0);
}

}  // extern "C"

static tg_status attn_fwd_impl(bool gph, const void *q, const void *k, const void *v, const float *g, const float *gamma,
                            const int32_t *pos, float rope_theta, float tau, const float *sigma, int64_t B,
                            int64_t M, int64_t Hq, int64_t Hkv, int64_t D, tg_dtype dt, void *o, float *lse,
                            void *o_lo, void *ws, size_t ws_bytes, void *stream) {
  tg_status st = check_attn(q, k, v, g, gamma, tau, B, M, Hq, Hkv, D, dt);
  if (st != TG_OK) return st;
  REQUIRE(o, TG_ERR_INVALID_ARG, "o is required");
  REQUIRE(!sigma || aligned16(sigma), TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  REQUIRE(aligned16(o) && aligned16(lse) && aligned16(o_lo), TG_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(!o_lo || dt == TG_BF16, TG_ERR_INVALID_ARG, "o_lo exists for bf16 only");
  if (pos) REQUIRE(std::isfinite(rope_theta) && rope_theta > 1.f, TG_ERR_INVALID_ARG, "rope_theta must be > 1");
  const size_t need = tg::attn_workspace_bytes(B, M, Hq, Hkv, D, false);
  REQUIRE(ws && ws_bytes >= need, TG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  REQUIRE(reinterpret_cast<uintptr_t>(ws) % kAlign == 0, TG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (B * M == 0) return ok();
  const tg::AttnWs w = tg::carve_attn_ws(ws, B, M, Hq, Hkv, D);
  return hip_status(tg::launch_attn_fwd(q, k, v, g, gamma, pos, (double)rope_theta, tau, sigma, (int)B, (int)M,
                                        (int)Hq, (int)Hkv, (int)D, dt == TG_BF16, gph, o, lse, o_lo, w,
                                        (hipStream_t)stream),
                    "tg_gated_attn_fwd launch");
}

static tg_status attn_bwd_impl(bool gph, const void *q, const void *k, const void *v, const float *g, const float *gamma,
                            const int32_t *pos, float rope_theta, float tau, const float *sigma, const float *lse,
                            const void *dout, const void *o, const void *o_lo, int64_t B, int64_t M, int64_t Hq,
                            int64_t Hkv, int64_t D, tg_dtype dt,
                            float *dq, float *dk, float *dv, float *dg, float *dgamma, float *dsigma, void *ws,
                            size_t ws_bytes, void *stream) {
  tg_status st = check_attn(q, k, v, g, gamma, tau, B, M, Hq, Hkv, D, dt);
  if (st != TG_OK) return st;
  REQUIRE(lse && dout && dq && dk && dv && dg && dgamma, TG_ERR_INVALID_ARG,
          "lse, dout, dq, dk, dv, dg and dgamma are required");
  REQUIRE(!sigma == !dsigma, TG_ERR_INVALID_ARG, "sigma and dsigma go together");
  REQUIRE(!sigma || (aligned16(sigma) && aligned16(dsigma)), TG_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(aligned16(lse) && aligned16(dout) && aligned16(dq) && aligned16(dk) && aligned16(dv) && aligned16(dg) &&
              aligned16(dgamma) && aligned16(o) && aligned16(o_lo),
          TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  REQUIRE(!o == !o_lo, TG_ERR_INVALID_ARG, "o and o_lo go together");
  REQUIRE(!o || dt == TG_BF16, TG_ERR_INVALID_ARG, "o and o_lo are taken for bf16 only");
  if (pos) REQUIRE(std::isfinite(rope_theta) && rope_theta > 1.f, TG_ERR_INVALID_ARG, "rope_theta must be > 1");
  const size_t need = tg::attn_workspace_bytes(B, M, Hq, Hkv, D, true);
  REQUIRE(ws && ws_bytes >= need, TG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  REQUIRE(reinterpret_cast<uintptr_t>(ws) % kAlign == 0, TG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const tg::AttnWs w = tg::carve_attn_ws(ws, B, M, Hq, Hkv, D);
  const tg::RunRow run{0, 0, (int)B, (int)M, 0, 0};
  return hip_status(tg::launch_attn_bwd(q, k, v, g, gamma, pos, (double)rope_theta, tau, sigma, lse, dout, o, o_lo,
                                        &run, 1,
                                        (int)Hq, (int)Hkv, (int)D, dt == TG_BF16, gph, dq, dk, dv, dg, dgamma, dsigma,
                                        nullptr, w, (hipStream_t)stream),
                    "tg_gated_attn_bwd launch");
}

extern "C" {

tg_status tg_gated_attn_fwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                            const int32_t *pos, float rope_theta, float tau, const float *sigma, int64_t B,
                            int64_t M, int64_t Hq, int64_t Hkv, int64_t D, tg_dtype dt, void *o, float *lse,
                            void *o_lo, void *ws, size_t ws_bytes, void *stream) {
  return attn_fwd_impl(false, q, k, v, g, gamma, pos, rope_theta, tau, sigma, B, M, Hq, Hkv, D, dt, o, lse, o_lo,
                       ws, ws_bytes, stream);
}

tg_status tg_gated_attn_fwd_headgates(const void *q, const void *k, const void *v, const float *g,
                                      const float *gamma, const int32_t *pos, float rope_theta, float tau,
                                      const float *sigma, int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D,
                                      tg_dtype dt, void *o, float *lse, void *o_lo, void *ws, size_t ws_bytes,
                                      void *stream) {
  return attn_fwd_impl(true, q, k, v, g, gamma, pos, rope_theta, tau, sigma, B, M, Hq, Hkv, D, dt, o, lse, o_lo,
                       ws, ws_bytes, stream);
}

tg_status tg_gated_attn_bwd(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                            const int32_t *pos, float rope_theta, float tau, const float *sigma, const float *lse,
                            const void *dout, const void *o, const void *o_lo, int64_t B, int64_t M, int64_t Hq,
                            int64_t Hkv, int64_t D, tg_dtype dt, float *dq, float *dk, float *dv, float *dg,
                            float *dgamma, float *dsigma, void *ws, size_t ws_bytes, void *stream) {
  return attn_bwd_impl(false, q, k, v, g, gamma, pos, rope_theta, tau, sigma, lse, dout, o, o_lo, B, M, Hq, Hkv, D,
                       dt, dq, dk, dv, dg, dgamma, dsigma, ws, ws_bytes, stream);
}

tg_status tg_gated_attn_bwd_headgates(const void *q, const void *k, const void *v, const float *g,
                                      const float *gamma, const int32_t *pos, float rope_theta, float tau,
                                      const float *sigma, const float *lse, const void *dout, const void *o,
                                      const void *o_lo, int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D,
                                      tg_dtype dt, float *dq, float *dk, float *dv, float *dg, float *dgamma,
                                      float *dsigma, void *ws, size_t ws_bytes, void *stream) {
  return attn_bwd_impl(true, q, k, v, g, gamma, pos, rope_theta, tau, sigma, lse, dout, o, o_lo, B, M, Hq, Hkv, D,
                       dt, dq, dk, dv, dg, dgamma, dsigma, ws, ws_bytes, stream);
}

size_t tg_gated_attn_varlen_workspace_size(const int64_t *cu_seqlens, int64_t nseq, int64_t Hq, int64_t Hkv,
                                           int64_t D, int bwd) {
  std::vector<tg::RunRow> runs;
  if (Hq <= 0 || Hkv <= 0 || D <= 0 || varlen_runs(cu_seqlens, nseq, Hq, Hkv, D, runs) != TG_OK) return 0;
  return varlen_ws_bytes(runs, Hq, Hkv, D, bwd != 0, nullptr);
}

tg_status tg_gated_attn_fwd_varlen(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                                   const int32_t *pos, float rope_theta, float tau, const float *sigma,
                                   const int64_t *cu_seqlens, int64_t nseq, int64_t Hq, int64_t Hkv, int64_t D,
                                   tg_dtype dt, void *o, float *lse, void *o_lo, void *ws, size_t ws_bytes,
                                   void *stream) {
  REQUIRE(Hq > 0 && Hkv > 0 && D > 0, TG_ERR_INVALID_ARG, "Hq, Hkv and D must be > 0");
  std::vector<tg::RunRow> runs;
  tg_status st = varlen_runs(cu_seqlens, nseq, Hq, Hkv, D, runs);
  if (st != TG_OK) return st;
  const int64_t T = cu_seqlens[nseq];
  st = check_attn(q, k, v, g, gamma, tau, 1, T, Hq, Hkv, D, dt);
  if (st != TG_OK) return st;
  REQUIRE(o, TG_ERR_INVALID_ARG, "o is required");
  REQUIRE(aligned16(o) && aligned16(lse) && aligned16(sigma) && aligned16(o_lo), TG_ERR_INVALID_ARG,
          "tensor pointers must be 16-byte aligned");
  REQUIRE(!o_lo || dt == TG_BF16, TG_ERR_INVALID_ARG, "o_lo exists for bf16 only");
  if (pos) REQUIRE(std::isfinite(rope_theta) && rope_theta > 1.f, TG_ERR_INVALID_ARG, "rope_theta must be > 1");
  const size_t need = varlen_ws_bytes(runs, Hq, Hkv, D, false, nullptr);
  REQUIRE(ws && ws_bytes >= need, TG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  REQUIRE(reinterpret_cast<uintptr_t>(ws) % kAlign == 0, TG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const size_t esz = dt == TG_BF16 ? 2 : 4;
  const tg::AttnWs wall = tg::carve_attn_ws_runs(ws, runs.data(), (int)runs.size(), Hq, Hkv, D);
  if (dt == TG_BF16 && runs.size() > 1)  // every run's blocks in one launch per group of runs
    return hip_status(tg::launch_attn_fwd_runs(q, k, v, g, gamma, pos, (double)rope_theta, tau, sigma, runs.data(),
                                               (int)runs.size(), (int)Hq, (int)Hkv, (int)D, o, lse, o_lo, wall,
                                               (hipStream_t)stream),
                      "tg_gated_attn_fwd_varlen launch");
  for (const tg::RunRow &r : runs) {
    const tg::AttnWs w = tg::run_view(wall, r, Hq, Hkv, D);
    const int64_t off = r.off;
    const hipError_t e = tg::launch_attn_fwd(
        (const char *)q + off * Hq * D * esz, (const char *)k + off * Hkv * D * esz,
        (const char *)v + off * Hkv * D * esz, g + off, gamma, pos ? pos + off : nullptr, (double)rope_theta, tau,
        sigma, r.n, r.M, (int)Hq, (int)Hkv, (int)D, dt == TG_BF16, false, (char *)o + off * Hq * D * esz,
        lse ? lse + Hq * off : nullptr, o_lo ? (char *)o_lo + off * Hq * D * esz : nullptr, w, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "tg_gated_attn_fwd_varlen launch");
  }
  return ok();
}

tg_status tg_gated_attn_bwd_varlen(const void *q, const void *k, const void *v, const float *g, const float *gamma,
                                   const int32_t *pos, float rope_theta, float tau, const float *sigma,
                                   const float *lse, const void *dout, const void *o, const void *o_lo,
                                   const int64_t *cu_seqlens, int64_t nseq, int64_t Hq, int64_t Hkv, int64_t D,
                                   tg_dtype dt, float *dq, float *dk, float *dv, float *dg, float *dgamma,
                                   float *dsigma, void *ws, size_t ws_bytes, void *stream) {
  REQUIRE(Hq > 0 && Hkv > 0 && D > 0, TG_ERR_INVALID_ARG, "Hq, Hkv and D must be > 0");
  std::vector<tg::RunRow> runs;
  tg_status st = varlen_runs(cu_seqlens, nseq, Hq, Hkv, D, runs);
  if (st != TG_OK) return st;
  const int64_t T = cu_seqlens[nseq];
  st = check_attn(q, k, v, g, gamma, tau, 1, T, Hq, Hkv, D, dt);
  if (st != TG_OK) return st;
  REQUIRE(lse && dout && dq && dk && dv && dg && dgamma, TG_ERR_INVALID_ARG,
          "lse, dout, dq, dk, dv, dg and dgamma are required");
  REQUIRE(!sigma == !dsigma, TG_ERR_INVALID_ARG, "sigma and dsigma go together");
  REQUIRE(aligned16(lse) && aligned16(dout) && aligned16(dq) && aligned16(dk) && aligned16(dv) && aligned16(dg) &&
              aligned16(dgamma) && aligned16(sigma) && aligned16(dsigma) && aligned16(o) && aligned16(o_lo),
          TG_ERR_INVALID_ARG, "tensor pointers must be 16-byte aligned");
  REQUIRE(!o == !o_lo, TG_ERR_INVALID_ARG, "o and o_lo go together");
  REQUIRE(!o || dt == TG_BF16, TG_ERR_INVALID_ARG, "o and o_lo are taken for bf16 only");
  if (pos) REQUIRE(std::isfinite(rope_theta) && rope_theta > 1.f, TG_ERR_INVALID_ARG, "rope_theta must be > 1");
  size_t part_off = 0;
  const size_t need = varlen_ws_bytes(runs, Hq, Hkv, D, true, &part_off);
  REQUIRE(ws && ws_bytes >= need, TG_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
  REQUIRE(reinterpret_cast<uintptr_t>(ws) % kAlign == 0, TG_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const tg::AttnWs w = tg::carve_attn_ws_runs(ws, runs.data(), (int)runs.size(), Hq, Hkv, D);
  return hip_status(tg::launch_attn_bwd(q, k, v, g, gamma, pos, (double)rope_theta, tau, sigma, lse, dout, o, o_lo,
                                        runs.data(), (int)runs.size(), (int)Hq, (int)Hkv, (int)D, dt == TG_BF16,
                                        false, dq, dk, dv, dg, dgamma, dsigma, (float *)((char *)ws + part_off), w,
                                        (hipStream_t)stream),
                    "tg_gated_attn_bwd_varlen launch");
}

}  // extern "C"
