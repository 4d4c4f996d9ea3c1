/*
 * tokengate.h -- C ABI of libtokengate, the gate-layer hot path of TokenGate
 * (learned token pruning with gate scores) for AMD Instinct MI355X (gfx950).
 *
 * The calls follow the method's statement of the problem:
 *   score every context token, keep the top K prunable tokens plus every
 *   non-prunable (scaffold) token in original order, gather the kept hidden
 *   states, positions and gate values, and run causal attention whose weights
 *   are multiplied by each key's gate value; plus the backward of that
 *   attention, through which the task gradient reaches the scores.
 *
 * Sources cited below (page title, then section / equation):
 *   [DeepDive] "TokenGate: Learnable Token Pruning for Fast, Memory-Efficient
 *              LLM Prefill" (agientry.com paper deep dive).
 *   [Summary]  "TokenGate: Adapting LLMs for Fast and Memory-Efficient Prefill
 *              with Learned Token Pruning" (thelatestinai.com).
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer owned by the caller, contiguous
 *     row-major, 16-byte aligned.  The library allocates no device memory and
 *     keeps no pointer after a call returns; scratch memory comes from a
 *     caller workspace sized by the matching *_workspace_size call.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All device work
 *     is enqueued asynchronously on it; no call synchronises with the host.
 *     Keep buffers alive until the stream has passed the work.
 *   - `dt` gives the storage type of hidden, w1, w2, q, k, v, o and dout
 *     (TG_BF16 or TG_F32).  Scores, gates, lse and every gradient are fp32.
 *   - Errors that the host can see (a NULL required pointer, a bad size, a
 *     misaligned pointer, an unsupported shape, a small workspace) return
 *     before anything is launched.  A failed launch returns TG_ERR_HIP; the
 *     text is in tg_last_error() (thread-local).
 *   - Data conditions are defined behaviour, not errors: NaN or infinite
 *     scores, ties, K = 0, K >= the number of prunable tokens, and a forced
 *     mask whose count differs from n_forced (see tg_select_topk).
 *   - Calls are stateless and may be made from several threads; device
 *     properties are cached once per device.
 */
#ifndef TOKENGATE_H
#define TOKENGATE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TG_OK = 0,
    TG_ERR_INVALID_ARG = 1, /* NULL / negative / inconsistent / misaligned argument */
    TG_ERR_UNSUPPORTED = 2, /* valid but not implemented shape or dtype */
    TG_ERR_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size */
    TG_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} tg_status;

typedef enum { TG_F32 = 0, TG_BF16 = 1 } tg_dtype;

/* Library version as major*10000 + minor*100 + patch. */
int tg_version(void);

/* Static description of a status code. */
const char *tg_status_string(tg_status s);

/* Detail of the last non-OK status returned on this thread ("" if none). */
const char *tg_last_error(void);

/*
 * tg_gate_score -- the scoring MLP and the gate value of every token.
 * [DeepDive] section 3.1, Eq. 3 (first part): a small MLP maps each token's
 * normalised post-attention residual to one scalar; section 3.4 shows the
 * scorer applied to the residual before selection.  Form computed:
 *     s_t = sum_k w2[k] * SiLU( sum_i w1[k, i] * hidden[t, i] ),
 *     gates[t] = 1 if forced_keep[t] != 0, else 1 / (1 + exp(-s_t)).
 *   hidden      [B, N, d]  (dt)     token states at the gate layer
 *   w1          [d_ff, d]  (dt)     first layer, stored out x in
 *   w2          [d_ff]     (dt)     second layer
 *   forced_keep [B, N] u8 or NULL   nonzero = non-prunable token (gate 1)
 *   scores      [B, N] f32 out      raw scores (the ranking key)
 *   gates       [B, N] f32 out or NULL
 * bf16 runs on matrix cores with fp32 accumulation; SiLU, the w2 dot and the
 * sigmoid are fp32.  Needs d % 32 == 0 for bf16 and d % 4 == 0 for f32.
 *   ws, ws_bytes                     bf16: device scratch of at least
 *                                    tg_gate_score_workspace_size(d, d_ff, dt)
 *                                    bytes, 16-byte aligned, owned by the
 *                                    caller (W1 is rewritten there in matrix-
 *                                    core fragment order before scoring);
 *                                    f32: unused (may be NULL).
 * Errors: TG_ERR_WORKSPACE when the bf16 workspace is missing or too small.
 */
tg_status tg_gate_score(const void *hidden, const void *w1, const void *w2,
                        const uint8_t *forced_keep, int64_t B, int64_t N, int64_t d,
                        int64_t d_ff, tg_dtype dt, float *scores, float *gates,
                        void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace tg_gate_score needs: the fragment-ordered copy of W1
 * for TG_BF16 (d_ff rounded up to 512 units, d to 128 inputs, 2 bytes each);
 * 0 for TG_F32 or invalid sizes. */
size_t tg_gate_score_workspace_size(int64_t d, int64_t d_ff, tg_dtype dt);

/*
 * tg_gate_pack_w1 / tg_gate_score_packed -- the same scoring MLP split into
 * a one-off weight transform and the per-call product, for callers that
 * keep the scorer's weights resident (section 3.1: the scorer is a fixed,
 * trained MLP at inference).  tg_gate_pack_w1 writes W1 [d_ff, d] bf16 in
 * fragment order into w1_packed (bytes >= tg_gate_score_workspace_size);
 * tg_gate_score_packed then computes exactly what tg_gate_score computes
 * from that copy.  bf16 only (TG_ERR_UNSUPPORTED otherwise).
 */
tg_status tg_gate_pack_w1(const void *w1, int64_t d, int64_t d_ff, tg_dtype dt,
                          void *w1_packed, size_t bytes, void *stream);
tg_status tg_gate_score_packed(const void *hidden, const void *w1_packed, const void *w2,
                               const uint8_t *forced_keep, int64_t B, int64_t N, int64_t d,
                               int64_t d_ff, tg_dtype dt, float *scores, float *gates,
                               void *stream);

/*
 * tg_gate_score_ln -- tg_gate_score on the raw post-attention residual, with
 * the layer's second normalisation in front.  [DeepDive] section 2, Eq. 1 (the
 * gate reads a~ = LN2(a)) and section 3.1, Eq. 3 (the scorer maps a~_j).  The
 * normaliser is RMSNorm with a per-channel weight (the Qwen3 models' LN2):
 *     a~[t,i] = a[t,i] / sqrt(mean_i a[t,i]^2 + ln_eps) * ln_w[i]
 * followed by exactly the scorer of tg_gate_score.
 *   hidden [B, N, d] (dt) raw residual; ln_w [d] (dt) or NULL (= 1);
 *   ln_eps finite >= 0 (an all-zero row with ln_eps = 0 gives NaN).
 * Other arguments, outputs, workspace (the same size) and errors as
 * tg_gate_score.  bf16: ln_w is folded into the packed W1 (one bf16 rounding
 * of w1 * ln_w) and each token's 1 / sqrt(mean square + eps), formed in fp32
 * from the bf16 inputs, scales its pre-activations before SiLU.
 */
tg_status tg_gate_score_ln(const void *hidden, const void *ln_w, float ln_eps, const void *w1,
                           const void *w2, const uint8_t *forced_keep, int64_t B, int64_t N,
                           int64_t d, int64_t d_ff, tg_dtype dt, float *scores, float *gates,
                           void *ws, size_t ws_bytes, void *stream);

/*
 * tg_score_normalize -- sequence RMS normalisation of one request's scores.
 * [DeepDive] section 3.1, Eq. 3 (second part): per row b,
 *     out_j = s_j / sqrt((1/|P|) sum_{j' in P} s_{j'}^2 + eps)   (j prunable)
 *     out_j = 0                                                 (j forced)
 * with P the positions whose forced_keep is 0.  A row with no prunable
 * position is all zeros.  Ranking out instead of s keeps the order of the
 * prunable scores (a positive scale); out feeds tg_select_topk and, gathered
 * by tg_compact, tg_gate_softmax.
 *   scores [B, N] f32; forced_keep [B, N] u8 or NULL (every position prunable);
 *   out [B, N] f32 (may equal scores: in place); eps finite >= 0; N <= 2^24.
 * fp32 arithmetic (out_j = s_j times the fp32 reciprocal of the root, within
 * an ulp of the quotient), fixed-order reductions (deterministic).
 */
tg_status tg_score_normalize(const float *scores, const uint8_t *forced_keep, int64_t B,
                             int64_t N, float eps, float *out, void *stream);

/*
 * tg_gate_softmax -- gate values as the softmax of the normalised scores over
 * the kept set.  [DeepDive] section 3.2, Eq. 5:
 *     g_j = exp(b_j) / sum_{j' in S} exp(b_j')
 * per row, over the kept tokens (b gathered by tg_compact).  Entries whose
 * kept_idx is negative (padding) are not in S and get g = 0.  Eq. 6's per-head
 * gain: tg_gated_attn_fwd with these g and gamma_h = the gain (the softplus of
 * the raw parameter) gives softmax_j(z_ij + gamma_h b_j), i.e. Eq. 6's gate
 * with the per-head normaliser removed by the attention softmax.
 *   b [B, M] f32; kept_idx [B, M] i32 or NULL; g [B, M] f32 out.
 * fp32 arithmetic (expf), fixed-order reductions (deterministic).
 */
tg_status tg_gate_softmax(const float *b, const int32_t *kept_idx, int64_t B, int64_t M,
                          float *g, void *stream);

/*
 * tg_gate_softmax_bwd -- backward of tg_gate_softmax: per row
 *     db_j = g_j (dg_j - sum_k g_k dg_k)
 * with g the forward's output and dg = dL/dg (e.g. from tg_gated_attn_bwd).
 *   g, dg, db [B, M] f32 (db fully overwritten; 0 where g = 0).
 */
tg_status tg_gate_softmax_bwd(const float *g, const float *dg, int64_t B, int64_t M, float *db,
                              void *stream);

/* Kept tokens per row: n_forced + min(K, N - n_forced); -1 for invalid input. */
int64_t tg_kept_count(int64_t N, int64_t n_forced, int64_t K);

/* Workspace bytes tg_select_topk needs: 256 when N <= 32768 (one work-group
 * per row, nothing kept in it); otherwise, per row, per-work-group histograms
 * (4356 words per 4096 tokens) and 8 bytes per token for the threshold bin's
 * candidates.  0 for invalid sizes or N > 2^22. */
size_t tg_select_topk_workspace_size(int64_t B, int64_t N);

/*
 * tg_select_topk -- scaffold-aware top-K, kept in original order.
 * [DeepDive] section 3.1, Eq. 4: S = top-K of the prunable set P by score,
 * united with the non-prunable set; section 3.4: the budget is clamped and a
 * keep mask over the whole sequence is built.
 *   scores      [B, N] f32           ranking key
 *   forced_keep [B, N] u8 or NULL    nonzero = always kept (NULL: none forced)
 *   K >= 0                           budget of prunable tokens
 *   n_forced                         forced tokens per row the caller expects;
 *                                    sets the row length M = tg_kept_count(N, n_forced, K)
 *   kept_idx    [B, M] i32 out       strictly ascending token indices
 *   kept_count  [B] i32 out or NULL  true kept count of each row
 * Order: a non-NaN score ranks above NaN; larger ranks above smaller, with
 * -0 == +0 and -inf < finite < +inf; equal scores rank the lower index first.
 * A row whose forced count differs from n_forced keeps its true count
 * M_true = F + min(K, N - F): it writes min(M_true, M) indices, pads the rest
 * with -1 and reports M_true in kept_count.
 *   ws, ws_bytes                     device scratch of at least
 *                                    tg_select_topk_workspace_size(B, N) bytes,
 *                                    256-byte aligned, owned by the caller; its
 *                                    contents need no initial value and carry
 *                                    nothing between calls
 * Exact radix select over a monotone 32-bit key of the score (digits of 12,
 * 10 and 10 bits), deterministic: rows of up to 32768 tokens in one
 * work-group each with the keys in registers; longer rows in three launches
 * of 4096-token work-groups (histograms of the top 12 key bits, threshold bin
 * and exact threshold, output).  N <= 2^22, B <= 65535 (TG_ERR_UNSUPPORTED
 * otherwise); TG_ERR_WORKSPACE when the workspace is missing or too small.
 */
tg_status tg_select_topk(const float *scores, const uint8_t *forced_keep, int64_t B,
                         int64_t N, int64_t K, int64_t n_forced, int32_t *kept_idx,
                         int32_t *kept_count, void *ws, size_t ws_bytes, void *stream);

/*
 * tg_select_topk_noalloc -- tg_select_topk with no workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Arguments, results
 * and errors as tg_select_topk.  Its scratch is a 16 MiB device array inside
 * the library, one per GPU, held until the process ends: a call needing more
 * than that (tg_select_topk_workspace_size(B, N) > 16 MiB: rows of up to
 * 32768 tokens need none; a single row fits up to about 1.3 M tokens) returns
 * TG_ERR_UNSUPPORTED before any launch.  It allocates nothing.  Calls on one GPU share that array: calls that overlap
 * on one GPU (several streams or threads at once) race and must be ordered by
 * the caller; no state carries over from one call to the next.
 */
tg_status tg_select_topk_noalloc(const float *scores, const uint8_t *forced_keep, int64_t B,
                                 int64_t N, int64_t K, int64_t n_forced, int32_t *kept_idx,
                                 int32_t *kept_count, void *stream);

/*
 * tg_compact -- gather of the kept tokens' hidden states, original positions
 * and gate values.  [DeepDive] section 3.4: the hidden states are sliced with
 * the keep indices and the position ids are taken at the same indices.
 *   hidden     [B, N, d] (dt)        source rows
 *   pos        [B, N] i32 or NULL    position ids (NULL: position = index)
 *   gates      [B, N] f32 or NULL
 *   kept_idx   [B, M] i32            indices from tg_select_topk
 *   hidden_out [B, M, d] (dt) or NULL, pos_out [B, M] i32 or NULL,
 *   gates_out  [B, M] f32 or NULL (needs gates)
 * An index outside [0, N) (the -1 padding) yields a zero row, position -1
 * and gate 0.  The copy is bit-exact.
 */
tg_status tg_compact(const void *hidden, const int32_t *pos, const float *gates,
                     const int32_t *kept_idx, int64_t B, int64_t N, int64_t M, int64_t d,
                     tg_dtype dt, void *hidden_out, int32_t *pos_out, float *gates_out,
                     void *stream);

/* Workspace bytes the attention calls need (bwd = 0: forward, 1: backward).
 * Both attention calls require a workspace of at least this size, 256-byte
 * aligned: it holds the cos/sin table of the kept positions, the rotated keys,
 * the per-head bias gamma_h log2 g_j, the partial results and arrival
 * counters of the forward's split rows, the temperature's row factors and,
 * for the backward, the rotated queries, the row statistics (-lse / c, D_i),
 * the per-head column sums of dL/dZ and the per-row temperatures and their
 * gradient terms.  Its contents are scratch: nothing is carried between
 * calls. */
size_t tg_gated_attn_workspace_size(int64_t B, int64_t M, int64_t Hq, int64_t Hkv,
                                    int64_t D, int bwd);

/*
 * tg_gated_attn_fwd -- token-gated causal attention over the kept tokens.
 * [DeepDive] section 2, Eq. 2 (causal attention); section 3.2, Eq. 5 (each
 * weight multiplied by its key's gate value g_j, renormalised) and Eq. 6
 * (per-head non-negative gain); section 3.4 (temperature folded into the
 * query scale, gate passed as a per-key bias); [Summary] Figure 1(c).
 * For batch b, query head h, kv head h / (Hq / Hkv), rows i and keys j <= i
 * of the compacted sequence:
 *     S_ij = (q^_i . k^_j) / (sqrt(D) * tau) + gamma[h] * ln g_j
 *     o_i  = sum_j softmax_j(S_ij) v_j,     lse_i = ln sum_{j <= i} exp(S_ij)
 * q^, k^ are q, k rotated by rotary embedding at pos (rotate-half pairs
 * (x_i, x_{i+D/2}), angle pos * rope_theta^(-2i/D), computed in fp64); pos
 * NULL means no rotation.  A key with g_j = 0 gets weight 0; a row with no
 * visible key gets o = 0, lse = -inf.
 * With sigma (non-NULL) the logits follow the operative rule of [DeepDive]
 * section 3.2, Eq. 8, with the pruning-ratio temperature of Eq. 7:
 *     S_ij = t_ih * Z_ij,  Z_ij = (q^_i . k^_j) / (sqrt(D) * tau) + gamma[h] ln g_j
 *     t_ih = softplus(sigma[h]) * ln m_i / ln max(2, p_i)
 * with m_i = i + 1 the keys row i sees after pruning and p_i = pos_i + 1 the
 * positions it saw before (p_i = i + 1 when pos is NULL).  t is computed in
 * fp32 and kept >= 1e-30 (t = 0 at row 0, whose only live key gets weight 1
 * either way), so a sigma below about -69 behaves as that floor.
 *   q [B, M, Hq, D], k, v [B, M, Hkv, D], o [B, M, Hq, D] (dt)
 *   g [B, M] f32 > = 0, gamma [Hq] f32, pos [B, M] i32 or NULL
 *   sigma [Hq] f32 or NULL (no temperature: t = 1)
 *   lse [B, Hq, M] f32 out or NULL (needed by the backward)
 *   o_lo [B, M, Hq, D] bf16 out or NULL (bf16 only): the residual of o's
 *     rounding, o_lo = bf16(o32 - o) for the fp32 output o32, so that
 *     o + o_lo is o32 to about 2^-18 relative (for the backward)
 * bf16: D in {64, 128}, Hq / Hkv in {1, 2, 4, 8}; q.k and
 * P.v on matrix cores with fp32 accumulation, softmax in fp32, P rounded to
 * bf16 for the P.v product.  f32: D <= 128, plain fp32 arithmetic.
 * The bf16 softmax of a stretch of keys is taken against a fixed reference:
 * the largest live logit of its first 32 keys, or, when g = 0 on every key of
 * those 32 that a row sees, the logit of the stretch's first key with g > 0;
 * a stretch whose sum would overflow is recomputed with the reference raised.
 * Live logits count at any scale.
 */
tg_status tg_gated_attn_fwd(const void *q, const void *k, const void *v, const float *g,
                            const float *gamma, const int32_t *pos, float rope_theta,
                            float tau, const float *sigma, int64_t B, int64_t M, int64_t Hq,
                            int64_t Hkv, int64_t D, tg_dtype dt, void *o, float *lse, void *o_lo,
                            void *ws, size_t ws_bytes, void *stream);

/*
 * tg_gated_attn_bwd -- gradients of tg_gated_attn_fwd.  The task gradient
 * reaches the scorer through the attention bias ([DeepDive] section 3.1 last
 * paragraph, section 3.2, and the flowchart's "task gradient through bias").
 * Given dout = dL/do and the forward's lse:
 *     dP_ij = dout_i . v_j,  D_i = sum_j P_ij dP_ij,  dS_ij = P_ij (dP_ij - D_i)
 *     dq = R(-phi_i) c sum_j dS_ij k^_j,   dk = R(-phi_j) c sum_i dS_ij q^_i
 *     dv_j = sum_i P_ij dout_i,            (dk, dv summed over the group)
 *     dg_j = sum_h gamma_h colsum_h(j) / g_j      (0 where g_j = 0)
 *     dgamma_h = sum_b sum_j colsum_h(j) ln g_j,   colsum_h(j) = sum_i dS_ij
 * with c = 1 / (sqrt(D) tau).  D_i is formed exactly from fp32 P and dP.
 * Without o and o_lo that takes one more pass over the keys.  With them (bf16,
 * both given or both NULL: the forward's o and o_lo of the same inputs) the
 * dq pass takes D_o = dout_i . (o_i + o_lo_i) in its dS and sums that dS's row,
 * which yields the exact D_i for dk, dv, dg, dgamma and dsigma; dq alone keeps
 * D_o, off by the forward's bf16 rounding of P (an error in dq of about
 * 2^-9 c |D_i| |sum_j P_ij k^_j|, 2e-3 at the training shape's inputs).  With sigma (the temperature of Eq. 7/8, as in the
 * forward) dS_ij is dL/dS of S = t Z, dL/dZ_ij = t_ih dS_ij takes its place in
 * dq, dk and colsum, and
 *     dsigma_h = sigmoid(sigma_h) sum_b sum_i (ln m_i / ln max(2, p_i)) sum_j dS_ij Z_ij
 * (sigma and dsigma both given or both NULL).  Outputs are fp32 and fully
 * overwritten:
 *   dq [B, M, Hq, D], dk, dv [B, M, Hkv, D], dg [B, M], dgamma [Hq], dsigma [Hq].
 * Deterministic: repeated calls give bitwise-identical results.
 */
tg_status tg_gated_attn_bwd(const void *q, const void *k, const void *v, const float *g,
                            const float *gamma, const int32_t *pos, float rope_theta,
                            float tau, const float *sigma, const float *lse, const void *dout,
                            const void *o, const void *o_lo, int64_t B, int64_t M, int64_t Hq,
                            int64_t Hkv, int64_t D,
                            tg_dtype dt, float *dq, float *dk, float *dv, float *dg,
                            float *dgamma, float *dsigma, void *ws, size_t ws_bytes,
                            void *stream);

/*
 * Per-head scores with a uniform head aggregation for selection, and per-head
 * gates ([DeepDive] section 3.4: the released code keeps a per-layer, per-head
 * bias and aggregates the heads uniformly for selection).  Reading: the
 * scorer's second layer has H outputs (w2 [H, d_ff]); each head's scores are
 * normalised as in tg_score_normalize; selection ranks their mean over heads;
 * each head's gate is the softmax over the kept set of its own scores; and
 * query head h attends with bias gamma_h ln g_hj.
 *
 * tg_gate_score_heads: b~[b][h][n] = sum_k w2[h,k] SiLU(sum_i w1[k,i] a~[b,n,i])
 *   with a~ = RMSNorm(hidden) (weight ln_w or NULL = 1, ln_eps) when ln != 0,
 *   else a~ = hidden.  hidden [B, N, d] (dt), w1 [d_ff, d], w2 [H, d_ff] (dt),
 *   1 <= H <= 16; scores [B, H, N] f32 out; workspace and errors as
 *   tg_gate_score (bf16: the packed W1).  bf16: both products on the matrix
 *   cores with fp32 accumulation; the second takes SiLU as two bf16 parts
 *   (hi + lo, within 2^-17 of the fp32 value) and w2 as stored.
 * tg_score_normalize_heads: tg_score_normalize on each (b, h) row of
 *   scores [B, H, N], with b's forced mask [B, N] (or NULL); out may be scores.
 * tg_aggregate_heads: out[b][n] = (sum_h b[b][h][n]) / H (heads in order),
 *   b [B, H, N], out [B, N] f32: the vector tg_select_topk ranks.
 * tg_gather_heads: out[b][h][m] = b[b][h][kept_idx[b][m]] (0 where the index is
 *   negative): b [B, H, N], kept_idx [B, M], out [B, H, M].
 * tg_gate_softmax_heads: tg_gate_softmax on each (b, h) row of b [B, H, M]
 *   with b's kept_idx [B, M] (or NULL); g [B, H, M].  (tg_gate_softmax_bwd
 *   applies to [B * H, M] as it is.)
 * tg_gated_attn_fwd_headgates / _bwd_headgates: tg_gated_attn_fwd / _bwd with
 *   one gate per (query head, key): g [B, Hq, M] f32 (> = 0), bias
 *   gamma_h ln g_hj; the backward's dg is [B, Hq, M],
 *   dg_hj = gamma_h colsum_h(j) / g_hj (0 where g_hj = 0), and dgamma uses
 *   ln g_hj.  Everything else (sigma, o_lo / o, workspace, dtypes, errors) as
 *   the shared-gate calls.
 */
tg_status tg_gate_score_heads(const void *hidden, int ln, const void *ln_w, float ln_eps,
                              const void *w1, const void *w2, int64_t B, int64_t N, int64_t d,
                              int64_t d_ff, int64_t H, tg_dtype dt, float *scores, void *ws,
                              size_t ws_bytes, void *stream);
tg_status tg_score_normalize_heads(const float *scores, const uint8_t *forced_keep, int64_t B,
                                   int64_t H, int64_t N, float eps, float *out, void *stream);
tg_status tg_aggregate_heads(const float *b, int64_t B, int64_t H, int64_t N, float *out,
                             void *stream);
tg_status tg_gather_heads(const float *b, const int32_t *kept_idx, int64_t B, int64_t H,
                          int64_t N, int64_t M, float *out, void *stream);
tg_status tg_gate_softmax_heads(const float *b, const int32_t *kept_idx, int64_t B, int64_t H,
                                int64_t M, float *g, void *stream);
tg_status tg_gated_attn_fwd_headgates(const void *q, const void *k, const void *v, const float *g,
                                      const float *gamma, const int32_t *pos, float rope_theta,
                                      float tau, const float *sigma, int64_t B, int64_t M,
                                      int64_t Hq, int64_t Hkv, int64_t D, tg_dtype dt, void *o,
                                      float *lse, void *o_lo, void *ws, size_t ws_bytes,
                                      void *stream);
tg_status tg_gated_attn_bwd_headgates(const void *q, const void *k, const void *v, const float *g,
                                      const float *gamma, const int32_t *pos, float rope_theta,
                                      float tau, const float *sigma, const float *lse,
                                      const void *dout, const void *o, const void *o_lo,
                                      int64_t B, int64_t M, int64_t Hq,
                                      int64_t Hkv, int64_t D, tg_dtype dt, float *dq, float *dk,
                                      float *dv, float *dg, float *dgamma, float *dsigma, void *ws,
                                      size_t ws_bytes, void *stream);

/*
 * tg_gate_score_clone -- raw scores from a scoring branch cloned from the gate
 * layer's MLP ([DeepDive] section 3.4, and the section 3 pipeline figure's
 * "MLP clone of gate-layer MLP" feeding the sequence-normalised scores of
 * Eq. 3).  The pages give the branch no shape.  Reading: the gated (SwiGLU)
 * MLP of the Qwen3 models the pages evaluate, with its shapes, followed by a
 * head projection P of H rows (zero at initialisation, so the scores start
 * at zero as section 3.1 states):
 *   m_k    = SiLU(sum_i w_gate[k,i] a~[b,n,i]) * (sum_i w_up[k,i] a~[b,n,i])
 *   b~[b][h][n] = sum_o w_head[h,o] sum_k w_down[o,k] m_k
 * with a~ = RMSNorm(hidden) (weight ln_w or NULL = 1, ln_eps) when ln != 0,
 * else a~ = hidden.  The outputs feed tg_score_normalize_heads (or, with
 * H = 1, tg_score_normalize) exactly as the per-head scorer's do.
 *   hidden [B, N, d] (dt); w_gate, w_up [d_i, d]; w_down [d, d_i];
 *   w_head [H, d] (dt), 1 <= H <= 16, d_i <= 32768; scores [B, H, N] f32 out.
 *   The call computes U = w_head w_down ([H, d_i], fp32) into the workspace and
 *   then b~ = U m, the same sum taken in the other order.  bf16: d % 32 == 0;
 *   ln_w is folded into the packed gate and up weights (one bf16 rounding of
 *   each product, as tg_gate_score_ln); the gate and up products on the matrix
 *   cores (fp32 accumulation), SiLU and
 *   m in fp32, and U m as a matrix-core product of bf16 pairs (U and m each as
 *   hi + lo, within 2^-16 of the fp32 product).  f32: d % 4 == 0,
 *   d + d_i <= 16000, plain fp32.
 *   ws: tg_gate_score_clone_workspace_size(d, d_i, H, dt) bytes, 16-byte
 *   aligned (bf16: the gate/up weights packed in fragment order; then U and
 *   the partial sums that form it), owned by the caller, overwritten.
 *   Errors as tg_gate_score; TG_ERR_UNSUPPORTED for H or d_i out of range.
 *   Deterministic: fixed-order sums throughout.
 */
size_t tg_gate_score_clone_workspace_size(int64_t d, int64_t d_i, int64_t H, tg_dtype dt);
tg_status tg_gate_score_clone(const void *hidden, int ln, const void *ln_w, float ln_eps,
                              const void *w_gate, const void *w_up, const void *w_down,
                              const void *w_head, int64_t B, int64_t N, int64_t d, int64_t d_i,
                              int64_t H, tg_dtype dt, float *scores, void *ws, size_t ws_bytes,
                              void *stream);

/*
 * Packed variable-length attention: the training path evaluates both budgets'
 * targets in one call ([DeepDive] section 3.3), i.e. several sequences of
 * different lengths packed back to back.  Sequence s holds tokens
 * cu_seqlens[s] .. cu_seqlens[s+1]-1 and attends causally within itself only,
 * exactly as tg_gated_attn_fwd / _bwd on that sequence alone (row index, and
 * the temperature's m_i, counted from the sequence start; positions, if given,
 * are the caller's per token).
 *   cu_seqlens: HOST array of nseq + 1 int64 offsets, cu_seqlens[0] = 0,
 *     non-decreasing (empty sequences allowed); T = cu_seqlens[nseq] tokens.
 *   q [T, Hq, D], k, v [T, Hkv, D], o [T, Hq, D] (dt); g [T] f32; pos [T] i32
 *     or NULL; sigma [Hq] or NULL (as in tg_gated_attn_fwd);
 *   lse: Hq * T f32, sequence s's [Hq, M_s] block at offset Hq * cu_seqlens[s];
 *   o_lo (forward, optional) and o, o_lo (backward, optional): [T, Hq, D]
 *     bf16, as in tg_gated_attn_fwd / _bwd;
 *   backward: dq [T, Hq, D], dk, dv [T, Hkv, D], dg [T] f32 per token; dgamma
 *     (and dsigma) [Hq] summed over all sequences.
 * Maximal runs of adjacent equal-length sequences (empty ones skipped) are
 * the unit of work.  The matrix-core kernels take up to 16 runs per launch:
 * each work-group holds one block (the forward: one piece of a block) of one
 * sequence of one run, with the blocks of all runs ordered longest first, so
 * sequences of different lengths share the compute units.  The bf16 forward
 * picks its key-split length once for the 16 runs of a launch; the prep
 * passes, and the backward's dg pass, also take 16 runs per launch, and one
 * reduction gives dgamma (dsigma) (f32: one launch of each kernel per run).
 * The workspace (tg_gated_attn_varlen_workspace_size,
 * 256-byte aligned) holds every run's arrays side by side.  Validation,
 * dtypes and errors as the batched calls; dgamma / dsigma are summed in run
 * order (deterministic).
 */
size_t tg_gated_attn_varlen_workspace_size(const int64_t *cu_seqlens, int64_t nseq, int64_t Hq,
                                           int64_t Hkv, int64_t D, int bwd);
tg_status tg_gated_attn_fwd_varlen(const void *q, const void *k, const void *v, const float *g,
                                   const float *gamma, const int32_t *pos, float rope_theta,
                                   float tau, const float *sigma, const int64_t *cu_seqlens,
                                   int64_t nseq, int64_t Hq, int64_t Hkv, int64_t D, tg_dtype dt,
                                   void *o, float *lse, void *o_lo, void *ws, size_t ws_bytes,
                                   void *stream);
tg_status tg_gated_attn_bwd_varlen(const void *q, const void *k, const void *v, const float *g,
                                   const float *gamma, const int32_t *pos, float rope_theta,
                                   float tau, const float *sigma, const float *lse,
                                   const void *dout, const void *o, const void *o_lo,
                                   const int64_t *cu_seqlens, int64_t nseq,
                                   int64_t Hq, int64_t Hkv, int64_t D, tg_dtype dt, float *dq,
                                   float *dk, float *dv, float *dg, float *dgamma, float *dsigma,
                                   void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* TOKENGATE_H */
