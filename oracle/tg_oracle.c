/*
 * tg_oracle.c -- plain, slow CPU oracle for the TokenGate gate-layer path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or helper with the
 * HIP library: every function below is written from the method's definition.
 *
 * Sources (cited by page title and section / equation):
 *   [DeepDive]  "TokenGate: Learnable Token Pruning for Fast, Memory-Efficient
 *               LLM Prefill" (agientry.com paper deep dive), sections 2, 3.1,
 *               3.2 and 3.4, equations 2-8.
 *   [Summary]   "TokenGate: Adapting LLMs for Fast and Memory-Efficient Prefill
 *               with Learned Token Pruning" (thelatestinai.com), Figure 1.
 *
 * Conventions:
 *   - All floating-point arithmetic is fp64 (double).  Inputs arrive already
 *     widened exactly from their storage type (bf16 or fp32) to double.
 *   - Plain loops; OpenMP only over independent rows / heads.
 *   - Compiled without fast-math and with -ffp-contract=off.
 *
 * Parity pins: every function is checked in tests/test_oracle_*.py against
 * something other than itself (brute force, closed forms, NumPy/PyTorch CPU
 * library routines, autograd, finite differences).  The readings listed as
 * contract choices (scorer shape without biases, gate of forced tokens = 1,
 * scalar temperature on q.k only, RoPE pairing and theta, where bf16 rounding
 * happens, the clone scorer's SwiGLU form and head projection) are "parity
 * unpinned" by the pages: the pages do not fix them.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* a1. Scoring MLP and gate value                                            */
/* ------------------------------------------------------------------------ */
/*
 * [DeepDive] section 3.1, Eq. 3 (first part): a small MLP maps each token's
 * normalised post-attention residual to one scalar score, b~_j = MLP(a~_j).
 * Reading used here: two layers d -> d_ff -> 1, SiLU in between, no biases:
 *     u_k = sum_i W1[k,i] h[i]            (W1 is stored out x in: [d_ff, d])
 *     s   = sum_k w2[k] * SiLU(u_k),      SiLU(u) = u / (1 + exp(-u))
 * Gate value: g = sigmoid(s) = 1 / (1 + exp(-s)) for prunable tokens.  For a
 * forced (non-prunable) token, Eq. 3 sets its score to zero bias, so its gate
 * enters attention as g = 1 (log g = 0, no bias).
 *
 * hidden: [T, d]; forced: [T] or NULL; scores, gates: [T] (gates may be NULL).
 */
void tgo_gate_score(const double *hidden, const double *w1, const double *w2,
                    const uint8_t *forced, int64_t T, int64_t d, int64_t d_ff,
                    double *scores, double *gates)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < T; ++t) {
        const double *h = hidden + t * d;
        double s = 0.0;
        for (int64_t k = 0; k < d_ff; ++k) {
            const double *row = w1 + k * d;
            double u = 0.0;
            for (int64_t i = 0; i < d; ++i)
                u += row[i] * h[i];
            double a = u / (1.0 + exp(-u));
            s += w2[k] * a;
        }
        scores[t] = s;
        if (gates) {
            if (forced && forced[t])
                gates[t] = 1.0;
            else
                gates[t] = 1.0 / (1.0 + exp(-s));
        }
    }
}

/* ------------------------------------------------------------------------ */
/* a2. Scaffold-aware top-K selection                                        */
/* ------------------------------------------------------------------------ */
/*
 * [DeepDive] section 3.1, Eq. 4: S = topK over the prunable set P of the
 * scores, united with the non-prunable set N.  Section 3.4: the budget is
 * clamped (K' = min(K, |P|)) and a keep mask over the full sequence is built,
 * so the kept tokens come out in their original (ascending) order.
 *
 * Order used to rank prunable tokens (a total order on (score, index)):
 *   1. any non-NaN score ranks above NaN;
 *   2. among non-NaN scores, the larger ranks higher, with -0 == +0 and
 *      -inf < every finite value < +inf (plain IEEE comparison);
 *   3. equal scores (and NaN vs NaN): the lower index ranks higher.
 * Scores are compared as the fp32 values the caller holds.
 */
typedef struct {
    float s;
    int64_t idx;
} ranked_t;

/* qsort comparator: negative when a ranks before b. */
static int rank_cmp(const void *pa, const void *pb)
{
    const ranked_t *a = (const ranked_t *)pa, *b = (const ranked_t *)pb;
    int na = isnan(a->s), nb = isnan(b->s);
    if (na != nb)
        return na ? 1 : -1;
    if (!na && a->s != b->s)
        return a->s > b->s ? -1 : 1;
    return a->idx < b->idx ? -1 : (a->idx > b->idx ? 1 : 0);
}

/*
 * One batch row.  scores: [N]; forced: [N] or NULL (no forced token).
 * Writes min(true M, M_alloc) ascending indices into kept[0..M_alloc) and pads
 * the rest with -1.  Returns the true kept count M = |N| + min(K, |P|), where
 * |N| is the number of forced tokens actually present in `forced`.
 * Returns -1 if K < 0 or memory cannot be allocated.
 */
int64_t tgo_select_topk(const float *scores, const uint8_t *forced, int64_t N,
                        int64_t K, int64_t M_alloc, int32_t *kept)
{
    if (K < 0)
        return -1;
    int64_t nF = 0;
    for (int64_t n = 0; n < N; ++n)
        if (forced && forced[n])
            ++nF;
    int64_t nP = N - nF;
    int64_t Kc = K < nP ? K : nP;

    ranked_t *cand = (ranked_t *)malloc(sizeof(ranked_t) * (size_t)(nP > 0 ? nP : 1));
    uint8_t *keep = (uint8_t *)calloc((size_t)(N > 0 ? N : 1), 1);
    if (!cand || !keep) {
        free(cand);
        free(keep);
        return -1;
    }
    int64_t c = 0;
    for (int64_t n = 0; n < N; ++n) {
        if (forced && forced[n]) {
            keep[n] = 1; /* every non-prunable token survives */
        } else {
            cand[c].s = scores[n];
            cand[c].idx = n;
            ++c;
        }
    }
    qsort(cand, (size_t)nP, sizeof(ranked_t), rank_cmp);
    for (int64_t r = 0; r < Kc; ++r)
        keep[cand[r].idx] = 1;

    int64_t m = 0;
    for (int64_t n = 0; n < N; ++n) {
        if (keep[n]) {
            if (m < M_alloc)
                kept[m] = (int32_t)n;
            ++m;
        }
    }
    for (int64_t r = m; r < M_alloc; ++r)
        kept[r] = -1;
    free(cand);
    free(keep);
    return m;
}

/* ------------------------------------------------------------------------ */
/* a3. Compaction                                                            */
/* ------------------------------------------------------------------------ */
/*
 * [DeepDive] section 3.4: the kept hidden states are sliced with the keep
 * indices and the position ids are taken at the same indices (the original
 * positions); the gate values of the kept tokens are handed to attention.
 * A plain gather.  Rows whose index is outside [0, N) (padding, -1) give a
 * zero hidden row, position -1 and gate 0.
 *
 * One batch row.  hidden: N rows of row_bytes bytes; pos: [N] or NULL
 * (NULL means position = index); gates: [N] or NULL.
 */
void tgo_compact(const uint8_t *hidden, const int32_t *pos, const float *gates,
                 const int32_t *kept, int64_t N, int64_t M, int64_t row_bytes,
                 uint8_t *hidden_out, int32_t *pos_out, float *gates_out)
{
    for (int64_t m = 0; m < M; ++m) {
        int64_t n = kept[m];
        int valid = (n >= 0 && n < N);
        if (hidden_out) {
            if (valid)
                memcpy(hidden_out + m * row_bytes, hidden + n * row_bytes, (size_t)row_bytes);
            else
                memset(hidden_out + m * row_bytes, 0, (size_t)row_bytes);
        }
        if (pos_out)
            pos_out[m] = valid ? (pos ? pos[n] : (int32_t)n) : -1;
        if (gates_out)
            gates_out[m] = valid ? (gates ? gates[n] : 1.0f) : 0.0f;
    }
}

/* ------------------------------------------------------------------------ */
/* Rotary position embedding at the kept tokens' original positions          */
/* ------------------------------------------------------------------------ */
/*
 * The pages say the kept positions are the original position ids
 * ([DeepDive] section 3.4); the rotation itself is the backbone's (Qwen3 uses
 * rotary embeddings).  Reading: rotate-half pairing (x_i, x_{i+D/2}) for
 * i < D/2, angle phi_i = p * theta^(-2i/D), computed in fp64:
 *     x_i'       = x_i cos(phi) - x_{i+D/2} sin(phi)
 *     x_{i+D/2}' = x_{i+D/2} cos(phi) + x_i sin(phi)
 */
static void rope_rotate(double *x, int64_t D, double p, double theta, int sign)
{
    int64_t h = D / 2;
    for (int64_t i = 0; i < h; ++i) {
        double phi = p * pow(theta, -2.0 * (double)i / (double)D);
        double cs = cos(phi), sn = sign * sin(phi);
        double a = x[i], b = x[i + h];
        x[i] = a * cs - b * sn;
        x[i + h] = b * cs + a * sn;
    }
}

/*
 * Round a double to the nearest bf16 value (ties to even), returned as a
 * double.  bf16 keeps 8 significant bits: clear the low 45 of the 52
 * fraction bits of the double with round-to-nearest-even.  Values below the
 * normal range of bf16 go through float (not reached by these workloads).
 */
static double round_bf16(double x)
{
    if (isnan(x) || isinf(x) || x == 0.0)
        return x;
    if (fabs(x) < 1.1754943508222875e-38) {
        float f = (float)x;
        uint32_t u;
        memcpy(&u, &f, 4);
        u += 0x7FFFu + ((u >> 16) & 1u);
        u &= 0xFFFF0000u;
        memcpy(&f, &u, 4);
        return (double)f;
    }
    uint64_t u;
    memcpy(&u, &x, 8);
    uint64_t lsb = (u >> 45) & 1u;
    u += ((uint64_t)1 << 44) - 1u + lsb;
    u &= ~(((uint64_t)1 << 45) - 1u);
    memcpy(&x, &u, 8);
    return x;
}

/* Rotate (and optionally bf16-round) a [B, M, H, D] tensor into `out`. */
static void rotate_all(const double *x, double *out, const int32_t *pos, double theta,
                       int64_t B, int64_t M, int64_t H, int64_t D, int round)
{
#pragma omp parallel for schedule(static)
    for (int64_t bm = 0; bm < B * M; ++bm) {
        for (int64_t h = 0; h < H; ++h) {
            double *y = out + (bm * H + h) * D;
            memcpy(y, x + (bm * H + h) * D, sizeof(double) * (size_t)D);
            if (pos) {
                rope_rotate(y, D, (double)pos[bm], theta, +1);
                if (round)
                    for (int64_t e = 0; e < D; ++e)
                        y[e] = round_bf16(y[e]);
            }
        }
    }
}

/*
 * Temperature of the operative attention rule ([DeepDive] section 3.2, Eq. 7):
 *     tau_ih = softplus(sigma_h) * ln m_i / ln max(2, p_i)
 * with m_i = i + 1 the kept keys visible to compacted row i and p_i = pos_i + 1
 * the original positions visible to it (p_i = m_i without positions).
 */
static double softplus_d(double x) { return x > 30.0 ? x : log1p(exp(x)); }
static double temp_ratio(int64_t i, const int32_t *pos, int64_t bm)
{
    double m = (double)(i + 1);
    double p = pos ? (double)pos[bm] + 1.0 : m;
    return log(m) / log(p > 2.0 ? p : 2.0);
}

/* ------------------------------------------------------------------------ */
/* a4. Token-gated causal attention, forward                                 */
/* ------------------------------------------------------------------------ */
/*
 * [DeepDive] section 2, Eq. 2 (causal attention, z = q.k / sqrt(d_head)) and
 * section 3.2, Eq. 5 (each attention weight multiplied by its key's gate value
 * g_j and renormalised; [Summary] Figure 1(c)), with the per-head gain of
 * Eq. 6 and a temperature.  Form computed here, for query row i, query head h,
 * kv head kv = floor(h / (Hq/Hkv)), keys j <= i (indices in the compacted
 * sequence):
 *     S_ij = q^_i . k^_j / (sqrt(D) * tau) + gamma_h * ln g_j
 *     P_ij = exp(S_ij - lse_i),   lse_i = ln sum_{j<=i} exp(S_ij)
 *     O_i  = sum_j P_ij v_j
 * which equals exp(z_ij / tau) * g_j^gamma_h renormalised over j <= i.
 * q^, k^ are q, k rotated at their positions (identity when pos == NULL) and,
 * when round is set, rounded to bf16 (the precision the tensor cores consume).
 * A key with g_j = 0 has ln g_j = -inf and weight 0; a row whose every logit
 * is -inf gets O = 0 and lse = -inf.
 *
 * With sigma (per query head, NULL for none) the rule is the operative one of
 * [DeepDive] section 3.2, Eq. 8: the whole logit is scaled by the temperature
 * tau_ih of Eq. 7 (see temp_ratio above),
 *     S_ij = tau_ih * (q^_i . k^_j / (sqrt(D) * tau) + gamma_h * ln g_j),
 * a key with g_j = 0 still getting weight 0.
 *
 * rows: optional list of nrows flattened (b * M + i) query rows to compute;
 * NULL computes all B*M rows.  o: [B, M, Hq, D], lse: [B, Hq, M]; entries of
 * rows not listed are left untouched.
 */
int tgo_attn_fwd(const double *q, const double *k, const double *v, const double *g,
                 const double *gamma, const int32_t *pos, double theta, double tau,
                 const double *sigma, int64_t B, int64_t M, int64_t Hq, int64_t Hkv, int64_t D,
                 int round, const int64_t *rows, int64_t nrows, int g_per_head, double *o, double *lse)
{
    if (Hkv <= 0 || Hq % Hkv != 0)
        return -1;
    int64_t grp = Hq / Hkv;
    double c = 1.0 / (sqrt((double)D) * tau);
    double *qr = (double *)malloc(sizeof(double) * (size_t)(B * M * Hq * D));
    double *kr = (double *)malloc(sizeof(double) * (size_t)(B * M * Hkv * D));
    if (!qr || !kr) {
        free(qr);
        free(kr);
        return -1;
    }
    rotate_all(q, qr, pos, theta, B, M, Hq, D, round);
    rotate_all(k, kr, pos, theta, B, M, Hkv, D, round);
    int64_t R = rows ? nrows : B * M;

#pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t r = 0; r < R; ++r) {
            for (int64_t h = 0; h < Hq; ++h) {
                int64_t bi = rows ? rows[r] : r;
                int64_t b = bi / M, i = bi % M;
                int64_t kv = h / grp;
                const double *qi = qr + ((b * M + i) * Hq + h) * D;
                double t = sigma ? softplus_d(sigma[h]) * temp_ratio(i, pos, b * M + i) : 1.0;
                double mx = -INFINITY;
                for (int64_t j = 0; j <= i; ++j) {
                    const double *kj = kr + ((b * M + j) * Hkv + kv) * D;
                    double dot = 0.0;
                    for (int64_t e = 0; e < D; ++e)
                        dot += qi[e] * kj[e];
                    double gj = g[g_per_head ? (b * Hq + h) * M + j : b * M + j];
                    logit[j] = gj > 0.0 ? t * (c * dot + gamma[h] * log(gj)) : -INFINITY;
                    if (logit[j] > mx)
                        mx = logit[j];
                }
                double *oi = o + ((b * M + i) * Hq + h) * D;
                for (int64_t e = 0; e < D; ++e)
                    oi[e] = 0.0;
                if (mx == -INFINITY) {
                    lse[(b * Hq + h) * M + i] = -INFINITY;
                    continue;
                }
                double sum = 0.0;
                for (int64_t j = 0; j <= i; ++j)
                    sum += exp(logit[j] - mx);
                double l = mx + log(sum);
                lse[(b * Hq + h) * M + i] = l;
                for (int64_t j = 0; j <= i; ++j) {
                    double p = exp(logit[j] - l);
                    const double *vj = v + ((b * M + j) * Hkv + kv) * D;
                    for (int64_t e = 0; e < D; ++e)
                        oi[e] += p * vj[e];
                }
            }
        }
        free(logit);
    }
    free(qr);
    free(kr);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* a5. Token-gated causal attention, backward                                */
/* ------------------------------------------------------------------------ */
/*
 * The task gradient reaches the scorer through the attention bias
 * ([DeepDive] section 3.1 last paragraph, section 3.2, and the flowchart's
 * "task gradient through bias" edge).  Derivatives of the forward above,
 * given dO, for each (b, h, i) and j <= i:
 *     dP_ij = dO_i . v_j
 *     D_i   = sum_j P_ij dP_ij
 *     dS_ij = P_ij (dP_ij - D_i)
 *     dq^_i += c dS_ij k^_j      dk^_j += c dS_ij q^_i      dv_j += P_ij dO_i
 *     colsum_h(j) += dS_ij
 * then dq = R(-phi_i) dq^, dk = R(-phi_j) dk^ (the bf16 rounding of q^, k^ is
 * passed straight through), dk and dv summed over the query heads of the
 * group, and for the gate terms (S depends on g_j through gamma_h ln g_j):
 *     dg_j     = sum_h gamma_h colsum_h(j) / g_j      (0 where g_j = 0)
 *     dgamma_h = sum_b sum_j colsum_h(j) ln g_j       (terms with g_j = 0 skipped)
 * With sigma (Eq. 8, S_ij = tau_ih Z_ij, Z_ij the bracket of the forward), the
 * bracket's gradient is dZ_ij = tau_ih dS_ij: it replaces dS_ij in dq^, dk^ and
 * colsum, and the temperature gets dtau_ih = sum_j dS_ij Z_ij, so
 *     dsigma_h = sum_b sum_i dtau_ih * ln m_i / ln max(2, p_i) * sigmoid(sigma_h).
 *
 * dq: [B,M,Hq,D]; dk, dv: [B,M,Hkv,D]; dg: [B,M]; dgamma: [Hq]; dsigma: [Hq]
 * (written when sigma is given).
 */
int tgo_attn_bwd(const double *q, const double *k, const double *v, const double *g,
                 const double *gamma, const int32_t *pos, double theta, double tau,
                 const double *sigma, const double *dout, int64_t B, int64_t M, int64_t Hq,
                 int64_t Hkv, int64_t D, int round, int g_per_head, double *dq, double *dk,
                 double *dv, double *dg, double *dgamma, double *dsigma)
{
    if (Hkv <= 0 || Hq % Hkv != 0)
        return -1;
    int64_t grp = Hq / Hkv;
    double c = 1.0 / (sqrt((double)D) * tau);
    double *qr = (double *)malloc(sizeof(double) * (size_t)(B * M * Hq * D));
    double *kr = (double *)malloc(sizeof(double) * (size_t)(B * M * Hkv * D));
    double *colsum = (double *)calloc((size_t)(B * Hq * M), sizeof(double));
    double *dsig = (double *)calloc((size_t)(B * Hq), sizeof(double)); /* per (b, h): no races */
    if (!qr || !kr || !colsum || !dsig) {
        free(qr);
        free(kr);
        free(colsum);
        free(dsig);
        return -1;
    }
    rotate_all(q, qr, pos, theta, B, M, Hq, D, round);
    rotate_all(k, kr, pos, theta, B, M, Hkv, D, round);
    memset(dq, 0, sizeof(double) * (size_t)(B * M * Hq * D));
    memset(dk, 0, sizeof(double) * (size_t)(B * M * Hkv * D));
    memset(dv, 0, sizeof(double) * (size_t)(B * M * Hkv * D));

    /* One task per (b, kv head): it owns dk/dv of that kv head, so no races. */
#pragma omp parallel
    {
        double *P = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
        double *dP = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
        double *Z = (double *)malloc(sizeof(double) * (size_t)(M > 0 ? M : 1));
#pragma omp for schedule(dynamic, 1) collapse(2)
        for (int64_t b = 0; b < B; ++b) {
            for (int64_t kv = 0; kv < Hkv; ++kv) {
                for (int64_t h = kv * grp; h < (kv + 1) * grp; ++h) {
                    for (int64_t i = 0; i < M; ++i) {
                        const double *qi = qr + ((b * M + i) * Hq + h) * D;
                        const double *doi = dout + ((b * M + i) * Hq + h) * D;
                        double ratio = sigma ? temp_ratio(i, pos, b * M + i) : 1.0;
                        double t = sigma ? softplus_d(sigma[h]) * ratio : 1.0;
                        double mx = -INFINITY;
                        for (int64_t j = 0; j <= i; ++j) {
                            const double *kj = kr + ((b * M + j) * Hkv + kv) * D;
                            double dot = 0.0;
                            for (int64_t e = 0; e < D; ++e)
                                dot += qi[e] * kj[e];
                            double gj = g[g_per_head ? (b * Hq + h) * M + j : b * M + j];
                            Z[j] = gj > 0.0 ? c * dot + gamma[h] * log(gj) : -INFINITY;
                            P[j] = gj > 0.0 ? t * Z[j] : -INFINITY;
                            if (P[j] > mx)
                                mx = P[j];
                        }
                        if (mx == -INFINITY)
                            continue; /* no visible key: zero gradient */
                        double sum = 0.0;
                        for (int64_t j = 0; j <= i; ++j)
                            sum += exp(P[j] - mx);
                        double l = mx + log(sum);
                        double Di = 0.0;
                        for (int64_t j = 0; j <= i; ++j) {
                            P[j] = exp(P[j] - l);
                            const double *vj = v + ((b * M + j) * Hkv + kv) * D;
                            double d = 0.0;
                            for (int64_t e = 0; e < D; ++e)
                                d += doi[e] * vj[e];
                            dP[j] = d;
                            Di += P[j] * d;
                        }
                        double *dqi = dq + ((b * M + i) * Hq + h) * D;
                        double dt = 0.0;
                        for (int64_t j = 0; j <= i; ++j) {
                            double dS = P[j] * (dP[j] - Di);
                            double dZ = t * dS;
                            const double *kj = kr + ((b * M + j) * Hkv + kv) * D;
                            double *dkj = dk + ((b * M + j) * Hkv + kv) * D;
                            double *dvj = dv + ((b * M + j) * Hkv + kv) * D;
                            for (int64_t e = 0; e < D; ++e) {
                                dqi[e] += c * dZ * kj[e];
                                dkj[e] += c * dZ * qi[e];
                                dvj[e] += P[j] * doi[e];
                            }
                            colsum[(b * Hq + h) * M + j] += dZ;
                            if (g[g_per_head ? (b * Hq + h) * M + j : b * M + j] > 0.0)
                                dt += dS * Z[j];
                        }
                        dsig[b * Hq + h] += dt * ratio;
                    }
                }
            }
        }
        free(P);
        free(dP);
        free(Z);
    }

    /* Undo the rotation on the gradients of the rotated q and k. */
    if (pos) {
#pragma omp parallel for schedule(static)
        for (int64_t bm = 0; bm < B * M; ++bm) {
            for (int64_t h = 0; h < Hq; ++h)
                rope_rotate(dq + (bm * Hq + h) * D, D, (double)pos[bm], theta, -1);
            for (int64_t h = 0; h < Hkv; ++h)
                rope_rotate(dk + (bm * Hkv + h) * D, D, (double)pos[bm], theta, -1);
        }
    }

    /* dg: per key (summed over heads) for a shared gate, per (head, key) for per-head gates
     * (dL/dg_hj = gamma_h colsum_h(j) / g_hj). */
    if (g_per_head) {
        for (int64_t bh = 0; bh < B * Hq; ++bh)
            for (int64_t j = 0; j < M; ++j) {
                double gj = g[bh * M + j];
                dg[bh * M + j] = gj > 0.0 ? gamma[bh % Hq] * colsum[bh * M + j] / gj : 0.0;
            }
    } else {
        for (int64_t bm = 0; bm < B * M; ++bm) {
            int64_t b = bm / M, j = bm % M;
            double gj = g[bm];
            double acc = 0.0;
            for (int64_t h = 0; h < Hq; ++h)
                acc += gamma[h] * colsum[(b * Hq + h) * M + j];
            dg[bm] = gj > 0.0 ? acc / gj : 0.0;
        }
    }
    for (int64_t h = 0; h < Hq; ++h) {
        double acc = 0.0;
        for (int64_t b = 0; b < B; ++b)
            for (int64_t j = 0; j < M; ++j) {
                double gj = g[g_per_head ? (b * Hq + h) * M + j : b * M + j];
                if (gj > 0.0)
                    acc += colsum[(b * Hq + h) * M + j] * log(gj);
            }
        dgamma[h] = acc;
    }
    if (sigma && dsigma) {
        for (int64_t h = 0; h < Hq; ++h) {
            double acc = 0.0;
            for (int64_t b = 0; b < B; ++b)
                acc += dsig[b * Hq + h];
            dsigma[h] = acc / (1.0 + exp(-sigma[h])); /* d softplus / d sigma = sigmoid(sigma) */
        }
    }
    free(qr);
    free(kr);
    free(colsum);
    free(dsig);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* The rest of the scoring definition: LN2 before the scorer, the sequence  */
/* RMS normalisation of the scores, and the softmax-over-S gate             */
/* ------------------------------------------------------------------------ */
/*
 * [DeepDive] section 2, Eq. 1: the gate reads the post-attention residual
 * after the layer's second normalisation, a~_j = LN2(a_j), and section 3.1,
 * Eq. 3 feeds a~_j to the scorer.  Reading used here (the pages name the
 * normaliser, not its kind): RMSNorm with a per-channel weight w,
 *     a~_j[i] = a_j[i] / sqrt((1/d) sum_i a_j[i]^2 + eps) * w[i],
 * the normaliser of the Qwen3 models the pages evaluate; ln_w NULL means
 * w = 1.  Then the scorer of section a1 above on a~.
 */
void tgo_rms_norm(const double *hidden, const double *ln_w, double eps, int64_t T, int64_t d, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const double *h = hidden + t * d;
        double ss = 0.0;
        for (int64_t i = 0; i < d; ++i)
            ss += h[i] * h[i];
        double r = 1.0 / sqrt(ss / (double)d + eps);
        for (int64_t i = 0; i < d; ++i)
            out[t * d + i] = h[i] * r * (ln_w ? ln_w[i] : 1.0);
    }
}

void tgo_gate_score_ln(const double *hidden, const double *ln_w, double eps, const double *w1,
                       const double *w2, const uint8_t *forced, int64_t T, int64_t d, int64_t d_ff,
                       double *scores, double *gates)
{
    double *norm = (double *)malloc((size_t)(T * d) * sizeof(double));
    tgo_rms_norm(hidden, ln_w, eps, T, d, norm);
    tgo_gate_score(norm, w1, w2, forced, T, d, d_ff, scores, gates);
    free(norm);
}

/*
 * [DeepDive] section 3.1, Eq. 3 (second part): the raw scores of one request
 * are divided by their root mean square over the prunable positions P, and
 * the non-prunable positions N get 0:
 *     b_j = b~_j / sqrt((1/|P|) sum_{j' in P} b~_{j'}^2 + eps)   (j in P)
 *     b_j = 0                                                   (j in N)
 * A row with no prunable position is all zeros.  scores, out: [B, N];
 * forced: [B, N] (nonzero = in N) or NULL (every position prunable).
 */
void tgo_score_normalize(const double *scores, const uint8_t *forced, int64_t B, int64_t N, double eps,
                         double *out)
{
    for (int64_t b = 0; b < B; ++b) {
        const double *s = scores + b * N;
        const uint8_t *f = forced ? forced + b * N : NULL;
        double ss = 0.0;
        int64_t np = 0;
        for (int64_t j = 0; j < N; ++j)
            if (!(f && f[j])) {
                ss += s[j] * s[j];
                ++np;
            }
        double r = np > 0 ? sqrt(ss / (double)np + eps) : 1.0;
        for (int64_t j = 0; j < N; ++j)
            out[b * N + j] = (f && f[j]) ? 0.0 : s[j] / r;
    }
}

/*
 * [DeepDive] section 3.2, Eq. 5: the gate of a kept token is the softmax of
 * the normalised scores over the kept set S,
 *     g_j = exp(b_j) / sum_{j' in S} exp(b_j').
 * b: [B, M] normalised scores of the kept tokens; kept: [B, M] kept indices
 * or NULL: an entry whose index is negative (padding) is not in S and gets
 * g = 0.  Eq. 6 scales b by a per-head gain c before the softmax; since
 * softmax_S(c b)_j = softmax_S(b)_j^c / Z_c, the attention bias c ln g_j of
 * this gate equals Eq. 6's ln g_j^h up to a per-head constant, which the
 * attention softmax over keys removes.
 */
void tgo_gate_softmax(const double *bsc, const int32_t *kept, int64_t B, int64_t M, double *g)
{
    for (int64_t b = 0; b < B; ++b) {
        const double *x = bsc + b * M;
        const int32_t *k = kept ? kept + b * M : NULL;
        double mx = -INFINITY;
        for (int64_t j = 0; j < M; ++j)
            if (!(k && k[j] < 0) && x[j] > mx)
                mx = x[j];
        double z = 0.0;
        for (int64_t j = 0; j < M; ++j)
            if (!(k && k[j] < 0))
                z += exp(x[j] - mx);
        for (int64_t j = 0; j < M; ++j)
            g[b * M + j] = (k && k[j] < 0) ? 0.0 : exp(x[j] - mx) / z;
    }
}

/* Backward of tgo_gate_softmax: db_j = g_j (dg_j - sum_{k in S} g_k dg_k)
 * (padding has g = 0, so db = 0 there). */
void tgo_gate_softmax_bwd(const double *g, const double *dg, int64_t B, int64_t M, double *db)
{
    for (int64_t b = 0; b < B; ++b) {
        double dot = 0.0;
        for (int64_t j = 0; j < M; ++j)
            dot += g[b * M + j] * dg[b * M + j];
        for (int64_t j = 0; j < M; ++j)
            db[b * M + j] = g[b * M + j] * (dg[b * M + j] - dot);
    }
}

/*
 * [DeepDive] section 3.4 (the released code's invariants): per-head scores and
 * a uniform aggregation over heads for selection.  Reading used here: the
 * scorer's second layer has H outputs, one per attention head,
 *     b~_j^h = sum_k w2[h, k] SiLU(sum_i W1[k, i] a~_j[i]),
 * i.e. the a1 scorer with H rows in w2.  scores: [H, T] (head-major).
 */
void tgo_gate_score_heads(const double *hidden, const double *w1, const double *w2, int64_t T,
                          int64_t d, int64_t d_ff, int64_t H, double *scores)
{
#pragma omp parallel
    {
        double *act = (double *)malloc((size_t)(d_ff > 0 ? d_ff : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t t = 0; t < T; ++t) {
            const double *h = hidden + t * d;
            for (int64_t k = 0; k < d_ff; ++k) {
                const double *row = w1 + k * d;
                double u = 0.0;
                for (int64_t i = 0; i < d; ++i)
                    u += row[i] * h[i];
                act[k] = u / (1.0 + exp(-u));
            }
            for (int64_t hh = 0; hh < H; ++hh) {
                double s = 0.0;
                for (int64_t k = 0; k < d_ff; ++k)
                    s += w2[hh * d_ff + k] * act[k];
                scores[hh * T + t] = s;
            }
        }
        free(act);
    }
}

/* Exposed for the pin tests of the bf16 rounding helper. */
double tgo_round_bf16(double x) { return round_bf16(x); }

/*
 * [DeepDive] section 3.4 (the released code keeps a scoring branch cloned from
 * the gate layer's MLP) and the pipeline figure of section 3 ("MLP clone of
 * gate-layer MLP", whose outputs become the raw scores of Eq. 3).  The pages
 * give neither the MLP's form nor how a scalar (or one value per head) is read
 * off it.  Reading used here: the gate layer's MLP is the gated (SwiGLU) MLP of
 * the Qwen3 models the pages evaluate, cloned with its shapes, followed by a
 * head projection P with H rows (zero at initialisation, which gives the
 * "score MLP starts at zero" of section 3.1):
 *     gt_k = sum_i Wg[k, i] a~[i],   up_k = sum_i Wu[k, i] a~[i]   (k < d_i)
 *     m_k  = SiLU(gt_k) * up_k
 *     y_o  = sum_k Wd[o, k] m_k                                    (o < d)
 *     b~^h = sum_o P[h, o] y_o                                     (h < H)
 * Wg, Wu: [d_i, d]; Wd: [d, d_i]; P: [H, d] (all out x in).  hidden: [T, d]
 * (already normalised); scores: [H, T] (head-major).
 */
void tgo_gate_score_clone(const double *hidden, const double *wg, const double *wu, const double *wd,
                          const double *wh, int64_t T, int64_t d, int64_t d_i, int64_t H, double *scores)
{
#pragma omp parallel
    {
        double *m = (double *)malloc((size_t)(d_i > 0 ? d_i : 1) * sizeof(double));
        double *y = (double *)malloc((size_t)(d > 0 ? d : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t t = 0; t < T; ++t) {
            const double *h = hidden + t * d;
            for (int64_t k = 0; k < d_i; ++k) {
                double gt = 0.0, up = 0.0;
                for (int64_t i = 0; i < d; ++i) {
                    gt += wg[k * d + i] * h[i];
                    up += wu[k * d + i] * h[i];
                }
                m[k] = gt / (1.0 + exp(-gt)) * up;
            }
            for (int64_t o = 0; o < d; ++o) {
                double s = 0.0;
                for (int64_t k = 0; k < d_i; ++k)
                    s += wd[o * d_i + k] * m[k];
                y[o] = s;
            }
            for (int64_t hh = 0; hh < H; ++hh) {
                double s = 0.0;
                for (int64_t o = 0; o < d; ++o)
                    s += wh[hh * d + o] * y[o];
                scores[hh * T + t] = s;
            }
        }
        free(m);
        free(y);
    }
}
