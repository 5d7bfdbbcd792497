/* oracle.c - plain fp64 CPU oracle for batched speculative-sampling verification.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * benchmark's CPU baseline to define the right answer. It is deliberately
 * slow and literal: one sequence at a time, rows widened to fp64, softmax
 * written out, a sequential accept loop with early stop, a sequential
 * cumulative sum for the correction draw. It shares no code with the HIP path.
 *
 * Page citations are by title and section (see oracle.h for the legend):
 *  - softmax at temperature T: [Ch15] 15.1.2 step 2 and the notation list
 *    (temperature T); [CSDN] 2.1 (F.softmax of target and draft logits).
 *  - accept test and early stop: [Ch15] 15.1.2 step 3; [CSDN] 2.1 (r < alpha).
 *  - correction draw from max(0, p - q)/Z: [Ch15] 15.1.2 step 4; [CSDN] 2.1.
 *  - bonus draw from the last target row after full acceptance: [HSD] 3.3.
 *  - draft-side sampling (the step before verification): [Ch15] 15.1.2 step 1
 *    (draw from q, keep q of the drawn token); [CSDN] 2.1 stage 1.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - accept iff u < alpha with u on the 2^-53 grid in [0, 1) ([CSDN] uses
 *    "<", [Ch15] "<="; they differ on a set of probability 2^-53 per draw);
 *  - alpha = 0 when p(x) = 0; alpha = 1 when q(x) = 0 < p(x);
 *  - target row i scores draft token i; row gamma is the bonus row;
 *  - correction token = smallest j with C_j > u*Z, C the ascending cumulative
 *    sum; if rounding leaves none, the last j with r_j > 0;
 *  - Z == 0 at a rejected row (rounding only) falls back to r = p;
 *  - T == 0 is greedy: accept while the draft token is the target argmax
 *    (lowest index on ties), then emit that argmax;
 *  - a sequence is invalid (-1) when the loop reaches a position whose target
 *    or draft row holds NaN or +inf or no finite entry, or whose draft token is
 *    outside [0, V); the bonus row is checked only when it is reached.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* Philox4x32-10 (Salmon et al., SC'11): 10 rounds of the S-box                */
/*   (c0, c1, c2, c3) -> (hi(M1*c2) ^ c1 ^ k0, lo(M1*c2), hi(M0*c0) ^ c3 ^ k1,  */
/*   lo(M0*c0)), with the key bumped by the Weyl constants between rounds.    */
/* ------------------------------------------------------------------------- */
static const uint32_t PHILOX_MUL0 = 0xD2511F53u;
static const uint32_t PHILOX_MUL1 = 0xCD9E8D57u;
static const uint32_t PHILOX_WEYL0 = 0x9E3779B9u;
static const uint32_t PHILOX_WEYL1 = 0xBB67AE85u;

void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += PHILOX_WEYL0;
            k1 += PHILOX_WEYL1;
        }
        uint64_t prod0 = (uint64_t)PHILOX_MUL0 * (uint64_t)c0;
        uint64_t prod1 = (uint64_t)PHILOX_MUL1 * (uint64_t)c2;
        uint32_t n0 = (uint32_t)(prod1 >> 32) ^ c1 ^ k0;
        uint32_t n1 = (uint32_t)prod1;
        uint32_t n2 = (uint32_t)(prod0 >> 32) ^ c3 ^ k1;
        uint32_t n3 = (uint32_t)prod0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

double orc_uniform(uint64_t seed, uint32_t b, uint32_t i, uint32_t purpose) {
    uint32_t ctr[4] = {b, i, purpose, 0u};
    uint32_t key[2] = {(uint32_t)(seed & 0xFFFFFFFFu), (uint32_t)(seed >> 32)};
    uint32_t x[4];
    orc_philox4x32_10(ctr, key, x);
    uint64_t bits = (((uint64_t)x[1] << 32) | (uint64_t)x[0]) >> 11;
    return (double)bits * 0x1.0p-53;
}

void orc_uniform_batch(uint64_t seed, const uint32_t* b, const uint32_t* i,
                       const uint32_t* purpose, int64_t n, double* u) {
    for (int64_t k = 0; k < n; ++k) u[k] = orc_uniform(seed, b[k], i[k], purpose[k]);
}

/* ------------------------------------------------------------------------- */
/* Rows                                                                        */
/* ------------------------------------------------------------------------- */
static double widen(const void* row, int dtype, int64_t j) {
    if (dtype == ORC_F32) return (double)((const float*)row)[j];
    uint32_t bits = (uint32_t)((const uint16_t*)row)[j] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static const void* row_ptr(const void* base, int dtype, int64_t row, int64_t V) {
    size_t es = dtype == ORC_F32 ? 4 : 2;
    return (const char*)base + (size_t)row * (size_t)V * es;
}

/* Softmax at temperature T of one row: x_j = l_j / T, M = max_j x_j,
 * e_j = exp(x_j - M), S = sum e_j, p_j = e_j / S ([Ch15] 15.1.2 step 2). */
int orc_row_softmax(const void* row, int dtype, int64_t V, double T,
                    double* p, double* m_raw, double* S) {
    double mx = -INFINITY;
    int usable = 1;
    for (int64_t j = 0; j < V; ++j) {
        double l = widen(row, dtype, j);
        if (isnan(l) || l == INFINITY) usable = 0;
        if (l > mx) mx = l;
    }
    if (m_raw) *m_raw = mx;
    if (!usable || mx == -INFINITY) {
        if (S) *S = NAN;
        return 0;
    }
    double M = mx / T;
    double sum = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        double e = exp(widen(row, dtype, j) / T - M);
        if (p) p[j] = e;
        sum += e;
    }
    if (p)
        for (int64_t j = 0; j < V; ++j) p[j] /= sum;
    if (S) *S = sum;
    return 1;
}

/* Inverse-CDF draw: smallest j with C_j > u * Z over the ascending cumulative
 * sum C of r; C is written to cdf (unnormalised). */
static int64_t draw_from(const double* r, int64_t V, double u, double* cdf, double* Z_out) {
    double c = 0.0;
    for (int64_t j = 0; j < V; ++j) {
        c += r[j];
        cdf[j] = c;
    }
    double Z = c;
    *Z_out = Z;
    double t = u * Z;
    for (int64_t j = 0; j < V; ++j)
        if (cdf[j] > t) return j;
    for (int64_t j = V - 1; j >= 0; --j) /* rounding guard */
        if (r[j] > 0.0) return j;
    return 0;
}

double orc_residual_cdf(const void* p_row, const void* q_row, int dtype, int64_t V,
                        double T, double* cdf) {
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* q = q_row ? (double*)malloc(sizeof(double) * (size_t)V) : NULL;
    double* r = (double*)malloc(sizeof(double) * (size_t)V);
    double Z = NAN;
    int ok = orc_row_softmax(p_row, dtype, V, T, p, NULL, NULL);
    if (ok && q_row) ok = orc_row_softmax(q_row, dtype, V, T, q, NULL, NULL);
    if (ok) {
        for (int64_t j = 0; j < V; ++j) r[j] = q_row ? fmax(0.0, p[j] - q[j]) : p[j];
        double Zr;
        draw_from(r, V, 0.0, cdf, &Zr);
        Z = Zr;
        if (Zr == 0.0) { /* fallback r = p */
            draw_from(p, V, 0.0, cdf, &Zr);
        }
        for (int64_t j = 0; j < V; ++j) cdf[j] /= Zr;
    }
    free(p); free(q); free(r);
    return Z;
}

/* ------------------------------------------------------------------------- */
/* Greedy verification, T == 0                                                 */
/* ------------------------------------------------------------------------- */
static int argmax_row(const void* row, int dtype, int64_t V, int64_t* arg) {
    double best = -INFINITY;
    int64_t at = 0;
    int usable = 1;
    for (int64_t j = 0; j < V; ++j) {
        double l = widen(row, dtype, j);
        if (isnan(l) || l == INFINITY) usable = 0;
        if (l > best) { best = l; at = j; }
    }
    *arg = at;
    return usable && best > -INFINITY;
}

static void verify_greedy_one(const void* target, const int32_t* tokens, int32_t b,
                              int32_t gamma, int64_t V, int dtype,
                              int32_t* out_tokens, int32_t* out_n) {
    int32_t* out = out_tokens + (size_t)b * (gamma + 1);
    for (int i = 0; i <= gamma; ++i) out[i] = -1;
    int32_t k = gamma;
    for (int32_t i = 0; i <= gamma; ++i) {
        int64_t a;
        int usable = argmax_row(row_ptr(target, dtype, (int64_t)b * (gamma + 1) + i, V), dtype, V, &a);
        if (i == gamma) {
            if (!usable) goto invalid;
            out[gamma] = (int32_t)a;
            break;
        }
        int32_t x = tokens[(size_t)b * gamma + i];
        if (!usable || x < 0 || (int64_t)x >= V) goto invalid;
        if ((int64_t)x == a) {
            out[i] = x;
        } else {
            k = i;
            out[i] = (int32_t)a;
            break;
        }
    }
    out_n[b] = k;
    return;
invalid:
    for (int i = 0; i <= gamma; ++i) out[i] = -1;
    out_n[b] = -1;
}

/* ------------------------------------------------------------------------- */
/* Sampling verification, T > 0                                                */
/* ------------------------------------------------------------------------- */
static void verify_sample_one(const void* target, const void* draft, const int32_t* tokens,
                              int32_t b, int32_t gamma, int64_t V, int dtype, double T,
                              const double* u_accept, const double* u_sample,
                              int32_t* out_tokens, int32_t* out_n, const orc_diag_t* dg) {
    const int32_t R = 2 * gamma + 1;
    int32_t* out = out_tokens + (size_t)b * (gamma + 1);
    for (int i = 0; i <= gamma; ++i) out[i] = -1;

    /* Step 2: the distribution of every target row (0..gamma) and every
     * draft row (0..gamma-1), all computed before the accept loop. */
    double* probs = (double*)malloc(sizeof(double) * (size_t)R * (size_t)V);
    int* usable = (int*)malloc(sizeof(int) * (size_t)R);
    for (int32_t r = 0; r < R; ++r) {
        const void* row = r <= gamma
            ? row_ptr(target, dtype, (int64_t)b * (gamma + 1) + r, V)
            : row_ptr(draft, dtype, (int64_t)b * gamma + (r - gamma - 1), V);
        double m, S;
        usable[r] = orc_row_softmax(row, dtype, V, T, probs + (size_t)r * V, &m, &S);
        if (dg && dg->row_max) dg->row_max[(size_t)b * R + r] = m;
        if (dg && dg->row_sumexp) dg->row_sumexp[(size_t)b * R + r] = S;
    }
    const double* P = probs;                         /* target row i: P + i*V */
    const double* Q = probs + (size_t)(gamma + 1) * V; /* draft row i: Q + i*V */
    for (int32_t i = 0; i < gamma; ++i) {
        if (dg && dg->p_tok) dg->p_tok[(size_t)b * gamma + i] = NAN;
        if (dg && dg->q_tok) dg->q_tok[(size_t)b * gamma + i] = NAN;
        if (dg && dg->alpha) dg->alpha[(size_t)b * gamma + i] = NAN;
    }
    if (dg && dg->Z) dg->Z[b] = NAN;
    if (dg && dg->cdf_lo) dg->cdf_lo[b] = NAN;
    if (dg && dg->cdf_hi) dg->cdf_hi[b] = NAN;
    if (dg && dg->degenerate) dg->degenerate[b] = 0;

    /* Step 3: accept draft token i with probability min(1, p_i/q_i); stop at
     * the first rejection. */
    int32_t k = gamma;
    for (int32_t i = 0; i < gamma; ++i) {
        int32_t x = tokens[(size_t)b * gamma + i];
        if (!usable[i] || !usable[gamma + 1 + i] || x < 0 || (int64_t)x >= V) goto invalid;
        double p = P[(size_t)i * V + x];
        double q = Q[(size_t)i * V + x];
        double alpha;
        if (p == 0.0) alpha = 0.0;
        else if (q == 0.0) alpha = 1.0;
        else alpha = fmin(1.0, p / q);
        if (dg && dg->p_tok) dg->p_tok[(size_t)b * gamma + i] = p;
        if (dg && dg->q_tok) dg->q_tok[(size_t)b * gamma + i] = q;
        if (dg && dg->alpha) dg->alpha[(size_t)b * gamma + i] = alpha;
        double u = u_accept[(size_t)b * gamma + i];
        if (u < alpha) {
            out[i] = x;
        } else {
            k = i;
            break;
        }
    }
    if (k == gamma && !usable[gamma]) goto invalid;

    {
        /* Step 4: correction draw from max(0, p_k - q_k)/Z at the rejected row,
         * or the bonus draw from p_gamma when every draft token was accepted. */
        double* r = (double*)malloc(sizeof(double) * (size_t)V);
        double* cdf = (double*)malloc(sizeof(double) * (size_t)V);
        const double* pk = P + (size_t)k * V;
        if (k < gamma) {
            const double* qk = Q + (size_t)k * V;
            for (int64_t j = 0; j < V; ++j) r[j] = fmax(0.0, pk[j] - qk[j]);
        } else {
            for (int64_t j = 0; j < V; ++j) r[j] = pk[j];
        }
        double u = u_sample[(size_t)b * (gamma + 1) + k];
        double Z;
        int64_t j = draw_from(r, V, u, cdf, &Z);
        if (dg && dg->Z) dg->Z[b] = Z;
        if (Z == 0.0) { /* only reachable through rounding: sample from p_k */
            if (dg && dg->degenerate) dg->degenerate[b] = 1;
            j = draw_from(pk, V, u, cdf, &Z);
        }
        if (dg && dg->cdf_lo) dg->cdf_lo[b] = (j > 0 ? cdf[j - 1] : 0.0) / Z;
        if (dg && dg->cdf_hi) dg->cdf_hi[b] = cdf[j] / Z;
        out[k] = (int32_t)j;
        out_n[b] = k;
        free(r);
        free(cdf);
    }
    free(probs);
    free(usable);
    return;
invalid:
    for (int i = 0; i <= gamma; ++i) out[i] = -1;
    out_n[b] = -1;
    free(probs);
    free(usable);
}

int orc_verify_u(const void* target, const void* draft, const int32_t* tokens,
                 int32_t B, int32_t gamma, int64_t V, int dtype, double T,
                 const double* u_accept, const double* u_sample,
                 int32_t* out_tokens, int32_t* out_n, const orc_diag_t* diag) {
    if (!target || !tokens || !out_tokens || !out_n) return -1;
    if (B < 0 || gamma < 1 || V < 1 || (dtype != ORC_F32 && dtype != ORC_BF16)) return -1;
    if (!(T >= 0.0)) return -1;
    if (T > 0.0 && (!draft || !u_accept || !u_sample)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t b = 0; b < B; ++b) {
        if (T == 0.0)
            verify_greedy_one(target, tokens, b, gamma, V, dtype, out_tokens, out_n);
        else
            verify_sample_one(target, draft, tokens, b, gamma, V, dtype, T, u_accept,
                              u_sample, out_tokens, out_n, diag);
    }
    return 0;
}

int orc_verify(const void* target, const void* draft, const int32_t* tokens,
               int32_t B, int32_t gamma, int64_t V, int dtype, double T, uint64_t seed,
               int64_t b_offset, int32_t* out_tokens, int32_t* out_n, const orc_diag_t* diag) {
    if (B < 0 || gamma < 1) return -1;
    double* ua = (double*)malloc(sizeof(double) * ((size_t)B * gamma + 1));
    double* us = (double*)malloc(sizeof(double) * ((size_t)B * (gamma + 1) + 1));
    for (int64_t b = 0; b < B; ++b) {
        uint32_t gb = (uint32_t)(b + b_offset);
        for (int32_t i = 0; i < gamma; ++i)
            ua[b * gamma + i] = orc_uniform(seed, gb, (uint32_t)i, ORC_PURPOSE_ACCEPT);
        for (int32_t k = 0; k <= gamma; ++k)
            us[b * (gamma + 1) + k] = orc_uniform(seed, gb, (uint32_t)k, ORC_PURPOSE_SAMPLE);
    }
    int rc = orc_verify_u(target, draft, tokens, B, gamma, V, dtype, T, ua, us,
                          out_tokens, out_n, diag);
    free(ua);
    free(us);
    return rc;
}

/* ------------------------------------------------------------------------- */
/* Draft-side sampling ([Ch15] 15.1.2 step 1; [CSDN] 2.1 stage 1)              */
/* ------------------------------------------------------------------------- */
static void draft_one(const void* row, int64_t V, int dtype, double T, double u,
                      int32_t* tok, double* q, double* lo, double* hi) {
    *tok = -1;
    *q = NAN;
    *lo = NAN;
    *hi = NAN;
    if (T == 0.0) {
        int64_t a;
        if (argmax_row(row, dtype, V, &a)) {
            *tok = (int32_t)a;
            *q = 1.0;
        }
        return;
    }
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* cdf = (double*)malloc(sizeof(double) * (size_t)V);
    if (orc_row_softmax(row, dtype, V, T, p, NULL, NULL)) {
        double Z;
        int64_t j = draw_from(p, V, u, cdf, &Z);
        *tok = (int32_t)j;
        *q = p[j];
        *lo = (j > 0 ? cdf[j - 1] : 0.0) / Z;
        *hi = cdf[j] / Z;
    }
    free(p);
    free(cdf);
}

int orc_draft_sample(const void* logits, int32_t B, int32_t n, int64_t V, int dtype, double T,
                     uint64_t seed, int64_t pos0, int64_t b_offset, int32_t* out_tokens,
                     double* out_q, double* cdf_lo, double* cdf_hi) {
    if (!logits || !out_tokens) return -1;
    if (B < 0 || n < 1 || V < 1 || pos0 < 0 || (dtype != ORC_F32 && dtype != ORC_BF16)) return -1;
    if (!(T >= 0.0)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < (int64_t)B * n; ++r) {
        const int64_t b = r / n, t = r % n;
        const double u = T > 0.0 ? orc_uniform(seed, (uint32_t)(b + b_offset), (uint32_t)(pos0 + t),
                                                ORC_PURPOSE_DRAFT)
                                 : 0.0;
        double q, lo, hi;
        draft_one(row_ptr(logits, dtype, r, V), V, dtype, T, u, out_tokens + r, &q, &lo, &hi);
        if (out_q) out_q[r] = q;
        if (cdf_lo) cdf_lo[r] = lo;
        if (cdf_hi) cdf_hi[r] = hi;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Diagnostics: entropy of a row, expected acceptance per position             */
/* ------------------------------------------------------------------------- */
double orc_row_entropy(const void* row, int dtype, int64_t V, double T) {
    if (T == 0.0) {
        int64_t a;
        return argmax_row(row, dtype, V, &a) ? 0.0 : NAN;
    }
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double H = NAN;
    if (orc_row_softmax(row, dtype, V, T, p, NULL, NULL)) {
        H = 0.0;
        for (int64_t j = 0; j < V; ++j)
            if (p[j] > 0.0) H -= p[j] * log(p[j]);
    }
    free(p);
    return H;
}

int orc_expected_accept(const void* target, const void* draft, int32_t B, int32_t gamma,
                        int64_t V, int dtype, double T, double* beta) {
    if (!target || !draft || !beta) return -1;
    if (B < 0 || gamma < 1 || V < 1 || (dtype != ORC_F32 && dtype != ORC_BF16)) return -1;
    if (!(T > 0.0)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < (int64_t)B * gamma; ++r) {
        const int64_t b = r / gamma, i = r % gamma;
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        double* q = (double*)malloc(sizeof(double) * (size_t)V);
        double s = NAN;
        if (orc_row_softmax(row_ptr(target, dtype, b * (gamma + 1) + i, V), dtype, V, T, p, NULL, NULL) &&
            orc_row_softmax(row_ptr(draft, dtype, b * gamma + i, V), dtype, V, T, q, NULL, NULL)) {
            s = 0.0;
            for (int64_t j = 0; j < V; ++j) s += fmin(p[j], q[j]);
        }
        beta[r] = s;
        free(p);
        free(q);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Token-tree verification ([CSDN] 3.2; [Ch15] 15.2.4), the page's heuristic  */
/* ------------------------------------------------------------------------- */
static void tree_one(const void* target, const void* draft, const int32_t* parent, const int32_t* token,
                     int64_t b, int32_t N, int64_t V, int dtype, double T, double threshold,
                     int32_t* out_tokens, int32_t* out_nodes, int32_t* out_n) {
    const int32_t* par = parent + b * N;
    const int32_t* tok = token + b * N;
    int32_t* ot = out_tokens + b * (N - 1);
    int32_t* on = out_nodes ? out_nodes + b * (N - 1) : NULL;
    for (int32_t j = 0; j < N - 1; ++j) {
        ot[j] = -1;
        if (on) on[j] = -1;
    }
    for (int32_t j = 1; j < N; ++j)
        if (par[j] < 0 || par[j] >= j) goto invalid;
    double* p = (double*)malloc(sizeof(double) * (size_t)V);
    double* q = (double*)malloc(sizeof(double) * (size_t)V);
    int32_t v = 0, n = 0;
    for (;;) {
        int32_t best = -1;
        double best_score = -1.0;
        int has_child = 0;
        for (int32_t c = v + 1; c < N; ++c)
            if (par[c] == v) has_child = 1;
        if (!has_child) break;
        const void* trow = row_ptr(target, dtype, b * N + v, V);
        if (T == 0.0) {
            int64_t a;
            if (!argmax_row(trow, dtype, V, &a)) goto invalid_free;
            for (int32_t c = v + 1; c < N; ++c) {
                if (par[c] != v) continue;
                if (tok[c] < 0 || (int64_t)tok[c] >= V) goto invalid_free;
                if (best < 0 && (int64_t)tok[c] == a) best = c;
            }
            if (best < 0) break;
        } else {
            if (!orc_row_softmax(trow, dtype, V, T, p, NULL, NULL) ||
                !orc_row_softmax(row_ptr(draft, dtype, b * N + v, V), dtype, V, T, q, NULL, NULL))
                goto invalid_free;
            for (int32_t c = v + 1; c < N; ++c) {
                if (par[c] != v) continue;
                if (tok[c] < 0 || (int64_t)tok[c] >= V) goto invalid_free;
                const double pp = p[tok[c]], qq = q[tok[c]];
                double score;
                if (pp == 0.0) score = 0.0;
                else if (qq == 0.0) score = 1.0;
                else score = fmin(1.0, pp / qq);
                if (score > best_score) {
                    best_score = score;
                    best = c;
                }
            }
            if (best_score < threshold) break;
        }
        ot[n] = tok[best];
        if (on) on[n] = best;
        ++n;
        v = best;
    }
    out_n[b] = n;
    free(p);
    free(q);
    return;
invalid_free:
    free(p);
    free(q);
invalid:
    for (int32_t j = 0; j < N - 1; ++j) {
        ot[j] = -1;
        if (on) on[j] = -1;
    }
    out_n[b] = -1;
}

int orc_tree_verify(const void* target, const void* draft, const int32_t* parent,
                    const int32_t* token, int32_t B, int32_t N, int64_t V, int dtype,
                    double T, double threshold, int32_t* out_tokens, int32_t* out_nodes,
                    int32_t* out_n) {
    if (!target || !parent || !token || !out_tokens || !out_n) return -1;
    if (B < 0 || N < 2 || V < 1 || (dtype != ORC_F32 && dtype != ORC_BF16)) return -1;
    if (!(T >= 0.0) || (T > 0.0 && !draft)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t b = 0; b < B; ++b)
        tree_one(target, draft, parent, token, b, N, V, dtype, T, threshold, out_tokens, out_nodes, out_n);
    return 0;
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
