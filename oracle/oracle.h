/* oracle.h - fp64 CPU oracle for batched speculative-sampling verification.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline use this library. It shares no code with the HIP path (no headers,
 * helpers or tables) and exists to say what the right answer is.
 *
 * Pages (cited by title and section):
 *  [Ch15] "Chapter 15: Decoding acceleration techniques" (zsc.github.io, LLM edge
 *         inference), section 15.1.2 "The mathematical framework of speculative
 *         decoding": step 2 (parallel verification, softmax of the target
 *         logits), step 3 (accept with probability min(1, p/q), stop at the first
 *         rejection), step 4 (resample from max(0, p - q) / Z), Lemma 1 and the
 *         main theorem (output distribution equals p).
 *  [CSDN] devpress.csdn.net speculative-inference post, section 2.1 "The
 *         mathematical essence: parallelising rejection sampling": the
 *         speculative_decode() listing (same steps, strict u < alpha test).
 *  [HSD]  "LLM inference optimisation: hidden-state speculative decoding"
 *         (jsqmd.com), section 3.3: the bonus token after full acceptance.
 *  Philox4x32-10: Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 *         as 1, 2, 3", SC'11.
 */
#ifndef SPECVERIFY_ORACLE_H
#define SPECVERIFY_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_PURPOSE_ACCEPT = 0, ORC_PURPOSE_SAMPLE = 1, ORC_PURPOSE_DRAFT = 2 };

/* Philox4x32-10 block function: out = Philox(counter, key). */
void orc_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* Uniform in [0, 1) on the 2^-53 grid from counter (b, i, purpose, 0) and
 * key (seed low word, seed high word): ((x1 << 32 | x0) >> 11) * 2^-53. */
double orc_uniform(uint64_t seed, uint32_t b, uint32_t i, uint32_t purpose);

/* Fill u[n] with orc_uniform(seed, b[n], i[n], purpose[n]). */
void orc_uniform_batch(uint64_t seed, const uint32_t* b, const uint32_t* i,
                       const uint32_t* purpose, int64_t n, double* u);

/* Softmax statistics of one row of logits at temperature T > 0.
 * m_raw = max_j l_j;  S = sum_j exp(l_j/T - m_raw/T);  p_j = exp(l_j/T - m_raw/T) / S.
 * p may be NULL. Returns 1 if the row is usable (no NaN, no +inf, at least one
 * entry > -inf), else 0 (then S is NaN and p is untouched). */
int orc_row_softmax(const void* row, int dtype, int64_t V, double T,
                    double* p, double* m_raw, double* S);

/* Normalised residual CDF used by the correction step:
 * r_j = max(0, p_j - q_j) (q row given) or r_j = p_j (q_row == NULL, bonus row);
 * if sum r == 0 the row falls back to r = p. cdf[j] = (r_0 + ... + r_j) / Z.
 * Returns Z (before the fallback), or NaN if a row is unusable. */
double orc_residual_cdf(const void* p_row, const void* q_row, int dtype, int64_t V,
                        double T, double* cdf);

/* Optional per-call diagnostics; every pointer may be NULL. */
typedef struct {
    double* row_max;     /* [B, 2*gamma+1]: target rows 0..gamma, then draft rows 0..gamma-1 */
    double* row_sumexp;  /* [B, 2*gamma+1]: S of each row (NaN when unusable) */
    double* p_tok;       /* [B, gamma]: p_i(x_i) for positions reached, else NaN */
    double* q_tok;       /* [B, gamma]: q_i(x_i) likewise */
    double* alpha;       /* [B, gamma]: acceptance probability for positions reached, else NaN */
    double* Z;           /* [B]: residual mass at row k (k < gamma), sum of p at the bonus row */
    double* cdf_lo;      /* [B]: normalised CDF just below the emitted correction/bonus token */
    double* cdf_hi;      /* [B]: normalised CDF at the emitted token */
    int32_t* degenerate; /* [B]: 1 if Z == 0 forced the fallback r = p */
} orc_diag_t;

/* The verification step with explicit uniforms.
 *  target  [B, gamma+1, V] (dtype), draft [B, gamma, V] (dtype; unused if T == 0),
 *  tokens  [B, gamma] int32,
 *  u_accept [B, gamma]   : uniform for the accept test at position i,
 *  u_sample [B, gamma+1] : uniform for the correction draw at row k (k < gamma)
 *                          or for the bonus draw (k == gamma).
 *  Outputs: out_tokens [B, gamma+1] (-1 after the emitted token), out_n [B]
 *  (0..gamma, or -1 when the sequence reaches an unusable input).
 *  T == 0 selects greedy verification (u arrays unused, may be NULL).
 *  Returns 0, or -1 on bad arguments. */
int orc_verify_u(const void* target, const void* draft, const int32_t* tokens,
                 int32_t B, int32_t gamma, int64_t V, int dtype, double T,
                 const double* u_accept, const double* u_sample,
                 int32_t* out_tokens, int32_t* out_n, const orc_diag_t* diag);

/* Same, with the uniforms drawn from Philox4x32-10 keyed by seed:
 * accept uniform (b, i, ACCEPT), correction/bonus uniform (b, k, SAMPLE).
 * b_offset is added to b in the counter (a shard of a larger batch). */
int orc_verify(const void* target, const void* draft, const int32_t* tokens,
               int32_t B, int32_t gamma, int64_t V, int dtype, double T, uint64_t seed,
               int64_t b_offset, int32_t* out_tokens, int32_t* out_n, const orc_diag_t* diag);

/* Draft-side sampling, the step before verification ([Ch15] 15.1.2 step 1:
 * draw each draft token from the draft distribution and keep its probability;
 * [CSDN] 2.1, stage 1 of speculative_decode()). Row (b, t) of logits
 * [B, n, V] (positions pos0 .. pos0 + n - 1 of sequence b):
 *   T > 0:  x = smallest j with C_j > u * Z, C the ascending cumulative sum of
 *           p = softmax(l / T) and Z its total, with
 *           u = orc_uniform(seed, b + b_offset, pos0 + t, DRAFT); q = p_x;
 *   T == 0: x = argmax_j l_j (lowest index on ties), q = 1;
 *   a row with NaN, +inf or no finite entry: x = -1, q = NaN.
 * out_q, cdf_lo, cdf_hi may be NULL; cdf_lo/cdf_hi receive the normalised
 * cumulative mass just below x and at x (NaN at T == 0 or for unusable rows).
 * Returns 0, or -1 on bad arguments. */
int orc_draft_sample(const void* logits, int32_t B, int32_t n, int64_t V, int dtype, double T,
                     uint64_t seed, int64_t pos0, int64_t b_offset, int32_t* out_tokens,
                     double* out_q, double* cdf_lo, double* cdf_hi);

/* Per-row diagnostics for choosing the draft length ([Ch15] 15.1.4, dynamic
 * strategy adjustment: the acceptance-rate window rule; 15.2.4, adaptive
 * draft length from the prediction entropy; Lemma 1 for the expected
 * acceptance).
 * orc_row_entropy: H = -sum_j p_j ln p_j of p = softmax(l / T) (natural log;
 *   0 terms for p_j = 0); NaN for an unusable row. At T == 0 the distribution
 *   is the point mass on the first argmax: H = 0 (NaN if unusable).
 * orc_expected_accept: beta[b, i] = sum_x min(p_i(x), q_i(x)) for every
 *   position i < gamma (target row i against draft row i; T > 0), the
 *   probability that position i accepts its draft token given that it is
 *   reached; NaN when either row is unusable. Returns 0, or -1 on bad
 *   arguments. */
double orc_row_entropy(const void* row, int dtype, int64_t V, double T);
int orc_expected_accept(const void* target, const void* draft, int32_t B, int32_t gamma,
                        int64_t V, int dtype, double T, double* beta);

/* Token-tree verification, a labelled heuristic mode ([CSDN] 3.2
 * TokenTreeVerifier.parallel_verify; [Ch15] 15.2.4 candidate trees). It does
 * NOT preserve the target distribution: it follows the page's rule.
 * Sequence b has a tree of N nodes: node 0 is the root (the context), node
 * j >= 1 holds token[b, j] and its parent parent[b, j] (0 <= parent < j).
 * target [B, N, V] row j scores the children of node j (the target model's
 * logits after the path to j); draft [B, N, V] row j likewise for the draft
 * model (unused at T == 0).
 * Walk from the root: among the children c of the current node v (ascending
 * index), T > 0: score(c) = min(1, p_v(token c) / q_v(token c)) with
 *   p_v = softmax(target row v / T), q_v = softmax(draft row v / T) (the
 *   acceptance rule, R5 for zeros); the best child is the first with the
 *   largest score; stop if there is no child or score(best) < threshold;
 * T == 0: the first child whose token is the argmax of target row v (lowest
 *   index on ties); stop if none.
 * Otherwise append the best child's token and node and continue from it.
 * Outputs: out_tokens [B, N-1] and out_nodes [B, N-1] (-1 after the path),
 * out_n [B] = path length, or -1 when the walk reaches a node whose row (at
 * T > 0 both rows) is unusable, a child token outside [0, V), or a parent
 * index outside [0, j). out_nodes may be NULL. Returns 0, or -1 on bad
 * arguments. */
int orc_tree_verify(const void* target, const void* draft, const int32_t* parent,
                    const int32_t* token, int32_t B, int32_t N, int64_t V, int dtype,
                    double T, double threshold, int32_t* out_tokens, int32_t* out_nodes,
                    int32_t* out_n);

/* Threads the OpenMP runtime will use (1 when built without OpenMP). */
int orc_max_threads(void);
void orc_set_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
