/* specverify.h - C ABI of libspecverify: batched speculative-sampling
 * verification on one AMD Instinct MI355X (gfx950).
 *
 * What the library computes (pages cited by title and section):
 *  [Ch15] "Chapter 15: Decoding acceleration techniques" (zsc.github.io, LLM
 *         edge inference), 15.1.2 "The mathematical framework of speculative
 *         decoding": step 2 (one target pass scores every drafted position;
 *         p_i = softmax(logits of row i)), step 3 (accept draft token i with
 *         probability min(1, p_i/q_i); stop at the first rejection), step 4
 *         (at the rejected row resample from max(0, p - q)/Z), and the main
 *         theorem (the emitted tokens are distributed as p).
 *  [CSDN] devpress.csdn.net speculative-inference post, 2.1: the same loop as
 *         a PyTorch listing, returning the emitted tokens and the accepted count.
 *  [HSD]  "LLM inference optimisation: hidden-state speculative decoding"
 *         (jsqmd.com), 3.3: after full acceptance the target's last row yields
 *         one more (bonus) token.
 * Around that step: the draft-side draw with its probabilities
 * (spec_draft_sample; [Ch15] 15.1.2 step 1), the diagnostics for choosing
 * the draft length (the row entropy beside that draw, the per-position
 * expected acceptance spec_expected_accept; [Ch15] 15.1.4 dynamic strategy
 * adjustment, 15.2.4), and token-tree verification as a labelled heuristic
 * mode (spec_tree_verify; [CSDN] 3.2, [Ch15] 15.2.4).
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    never frees or retains them. Rows are contiguous and row-major.
 *  - dtype: SPEC_F32 (float) or SPEC_BF16 (bfloat16 bits, uint16). Both logits
 *    tensors share it.
 *  - stream: a hipStream_t passed as void* (NULL = the legacy default
 *    stream). Every kernel is enqueued on it and the call returns without
 *    waiting; buffers must stay alive until the stream reaches the work.
 *  - Randomness: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with key =
 *    (seed low 32 bits, seed high 32 bits) and counter (b, i, purpose, 0);
 *    purpose 0 = accept test at position i, purpose 1 = correction draw at the
 *    rejected row k or the bonus draw (i = k = gamma), purpose 2 = the draft
 *    draw of spec_draft_sample at position i. The uniform is
 *    ((x1 << 32 | x0) >> 11) * 2^-53 in [0, 1). Results are a pure function of
 *    (inputs, seed): no state is carried between calls.
 *  - Host-detectable errors return a negative status before anything is
 *    launched; spec_verify_last_error() gives the message (thread-local).
 *    Input errors only visible on the device are reported in band: a sequence
 *    whose verification reaches a position with an unusable row (NaN, +inf, or
 *    no finite entry; at T > 0 both rows of the position, at T == 0 the target
 *    row) or an out-of-range draft token gets out_n_accepted[b] = -1 and an
 *    all -1 out_tokens row. -inf logits are legal (masked tokens).
 *  - Failure detection ([Ch15] 15.1.4, failure-mode detection and recovery:
 *    the host must be able to see that the fast path misbehaved and fall
 *    back). Inside a kernel, blocks wait for other blocks of the same launch
 *    (always blocks of lower index, which in-order dispatch has started, so
 *    in correct operation every wait ends). Every such wait is bounded (about
 *    2 s by default, see spec_verify_set_wait_limit). A wait that runs out
 *    sets a sticky word in the (device, stream) workspace, reports the
 *    sequence, row, pair or tree it was computing as invalid (-1, or NaN for
 *    the diagnostics) where it owns that output, and then drains: it goes on
 *    waiting, up to the default bound, for what it waited for, so that the
 *    workspace's counters are left at zero and the next call on the stream is
 *    unaffected. spec_verify_status reads and clears the sticky word.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SPEC_OK = 0,
    SPEC_EINVAL = -1,  /* bad pointer, size, temperature or dtype combination */
    SPEC_EDTYPE = -2,  /* dtype is neither SPEC_F32 nor SPEC_BF16 */
    SPEC_EHIP = -3,    /* a HIP runtime call or kernel launch failed */
    SPEC_ENOMEM = -4   /* the library's device workspace could not be allocated */
} spec_status_t;

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype_t;

#define SPEC_MAX_GAMMA 63

/* spec_verify: one batched verification step ([Ch15] 15.1.2 steps 2-4,
 * [CSDN] 2.1, bonus token [HSD] 3.3).
 *
 *  target_logits  [B, gamma+1, V] dtype. Row i < gamma scores draft token i;
 *                 row gamma is the bonus row.
 *  draft_logits   [B, gamma, V] dtype: row i is the distribution draft token i
 *                 was drawn from. May be NULL iff temperature == 0.
 *  draft_tokens   [B, gamma] int32.
 *  B >= 1, 1 <= gamma <= SPEC_MAX_GAMMA, V >= 1.
 *  temperature    > 0: p = softmax(target/T), q = softmax(draft/T), accept
 *                 token i iff u_i < min(1, p_i(x_i)/q_i(x_i)) (alpha = 0 when
 *                 p_i(x_i) = 0, 1 when q_i(x_i) = 0 < p_i(x_i)); at the first
 *                 rejected row k draw from max(0, p_k - q_k)/Z (from p_k if Z
 *                 rounds to 0); if none is rejected draw the bonus token from
 *                 p_gamma. A draw takes the smallest j whose ascending
 *                 cumulative mass exceeds u*Z.
 *                 == 0: greedy; accept while draft token i equals the argmax of
 *                 target row i (lowest index on ties), then emit that argmax
 *                 (the bonus row's argmax when all are accepted).
 *                 < 0 or NaN: SPEC_EINVAL.
 *  seed           Philox key.
 *  out_tokens     [B, gamma+1] int32: the n accepted draft tokens, then the
 *                 correction (or bonus) token, then -1 padding.
 *  out_n_accepted [B] int32: n in 0..gamma, or -1 (invalid input, see above).
 *  Returns SPEC_OK or a negative spec_status_t (SPEC_EINVAL also when the
 *  problem exceeds the kernel's dispatch size). The
 *  library keeps a device workspace per (device, stream), grown on demand
 *  under a lock; concurrent calls on different streams are safe, calls on one
 *  stream are ordered. One kernel is launched per call. Inside it, blocks
 *  wait (bounded) for other blocks of the same sequence; should that bound
 *  ever run out, the failure is reported as described above (failure
 *  detection) rather than the kernel waiting on. */
int spec_verify(const void* target_logits, const void* draft_logits,
                const int32_t* draft_tokens, int32_t B, int32_t gamma, int32_t V,
                int32_t dtype, float temperature, uint64_t seed,
                int32_t* out_tokens, int32_t* out_n_accepted, void* stream);

/* Optional extras of spec_verify_ex. Every pointer may be NULL; device
 * pointers unless stated. */
typedef struct {
    float* row_max;        /* [B, 2*gamma+1]: max logit of target rows 0..gamma, then
                              draft rows 0..gamma-1 (T > 0: every row; T == 0: target
                              rows only, draft slots untouched) */
    double* row_sumexp;    /* [B, 2*gamma+1]: sum_j exp((l_j - max)/T) (T > 0 only) */
    double* p_draft;       /* [B, gamma]: p_i(x_i) (T > 0; NaN if the position is unusable) */
    double* q_draft;       /* [B, gamma]: q_i(x_i) */
    double* Z;             /* [B]: residual mass at row k, or sum of p at the bonus row
                              (T > 0 only; NaN for an invalid sequence) */
    int32_t* argmax;       /* [B, gamma+1]: argmax of each target row (T == 0 only) */
    int64_t b_offset;      /* added to b in the Philox counter, so that a shard of a
                              larger batch draws the same uniforms as the whole batch */
    void* events[3];       /* optional hipEvent_t (host handles): [0] and [1] are bound to
                              the start and end of the call's verification kernel
                              dispatch itself (no extra stream packets); [2] is
                              reserved and ignored */
    int32_t schedule;      /* a spec_schedule_t (0 = SPEC_SCHEDULE_AUTO), see below */
} spec_extras_t;

/* Grid schedules. Outputs do not depend on the schedule. At T == 0 GROUP and
 * GROUP_TWO_PHASE select the group-major order and every other value the
 * position-major order with the early stop.
 *  SPEC_SCHEDULE_GROUP       group-major: a sequence's 2*gamma+1 rows (T == 0:
 *                            its gamma+1 target rows) are streamed together;
 *                            the sequence's closing blocks (at the end of the
 *                            grid) take the accept step and the draw (T == 0:
 *                            one block, the greedy step). At T > 0 the bonus
 *                            row (target row gamma) is not streamed: only the
 *                            closing blocks of a sequence that accepts all
 *                            gamma draft tokens read it, for the bonus draw.
 *  SPEC_SCHEDULE_EARLY_STOP  position-major: all sequences' position 0, then
 *                            position 1, ...; each position is decided as soon
 *                            as its rows are streamed, and a block whose
 *                            sequence already stopped at an earlier position
 *                            reads nothing (the early stop of [Ch15] 15.1.2
 *                            step 3) and helps with that sequence's draw.
 *  SPEC_SCHEDULE_POSITION    the same order, reading every row.
 *  SPEC_SCHEDULE_GROUP_TWO_PHASE
 *                            group-major in two phases (T > 0, gamma >= 2):
 *                            every sequence's first p0 row pairs (p0 =
 *                            max(1, min((3 gamma + 4) / 8, gamma - 1)), in
 *                            integer division), then a
 *                            decider per sequence takes the accept step for
 *                            them; then the other row pairs, read only for
 *                            the sequences that accepted all of the first
 *                            (the early stop of [Ch15] 15.1.2 step 3 applied
 *                            per sequence); then the closing blocks. The
 *                            closing blocks of a sequence that stopped early
 *                            take k and row k's constants from its decider.
 *  SPEC_SCHEDULE_AUTO        EARLY_STOP once one position's row pairs come
 *                            to at least 152 MiB (2 B V times the element
 *                            size), else
 *                            GROUP_TWO_PHASE where the rows come to at least
 *                            112 MiB (2 gamma B V times the element size;
 *                            gamma >= 2), else GROUP.
 * Any of row_max, row_sumexp, p_draft, q_draft or argmax turns EARLY_STOP into
 * POSITION, and any of them or Z makes GROUP stream the bonus row with the
 * others and GROUP_TWO_PHASE run as GROUP (the per-row values are then
 * defined for every row). */
typedef enum {
    SPEC_SCHEDULE_AUTO = 0,
    SPEC_SCHEDULE_GROUP = 1,
    SPEC_SCHEDULE_EARLY_STOP = 2,
    SPEC_SCHEDULE_POSITION = 3,
    SPEC_SCHEDULE_GROUP_TWO_PHASE = 4
} spec_schedule_t;

/* spec_verify_noalloc: spec_verify for callers that cannot allocate device
 * memory - code under stream capture, tight serving loops, harnesses that
 * forbid hipMalloc. Same arguments, same results (the outputs do not depend
 * on the schedule). It calls no hipMalloc, hipFree or allocating library
 * routine: its kernel's scratch (partial slots, residual masses, counters,
 * the error word) is a fixed device array of the library, about 8.6 MiB per
 * GPU it runs on, held until the process ends; its address is looked up once
 * per device, and that first call also clears the array's counter words on
 * `stream` with a small kernel. Always the group-major order
 * (SPEC_SCHEDULE_GROUP), whose counters are reset by their last user, so the
 * array needs no clearing between calls.
 * Limits: B <= 1024, and the call's partial slots and residual masses within
 * 8 MiB (B = 1024, gamma = 8, V = 152064 in bf16 fits); larger problems get
 * SPEC_EINVAL before anything is launched. Every call on one GPU shares that
 * GPU's array: calls that overlap in time on one GPU (different streams, or
 * threads) race and must be serialised by the caller. The sticky error word
 * of spec_verify_status is the array's own (read with any stream of the
 * device that has no workspace of its own). */
int spec_verify_noalloc(const void* target_logits, const void* draft_logits,
                        const int32_t* draft_tokens, int32_t B, int32_t gamma, int32_t V,
                        int32_t dtype, float temperature, uint64_t seed,
                        int32_t* out_tokens, int32_t* out_n_accepted, void* stream);

/* spec_verify with extras (NULL extras == spec_verify, SPEC_SCHEDULE_AUTO).
 * SPEC_EINVAL for a schedule outside spec_schedule_t. */
int spec_verify_ex(const void* target_logits, const void* draft_logits,
                   const int32_t* draft_tokens, int32_t B, int32_t gamma, int32_t V,
                   int32_t dtype, float temperature, uint64_t seed,
                   int32_t* out_tokens, int32_t* out_n_accepted, void* stream,
                   const spec_extras_t* extras);

/* spec_row_stats: the softmax statistics pass alone ([Ch15] 15.1.2 step 2).
 *  logits [rows, V] dtype; 1 <= rows < 2^31; T > 0.
 *  row_max [rows] float  : max_j l_j;
 *  row_sumexp [rows] double : sum_j exp((l_j - row_max)/T); NaN when the row
 *  holds NaN or +inf or no finite entry. Same kernel and statistics code as
 *  spec_verify. */
int spec_row_stats(const void* logits, int64_t rows, int32_t V, int32_t dtype,
                   float temperature, float* row_max, double* row_sumexp, void* stream);

/* spec_draft_sample: draft-side sampling, the step before verification
 * ([Ch15] 15.1.2 step 1: each draft token is drawn from the draft model's
 * distribution and its probability kept; [CSDN] 2.1, stage 1 of
 * speculative_decode()).
 *  logits [B, n, V] dtype, DEVICE, row-major contiguous: row (b, t) holds the
 *      draft model's logits for position pos0 + t of sequence b (n = 1 for one
 *      autoregressive step, or a block of positions at once).
 *  temperature > 0: x = the smallest j whose ascending cumulative mass of
 *      softmax(l/T) exceeds u*S (S the total), with u the Philox4x32-10 uniform
 *      of counter (b + b_offset, pos0 + t, 2 = DRAFT, 0) keyed by seed (the
 *      verification's accept and correction draws use purposes 0 and 1, so
 *      the streams never meet); q = softmax(l/T)_x. temperature == 0: x = the
 *      first index of the maximum, q = 1.
 *  out_tokens [B, n] int32, DEVICE: x, or -1 for a row holding NaN, +inf or no
 *      finite entry (-inf entries are masked tokens and never drawn).
 *  out_q [B, n] double, DEVICE, or NULL: q, NaN where the token is -1.
 *  pos0 >= 0 and b_offset >= 0 (counter words are taken mod 2^32);
 *  B * n < 2^31. Enqueued on stream; returns without synchronising. Errors as
 *  spec_verify (checked before any launch). Uses the library's workspace of
 *  (device, stream), like spec_verify. Every row's logits are read once, plus
 *  one 4 KiB range again at T > 0. */
int spec_draft_sample(const void* logits, int32_t B, int32_t n, int32_t V, int32_t dtype,
                      float temperature, uint64_t seed, int64_t pos0, int64_t b_offset,
                      int32_t* out_tokens, double* out_q, void* stream);

/* Optional outputs and timing of spec_draft_sample_ex; every field may be
 * NULL. */
typedef struct {
    double* entropy;  /* [B, n] DEVICE: H = -sum_j p_j ln p_j of softmax(l/T) per row
                         (natural log; 0 at T == 0; NaN for an unusable row), the
                         confidence measure for choosing the draft length ([Ch15]
                         15.2.4, adaptive draft length). Formed in the same pass. */
    void* events[2];  /* hipEvent_t bound to the start and end of the dispatch */
} spec_draft_extras_t;

/* spec_draft_sample with optional extras (extras may be NULL). */
int spec_draft_sample_ex(const void* logits, int32_t B, int32_t n, int32_t V, int32_t dtype,
                         float temperature, uint64_t seed, int64_t pos0, int64_t b_offset,
                         int32_t* out_tokens, double* out_q, void* stream,
                         const spec_draft_extras_t* extras);

/* spec_expected_accept: the probability that position i accepts its draft
 * token when it is reached, beta[b, i] = sum_x min(p_i(x), q_i(x)) (Lemma 1
 * of [Ch15] 15.1.2; 1 - beta_i is the residual mass of the correction step),
 * for every position i < gamma: the per-position diagnostic behind the
 * acceptance-rate rule for the draft length ([Ch15] 15.1.4, dynamic strategy
 * adjustment).
 *  target_logits [B, gamma+1, V], draft_logits [B, gamma, V]: dtype, DEVICE,
 *      row-major contiguous (the bonus rows are not read); temperature > 0.
 *  out_beta [B, gamma] double, DEVICE: beta, NaN where either row holds NaN
 *      or +inf or no finite entry.
 *  B * (gamma + 1) < 2^31. Reads every row twice (statistics, then the
 *  overlap) in one launch on stream, no synchronisation. Errors as
 *  spec_verify. Uses the library's workspace of (device, stream). */
int spec_expected_accept(const void* target_logits, const void* draft_logits, int32_t B,
                         int32_t gamma, int32_t V, int32_t dtype, float temperature,
                         double* out_beta, void* stream);

/* spec_tree_verify: token-tree verification, a LABELLED HEURISTIC MODE that
 * does not preserve the target distribution ([CSDN] 3.2,
 * TokenTreeVerifier.parallel_verify; [Ch15] 15.2.4 candidate trees). From
 * the root, among the children of the last accepted node the first child
 * with the largest score is taken while its score reaches `threshold`;
 * score = min(1, p_v(token)/q_v(token)) under the parent v's target and draft
 * rows at temperature > 0; at temperature == 0 the child whose token is the
 * target argmax of row v (lowest index on ties) is taken, if any. No
 * correction or bonus token is emitted.
 *  target_logits [B, N, V], draft_logits [B, N, V] (NULL allowed only at
 *      temperature 0): dtype, DEVICE; row j = the model's logits after the
 *      path to node j (scores node j's children).
 *  parent [B, N], token [B, N] int32, DEVICE: node 0 is the root (its
 *      entries are ignored); node j >= 1 has parent 0 <= parent[j] < j and
 *      token token[j].
 *  out_tokens [B, N-1], out_nodes [B, N-1] (may be NULL) int32, DEVICE: the
 *      accepted path's tokens and nodes, -1 after it; out_n [B]: its length,
 *      or -1 when a parent index is out of order, or the walk meets a child
 *      token outside [0, V) or a needed row holding NaN, +inf or no finite
 *      entry.
 *  N >= 2, B * N < 2^31, threshold not NaN. Reads every row once (the
 *  statistics of all nodes), then walks each tree with one wavefront (at
 *  temperature > 0 with N <= 256, in the same launch). Errors as
 *  spec_verify. Uses the library's workspace of (device, stream). */
int spec_tree_verify(const void* target_logits, const void* draft_logits, const int32_t* parent,
                     const int32_t* token, int32_t B, int32_t N, int32_t V, int32_t dtype,
                     float temperature, float threshold, int32_t* out_tokens, int32_t* out_nodes,
                     int32_t* out_n, void* stream);

/* The schedule SPEC_SCHEDULE_AUTO takes for this shape with no per-row
 * outputs (SPEC_SCHEDULE_GROUP_TWO_PHASE, SPEC_SCHEDULE_GROUP or
 * SPEC_SCHEDULE_EARLY_STOP), or SPEC_EINVAL. A rule of the shape alone (see
 * SPEC_SCHEDULE_AUTO): it makes no HIP call. */
int32_t spec_verify_schedule(int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature);

/* spec_verify_status: whether any bounded wait of a kernel enqueued on
 * `stream` (current device) ran out since the last status call on that
 * stream ([Ch15] 15.1.4, failure-mode detection: the host's view of it).
 * Synchronises the stream, then sets *timed_out to 1 (and clears the word,
 * scrubbing the workspace's counters) or 0. With a timed-out wait, the
 * affected sequences of the calls since the last status call may be -1
 * (invalid), or may have been computed correctly after the wait drained;
 * no sequence holds a wrong token or count. Returns SPEC_OK, SPEC_EINVAL for
 * a NULL timed_out, or SPEC_EHIP. Every entry point on one (device, stream)
 * shares the word. */
int spec_verify_status(void* stream, int32_t* timed_out);

/* spec_verify_set_wait_limit: the bound on every in-kernel wait of calls
 * made after it, in ticks of the device's constant-rate wall clock (100 MHz
 * on gfx950); ticks < 0 restores the default (2e8 ticks, about 2 s).
 * Process-wide; returns the previous setting (-1 for the default). Meant for
 * tests of the failure path (0 makes every wait that is not satisfied at
 * its first poll give up), never needed for correct operation. The drain
 * after a wait gives up always uses the default bound. */
int64_t spec_verify_set_wait_limit(int64_t ticks);

/* Bytes of device workspace one call of this shape needs (the library
 * allocates and owns it). */
size_t spec_verify_workspace_bytes(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                                   float temperature);

/* Frees every cached workspace after synchronising the streams that own them. */
void spec_verify_release_workspace(void);

/* Message of the last non-OK return on this thread ("" if none). */
const char* spec_verify_last_error(void);

/* ABI version: 6 (2: spec_extras_t gained schedule; 3: spec_draft_sample;
 * 4: spec_draft_extras_t and spec_expected_accept; 5: spec_tree_verify;
 * 6: spec_verify_status and spec_verify_set_wait_limit). */
int32_t spec_verify_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* SPECVERIFY_H */
