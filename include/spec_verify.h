/*
 * spec_verify.h — C ABI of libspecverify.so: the batched verification step of
 * speculative sampling on AMD Instinct MI355X (gfx950).
 *
 * Sources for what each call computes:
 *   [P1] "Speculative Decoding" (atonlee.tistory.com/330), ch.2 "propose와 verify가 한
 *        round를 만드는 방식" and ch.3 "target distribution을 보존하는 acceptance rule";
 *   [P2] "Speculative Decoding으로 LLM 추론 속도 높이기" (donmain.dev), sections
 *        "미리 그려놓고 한 번에 검증한다" and "품질은 rejection sampling이 지킨다";
 *   [P3] "Fast Inference from Transformers via Speculative Decoding" (notes page),
 *        방법론 상세: 문제 설정 and 단계 1-3;
 *   [P4] "투기적 디코딩 — 초안 모델을 무엇으로 세울 것인가" (ailab.paldyn.com), section
 *        "출력이 변하지 않는다는 것이 핵심이다".
 *
 * Problem statement ([P3] 문제 설정, 단계 1-3): for each of B sequences the draft
 * proposed gamma_b tokens x_i ~ q_i, and one target forward produced gamma_b + 1
 * target rows. Verification computes p_i = softmax(l_i / T), judges the drafts
 * left to right, accepting x_i when u_i < min(1, p_i(x_i) / q_i(x_i)), stops at
 * the first rejection and draws the replacement there from
 * norm(max(0, p - q)); if all gamma_b drafts are accepted it draws a bonus
 * token from p at position gamma_b + 1 ([P1] ch.2-3; [P3] 단계 3). At T = 0 it
 * is greedy: accept iff the draft equals the target argmax (lowest index on
 * ties), and emit the target argmax at the first mismatch or at the bonus row
 * ([P1] ch.3 greedy paragraph; [P4]).
 *
 * Every draw is an inverse CDF over ascending token ids: with weights w and the
 * uniform u, t = u * sum(w) and the token is the first v whose inclusive prefix
 * sum exceeds t (the last positive-weight v if rounding leaves none). The
 * sampled row's arithmetic runs in float64 on the device; the pass over the
 * judged rows runs in float32 with a float64 accept test.
 *
 * Packing (ragged gamma_b, "cu_gamma" = exclusive prefix of gamma_b, length B+1):
 *   logits row of (b, i), i <= gamma_b : cu_gamma[b] + b + i
 *   q row / draft id of (b, i), i < gamma_b : cu_gamma[b] + i
 *   uniform of (b, i), i <= gamma_b   : cu_gamma[b] + b + i
 *   uniform slot i < gamma_b is the accept test of draft position i; slot
 *   gamma_b drives the single final draw (residual or bonus).
 * With a uniform gamma (cu_gamma == NULL) cu_gamma[b] = b * gamma.
 *
 * Ownership: the caller owns every input and output buffer. Pointers passed to
 * spec_verify_run are DEVICE pointers on the context's device and must stay
 * valid until the enqueued work has passed on the stream. The context owns its
 * device workspace, allocated once in spec_verify_create and freed in
 * spec_verify_destroy. spec_verify_run allocates nothing, never synchronizes and
 * returns once the kernels are enqueued. A context allows one run in flight at a
 * time (the workspace is shared) and is not thread-safe.
 *
 * Errors: functions return SV_* codes; nothing is thrown across the ABI.
 * Argument errors found on the host return SV_EINVAL and launch nothing. HIP
 * failures return SV_EHIP. Data errors are found on the device and raise a
 * sticky flag read by spec_verify_status (SV_EDATA), with defined fallbacks:
 *   - a draft id outside [0, V): that position is rejected (and its residual
 *     uses q as given);
 *   - a uniform outside [0, 1): used as is (u >= 1 rejects every judged
 *     position with thr <= 1 and makes a draw take the last positive weight);
 *   - a judged or sampled row whose softmax normaliser is not finite or not
 *     positive (NaN / +inf logits, or a row of -inf): flagged; outputs for that
 *     sequence are unspecified but in range. Row statistics are fp32 sums against a
 *     reference l log2(e)/T rounded to fp32, whose rounding passes the fp32
 *     exponent range once |l| log2(e)/T reaches about 2^30 (fp32 logits of 1e6 at
 *     T = 1e-3): such a row's normaliser overflows and is flagged the same way;
 *   - greedy mode (T == 0): a NaN logit in a judged row (a draft row up to the
 *     first mismatch, or the bonus row when it is read) raises the same flag
 *     (SV_DATA_NONFINITE); outputs for that sequence are unspecified but in range.
 *     -inf logits are values (a row of -inf has its argmax at index 0). A NaN in a
 *     row after the first mismatch is examined by the two-launch plan (which judges
 *     every draft row) and may or may not be by the one-launch plan;
 *   - malformed cu_gamma (decreasing, gamma_b > max_gamma, cu_gamma[B] !=
 *     total_draft_rows): flagged; that sequence's accepted_count is -1 and its
 *     other outputs are not written.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct spec_verify_ctx spec_verify_ctx; /* opaque; owns the workspace */

enum {
  SV_OK = 0,     /* success */
  SV_EINVAL = 1, /* bad argument found on the host; nothing launched */
  SV_ENOMEM = 2, /* workspace allocation failed in create */
  SV_EHIP = 3,   /* a HIP runtime call or launch failed */
  SV_EDATA = 4   /* (status only) the device flagged a data error since the last status call */
};

enum { SV_F32 = 0, SV_BF16 = 1 }; /* logits element type */

/* Data-error bits reported by spec_verify_status through spec_verify_last_error. */
enum {
  SV_DATA_DRAFT_ID = 1,   /* a draft id outside [0, V) */
  SV_DATA_NONFINITE = 2,  /* a row normaliser not finite / not positive */
  SV_DATA_UNIFORM = 4,    /* a uniform outside [0, 1) */
  SV_DATA_CU_GAMMA = 8,   /* malformed cu_gamma */
  SV_DATA_CONTEXT = 16,   /* malformed cu_ctx (spec_ngram_propose) */
  SV_DATA_STATE = 32,     /* adaptive draft-length state out of range (spec_adapt_gamma) */
  SV_DATA_STALL = 64      /* a wait between waves (of one workgroup, or of the workgroups of
                             one sequence in the small-batch plan) reached its bound: the
                             outputs of that call are not valid (not expected in use) */
};

/*
 * Create a context on HIP device `device` for vocabulary size `vocab` (1 <= V <= 2^24)
 * and logits element type `logits_dtype` (SV_F32 or SV_BF16). The workspace is
 * sized for at most `max_batch` sequences (<= 2^24; ragged runs <= 65536), `max_draft_rows` packed draft rows
 * (>= sum gamma_b of any run) and gamma_b <= `max_gamma` (<= 1024).
 * On success *out holds the context and SV_OK is returned; on failure *out is
 * NULL. Errors: SV_EINVAL (out NULL, vocab outside [1, 2^24], max_* < 0, max_gamma > 1024,
 * unknown dtype, or sizes whose packed tensors would not be addressable with
 * 64-bit offsets), SV_EHIP (bad device), SV_ENOMEM.
 */
int spec_verify_create(spec_verify_ctx **out, int device, int vocab, int logits_dtype,
                       int max_batch, int max_draft_rows, int max_gamma);

/*
 * Enqueue one verification step on `hip_stream` (a hipStream_t; NULL = the
 * default stream) of the context's device.
 *
 *   batch            B >= 0 sequences (B == 0: nothing is enqueued; returns SV_OK).
 *   gamma            uniform draft length (>= 0) when cu_gamma is NULL; must be -1
 *                    when cu_gamma is given.
 *   cu_gamma         device int32 [B+1] exclusive prefix of gamma_b, or NULL.
 *   total_draft_rows host copy of sum gamma_b (= B * gamma when uniform).
 *   temperature      T >= 0 and finite; T == 0 selects the greedy rule.
 *   logits           [sum(gamma_b + 1), V] row-major, element type from create.
 *   q                fp32 [sum gamma_b, V] draft distributions; required iff T > 0
 *                    (ignored when T == 0).
 *   draft_ids        int32 [sum gamma_b].
 *   uniforms         fp32 [sum(gamma_b + 1)] in [0, 1); required iff T > 0
 *                    (ignored when T == 0).
 * Outputs (device buffers, written completely for valid sequences):
 *   accepted_count   int32 [B]: n_b, the number of accepted drafts.
 *   emitted_tokens   int32 [sum(gamma_b + 1)]: per sequence, slots 0..n_b hold the
 *                    n_b accepted drafts and the drawn token; slots after are -1.
 *   residual_sum     fp32 [B]: S = sum max(0, p - q) at the rejected row; 0.0 when
 *                    every draft was accepted, and in greedy mode.
 *   p_draft          fp32 [sum gamma_b] or NULL: p_i(x_i) for every draft
 *                    position (NaN for an out-of-range id); not written when T == 0.
 * Errors: SV_EINVAL (ctx / required pointer NULL, B > max_batch,
 * total_draft_rows > max_draft_rows or inconsistent with B * gamma, gamma out of
 * range, T < 0 or not finite), SV_EHIP (launch failure). Data errors: see top.
 */
int spec_verify_run(spec_verify_ctx *ctx, void *hip_stream, int batch, int gamma,
                    const int32_t *cu_gamma, int total_draft_rows, float temperature,
                    const void *logits, const float *q, const int32_t *draft_ids,
                    const float *uniforms, int32_t *accepted_count, int32_t *emitted_tokens,
                    float *residual_sum, float *p_draft);

/*
 * spec_verify_run for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It takes no context and
 * allocates nothing (no hipMalloc, hipFree or allocating library call). Its workspace is
 * a static device array inside the library, SV_STATIC_SCRATCH_MAX_BYTES at most, of which
 * every GPU the library runs on holds one copy until the process ends; its address is
 * looked up once per device, on the first call there, which also enqueues a small kernel
 * on `hip_stream` that clears the workspace's counters.
 *   device        the HIP device of every pointer; the calling thread's current device
 *                 is left as it was.
 *   vocab, logits_dtype  as for spec_verify_create.
 *   batch .. p_draft     as for spec_verify_run, within the static workspace's limits:
 *                 batch <= SV_STATIC_MAX_BATCH, total_draft_rows <= SV_STATIC_MAX_ROWS,
 *                 gamma (or every gamma_b of a ragged run) <= SV_STATIC_MAX_GAMMA.
 *   data_flags    device int32 [1], caller-owned: the data-error bits (SV_DATA_*) found
 *                 by the kernels are OR-ed into it, never cleared (start it at 0).
 * The kernels and outputs are those of spec_verify_run under SV_PATH_AUTO, except that a
 * greedy batch never takes the helper plan (it runs one workgroup per sequence instead)
 * and a sampling batch never takes the small-batch plan's several workgroups per
 * sequence (short rows keep their one workgroup per sequence): both hand data between
 * workgroups under a per-call number kept on the host, and such a batch takes the
 * other plans. Nothing the kernels leave in the workspace is told apart by a host-side
 * number (its counters return to zero within each call), so calls captured into a HIP
 * graph can be replayed, also with new contents in the captured buffers.
 * Every call on one GPU shares that GPU's workspace, which keeps the last call's contents:
 * calls that overlap on one GPU (two streams, two threads) race and give undefined
 * results; calls in stream order are safe.
 * Errors: SV_EINVAL (a size beyond the static limits, the checks of spec_verify_run, a
 * NULL data_flags, no such device), SV_EHIP. The message of the calling thread's last
 * call is spec_verify_last_error(NULL).
 */
enum {
  SV_STATIC_MAX_BATCH = 1024,
  SV_STATIC_MAX_ROWS = 16384,
  SV_STATIC_MAX_GAMMA = 64,
  SV_STATIC_SCRATCH_MAX_BYTES = 4 << 20
};
int spec_verify_run_static(int device, void *hip_stream, int vocab, int logits_dtype, int batch, int gamma,
                           const int32_t *cu_gamma, int total_draft_rows, float temperature,
                           const void *logits, const float *q, const int32_t *draft_ids,
                           const float *uniforms, int32_t *accepted_count, int32_t *emitted_tokens,
                           float *residual_sum, float *p_draft, int32_t *data_flags);

/*
 * The same step for deterministic drafts, such as prompt-lookup (n-gram) proposals
 * ("Speculative Decoding", atonlee.tistory.com/330, ch.5; the pages do not say how such
 * drafts are verified, and this entry point takes the plain reading that the draft
 * distribution is one-hot at the proposed id, q = onehot(x)). No q is passed or read.
 * With the accept rule of ch.3 the test becomes u < p(x), and after a rejection at n
 * the draw is from max(0, p_n - onehot(x_n)) = p_n with x_n removed, S = 1 - p_n(x_n)
 * (p_n(x_n) = 1 draws from p_n and reports S = 0).
 * An id of -1 means "no draft at this slot" (spec_ngram_propose pads with it): the slot
 * is rejected, nothing is removed from p_n and no data flag is raised. Any other id
 * outside [0, V) is handled the same way but raises SV_DATA_DRAFT_ID.
 * Arguments, outputs and errors as spec_verify_run without q; with T == 0 it is the
 * greedy rule.
 */
int spec_verify_run_onehot(spec_verify_ctx *ctx, void *hip_stream, int batch, int gamma,
                           const int32_t *cu_gamma, int total_draft_rows, float temperature,
                           const void *logits, const int32_t *draft_ids, const float *uniforms,
                           int32_t *accepted_count, int32_t *emitted_tokens, float *residual_sum,
                           float *p_draft);

/*
 * Launch plan. A run either takes two launches (row statistics or argmaxes of every
 * draft row, then one workgroup per sequence for the first-rejection scan and the
 * draw; sampling runs with 16-byte aligned rows, V a multiple of 8 and at most half as
 * many sequences as compute units give each sequence two or four workgroups that
 * share the draw, fewer when the rows are too short to divide) or one launch (one
 * workgroup per sequence that judges its rows left to right,
 * stops reading at the first rejection and then draws; in greedy mode the argmax of
 * the first mismatching row, or of the bonus row, is the token). The one-launch plan
 * needs V a multiple of 8, 16-byte aligned logits (and q when T > 0), gamma_b <= 64
 * (for ragged runs: the context's max_gamma <= 64) and, under SV_PATH_AUTO, at least
 * 0.55 times as many sequences as the device has compute units (greedy: 0.8 times;
 * below that the two launches, which spread the rows over every compute unit, measured
 * faster on MI355X). With p_draft requested (T > 0)
 * it still reads every row. A ragged run with more sequences than compute units
 * first launches a one-workgroup kernel that orders the sequences by gamma_b,
 * longest first (the workspace holds the order); workgroups then take the sequences
 * in that order, so the short ones are dispatched last. A greedy one-launch run with
 * one to four times as many sequences as compute units adds two waves of one helper
 * workgroup per sequence, dispatched as slots free up, which take rows of a sequence
 * still being judged; the outputs are the same.
 * A third plan, one launch for small sampling batches (SV_PATH_POOLED): uniform gamma
 * <= 64, T > 0, V a multiple of 8 and 16-byte aligned logits and q, B x gamma x split
 * workgroups (split >= 1 chunks per draft row) no more than the device holds at once
 * (about 1024 on MI355X), B <= 2048 and the context's max_batch. Every draft row is read
 * in parallel, in chunks; the workgroups of a sequence wait (boundedly) for each other's
 * pass-1 records, all reach the same first rejection, and then sweep the drawn row
 * together, the wave of the first unit completing the draw. Rows of at most 4096
 * entries instead take one workgroup per sequence (any B), whose waves hand over through
 * LDS. The plan reads every draft row (as the two-launch plan does) and gives the same
 * outputs as the other plans. Under SV_PATH_AUTO it is taken when it applies and either
 * V <= 4096, or B is below the compute-unit count with fp32 logits (bf16 logits whose
 * values the draw's table covers take the two-launch plan, which measured faster there).
 * All plans return the same outputs, except that a draft id after the first rejection
 * is not examined by the one-launch plan (so it cannot raise SV_DATA_DRAFT_ID there).
 * Calls through a context are not meant to be captured into a HIP graph and replayed:
 * the greedy helper plan and the small-batch plan number their calls on the host, and a
 * replay would reuse the number. spec_verify_run_static takes neither and replays.
 *   spec_verify_set_path(ctx, mode): SV_PATH_AUTO (default), SV_PATH_TWO_LAUNCH,
 *     SV_PATH_ONE_LAUNCH (taken whenever the run allows it, whatever B) or
 *     SV_PATH_POOLED (taken whenever the run allows it; else the two-launch plan).
 *     Returns SV_OK or SV_EINVAL (NULL ctx, unknown mode).
 *   spec_verify_last_path(ctx): the plan of the last successful run
 *     (SV_PATH_TWO_LAUNCH, SV_PATH_ONE_LAUNCH or SV_PATH_POOLED), SV_PATH_AUTO if none
 *     yet, or -SV_EINVAL for a NULL ctx.
 */
enum { SV_PATH_AUTO = 0, SV_PATH_TWO_LAUNCH = 1, SV_PATH_ONE_LAUNCH = 2, SV_PATH_POOLED = 3 };
int spec_verify_set_path(spec_verify_ctx *ctx, int mode);
int spec_verify_last_path(const spec_verify_ctx *ctx);

/*
 * Vocabulary-parallel verification, one shard's part. The accept rule, the first
 * rejection and the draws are those of spec_verify_run ("Speculative Decoding",
 * atonlee.tistory.com/330, ch.3; "Fast Inference from Transformers via Speculative
 * Decoding" notes, 방법론 상세, 단계 3); only where the sums over the vocabulary are
 * taken moves. The vocabulary [0, vocab_total) is cut into `shards` contiguous column
 * ranges, shard k holding ids [bounds[k], bounds[k + 1]). A device that holds shard k
 * passes only its columns: logits [sum(gamma_b + 1), W_k] and q [sum gamma_b, W_k],
 * row-major with row pitch W_k = bounds[k + 1] - bounds[k], which must equal the
 * context's vocab. Batch, gamma, cu_gamma, temperature, draft ids and uniforms are those
 * of spec_verify_run and the same on every shard. A round is three calls per shard, with
 * two all-gathers between them (done by the caller, e.g. over RCCL; each record array
 * is gathered in shard order into one contiguous array):
 *   1. spec_vshard_rows writes `rec`: one 16-byte record per judged row (T > 0: the
 *      sum(gamma_b) draft rows; T == 0: those, then the B bonus rows), holding this
 *      shard's softmax state of the row and, on the shard owning the draft id, the id's
 *      logit and q entry (T == 0: the row's max and its lowest global index).
 *      All-gather -> rec_all [shards][records].
 *   2. spec_vshard_decide merges the records in shard order, so every shard takes the
 *      same decisions. It writes accepted_count, the accepted tokens and p_draft (T == 0:
 *      every output, and step 3 does nothing). T > 0: it then sweeps this shard's columns
 *      of the drawn row and writes `part` (fp64 [B][3], this shard's totals) and `local`
 *      (fp64 [B][52], kept on this device for step 3). All-gather part ->
 *      part_all [shards][B][3].
 *   3. spec_vshard_finish finds the shard whose columns hold each sequence's drawn
 *      token (the last shard when no column has weight). Only that shard writes
 *      emitted_tokens[n_b], the -1 padding after it and residual_sum[b]; the others
 *      leave those entries untouched, so a final exchange (or one shared buffer) gives
 *      every device the outputs.
 * The results are those of spec_verify_run on the whole vocabulary, up to the rounding
 * of the merged sums.
 *   sh         host struct: vocab_total, shards (1..64), shard (this device's index),
 *              bounds (host int32 [shards + 1], bounds[0] = 0, increasing,
 *              bounds[shards] = vocab_total).
 *   rec, rec_all, part, part_all, local: caller-owned device buffers of the sizes above.
 * Ownership, streams and the sticky data flag are as for spec_verify_run (ids are
 * checked against vocab_total); nothing is allocated and nothing synchronizes.
 * Errors: SV_EINVAL (NULL ctx, description or required pointer; bad bounds; a shard
 * width that differs from the context's vocab; the checks of spec_verify_run), SV_EHIP.
 */
typedef struct spec_vshard {
  int vocab_total;
  int shards;
  int shard;
  const int32_t *bounds;
} spec_vshard;
int spec_vshard_rows(spec_verify_ctx *ctx, void *hip_stream, const spec_vshard *sh, int batch,
                     int gamma, const int32_t *cu_gamma, int total_draft_rows, float temperature,
                     const void *logits, const float *q, const int32_t *draft_ids, void *rec);
int spec_vshard_decide(spec_verify_ctx *ctx, void *hip_stream, const spec_vshard *sh, int batch,
                       int gamma, const int32_t *cu_gamma, int total_draft_rows, float temperature,
                       const void *logits, const float *q, const int32_t *draft_ids,
                       const float *uniforms, const void *rec_all, int32_t *accepted_count,
                       int32_t *emitted_tokens, float *residual_sum, float *p_draft, double *part,
                       double *local);
int spec_vshard_finish(spec_verify_ctx *ctx, void *hip_stream, const spec_vshard *sh, int batch,
                       int gamma, const int32_t *cu_gamma, int total_draft_rows, float temperature,
                       const void *logits, const float *q, const float *uniforms,
                       const double *part_all, const double *local, int32_t *emitted_tokens,
                       float *residual_sum);

/*
 * Sampling one token per row from a given distribution: the draw of verification on
 * its own (decoding with the target alone, x ~ p, or drawing drafts, x ~ q), following
 * the draw's rule: t = u * sum(w) over the row's weights w, the token is the first id
 * whose inclusive prefix sum exceeds t, else the last id with positive weight.
 *   rows       number of rows (0 <= rows <= the context's max_batch; 0 enqueues nothing).
 *   mode       SV_SAMPLE_LOGITS: `x` is [rows, V] logits in the context's dtype and the
 *              weights are softmax(l / T); T == 0 takes the argmax (lowest index on ties)
 *              and ignores `uniforms`. This is spec_verify_run with gamma = 0.
 *              SV_SAMPLE_WEIGHTS: `x` is [rows, V] fp32 weights >= 0 (probabilities or
 *              any unnormalised weights; 4-byte aligned); T is ignored.
 *   uniforms   fp32 [rows] in [0, 1), one per row.
 *   tokens     int32 [rows] output.
 * Errors: SV_EINVAL (NULL ctx or pointer, rows out of range, unknown mode, bad T),
 * SV_EHIP. Data errors (sticky flag, spec_verify_status): negative or non-finite
 * weights count as 0 and set SV_DATA_NONFINITE, as does a row whose sum is not
 * positive (its token is then V - 1); a uniform outside [0, 1) sets SV_DATA_UNIFORM.
 */
enum { SV_SAMPLE_LOGITS = 0, SV_SAMPLE_WEIGHTS = 1 };
int spec_sample_run(spec_verify_ctx *ctx, void *hip_stream, int rows, int mode, float temperature,
                    const void *x, const float *uniforms, int32_t *tokens);

/*
 * Prompt-lookup (n-gram) draft proposer ("Speculative Decoding", atonlee.tistory.com/330,
 * ch.5 prompt lookup; "투기적 디코딩 — 초안 모델을 무엇으로 세울 것인가",
 * ailab.paldyn.com, "네 가지 방식"): for every context, the current suffix is looked up
 * earlier in the same context and the tokens that followed it there are proposed.
 * Readings of what the pages leave open: suffix lengths n = n_max .. n_min are tried and
 * the longest that occurs earlier wins; the occurrence must end before the last token
 * (it may overlap the suffix); of that length the most recent occurrence is used; at most
 * gamma following tokens are proposed, fewer where the context ends.
 *
 *   batch        B >= 0 contexts (B == 0: nothing is enqueued; returns SV_OK).
 *   tokens       device int32 [total_tokens], the contexts packed back to back; ids are
 *                only compared for equality (any int32 value).
 *   cu_ctx       device int32 [B+1], exclusive prefix of the context lengths.
 *   total_tokens host copy of cu_ctx[B] (>= 0).
 *   n_min, n_max 1 <= n_min <= n_max <= SV_NGRAM_MAX_N.
 *   gamma        0 <= gamma <= 1024 drafts per context.
 * Outputs (device, caller-owned, written completely):
 *   draft_ids    int32 [B, gamma]: row b holds its proposal, then -1 (the no-draft mark
 *                of spec_verify_run_onehot), so the rows feed that call with a uniform
 *                gamma.
 *   draft_len    int32 [B]: the proposal lengths (0 when nothing matched).
 * Errors: SV_EINVAL (ctx NULL, a required pointer NULL, sizes out of range; nothing is
 * launched), SV_EHIP. Offsets outside [0, total_tokens] or decreasing give that context
 * no proposal and set SV_DATA_CONTEXT (reported by spec_verify_status).
 * Runs on the context's device and stream like spec_verify_run; the vocabulary and
 * workspace of the context are not used.
 */
enum { SV_NGRAM_MAX_N = 64 };
int spec_ngram_propose(spec_verify_ctx *ctx, void *hip_stream, int batch, const int32_t *tokens,
                       const int32_t *cu_ctx, int total_tokens, int n_min, int n_max, int gamma,
                       int32_t *draft_ids, int32_t *draft_len);

/*
 * Adaptive draft length per sequence ("투기적 디코딩 — 초안 모델을 무엇으로 세울 것인가",
 * ailab.paldyn.com, "도입할 때 순서대로 확인할 것": after rejections in a row go down
 * to 1, raise again while acceptances continue; "Speculative Decoding",
 * atonlee.tistory.com/330, ch.4: the best length follows the acceptance rate). Run it
 * after a verification step to get the next round's draft lengths and packed layout.
 * Readings of what the pages leave open: a round "accepts" when every draft was accepted
 * (accepted_count[b] >= gamma[b]) and "rejects" when its first draft was rejected
 * (accepted_count[b] == 0); a partly accepted round breaks both runs. After up_after
 * accepting rounds in a row gamma[b] goes up by one (at most gamma_max), after
 * down_after rejecting rounds in a row it is cut to 1; a sequence with accepted_count -1
 * (its round was not run) keeps its state.
 *
 *   batch          0 <= B <= 65536 (B == 0: nothing is enqueued; returns SV_OK).
 *   accepted_count device int32 [B], the round's output of spec_verify_run.
 *   gamma          device int32 [B], in/out: the draft lengths of the round just
 *                  verified, replaced by the next round's, in [1, gamma_max] (0 stays 0
 *                  only when the round was not run).
 *   streak         device int32 [B], in/out: accepting (> 0) or rejecting (< 0) rounds
 *                  in a row; start at 0.
 *   gamma_max      1 <= gamma_max <= 1024; up_after, down_after >= 1.
 *   cu_gamma_next  device int32 [B+1], out: exclusive prefix of the new gamma, the
 *                  cu_gamma of the next spec_verify_run (its total_draft_rows is
 *                  cu_gamma_next[B]).
 * Errors: SV_EINVAL (ctx NULL, a NULL pointer, values out of range; nothing launched),
 * SV_EHIP. A gamma outside [0, gamma_max] or a streak outside [-down_after, up_after]
 * on entry is clamped into range and sets SV_DATA_STATE. One workgroup does the batch.
 */
int spec_adapt_gamma(spec_verify_ctx *ctx, void *hip_stream, int batch, const int32_t *accepted_count,
                     int32_t *gamma, int32_t *streak, int gamma_max, int up_after, int down_after,
                     int32_t *cu_gamma_next);

/*
 * Synchronize the stream of the last run, read and clear the device's sticky
 * data-error flag. Returns SV_OK, SV_EDATA (details in spec_verify_last_error),
 * SV_EHIP, or SV_EINVAL for a NULL ctx.
 */
int spec_verify_status(spec_verify_ctx *ctx);

/* Text of the last error on this context ("" if none). Owned by the context. With ctx NULL:
 * the message of the calling thread's last spec_verify_run_static call. */
const char *spec_verify_last_error(const spec_verify_ctx *ctx);

/* Free the workspace and the context. NULL-safe. Synchronizes the device first. */
void spec_verify_destroy(spec_verify_ctx *ctx);

/*
 * Measurement hook. spec_verify_set_timing(ctx, runs) with runs > 0 makes the
 * next `runs` calls of spec_verify_run launch each kernel with a start and a stop
 * HIP event (hipExtLaunchKernel), which take that dispatch's own begin and end
 * timestamps on the launch stream (runs == 0 switches recording off). It waits for the
 * device and allocates the events, so call it outside timed or captured code.
 * spec_verify_kernel_times waits for the last recorded run, writes up to `cap`
 * per-kernel mean durations in ms over the recorded runs and the kernels' names
 * (launch order; `names` may be NULL), stores the number of recorded runs in
 * *runs (may be NULL), restarts the recording and returns the number of kernels
 * per run (0 if nothing was recorded) or a negative SV_* code.
 */
int spec_verify_set_timing(spec_verify_ctx *ctx, int runs);
/* Record only one run in every `stride` (>= 1; default 1) of the runs that follow, so
 * that the events disturb a timed loop less. Returns SV_OK or SV_EINVAL. */
int spec_verify_set_timing_stride(spec_verify_ctx *ctx, int stride);
int spec_verify_kernel_times(spec_verify_ctx *ctx, float *ms, const char **names, int cap,
                             int *runs);

/*
 * Host-side argument check: the checks spec_verify_run performs before any
 * launch, without a context or a device. Returns SV_OK or SV_EINVAL (with the
 * reason copied into `msg`, NUL-terminated, when msg_cap > 0).
 */
int spec_verify_check_args(int vocab, int logits_dtype, int max_batch, int max_draft_rows,
                           int max_gamma, int batch, int gamma, int has_cu_gamma,
                           int total_draft_rows, float temperature, int has_logits, int has_q,
                           int has_draft_ids, int has_uniforms, int has_accepted_count,
                           int has_emitted_tokens, int has_residual_sum, char *msg, int msg_cap);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
