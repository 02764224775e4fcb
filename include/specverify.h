/*
 * specverify — batched verify-and-accept step of speculative decoding on MI355X (gfx950).
 *
 * For B sequences with K draft tokens each, the library takes the target model's and
 * the draft model's logits over a vocabulary of V ids at every draft position and
 * returns, per sequence, how many draft tokens are accepted and the tokens to emit.
 *
 * Operations and where they are defined (page title, section):
 *  - Sampling verify (also with early exit): "推测性拒绝采样" (speculative rejection sampling), steps 2-4
 *    (parallel verification, probability-ratio acceptance, truncation at the first
 *    rejection, replacement drawn at that position) and its "key guarantee" section
 *    (output distribution identical to the target's), which fixes the replacement law
 *    as the normalised residual max(0, p - q); the bonus token after K acceptances is
 *    the gamma+1 draw of the "Speculative Contrastive Decoding" review, SCD section.
 *  - Greedy blockwise verify (also with early exit): "Blockwise Parallel Decoding", section
 *    3.5 (Verify and Accept: longest prefix on which the target's argmax equals the proposals).
 *  - Contrastive-target verify: "Speculative Contrastive Decoding" review, sections on
 *    contrastive decoding (large-model minus small-model distribution) and SCD.
 *  - Draft-token sampler: "推测性拒绝采样", step 1 (the draft model proposes its tokens one
 *    at a time); SCD review (Ma drafts gamma tokens).
 *  - Greedy verify with the next block's proposals: "Blockwise Parallel Decoding", section
 *    3.6 (Predict and Verify merged into one pass of the heads).
 *  - Alpha-quantile cut: "Speculative Rejection" Best-of-N page, section 4.2 (rejection
 *    threshold r_cut at the alpha-quantile of the partial rewards).
 *
 * Conventions for every entry point below:
 *  - All array pointers are DEVICE pointers owned by the caller; arrays are row-major and
 *    contiguous.  Logits are float32 (SPECVERIFY_F32) or bfloat16 (SPECVERIFY_BF16) and
 *    must be aligned to their element size; int32 / float arrays to 4 bytes.
 *  - hip_stream is a hipStream_t (NULL = the default stream).  Calls only enqueue work on
 *    it and return; results are valid once the caller has synchronised that stream.
 *  - The context owns a device workspace sized at creation; one call may be in flight per
 *    context at a time (use one context per concurrent stream).  Only specverify_create
 *    allocates device memory.  The run_* calls only launch kernels (no allocation, memset
 *    or synchronisation), so a caller may capture them in a HIP graph and replay it; replays
 *    on one context must not overlap either.
 *  - Host-detectable errors return before anything is enqueued and leave all outputs
 *    untouched: NULL context or required pointer, negative sizes, V < 1, a non-positive or
 *    non-finite temperature, or a misaligned pointer -> SPECVERIFY_EINVAL; B, K or V above
 *    the context's capacity -> SPECVERIFY_ECAPACITY; an unknown dtype ->
 *    SPECVERIFY_EUNSUPPORTED; a failed launch -> SPECVERIFY_EHIP.
 *  - Token ids cannot be checked on the host without a synchronisation.  A sequence whose
 *    draft tokens / proposals fall outside [0, V) gets accepted_len = -1, all-(-1) tokens
 *    and NaN out_probs; the other sequences are unaffected.
 *  - B = 0 is a no-op.  K = 0 is plain sampling from p_0 (or the argmax of row 0).
 *  - Logits may be -inf (zero probability) provided every row has a finite entry; NaN
 *    and +inf are outside the contract.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct specverify_ctx specverify_ctx;

enum specverify_dtype { SPECVERIFY_F32 = 0, SPECVERIFY_BF16 = 1 };

enum specverify_status {
    SPECVERIFY_OK = 0,
    SPECVERIFY_EINVAL = -1,
    SPECVERIFY_EUNSUPPORTED = -2,
    SPECVERIFY_ENOMEM = -3,
    SPECVERIFY_EHIP = -4,
    SPECVERIFY_ECAPACITY = -5
};

/* Largest K a context accepts (one wave64 lane per draft position). */
#define SPECVERIFY_MAX_K 63

/* Largest vocabulary a context accepts (the draw keeps its per-slice weight sums on chip). */
#define SPECVERIFY_MAX_VOCAB (1 << 20)

/* Most scores per prompt the quantile cut accepts (they are selected on chip). */
#define SPECVERIFY_MAX_CUT_N 8192

/*
 * Create a context on HIP device `device` for calls with B <= max_batch, K <= max_k and
 * V <= max_vocab, allocating its device workspace there (a few MB for the largest
 * vocabularies; see specverify_workspace_bytes).  On success *out receives the context.
 * Errors: EINVAL (out NULL, sizes < 1, max_k > SPECVERIFY_MAX_K,
 * max_vocab > SPECVERIFY_MAX_VOCAB, or a capacity whose largest launch would exceed the
 * 2^32 - 1 work-items one dispatch can cover: with 256 threads per chunk of 8192 float32 ids,
 * max_batch * (2 * max_k + 1) * ceil(max_vocab / 8192) must stay below 2^24, and likewise
 * max_batch * (max_k + 1) * ceil(max_vocab / 4096); e.g. max_batch <= 8191 at max_k = 63 and
 * max_vocab = 128256), EHIP (bad device), ENOMEM (allocation failed).  These are checked
 * before the device is touched.
 */
int specverify_create(specverify_ctx **out, int device, int max_batch, int max_k, int max_vocab);

/* Bytes of device workspace the context holds. */
int64_t specverify_workspace_bytes(const specverify_ctx *ctx);

/*
 * Sampling verify.  With T the temperature, p_j = softmax(l_target[b,j,:] / T) for
 * j in [0, K] and q_j = softmax(l_draft[b,j,:] / T) for j < K:
 *  - draft token x_j is accepted iff p_j(x_j) > 0 and u[b,j] * q_j(x_j) <= p_j(x_j)
 *    (kept outright when the target favours it, else with probability p/q);
 *  - L = the first rejected position, or K if none;
 *  - the emitted token at position L is drawn by inverse CDF (ascending id, first id
 *    whose inclusive prefix sum exceeds u[b,K] * W) from w = max(0, p_L - q_L) when
 *    L < K, or from w = p_K when every draft token is accepted (if rounding leaves
 *    the residual empty, from p_L).
 *  target_logits [B][K+1][V], draft_logits [B][K][V] (dtype), draft_tokens [B][K] int32,
 *  uniforms [B][K+1] float in [0,1]: u[b,0..K-1] accept tests, u[b,K] the replacement or
 *  bonus draw.
 *  Outputs: accepted_len [B] int32 (L, or -1 for bad ids), out_tokens [B][K+1] int32
 *  (x_0..x_{L-1}, the drawn token, then -1), out_probs [B][K][2] float
 *  (p_j(x_j), q_j(x_j) for every j < K) or NULL.
 *  Arithmetic: fp32 row statistics from one read of every logit, fp64 combination and
 *  decisions.  The residual draw is computed in fp64 from the logits of row L (per-id terms
 *  and both normalising sums), so that its cumulative weights over W carry an fp64 error
 *  however small the residual mass W is.
 */
int specverify_run_sampling(specverify_ctx *ctx, void *hip_stream, int dtype, int B, int K,
                            int V, float temperature, const void *target_logits,
                            const void *draft_logits, const int32_t *draft_tokens,
                            const float *uniforms, int32_t *accepted_len, int32_t *out_tokens,
                            float *out_probs);

/*
 * Sampling verify that allocates nothing, for callers that cannot call hipMalloc: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.  Same arguments,
 * layouts, arithmetic and results as specverify_run_sampling, without a context: it runs on
 * the calling thread's current device, and its workspace is a file-scope device array of
 * SPECVERIFY_STATIC_SCRATCH_BYTES per device (held until the process ends; its address is
 * taken on the first call on each device).  A call needs B * (2K+1) * ceil(V / chunk) * 32
 * bytes of it for the row statistics (chunk = 8192 bfloat16 or 4096 float32 ids), plus about
 * 2.3 KB per sequence when B is at most half the device's compute units; larger inputs
 * return SPECVERIFY_ECAPACITY before any GPU work.  Every call on a device shares its array:
 * calls that overlap on one device (other streams, other threads) race and must be ordered
 * by the caller.  The statistics partials are rewritten and the arrival counts cleared by
 * each call (a kernel, not a memset, so a captured graph replays it).  Errors as
 * specverify_run_sampling (capacity: the array's size, SPECVERIFY_MAX_K, SPECVERIFY_MAX_VOCAB).
 */
#define SPECVERIFY_STATIC_SCRATCH_BYTES (4 << 20)
int specverify_run_sampling_static(void *hip_stream, int dtype, int B, int K, int V,
                                   float temperature, const void *target_logits,
                                   const void *draft_logits, const int32_t *draft_tokens,
                                   const float *uniforms, int32_t *accepted_len,
                                   int32_t *out_tokens, float *out_probs);

/*
 * Sampling verify with early exit: accepted_len and out_tokens exactly as
 * specverify_run_sampling (same arithmetic, same decisions), but a sequence's rows after its
 * first rejection are not read, since the tokens after that rejection are discarded
 * ("推测性拒绝采样", step 3).  Every sequence's first two positions (target and draft rows) are
 * read, then the remaining rows of the sequences that accepted both, then the draw.
 * out_probs [B][K][2] holds (p_j(x_j), q_j(x_j)) for j <= L only and NaN for j > L.
 * Same arguments, layouts and errors as specverify_run_sampling.
 */
int specverify_run_sampling_early_exit(specverify_ctx *ctx, void *hip_stream, int dtype, int B,
                                      int K, int V, float temperature, const void *target_logits,
                                      const void *draft_logits, const int32_t *draft_tokens,
                                      const float *uniforms, int32_t *accepted_len,
                                      int32_t *out_tokens, float *out_probs);

/*
 * Contrastive-target verify with early exit: accepted_len and out_tokens exactly as
 * specverify_run_contrastive, reading each sequence's row pairs only up to its first
 * rejection (as specverify_run_sampling_early_exit).  out_probs for j <= L, NaN after.
 * Same arguments, layouts and errors as specverify_run_contrastive.
 */
int specverify_run_contrastive_early_exit(specverify_ctx *ctx, void *hip_stream, int dtype, int B,
                                         int K, int V, float tau, const void *expert_logits,
                                         const void *amateur_logits, const int32_t *draft_tokens,
                                         const float *uniforms, int32_t *accepted_len,
                                         int32_t *out_tokens, float *out_probs);

/*
 * Greedy blockwise verify.  g_j = the lowest id among the maxima of l_target[b,j,:]
 * (raw value comparison) for j in [0, K]; L = the first j < K with proposals[b,j] != g_j,
 * else K.  target_logits [B][K+1][V] (dtype), proposals [B][K] int32.
 * Outputs: accepted_len [B] (L or -1 for bad ids), out_tokens [B][K+1] (g_0..g_L, then -1).
 */
int specverify_run_greedy(specverify_ctx *ctx, void *hip_stream, int dtype, int B, int K, int V,
                          const void *target_logits, const int32_t *proposals,
                          int32_t *accepted_len, int32_t *out_tokens);

/*
 * Greedy blockwise verify with early exit: accepted_len and out_tokens exactly as
 * specverify_run_greedy (the same argmaxes, bit for bit), but a sequence's rows after its
 * first mismatch are not read, since the emitted tokens stop there ("Blockwise Parallel
 * Decoding", section 3.5, Accept: the longest matching prefix and the target's token after
 * it).  Every sequence's first positions are read; the rows after them only for the
 * sequences whose proposals matched all of them.  Same arguments, layout and errors as
 * specverify_run_greedy.
 */
int specverify_run_greedy_early_exit(specverify_ctx *ctx, void *hip_stream, int dtype, int B,
                                     int K, int V, const void *target_logits,
                                     const int32_t *proposals, int32_t *accepted_len,
                                     int32_t *out_tokens);

/*
 * Contrastive-target verify: as specverify_run_sampling with the target law
 * p_j = softmax((l_expert[b,j,:] - l_amateur[b,j,:]) / tau) for j in [0, K] (the
 * difference formed in fp32) and the draft law q_j = softmax(l_amateur[b,j,:]) for j < K.
 * expert_logits and amateur_logits are both [B][K+1][V] (dtype); the amateur rows
 * 0..K-1 are the draft model's.
 */
int specverify_run_contrastive(specverify_ctx *ctx, void *hip_stream, int dtype, int B, int K,
                               int V, float tau, const void *expert_logits,
                               const void *amateur_logits, const int32_t *draft_tokens,
                               const float *uniforms, int32_t *accepted_len,
                               int32_t *out_tokens, float *out_probs);

/*
 * Draft-token sampler: one draw per row, out_tokens[n] = the first id (ascending) whose
 * inclusive prefix sum of p = softmax(logits[n,:] / T) exceeds uniforms[n] * sum(p).
 * logits [N][V] (dtype), uniforms [N] float in [0,1]; out_tokens [N] int32; out_probs [N]
 * float = p(out_tokens[n]) (fp64 from the row's statistics) or NULL.
 * N is limited by the context's max_batch and V by its max_vocab (ECAPACITY); other errors
 * as for specverify_run_sampling.  The same two kernels as sampling verify run, with no
 * draft positions.
 */
int specverify_sample(specverify_ctx *ctx, void *hip_stream, int dtype, int N, int V,
                      float temperature, const void *logits, const float *uniforms,
                      int32_t *out_tokens, float *out_probs);

/*
 * Greedy blockwise verify whose verify pass also carries the next block's proposals.
 * logits [B][K+1][H][V] (dtype): at position j (the prefix followed by proposals 0..j-1),
 * head h scores the token h places after it; head 0 is the base model.  accepted_len and
 * out_tokens are those of specverify_run_greedy on head 0 (L = longest prefix on which the
 * proposals equal head 0's first argmax; g_0..g_L emitted).  next_proposals [B][H-1] =
 * the first argmaxes of heads 1..H-1 at position L, the proposals for the positions after
 * the emitted g_L (-1 for a sequence with bad ids); may be NULL when H = 1.
 * Errors: EINVAL for H < 1 and as specverify_run_greedy; ECAPACITY for B, K or V above the
 * context's capacity, or B * (H - 1) >= 2^24 (one 256-thread workgroup per sequence and extra
 * head).
 */
int specverify_run_greedy_heads(specverify_ctx *ctx, void *hip_stream, int dtype, int B, int K,
                                int H, int V, const void *logits, const int32_t *proposals,
                                int32_t *accepted_len, int32_t *out_tokens,
                                int32_t *next_proposals);

/*
 * Alpha-quantile cut of P prompts' N partial-reward scores each (scores [P][N] float, finite):
 * with k = min(floor(alpha * N), N - 1) (computed in double on the host), r_cut[p] = the
 * (k+1)-th smallest score of prompt p, keep[p][i] = (scores[p][i] >= r_cut[p]) as 0/1 bytes,
 * n_keep[p] = the number kept (>= N - k; ties at r_cut are all kept).  Exact: comparisons
 * only.  Errors: EINVAL (NULL pointers, P < 0, N < 1, alpha outside [0, 1] or NaN),
 * ECAPACITY (N > SPECVERIFY_MAX_CUT_N, or P >= 2^22: one 1024-thread workgroup per prompt).
 * Needs no workspace: the context supplies the
 * device and the timing.
 */
int specverify_quantile_cut(specverify_ctx *ctx, void *hip_stream, int P, int N, float alpha,
                            const float *scores, float *r_cut, uint8_t *keep, int32_t *n_keep);

/*
 * Test hook: flags that force draw paths which data rarely reaches, so that tests can compare
 * them with a reference.  Normal callers never set them (a new context has 0).
 *   SPECVERIFY_TEST_CHUNK_FALLBACK  a draw from p_L alone (the bonus draw, the sampler) skips
 *                                   the one-chunk draw and weighs the whole row (the path taken
 *                                   when rounding leaves the chosen chunk without weight)
 *   SPECVERIFY_TEST_EXACT_TWO_PASS  the fp64 residual draw always runs its exact second pass
 *                                   (taken when an id lies too close to the residual's edge
 *                                   for the first pass to place it)
 * Every flag leaves the outputs within the same parity with the definitions above.  Applies to
 * the calls that follow on this context.  Errors: EINVAL (NULL ctx, unknown bits).
 */
#define SPECVERIFY_TEST_CHUNK_FALLBACK 1u
#define SPECVERIFY_TEST_EXACT_TWO_PASS 2u
int specverify_set_test_flags(specverify_ctx *ctx, unsigned flags);

/* Release the context and its workspace.  NULL-safe; returns SPECVERIFY_OK. */
int specverify_destroy(specverify_ctx *ctx);

/* Static description of a status code. */
const char *specverify_strerror(int status);

/*
 * Kernel timing.  Kernel kinds:
 *   0 row statistics (sampling, contrastive, sampler), 1 accept scan and draw (sampling,
 *   contrastive, sampler), 2 row argmax (greedy), 3 proposal compare and emit (greedy, with
 *   the next proposals for the heads variant), 4 quantile cut, 5 early-exit accept tests on
 *   the first positions, 6 early-exit statistics of the remaining rows.
 * specverify_profile_begin(ctx, max_calls, kinds, stride) creates hipEvent pairs for up to
 * max_calls timed calls: of the calls that follow, the 1st, (stride+1)-th, (2*stride+1)-th,
 * ... are timed (stride 1 = every call).  In a timed call every kernel whose kind k has bit
 * (1 << k) set in `kinds` (0 = every kind) is launched with its start and stop events
 * attached to the dispatch (hipExtLaunchKernel), on the call's stream; its duration is the
 * kernel's own execution.  A timed dispatch costs a few microseconds more than an untimed
 * one, so a stride above 1 keeps the timing out of the rate of a long run of calls.
 * specverify_profile_launches(ctx, kind, ms, cap), between begin and end, synchronises on the
 * events of the timed launches of kernel kind `kind` so far and writes their durations in
 * milliseconds, in call order, into the host array ms[0..cap) (cap 0 with ms NULL only
 * counts them).  It returns the number of such launches (which may exceed cap: only the
 * first cap are written) or a negative status.
 * specverify_profile_end(ctx, ms, launches) synchronises on the recorded events, writes the
 * summed milliseconds and launch counts per kind into the two SPECVERIFY_NUM_KERNELS-long
 * arrays (either may be NULL), and releases the events.
 * Errors: EINVAL (NULL ctx, max_calls < 1, stride < 1, unknown kind bits, begin twice, end
 * or launches without begin, kind outside [0, SPECVERIFY_NUM_KERNELS), cap < 0, cap > 0
 * with ms NULL), EHIP.
 */
#define SPECVERIFY_NUM_KERNELS 7
int specverify_profile_begin(specverify_ctx *ctx, int max_calls, unsigned kinds, int stride);
int specverify_profile_launches(specverify_ctx *ctx, int kind, float *ms, int cap);
int specverify_profile_end(specverify_ctx *ctx, double *ms, int *launches);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
