// C-ABI runtime: context and workspace, host-side argument validation, launch sequencing on
// the caller's stream, kernel timing.  The kernels live in sv_kernels.hip.
#include "specverify.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <vector>

#include "sv_internal.h"

struct specverify_ctx {
    int device;
    int max_batch, max_k, max_vocab, max_nch;
    int num_cus;                          // compute units of the device
    void *mem;
    size_t bytes;
    sv::Workspace ws;
    // timing
    bool prof;
    int prof_cap, prof_calls;
    long long prof_seen;                  // calls since profile_begin
    int prof_stride;                      // time every prof_stride-th of them
    unsigned prof_mask;                   // kernel kinds to time
    std::vector<hipEvent_t> events;       // prof_cap * 2 * SPECVERIFY_NUM_KERNELS
    std::vector<unsigned> launched;       // per recorded call: bit k = kernel kind k ran
};

namespace {

constexpr int NK = SPECVERIFY_NUM_KERNELS;
static_assert(NK == sv::NUM_KINDS, "kernel kinds out of step with the header");
static_assert(SPECVERIFY_MAX_CUT_N == sv::MAX_CUT_N, "cut capacity out of step with the header");
static_assert(SPECVERIFY_MAX_VOCAB == sv::MAX_VOCAB, "vocabulary cap out of step with the header");
static_assert(SPECVERIFY_STATIC_SCRATCH_BYTES == sv::STATIC_SCRATCH_BYTES,
              "scratch size out of step with the header");
static_assert(SPECVERIFY_TEST_CHUNK_FALLBACK == sv::TEST_CHUNK_FALLBACK &&
                  SPECVERIFY_TEST_EXACT_TWO_PASS == sv::TEST_EXACT_TWO_PASS,
              "test flags out of step with the header");

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    hipError_t err = hipSuccess;
    explicit DeviceGuard(int dev)
    {
        err = hipGetDevice(&prev);
        if (err == hipSuccess && prev != dev) {
            err = hipSetDevice(dev);
            changed = (err == hipSuccess);
        }
    }
    ~DeviceGuard()
    {
        if (changed)
            (void)hipSetDevice(prev);
    }
};

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

bool aligned_to(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_common(const specverify_ctx *ctx, int dtype, int B, int K, int V)
{
    if (!ctx)
        return SPECVERIFY_EINVAL;
    if (dtype != SPECVERIFY_F32 && dtype != SPECVERIFY_BF16)
        return SPECVERIFY_EUNSUPPORTED;
    if (B < 0 || K < 0 || V < 1)
        return SPECVERIFY_EINVAL;
    if (B > ctx->max_batch || K > ctx->max_k || V > ctx->max_vocab)
        return SPECVERIFY_ECAPACITY;
    return SPECVERIFY_OK;
}

bool bad_temperature(float t) { return !(t > 0.0f) || !isfinite(t); }

// A dispatch covers at most 2^32 - 1 work-items along its one grid dimension.
constexpr size_t MAX_ITEMS = 0xffffffffull;

// work-items of the largest launch a context of this capacity can make, over both dtypes: the
// row statistics and the greedy argmax (at most 2K+1 rows of float32 chunks of 8 vectors per
// thread; the statistics take two chunks per workgroup, so a row of an odd number of chunks
// launches one chunk's threads more), the contrastive pairs (K+1 rows of the smaller pair
// chunks) and the draw (one workgroup per sequence)
size_t largest_launch(int max_batch, int max_k, int max_vocab)
{
    const size_t k = (size_t)max_k;
    const size_t nch = (size_t)sv::num_chunks(sv::NV_STATS, 0, max_vocab);
    const size_t stats = (2 * k + 1) * (nch >= 2 ? (nch + 1) / 2 * 2 : nch);
    const size_t mc = (size_t)sv::max_chunks(max_vocab);
    const size_t pairs = (k + 1) * (mc >= 2 ? (mc + 1) / 2 * 2 : mc);
    const size_t per_seq = std::max(std::max(stats, pairs) * sv::WG, (size_t)sv::TAIL_WG);
    return (size_t)max_batch * per_seq;
}

// event pair array for the next call when timing is on, NULL otherwise
hipEvent_t *next_events(specverify_ctx *ctx)
{
    if (!ctx->prof)
        return nullptr;
    const bool timed = (ctx->prof_seen++ % ctx->prof_stride) == 0;
    if (!timed || ctx->prof_calls >= ctx->prof_cap)
        return nullptr;
    return ctx->events.data() + (size_t)ctx->prof_calls * 2 * NK;
}

void note_call(specverify_ctx *ctx, hipEvent_t *ev, unsigned kinds)
{
    if (ev) {
        ctx->launched[ctx->prof_calls] = kinds & ctx->prof_mask;
        ctx->prof_calls++;
    }
}

// sampling or contrastive verify, reading every row or (early_exit) only up to each
// sequence's first rejection
int run_sampling_like(specverify_ctx *ctx, void *stream, int mode, int dtype, int B, int K, int V,
                      float temperature, const void *tgt, const void *drf, const int32_t *tokens,
                      const float *unif, int32_t *acc_len, int32_t *out_tokens, float *out_probs,
                      bool early_exit)
{
    int rc = check_common(ctx, dtype, B, K, V);
    if (rc != SPECVERIFY_OK)
        return rc;
    if (bad_temperature(temperature))
        return SPECVERIFY_EINVAL;
    if (B == 0)
        return SPECVERIFY_OK;
    const bool need_draft = (mode == sv::CONTRASTIVE) || K > 0;
    if (!tgt || !unif || !acc_len || !out_tokens || (need_draft && !drf) || (K > 0 && !tokens))
        return SPECVERIFY_EINVAL;
    const size_t es = dtype == SPECVERIFY_BF16 ? 2 : 4;
    if (!aligned_to(tgt, es) || (drf && !aligned_to(drf, es)) || (tokens && !aligned_to(tokens, 4)) ||
        !aligned_to(unif, 4) || !aligned_to(acc_len, 4) || !aligned_to(out_tokens, 4) ||
        (out_probs && !aligned_to(out_probs, 4)))
        return SPECVERIFY_EINVAL;

    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess)
        return SPECVERIFY_EHIP;
    const sv::Scale sp = sv::make_scale((double)temperature);
    const sv::Scale sq = (mode == sv::CONTRASTIVE) ? sv::make_scale(1.0) : sp;
    hipEvent_t *ev = next_events(ctx);
    sv::Launch ln{static_cast<hipStream_t>(stream), ev, ctx->prof_mask};
    hipError_t e;
    unsigned kinds = (1u << sv::KIND_STATS) | (1u << sv::KIND_TAIL);
    if (early_exit) {
        // the survivors' rows: 24 256-thread workgroups per compute unit, most of which take
        // one or two items (fewer left the last items to a few workgroups)
        e = sv::launch_early_exit(ln, ctx->ws, mode, dtype, B, K, V, sp, sq, tgt, drf, tokens,
                                  unif, acc_len, out_tokens, out_probs, 24 * ctx->num_cus);
        kinds |= (1u << sv::KIND_EARLY_ACCEPT) | (1u << sv::KIND_EARLY_REST);
    } else {
        e = sv::launch_sampling(ln, ctx->ws, mode, dtype, B, K, V, sp, sq, tgt, drf, tokens, unif,
                                acc_len, out_tokens, out_probs, nullptr);
    }
    note_call(ctx, ev, kinds);
    return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_EHIP;
}

}  // namespace

extern "C" {

int specverify_create(specverify_ctx **out, int device, int max_batch, int max_k, int max_vocab)
{
    if (!out || max_batch < 1 || max_k < 0 || max_k > SPECVERIFY_MAX_K || max_vocab < 1 ||
        max_vocab > SPECVERIFY_MAX_VOCAB || largest_launch(max_batch, max_k, max_vocab) > MAX_ITEMS)
        return SPECVERIFY_EINVAL;
    *out = nullptr;
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || device < 0 || device >= ndev)
        return SPECVERIFY_EHIP;
    DeviceGuard g(device);
    if (g.err != hipSuccess)
        return SPECVERIFY_EHIP;

    const size_t nch = (size_t)sv::max_chunks(max_vocab);
    const size_t rows = (size_t)max_batch * (2 * (size_t)max_k + 1);
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess ||
        cus < 1)
        return SPECVERIFY_EHIP;
    // a sequence's draw is shared by several workgroups only when B <= cus / 2
    const int split_batch = std::min(max_batch, cus / 2);
    // per sequence of a shared draw: the fp64 pass's two sums per unit and three totals per
    // workgroup
    // per sequence: two fp64 sums per segment, three totals per workgroup
    const int nu_stride = 2 * sv::EXACT_MAX_SEGS + 3 * sv::TAIL_MAX_SPLIT;
    const size_t b_part = align_up(rows * nch * sv::WAVES * sizeof(float2));
    const size_t b_seq = align_up((size_t)max_batch * sizeof(int));
    const size_t b_gu = align_up((size_t)split_batch * nu_stride * sizeof(double));
    const size_t b_gc = align_up((size_t)split_batch * sizeof(int));
    const size_t b_tab = align_up((size_t)sv::GTAB_DOUBLES * sizeof(double));
    const size_t total = b_part + 2 * b_seq + align_up(sizeof(int)) + b_gu + b_gc + b_tab;

    specverify_ctx *ctx = new (std::nothrow) specverify_ctx();
    if (!ctx)
        return SPECVERIFY_ENOMEM;
    if (hipMalloc(&ctx->mem, total) != hipSuccess) {
        delete ctx;
        return SPECVERIFY_ENOMEM;
    }
    char *p = static_cast<char *>(ctx->mem);
    ctx->ws.part = reinterpret_cast<float2 *>(p);
    ctx->ws.alive = reinterpret_cast<int *>(p + b_part);
    ctx->ws.list = reinterpret_cast<int *>(p + b_part + b_seq);
    ctx->ws.count = reinterpret_cast<int *>(p + b_part + 2 * b_seq);
    ctx->ws.gunits = reinterpret_cast<double *>(p + b_part + 2 * b_seq + align_up(sizeof(int)));
    ctx->ws.gcount = reinterpret_cast<int *>(p + b_part + 2 * b_seq + align_up(sizeof(int)) + b_gu);
    ctx->ws.gtab = reinterpret_cast<double *>(p + b_part + 2 * b_seq + align_up(sizeof(int)) + b_gu +
                                              b_gc);
    ctx->ws.split_batch = split_batch;
    ctx->ws.nu_stride = nu_stride;
    ctx->ws.num_cus = cus;
    ctx->ws.test_flags = 0;
    // the arrival counts start at 0; every call leaves them at 0
    if (split_batch > 0 &&
        (hipMemset(ctx->ws.gcount, 0, (size_t)split_batch * sizeof(int)) != hipSuccess ||
         hipDeviceSynchronize() != hipSuccess)) {
        (void)hipFree(ctx->mem);
        delete ctx;
        return SPECVERIFY_EHIP;
    }
    ctx->num_cus = cus;
    ctx->device = device;
    ctx->max_batch = max_batch;
    ctx->max_k = max_k;
    ctx->max_vocab = max_vocab;
    ctx->max_nch = (int)nch;
    ctx->bytes = total;
    ctx->prof = false;
    ctx->prof_cap = ctx->prof_calls = 0;
    ctx->prof_seen = 0;
    ctx->prof_stride = 1;
    ctx->prof_mask = 0;
    *out = ctx;
    return SPECVERIFY_OK;
}

int64_t specverify_workspace_bytes(const specverify_ctx *ctx) { return ctx ? (int64_t)ctx->bytes : 0; }

int specverify_run_sampling(specverify_ctx *ctx, void *hip_stream, int dtype, int B, int K, int V,
                            float temperature, const void *target_logits, const void *draft_logits,
                            const int32_t *draft_tokens, const float *uniforms,
                            int32_t *accepted_len, int32_t *out_tokens, float *out_probs)
{
    return run_sampling_like(ctx, hip_stream, sv::SAMPLING, dtype, B, K, V, temperature,
                             target_logits, draft_logits, draft_tokens, uniforms, accepted_len,
                             out_tokens, out_probs, false);
}

int specverify_run_sampling_static(void *hip_stream, int dtype, int B, int K, int V,
                                   float temperature, const void *target_logits,
                                   const void *draft_logits, const int32_t *draft_tokens,
                                   const float *uniforms, int32_t *accepted_len,
                                   int32_t *out_tokens, float *out_probs)
{
    // the checks of specverify_run_sampling, with the scratch array's size as the capacity
    if (dtype != SPECVERIFY_F32 && dtype != SPECVERIFY_BF16)
        return SPECVERIFY_EUNSUPPORTED;
    if (B < 0 || K < 0 || V < 1 || bad_temperature(temperature))
        return SPECVERIFY_EINVAL;
    if (K > SPECVERIFY_MAX_K || V > SPECVERIFY_MAX_VOCAB ||
        (B > 0 && largest_launch(B, K, V) > MAX_ITEMS))
        return SPECVERIFY_ECAPACITY;
    if (B > 0 && (!target_logits || !uniforms || !accepted_len || !out_tokens ||
                  (K > 0 && (!draft_logits || !draft_tokens))))
        return SPECVERIFY_EINVAL;
    const size_t es = dtype == SPECVERIFY_BF16 ? 2 : 4;
    if (!aligned_to(target_logits, es) || (draft_logits && !aligned_to(draft_logits, es)) ||
        (draft_tokens && !aligned_to(draft_tokens, 4)) || !aligned_to(uniforms, 4) ||
        !aligned_to(accepted_len, 4) || !aligned_to(out_tokens, 4) ||
        (out_probs && !aligned_to(out_probs, 4)))
        return SPECVERIFY_EINVAL;
    // the scratch layout: the statistics' partials, then (a draw shared by several workgroups,
    // B <= compute units / 2) the segment sums and arrival counts of each sequence, then the
    // draw's tables
    const size_t nch = (size_t)sv::num_chunks(sv::NV_STATS, dtype, V);
    const size_t b_part = align_up((size_t)B * (2 * (size_t)K + 1) * nch * sv::WAVES * sizeof(float2));
    const int nu_stride = 2 * sv::EXACT_MAX_SEGS + 3 * sv::TAIL_MAX_SPLIT;
    if (b_part > sv::STATIC_SCRATCH_BYTES)
        return SPECVERIFY_ECAPACITY;
    if (B == 0)
        return SPECVERIFY_OK;
    int dev = -1, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
        return SPECVERIFY_EHIP;
    const bool split = B <= cus / 2;
    const size_t b_gu = split ? align_up((size_t)B * nu_stride * sizeof(double)) : 0;
    const size_t b_gc = split ? align_up((size_t)B * sizeof(int)) : 0;
    const size_t b_tab = align_up((size_t)sv::GTAB_DOUBLES * sizeof(double));
    if (b_part + b_gu + b_gc + b_tab > sv::STATIC_SCRATCH_BYTES)
        return SPECVERIFY_ECAPACITY;
    void *base = nullptr;
    if (sv::static_scratch(dev, &base) != hipSuccess)
        return SPECVERIFY_EHIP;
    char *p = static_cast<char *>(base);
    sv::Workspace ws = {};
    ws.part = reinterpret_cast<float2 *>(p);
    ws.gunits = split ? reinterpret_cast<double *>(p + b_part) : nullptr;
    ws.gcount = split ? reinterpret_cast<int *>(p + b_part + b_gu) : nullptr;
    ws.gtab = reinterpret_cast<double *>(p + b_part + b_gu + b_gc);
    ws.split_batch = split ? B : 0;
    ws.nu_stride = nu_stride;
    ws.num_cus = cus;
    ws.test_flags = 0;
    const hipStream_t st = static_cast<hipStream_t>(hip_stream);
    // the arrival counts must start at 0; the array keeps whatever the last call left
    if (split && sv::launch_zero_ints(st, ws.gcount, B) != hipSuccess)
        return SPECVERIFY_EHIP;
    const sv::Scale sc = sv::make_scale((double)temperature);
    sv::Launch ln{st, nullptr, 0u};
    const hipError_t e = sv::launch_sampling(ln, ws, sv::SAMPLING, dtype, B, K, V, sc, sc,
                                             target_logits, draft_logits, draft_tokens, uniforms,
                                             accepted_len, out_tokens, out_probs, nullptr);
    return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_EHIP;
}

int specverify_run_contrastive(specverify_ctx *ctx, void *hip_stream, int dtype, int B, int K,
                               int V, float tau, const void *expert_logits,
                               const void *amateur_logits, const int32_t *draft_tokens,
                               const float *uniforms, int32_t *accepted_len, int32_t *out_tokens,
                               float *out_probs)
{
    return run_sampling_like(ctx, hip_stream, sv::CONTRASTIVE, dtype, B, K, V, tau, expert_logits,
                             amateur_logits, draft_tokens, uniforms, accepted_len, out_tokens,
                             out_probs, false);
}

namespace {

int run_greedy_like(specverify_ctx *ctx, void *hip_stream, int dtype, int B, int K, int V,
                    const void *target_logits, const int32_t *proposals, int32_t *accepted_len,
                    int32_t *out_tokens, bool early_exit)
{
    int rc = check_common(ctx, dtype, B, K, V);
    if (rc != SPECVERIFY_OK)
        return rc;
    if (B == 0)
        return SPECVERIFY_OK;
    if (!target_logits || !accepted_len || !out_tokens || (K > 0 && !proposals))
        return SPECVERIFY_EINVAL;
    const size_t es = dtype == SPECVERIFY_BF16 ? 2 : 4;
    if (!aligned_to(target_logits, es) || (proposals && !aligned_to(proposals, 4)) ||
        !aligned_to(accepted_len, 4) || !aligned_to(out_tokens, 4))
        return SPECVERIFY_EINVAL;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess)
        return SPECVERIFY_EHIP;
    hipEvent_t *ev = next_events(ctx);
    sv::Launch ln{static_cast<hipStream_t>(hip_stream), ev, ctx->prof_mask};
    hipError_t e;
    unsigned kinds = (1u << sv::KIND_ARGMAX) | (1u << sv::KIND_GREEDY_EMIT);
    if (early_exit) {
        // the survivors' rows: as many workgroups as the sampling early exit uses
        e = sv::launch_greedy_early_exit(ln, ctx->ws, dtype, B, K, V, target_logits, proposals,
                                         accepted_len, out_tokens, 24 * ctx->num_cus);
        kinds |= (1u << sv::KIND_EARLY_ACCEPT) | (1u << sv::KIND_EARLY_REST);
    } else {
        e = sv::launch_greedy(ln, ctx->ws, dtype, B, K, V, target_logits, proposals,
                              accepted_len, out_tokens);
    }
    note_call(ctx, ev, kinds);
    return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_EHIP;
}

}  // namespace

int specverify_run_greedy(specverify_ctx *ctx, void *hip_stream, int dtype, int B, int K, int V,
                          const void *target_logits, const int32_t *proposals,
                          int32_t *accepted_len, int32_t *out_tokens)
{
    return run_greedy_like(ctx, hip_stream, dtype, B, K, V, target_logits, proposals,
                           accepted_len, out_tokens, false);
}

int specverify_run_greedy_early_exit(specverify_ctx *ctx, void *hip_stream, int dtype, int B,
                                     int K, int V, const void *target_logits,
                                     const int32_t *proposals, int32_t *accepted_len,
                                     int32_t *out_tokens)
{
    return run_greedy_like(ctx, hip_stream, dtype, B, K, V, target_logits, proposals,
                           accepted_len, out_tokens, true);
}

int specverify_run_sampling_early_exit(specverify_ctx *ctx, void *hip_stream, int dtype, int B,
                                      int K, int V, float temperature, const void *target_logits,
                                      const void *draft_logits, const int32_t *draft_tokens,
                                      const float *uniforms, int32_t *accepted_len,
                                      int32_t *out_tokens, float *out_probs)
{
    return run_sampling_like(ctx, hip_stream, sv::SAMPLING, dtype, B, K, V, temperature,
                             target_logits, draft_logits, draft_tokens, uniforms, accepted_len,
                             out_tokens, out_probs, true);
}

int specverify_run_contrastive_early_exit(specverify_ctx *ctx, void *hip_stream, int dtype, int B,
                                         int K, int V, float tau, const void *expert_logits,
                                         const void *amateur_logits, const int32_t *draft_tokens,
                                         const float *uniforms, int32_t *accepted_len,
                                         int32_t *out_tokens, float *out_probs)
{
    return run_sampling_like(ctx, hip_stream, sv::CONTRASTIVE, dtype, B, K, V, tau, expert_logits,
                             amateur_logits, draft_tokens, uniforms, accepted_len, out_tokens,
                             out_probs, true);
}

int specverify_sample(specverify_ctx *ctx, void *hip_stream, int dtype, int N, int V,
                      float temperature, const void *logits, const float *uniforms,
                      int32_t *out_tokens, float *out_probs)
{
    int rc = check_common(ctx, dtype, N, 0, V);
    if (rc != SPECVERIFY_OK)
        return rc;
    if (bad_temperature(temperature))
        return SPECVERIFY_EINVAL;
    if (N == 0)
        return SPECVERIFY_OK;
    if (!logits || !uniforms || !out_tokens)
        return SPECVERIFY_EINVAL;
    const size_t es = dtype == SPECVERIFY_BF16 ? 2 : 4;
    if (!aligned_to(logits, es) || !aligned_to(uniforms, 4) || !aligned_to(out_tokens, 4) ||
        (out_probs && !aligned_to(out_probs, 4)))
        return SPECVERIFY_EINVAL;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess)
        return SPECVERIFY_EHIP;
    const sv::Scale sp = sv::make_scale((double)temperature);
    hipEvent_t *ev = next_events(ctx);
    sv::Launch ln{static_cast<hipStream_t>(hip_stream), ev, ctx->prof_mask};
    // K = 0: each row is its own "sequence" whose only row is drawn from, u[n] the draw
    hipError_t e = sv::launch_sampling(ln, ctx->ws, sv::SAMPLING, dtype, N, 0, V, sp, sp, logits,
                                       nullptr, nullptr, uniforms, nullptr, out_tokens, nullptr,
                                       out_probs);
    note_call(ctx, ev, (1u << sv::KIND_STATS) | (1u << sv::KIND_TAIL));
    return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_EHIP;
}

int specverify_run_greedy_heads(specverify_ctx *ctx, void *hip_stream, int dtype, int B, int K,
                                int H, int V, const void *logits, const int32_t *proposals,
                                int32_t *accepted_len, int32_t *out_tokens,
                                int32_t *next_proposals)
{
    int rc = check_common(ctx, dtype, B, K, V);
    if (rc != SPECVERIFY_OK)
        return rc;
    if (H < 1)
        return SPECVERIFY_EINVAL;
    if ((size_t)B * (size_t)(H > 1 ? H - 1 : 1) * sv::WG > MAX_ITEMS)
        return SPECVERIFY_ECAPACITY;
    if (B == 0)
        return SPECVERIFY_OK;
    if (!logits || !accepted_len || !out_tokens || (K > 0 && !proposals) ||
        (H > 1 && !next_proposals))
        return SPECVERIFY_EINVAL;
    const size_t es = dtype == SPECVERIFY_BF16 ? 2 : 4;
    if (!aligned_to(logits, es) || (proposals && !aligned_to(proposals, 4)) ||
        !aligned_to(accepted_len, 4) || !aligned_to(out_tokens, 4) ||
        (next_proposals && !aligned_to(next_proposals, 4)))
        return SPECVERIFY_EINVAL;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess)
        return SPECVERIFY_EHIP;
    hipEvent_t *ev = next_events(ctx);
    sv::Launch ln{static_cast<hipStream_t>(hip_stream), ev, ctx->prof_mask};
    hipError_t e = sv::launch_greedy_heads(ln, ctx->ws, dtype, B, K, H, V, logits, proposals,
                                           accepted_len, out_tokens, next_proposals);
    note_call(ctx, ev, (1u << sv::KIND_ARGMAX) | (1u << sv::KIND_GREEDY_EMIT));
    return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_EHIP;
}

int specverify_quantile_cut(specverify_ctx *ctx, void *hip_stream, int P, int N, float alpha,
                            const float *scores, float *r_cut, uint8_t *keep, int32_t *n_keep)
{
    if (!ctx)
        return SPECVERIFY_EINVAL;
    if (P < 0 || N < 1 || !(alpha >= 0.0f && alpha <= 1.0f))
        return SPECVERIFY_EINVAL;
    if (N > SPECVERIFY_MAX_CUT_N || (size_t)P * sv::TAIL_WG > MAX_ITEMS)
        return SPECVERIFY_ECAPACITY;
    if (P == 0)
        return SPECVERIFY_OK;
    if (!scores || !r_cut || !keep || !n_keep)
        return SPECVERIFY_EINVAL;
    if (!aligned_to(scores, 4) || !aligned_to(r_cut, 4) || !aligned_to(n_keep, 4))
        return SPECVERIFY_EINVAL;
    // the number of responses cut, floor(alpha * N), taken once in double on the host
    long k = (long)floor((double)alpha * (double)N);
    if (k > N - 1)
        k = N - 1;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess)
        return SPECVERIFY_EHIP;
    hipEvent_t *ev = next_events(ctx);
    sv::Launch ln{static_cast<hipStream_t>(hip_stream), ev, ctx->prof_mask};
    hipError_t e = sv::launch_quantile_cut(ln, P, N, (int)k, scores, r_cut, keep, n_keep);
    note_call(ctx, ev, 1u << sv::KIND_CUT);
    return e == hipSuccess ? SPECVERIFY_OK : SPECVERIFY_EHIP;
}

int specverify_set_test_flags(specverify_ctx *ctx, unsigned flags)
{
    if (!ctx || (flags & ~(unsigned)sv::TEST_FLAGS_ALL) != 0)
        return SPECVERIFY_EINVAL;
    ctx->ws.test_flags = flags;
    return SPECVERIFY_OK;
}

int specverify_destroy(specverify_ctx *ctx)
{
    if (!ctx)
        return SPECVERIFY_OK;
    {
        DeviceGuard g(ctx->device);
        for (hipEvent_t e : ctx->events)
            (void)hipEventDestroy(e);
        if (ctx->mem)
            (void)hipFree(ctx->mem);
    }
    delete ctx;
    return SPECVERIFY_OK;
}

const char *specverify_strerror(int status)
{
    switch (status) {
    case SPECVERIFY_OK: return "ok";
    case SPECVERIFY_EINVAL: return "invalid argument (null or misaligned pointer, bad size or temperature)";
    case SPECVERIFY_EUNSUPPORTED: return "unsupported dtype";
    case SPECVERIFY_ENOMEM: return "device memory allocation failed";
    case SPECVERIFY_EHIP: return "HIP runtime or launch error";
    case SPECVERIFY_ECAPACITY: return "batch, draft length or vocabulary exceeds the context's capacity";
    default: return "unknown status";
    }
}

int specverify_profile_begin(specverify_ctx *ctx, int max_calls, unsigned kinds, int stride)
{
    if (!ctx || max_calls < 1 || stride < 1 || ctx->prof || (kinds >> NK) != 0)
        return SPECVERIFY_EINVAL;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess)
        return SPECVERIFY_EHIP;
    ctx->events.assign((size_t)max_calls * 2 * NK, nullptr);
    for (auto &e : ctx->events) {
        if (hipEventCreate(&e) != hipSuccess) {
            for (auto &f : ctx->events)
                if (f)
                    (void)hipEventDestroy(f);
            ctx->events.clear();
            return SPECVERIFY_EHIP;
        }
    }
    ctx->launched.assign((size_t)max_calls, 0u);
    ctx->prof = true;
    ctx->prof_cap = max_calls;
    ctx->prof_calls = 0;
    ctx->prof_seen = 0;
    ctx->prof_stride = stride;
    ctx->prof_mask = kinds ? kinds : (1u << NK) - 1;
    return SPECVERIFY_OK;
}

int specverify_profile_launches(specverify_ctx *ctx, int kind, float *ms, int cap)
{
    if (!ctx || !ctx->prof || kind < 0 || kind >= NK || cap < 0 || (cap > 0 && !ms))
        return SPECVERIFY_EINVAL;
    DeviceGuard g(ctx->device);
    if (g.err != hipSuccess)
        return SPECVERIFY_EHIP;
    int n = 0;
    for (int c = 0; c < ctx->prof_calls; ++c) {
        if (!(ctx->launched[c] & (1u << kind)))
            continue;
        if (n < cap) {
            hipEvent_t a = ctx->events[((size_t)c * NK + kind) * 2];
            hipEvent_t b = ctx->events[((size_t)c * NK + kind) * 2 + 1];
            float t = 0.0f;
            if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&t, a, b) != hipSuccess)
                return SPECVERIFY_EHIP;
            ms[n] = t;
        }
        ++n;
    }
    return n;
}

int specverify_profile_end(specverify_ctx *ctx, double *ms, int *launches)
{
    if (!ctx || !ctx->prof)
        return SPECVERIFY_EINVAL;
    DeviceGuard g(ctx->device);
    double tot[NK] = {0};
    int cnt[NK] = {0};
    int rc = (g.err == hipSuccess) ? SPECVERIFY_OK : SPECVERIFY_EHIP;
    for (int c = 0; c < ctx->prof_calls && rc == SPECVERIFY_OK; ++c) {
        for (int k = 0; k < NK; ++k) {
            if (!(ctx->launched[c] & (1u << k)))
                continue;
            hipEvent_t a = ctx->events[((size_t)c * NK + k) * 2];
            hipEvent_t b = ctx->events[((size_t)c * NK + k) * 2 + 1];
            float t = 0.0f;
            if (hipEventSynchronize(b) != hipSuccess || hipEventElapsedTime(&t, a, b) != hipSuccess) {
                rc = SPECVERIFY_EHIP;
                break;
            }
            tot[k] += t;
            cnt[k] += 1;
        }
    }
    for (hipEvent_t e : ctx->events)
        (void)hipEventDestroy(e);
    ctx->events.clear();
    ctx->launched.clear();
    ctx->prof = false;
    ctx->prof_cap = ctx->prof_calls = 0;
    ctx->prof_seen = 0;
    ctx->prof_stride = 1;
    if (ms)
        for (int k = 0; k < NK; ++k)
            ms[k] = tot[k];
    if (launches)
        for (int k = 0; k < NK; ++k)
            launches[k] = cnt[k];
    return rc;
}

}  // extern "C"
