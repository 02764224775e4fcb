/*
 * Plain, slow CPU oracle for the batched verify-and-accept step of speculative
 * decoding.  Every intermediate is an IEEE double; loops run in ascending order.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or load
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code with the GPU library.
 *
 * What it follows (the pages are cited by title and section):
 *  - "推测性拒绝采样" (speculative rejection sampling), steps 2-4: the target scores
 *    every draft prefix, each draft token is kept outright when the target gives it
 *    more probability than the draft, otherwise kept with probability
 *    P_target / P_draft; everything after the first rejected token is dropped and a
 *    replacement is drawn at that position.  Its "key guarantee" section (output
 *    distribution identical to the target's) fixes the replacement law: it must be
 *    the normalised residual max(0, p - q), the only law that makes the emitted token
 *    distributed as p.
 *  - "Speculative Contrastive Decoding" review, SCD section: if every draft token is
 *    accepted one more token is drawn at position gamma+1 from the target-side law;
 *    in SCD the target law is the contrastive one, large-model minus small-model.
 *  - "Blockwise Parallel Decoding", section 3.5 (Verify / Accept): greedy argmax at
 *    every position, keep the longest prefix on which it equals the proposals, the
 *    argmax at the first mismatch is the next token.
 *
 * Readings taken where the pages are silent (all listed in the design notes):
 *  temperature divides both target and draft logits in sampling mode; the
 *  contrastive target is softmax((l_e - l_a) / tau) and its draft law softmax(l_a);
 *  accept iff P > 0 and u * Q <= P; inverse CDF in ascending token id with a strict
 *  ">" so zero-mass ids are never drawn; argmax ties go to the lowest id.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_BF16 = 1 };
enum { OR_OK = 0, OR_EINVAL = -1, OR_ENOMEM = -3 };

/* Exact widening of one stored logit to double. bf16 is the top half of an fp32. */
static double logit_at(int dtype, const void *base, size_t i)
{
    if (dtype == OR_F32)
        return (double)((const float *)base)[i];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/*
 * softmax over one row of scaled logits z[0..V): m = max z, S = sum exp(z - m),
 * p[v] = exp(z[v] - m) / S.
 */
void oracle_softmax(const double *z, int V, double *p)
{
    double m = -INFINITY;
    for (int v = 0; v < V; ++v)
        if (z[v] > m)
            m = z[v];
    double S = 0.0;
    for (int v = 0; v < V; ++v)
        S += exp(z[v] - m);
    for (int v = 0; v < V; ++v)
        p[v] = exp(z[v] - m) / S;
}

/* first index of the largest value (raw comparison, lowest id on ties) */
static int first_argmax(int dtype, const void *base, size_t off, int V)
{
    int best = 0;
    double bv = logit_at(dtype, base, off);
    for (int v = 1; v < V; ++v) {
        double x = logit_at(dtype, base, off + (size_t)v);
        if (x > bv) {
            bv = x;
            best = v;
        }
    }
    return best;
}

/*
 * Draw from weights w[0..V) with one uniform: t = u * W, return the first id whose
 * inclusive prefix sum exceeds t.  If rounding leaves no such id (u next to 1), the
 * last id of positive weight.  *mu receives the distance from t to the nearer edge of
 * the chosen id's interval, divided by W; *alt the positive-weight id on the other
 * side of that nearer edge (the id a slightly different rounding could pick instead).
 */
static int inverse_cdf(const double *w, int V, double u, double *mu, int *alt)
{
    double W = 0.0;
    for (int v = 0; v < V; ++v)
        W += w[v];
    double t = u * W;
    double c = 0.0;
    for (int v = 0; v < V; ++v) {
        double prev = c;
        c += w[v];
        if (c > t) {
            double lo = t - prev, hi = c - t;
            *mu = (lo < hi ? lo : hi) / W;
            *alt = v;
            if (lo < hi) {
                for (int k = v - 1; k >= 0; --k)
                    if (w[k] > 0.0) {
                        *alt = k;
                        break;
                    }
            } else {
                for (int k = v + 1; k < V; ++k)
                    if (w[k] > 0.0) {
                        *alt = k;
                        break;
                    }
            }
            return v;
        }
    }
    int last = -1;
    for (int v = 0; v < V; ++v)
        if (w[v] > 0.0)
            last = v;
    *mu = 0.0;
    *alt = last;
    return last;
}

/* per-sequence decision margins */
typedef struct {
    double accept; /* min over the accept tests that were made (j <= L) of |u_j - min(1, P/Q)| */
    double sample; /* distance of t to the nearer edge of the drawn id's interval, / W */
    int alt;       /* positive-weight id across that nearer edge */
} margins_t;

/*
 * Verify one sequence given its per-position target laws p[0..K] and draft laws
 * q[0..K-1] (each V doubles), draft tokens x[0..K-1] and uniforms u[0..K].
 * Writes L, the emitted tokens (x_0..x_{L-1}, y, then -1), (P_j, Q_j) for every
 * j < K, and the decision margins.
 */
static void verify_sequence(int K, int V, const double *p, const double *q, const int32_t *x,
                            const float *u, double *w, int32_t *acc_len, int32_t *tokens,
                            double *probs, margins_t *mg)
{
    int L = K;
    double mu_min = INFINITY;
    for (int j = 0; j < K; ++j) {
        double P = p[(size_t)j * V + x[j]];
        double Q = q[(size_t)j * V + x[j]];
        if (probs) {
            probs[2 * j] = P;
            probs[2 * j + 1] = Q;
        }
        if (L < K)
            continue; /* already rejected: later tokens are discarded */
        double uj = (double)u[j];
        double ratio = (Q > 0.0) ? P / Q : (P > 0.0 ? INFINITY : 0.0);
        double keep = ratio < 1.0 ? ratio : 1.0;
        double mu = fabs(uj - keep);
        if (mu < mu_min)
            mu_min = mu;
        int accept = (P > 0.0) && (uj * Q <= P);
        if (!accept)
            L = j;
    }
    /* replacement law at the first rejection, or the bonus law after K acceptances */
    const double *pL = p + (size_t)L * V;
    double W = 0.0;
    if (L < K) {
        const double *qL = q + (size_t)L * V;
        for (int v = 0; v < V; ++v) {
            double d = pL[v] - qL[v];
            w[v] = d > 0.0 ? d : 0.0;
            W += w[v];
        }
    } else {
        for (int v = 0; v < V; ++v) {
            w[v] = pL[v];
            W += w[v];
        }
    }
    if (W == 0.0) /* only reachable by rounding: fall back to the target law */
        for (int v = 0; v < V; ++v)
            w[v] = pL[v];
    double mu_y;
    int alt;
    int y = inverse_cdf(w, V, (double)u[K], &mu_y, &alt);
    for (int j = 0; j < L; ++j)
        tokens[j] = x[j];
    tokens[L] = y;
    for (int j = L + 1; j <= K; ++j)
        tokens[j] = -1;
    *acc_len = L;
    mg->accept = mu_min;
    mg->sample = mu_y;
    mg->alt = alt;
}

static void mark_bad(int K, int32_t *acc_len, int32_t *tokens, double *probs, margins_t *mg)
{
    *acc_len = -1;
    for (int j = 0; j <= K; ++j)
        tokens[j] = -1;
    if (probs)
        for (int j = 0; j < 2 * K; ++j)
            probs[j] = NAN;
    mg->accept = INFINITY;
    mg->sample = INFINITY;
    mg->alt = -1;
}

static void put_margins(const margins_t *m, double *margin, int *alt)
{
    if (margin) {
        margin[0] = m->accept;
        margin[1] = m->sample;
    }
    if (alt)
        *alt = m->alt;
}

static int ids_ok(const int32_t *x, int K, int V)
{
    for (int j = 0; j < K; ++j)
        if (x[j] < 0 || x[j] >= V)
            return 0;
    return 1;
}

/*
 * Sampling verify. target [B][K+1][V], draft [B][K][V] (dtype), draft_tokens [B][K],
 * uniforms [B][K+1] (u[0..K-1] accept tests, u[K] replacement/bonus draw).
 * Outputs accepted_len [B], out_tokens [B][K+1], out_probs [B][K][2] (may be NULL),
 * margin [B][2] = (accept-test margin, sample margin) and alt_token [B] (both may be NULL).
 */
int oracle_run_sampling(int dtype, int B, int K, int V, double T, const void *target,
                        const void *draft, const int32_t *draft_tokens, const float *uniforms,
                        int32_t *accepted_len, int32_t *out_tokens, double *out_probs,
                        double *margin, int32_t *alt_token)
{
    if (B < 0 || K < 0 || V < 1 || !(T > 0.0) || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_EINVAL;
    double *p = malloc(sizeof(double) * (size_t)(K + 1) * V);
    double *q = malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * V);
    double *z = malloc(sizeof(double) * (size_t)V);
    double *w = malloc(sizeof(double) * (size_t)V);
    if (!p || !q || !z || !w) {
        free(p); free(q); free(z); free(w);
        return OR_ENOMEM;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t *x = draft_tokens + (size_t)b * K;
        int32_t *tok = out_tokens + (size_t)b * (K + 1);
        double *pr = out_probs ? out_probs + (size_t)b * K * 2 : NULL;
        margins_t mg;
        if (!ids_ok(x, K, V)) {
            mark_bad(K, accepted_len + b, tok, pr, &mg);
            put_margins(&mg, margin ? margin + 2 * (size_t)b : NULL, alt_token ? alt_token + b : NULL);
            continue;
        }
        for (int j = 0; j <= K; ++j) {
            size_t off = ((size_t)b * (K + 1) + j) * V;
            for (int v = 0; v < V; ++v)
                z[v] = logit_at(dtype, target, off + v) / T;
            oracle_softmax(z, V, p + (size_t)j * V);
        }
        for (int j = 0; j < K; ++j) {
            size_t off = ((size_t)b * K + j) * V;
            for (int v = 0; v < V; ++v)
                z[v] = logit_at(dtype, draft, off + v) / T;
            oracle_softmax(z, V, q + (size_t)j * V);
        }
        verify_sequence(K, V, p, q, x, uniforms + (size_t)b * (K + 1), w, accepted_len + b, tok,
                        pr, &mg);
        put_margins(&mg, margin ? margin + 2 * (size_t)b : NULL, alt_token ? alt_token + b : NULL);
    }
    free(p); free(q); free(z); free(w);
    return OR_OK;
}

/*
 * Contrastive-target verify. expert and amateur are [B][K+1][V]; the target law at
 * position j is softmax((l_e - l_a) / tau), the draft law softmax(l_a) for j < K.
 */
int oracle_run_contrastive(int dtype, int B, int K, int V, double tau, const void *expert,
                           const void *amateur, const int32_t *draft_tokens,
                           const float *uniforms, int32_t *accepted_len, int32_t *out_tokens,
                           double *out_probs, double *margin, int32_t *alt_token)
{
    if (B < 0 || K < 0 || V < 1 || !(tau > 0.0) || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_EINVAL;
    double *p = malloc(sizeof(double) * (size_t)(K + 1) * V);
    double *q = malloc(sizeof(double) * (size_t)(K > 0 ? K : 1) * V);
    double *z = malloc(sizeof(double) * (size_t)V);
    double *w = malloc(sizeof(double) * (size_t)V);
    if (!p || !q || !z || !w) {
        free(p); free(q); free(z); free(w);
        return OR_ENOMEM;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t *x = draft_tokens + (size_t)b * K;
        int32_t *tok = out_tokens + (size_t)b * (K + 1);
        double *pr = out_probs ? out_probs + (size_t)b * K * 2 : NULL;
        margins_t mg;
        if (!ids_ok(x, K, V)) {
            mark_bad(K, accepted_len + b, tok, pr, &mg);
            put_margins(&mg, margin ? margin + 2 * (size_t)b : NULL, alt_token ? alt_token + b : NULL);
            continue;
        }
        for (int j = 0; j <= K; ++j) {
            size_t off = ((size_t)b * (K + 1) + j) * V;
            for (int v = 0; v < V; ++v)
                z[v] = (logit_at(dtype, expert, off + v) - logit_at(dtype, amateur, off + v)) / tau;
            oracle_softmax(z, V, p + (size_t)j * V);
            if (j < K) {
                for (int v = 0; v < V; ++v)
                    z[v] = logit_at(dtype, amateur, off + v);
                oracle_softmax(z, V, q + (size_t)j * V);
            }
        }
        verify_sequence(K, V, p, q, x, uniforms + (size_t)b * (K + 1), w, accepted_len + b, tok,
                        pr, &mg);
        put_margins(&mg, margin ? margin + 2 * (size_t)b : NULL, alt_token ? alt_token + b : NULL);
    }
    free(p); free(q); free(z); free(w);
    return OR_OK;
}

/*
 * Greedy blockwise verify. target [B][K+1][V], proposals [B][K].
 * g_j = first argmax of row j; L = first j < K with proposal_j != g_j, else K;
 * emits g_0..g_L then -1.  A proposal outside [0, V) marks the sequence bad
 * (accepted_len -1, all tokens -1).
 */
int oracle_run_greedy(int dtype, int B, int K, int V, const void *target,
                      const int32_t *proposals, int32_t *accepted_len, int32_t *out_tokens)
{
    if (B < 0 || K < 0 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_EINVAL;
    for (int b = 0; b < B; ++b) {
        const int32_t *x = proposals + (size_t)b * K;
        int32_t *tok = out_tokens + (size_t)b * (K + 1);
        if (!ids_ok(x, K, V)) {
            margins_t mg;
            mark_bad(K, accepted_len + b, tok, NULL, &mg);
            continue;
        }
        int L = K;
        for (int j = 0; j <= K; ++j) {
            int g = first_argmax(dtype, target, ((size_t)b * (K + 1) + j) * V, V);
            tok[j] = g;
            if (j < K && x[j] != g) {
                L = j;
                break;
            }
        }
        for (int j = L + 1; j <= K; ++j)
            tok[j] = -1;
        accepted_len[b] = L;
    }
    return OR_OK;
}

/*
 * Draft-token sampler: one draw per row, x_n ~ softmax(l[n,:] / T) by the inverse CDF at
 * u[n] (ascending id, strict ">"), the draft model proposing its next token ("推测性拒绝采样",
 * step 1; Speculative Contrastive Decoding review, Ma drafting gamma tokens).
 * logits [N][V] (dtype), uniforms [N].  Outputs out_tokens [N], out_probs [N] (the drawn
 * token's probability, may be NULL), margin [N] (distance of t to the nearer edge of the
 * drawn id's interval / W) and alt_token [N] (the id across that edge); both may be NULL.
 */
int oracle_sample_rows(int dtype, int N, int V, double T, const void *logits,
                       const float *uniforms, int32_t *out_tokens, double *out_probs,
                       double *margin, int32_t *alt_token)
{
    if (N < 0 || V < 1 || !(T > 0.0) || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_EINVAL;
    double *z = malloc(sizeof(double) * (size_t)V);
    double *p = malloc(sizeof(double) * (size_t)V);
    if (!z || !p) {
        free(z); free(p);
        return OR_ENOMEM;
    }
    for (int n = 0; n < N; ++n) {
        size_t off = (size_t)n * V;
        for (int v = 0; v < V; ++v)
            z[v] = logit_at(dtype, logits, off + v) / T;
        oracle_softmax(z, V, p);
        double mu;
        int alt;
        int y = inverse_cdf(p, V, (double)uniforms[n], &mu, &alt);
        out_tokens[n] = y;
        if (out_probs)
            out_probs[n] = p[y];
        if (margin)
            margin[n] = mu;
        if (alt_token)
            alt_token[n] = alt;
    }
    free(z); free(p);
    return OR_OK;
}

/*
 * Greedy blockwise verify with the next block's proposals from the same pass ("Blockwise
 * Parallel Decoding", section 3.6, Predict and Verify merged).  logits [B][K+1][H][V]: at
 * position j (the prefix followed by proposals 0..j-1) head h scores the token h places
 * after that position; head 0 is the base model.  g_j = first argmax of head 0 at position
 * j; L = first j < K with proposal_j != g_j, else K; emits g_0..g_L then -1 (as
 * oracle_run_greedy); next_proposals [B][H-1] = first argmaxes of heads 1..H-1 at position L,
 * the heads that condition on the emitted prefix.  A proposal outside [0, V) marks the
 * sequence bad (accepted_len -1, all tokens and next proposals -1).
 */
int oracle_run_greedy_heads(int dtype, int B, int K, int H, int V, const void *logits,
                            const int32_t *proposals, int32_t *accepted_len, int32_t *out_tokens,
                            int32_t *next_proposals)
{
    if (B < 0 || K < 0 || H < 1 || V < 1 || (dtype != OR_F32 && dtype != OR_BF16))
        return OR_EINVAL;
    for (int b = 0; b < B; ++b) {
        const int32_t *x = proposals + (size_t)b * K;
        int32_t *tok = out_tokens + (size_t)b * (K + 1);
        int32_t *nxt = next_proposals + (size_t)b * (H - 1);
        if (!ids_ok(x, K, V)) {
            margins_t mg;
            mark_bad(K, accepted_len + b, tok, NULL, &mg);
            for (int h = 1; h < H; ++h)
                nxt[h - 1] = -1;
            continue;
        }
        int L = K;
        for (int j = 0; j <= K; ++j) {
            size_t row = ((size_t)b * (K + 1) + j) * H;
            int g = first_argmax(dtype, logits, row * V, V);
            tok[j] = g;
            if (j < K && x[j] != g) {
                L = j;
                break;
            }
        }
        for (int j = L + 1; j <= K; ++j)
            tok[j] = -1;
        accepted_len[b] = L;
        size_t rowL = ((size_t)b * (K + 1) + L) * H;
        for (int h = 1; h < H; ++h)
            nxt[h - 1] = first_argmax(dtype, logits, (rowL + h) * V, V);
    }
    return OR_OK;
}

static int cmp_float(const void *a, const void *b)
{
    float x = *(const float *)a, y = *(const float *)b;
    return (x > y) - (x < y);
}

/*
 * Speculative Rejection's cut ("Speculative Rejection" Best-of-N page, section 4.2: score the
 * partial responses with the reward model, take the rejection threshold r_cut at the
 * alpha-quantile of the scores, keep the responses that reach it).  For each of P prompts with
 * N scores: r_cut = the (k+1)-th smallest score with k = min(floor(alpha * N), N - 1), so the
 * floor(alpha * N) lowest-scoring responses fall below it; keep[i] = (score_i >= r_cut), so
 * ties at r_cut are all kept and at least one response survives.  scores [P][N] (finite);
 * outputs r_cut [P], keep [P][N] (0/1), n_keep [P].
 */
int oracle_quantile_cut(int P, int N, double alpha, const float *scores, float *r_cut,
                        uint8_t *keep, int32_t *n_keep)
{
    if (P < 0 || N < 1 || !(alpha >= 0.0 && alpha <= 1.0))
        return OR_EINVAL;
    long k = (long)floor(alpha * (double)N);
    if (k > N - 1)
        k = N - 1;
    float *s = malloc(sizeof(float) * (size_t)N);
    if (!s)
        return OR_ENOMEM;
    for (int p = 0; p < P; ++p) {
        const float *row = scores + (size_t)p * N;
        memcpy(s, row, sizeof(float) * (size_t)N);
        qsort(s, (size_t)N, sizeof(float), cmp_float);
        float cut = s[k];
        r_cut[p] = cut;
        int32_t c = 0;
        for (int i = 0; i < N; ++i) {
            uint8_t kk = row[i] >= cut;
            keep[(size_t)p * N + i] = kk;
            c += kk;
        }
        n_keep[p] = c;
    }
    free(s);
    return OR_OK;
}
