// gfx950 kernels for the batched verify-and-accept step of speculative decoding.
//
// Data path for one sampling / contrastive call (all on the caller's stream):
//   k_stats_*      one read of every logit row: per 32 KiB chunk, the row maximum m and
//                  S = sum exp2((l - m) * log2(e)/T) (fp32 terms, fp64 across threads)
//   k_accept       one wave64 per sequence: merge chunk statistics (fp64), gather
//                  p_j(x_j), q_j(x_j), accept iff p > 0 and u * q <= p, first rejection L
//   k_resid_chunks re-read row L (target and draft, or target alone for the bonus draw):
//                  per chunk, sum of w = max(0, p - q) (or p) and of p, in fp64
//   k_draw         one workgroup per sequence: locate the chunk holding t = u_K * W, scan
//                  it (fp64 block scan), emit the first id whose prefix sum exceeds t
// Greedy blockwise calls run k_argmax (first maximum per chunk) and k_greedy_final.
//
// The operations follow the speculative rejection sampling page (steps 2-4, and the
// "key guarantee" that fixes the residual law), the blockwise parallel decoding page
// (section 3.5, Verify/Accept) and the speculative contrastive decoding review (SCD).
#include <float.h>
#include <math.h>

#include "sv_internal.h"

namespace sv {

Scale make_scale(double temperature)
{
    const double c = 1.4426950408889634074 / temperature;  // log2(e) / T
    float hi = (float)c;
    if ((double)hi > c)
        hi = nextafterf(hi, 0.0f);
    float lo = (float)(c - (double)hi);
    if (!(lo > 0.0f))
        lo = FLT_MIN;
    Scale s;
    s.hi = hi;
    s.lo = lo;
    s.c = c;
    s.inv_t = 1.0 / temperature;
    return s;
}

// ------------------------------------------------------------------ element access

template <int DT> struct Elt;

template <> struct Elt<0> {  // float32
    static constexpr int EPV = 4;
    static constexpr int BYTES = 4;
    __device__ static inline void vec(const char *p, float (&x)[4])
    {
        const uint4 v = *reinterpret_cast<const uint4 *>(p);
        x[0] = __uint_as_float(v.x);
        x[1] = __uint_as_float(v.y);
        x[2] = __uint_as_float(v.z);
        x[3] = __uint_as_float(v.w);
    }
    __device__ static inline float one(const char *base, size_t i)
    {
        return reinterpret_cast<const float *>(base)[i];
    }
};

template <> struct Elt<1> {  // bfloat16 = the upper half of a float32: widening is exact
    static constexpr int EPV = 8;
    static constexpr int BYTES = 2;
    __device__ static inline void vec(const char *p, float (&x)[8])
    {
        const uint4 v = *reinterpret_cast<const uint4 *>(p);
        x[0] = __uint_as_float(v.x << 16);
        x[1] = __uint_as_float(v.x & 0xffff0000u);
        x[2] = __uint_as_float(v.y << 16);
        x[3] = __uint_as_float(v.y & 0xffff0000u);
        x[4] = __uint_as_float(v.z << 16);
        x[5] = __uint_as_float(v.z & 0xffff0000u);
        x[6] = __uint_as_float(v.w << 16);
        x[7] = __uint_as_float(v.w & 0xffff0000u);
    }
    __device__ static inline float one(const char *base, size_t i)
    {
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(base)[i] << 16);
    }
};

__device__ inline bool aligned16(const char *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// EPV ids e0..e0+EPV-1 of a row; ids >= V read as `fill`.  One 16-byte load when the
// row is 16-byte aligned and the vector is whole, element loads otherwise.
template <int DT>
__device__ inline void load_elems(const char *row, bool aligned, int e0, int V, float fill,
                                  float (&x)[Elt<DT>::EPV])
{
    constexpr int E = Elt<DT>::EPV;
    if (aligned && e0 + E <= V) {
        Elt<DT>::vec(row + (size_t)e0 * Elt<DT>::BYTES, x);
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k)
            x[k] = (e0 + k < V) ? Elt<DT>::one(row, (size_t)(e0 + k)) : fill;
    }
}

// 2^((d) * log2(e)/T) for d <= 0 with the scale split in two floats (see Scale).
__device__ inline float exp2s(float d, float hi, float lo)
{
    float a = d * hi;
    a = __builtin_fmaf(d, lo, a);
    return __builtin_amdgcn_exp2f(a);
}

template <int E> __device__ inline float tree_sum(const float (&t)[E]);
template <> __device__ inline float tree_sum<4>(const float (&t)[4]) { return (t[0] + t[1]) + (t[2] + t[3]); }
template <> __device__ inline float tree_sum<8>(const float (&t)[8])
{
    return ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
}

// ------------------------------------------------------------------ wave64 / block reductions
// Butterfly reductions: every lane ends with the same bits (each step adds the same two
// operands in both lanes), so the results are deterministic.

__device__ inline float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

__device__ inline double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// lexicographic "better": larger value, then lower id
__device__ inline void take_better(float &v, int &i, float v2, int i2)
{
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

__device__ inline void wave_argmax(float &v, int &i)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float v2 = __shfl_xor(v, o);
        const int i2 = __shfl_xor(i, o);
        take_better(v, i, v2, i2);
    }
}

// Combine per-thread (m, s) with s relative to m into the block's (M, S), S relative to M;
// thread 0 stores them.  The rescale factors are formed in fp64.
__device__ inline void block_stats(float m, float s, double c, float *out_m, double *out_s)
{
    __shared__ float sm[WG / 64];
    __shared__ double ss[WG / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __syncthreads();  // the arrays may still be read by a previous call
    float M = wave_max(m);
    if (lane == 0)
        sm[w] = M;
    __syncthreads();
    M = fmaxf(fmaxf(sm[0], sm[1]), fmaxf(sm[2], sm[3]));
    double e = (s > 0.0f) ? (double)s * exp2(((double)m - (double)M) * c) : 0.0;
    e = wave_sum(e);
    if (lane == 0)
        ss[w] = e;
    __syncthreads();
    if (threadIdx.x == 0) {
        *out_m = M;
        *out_s = ((ss[0] + ss[1]) + ss[2]) + ss[3];
    }
}

__device__ inline void block_sum2(double a, double b, double *out_a, double *out_b)
{
    __shared__ double sa[WG / 64], sb[WG / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) {
        sa[w] = a;
        sb[w] = b;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        *out_a = ((sa[0] + sa[1]) + sa[2]) + sa[3];
        *out_b = ((sb[0] + sb[1]) + sb[2]) + sb[3];
    }
}

// exclusive prefix sum over the workgroup in thread order (fp64, fixed order)
__device__ inline double block_exclusive_scan(double v)
{
    __shared__ double wtot[WG / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    double inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double n = __shfl_up(inc, o);
        if (lane >= o)
            inc += n;
    }
    double exc = __shfl_up(inc, 1);
    if (lane == 0)
        exc = 0.0;
    if (lane == 63)
        wtot[w] = inc;
    __syncthreads();
    double off = 0.0;
    for (int k = 0; k < w; ++k)
        off += wtot[k];
    return off + exc;
}

// ------------------------------------------------------------------ K1: row statistics

// Per-thread (max, sum of exp2) over NV vectors already in registers.
template <int E>
__device__ inline void thread_stats(float (&x)[NV][E], const Scale &sc, float &m, float &s)
{
    m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < E; ++k)
            m = fmaxf(m, x[i][k]);
    const float mr = (m == -INFINITY) ? 0.0f : m;  // an all -inf thread sums exact zeros
    s = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        float t[E];
#pragma unroll
        for (int k = 0; k < E; ++k)
            t[k] = exp2s(x[i][k] - mr, sc.hi, sc.lo);
        s += tree_sum<E>(t);
    }
}

// rows b*(2K+1)+k: k <= K target row (b, k), else draft row (b, k-K-1)
template <int DT>
__global__ __launch_bounds__(WG) void k_stats_sampling(const char *__restrict__ tgt,
                                                       const char *__restrict__ drf, int K, int V,
                                                       int nch, Scale sc, float *part_m,
                                                       double *part_s)
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    const int R = 2 * K + 1;
    const int row = blockIdx.x / nch, c = blockIdx.x - row * nch;
    const int b = row / R, k = row - b * R;
    const char *rp = (k <= K) ? tgt + ((size_t)b * (K + 1) + k) * (size_t)V * BY
                              : drf + ((size_t)b * K + (k - K - 1)) * (size_t)V * BY;
    const int cbase = c * CHUNK_VECS * E;
    const bool al = aligned16(rp);
    float x[NV][E];
    if (al && cbase + CHUNK_VECS * E <= V) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            Elt<DT>::vec(rp + (size_t)(cbase + (i * WG + threadIdx.x) * E) * BY, x[i]);
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            load_elems<DT>(rp, al, cbase + (i * WG + threadIdx.x) * E, V, -INFINITY, x[i]);
    }
    float m, s;
    thread_stats<E>(x, sc, m, s);
    block_stats(m, s, sc.c, part_m + blockIdx.x, part_s + blockIdx.x);
}

// one workgroup per (row pair (b, j), chunk): target values l_e - l_a (fp32), draft values l_a
template <int DT>
__global__ __launch_bounds__(WG) void k_stats_contrastive(const char *__restrict__ ex,
                                                          const char *__restrict__ am, int K, int V,
                                                          int nch, Scale sp, Scale sq,
                                                          float *part_m, double *part_s)
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    const int P = K + 1, R = 2 * K + 1;
    const int pr = blockIdx.x / nch, c = blockIdx.x - pr * nch;
    const int b = pr / P, j = pr - b * P;
    const size_t off = ((size_t)b * P + j) * (size_t)V * BY;
    const char *re = ex + off, *ra = am + off;
    const int cbase = c * CHUNK_VECS * E;
    const bool al = aligned16(re) && aligned16(ra);
    float xd[NV][E], xa[NV][E];
    if (al && cbase + CHUNK_VECS * E <= V) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const size_t o = (size_t)(cbase + (i * WG + threadIdx.x) * E) * BY;
            Elt<DT>::vec(re + o, xd[i]);
            Elt<DT>::vec(ra + o, xa[i]);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
#pragma unroll
            for (int k = 0; k < E; ++k)
                xd[i][k] = xd[i][k] - xa[i][k];
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e0 = cbase + (i * WG + threadIdx.x) * E;
            load_elems<DT>(re, al, e0, V, -INFINITY, xd[i]);
            load_elems<DT>(ra, al, e0, V, -INFINITY, xa[i]);
#pragma unroll
            for (int k = 0; k < E; ++k)
                xd[i][k] = (e0 + k < V) ? xd[i][k] - xa[i][k] : -INFINITY;
        }
    }
    float m, s;
    thread_stats<E>(xd, sp, m, s);
    const size_t prow = (size_t)b * R + j;
    block_stats(m, s, sp.c, part_m + prow * nch + c, part_s + prow * nch + c);
    if (j < K) {  // uniform across the workgroup
        thread_stats<E>(xa, sq, m, s);
        const size_t qrow = (size_t)b * R + K + 1 + j;
        block_stats(m, s, sq.c, part_m + qrow * nch + c, part_s + qrow * nch + c);
    }
}

// ------------------------------------------------------------------ K2+K3: accept and scan

template <int DT, int MODE>
__global__ __launch_bounds__(64) void k_accept(const char *__restrict__ tgt,
                                               const char *__restrict__ drf,
                                               const int32_t *__restrict__ tokens,
                                               const float *__restrict__ unif, int K, int V,
                                               int nch, Scale sp, Scale sq,
                                               const float *__restrict__ part_m,
                                               const double *__restrict__ part_s, int32_t *acc_len,
                                               int32_t *out_tokens, float *out_probs, SeqInfo *seq)
{
    extern __shared__ double smem[];
    const int R = 2 * K + 1, b = blockIdx.x, lane = threadIdx.x;
    double *sS = smem;
    float *sM = reinterpret_cast<float *>(smem + R);
    for (int r = 0; r < R; ++r) {
        const size_t base = ((size_t)b * R + r) * nch;
        float ml = -INFINITY;
        for (int c = lane; c < nch; c += 64)
            ml = fmaxf(ml, part_m[base + c]);
        const float M = wave_max(ml);
        const double cc = (r <= K) ? sp.c : sq.c;
        double sl = 0.0;
        for (int c = lane; c < nch; c += 64) {
            const double s = part_s[base + c];
            if (s > 0.0)
                sl += s * exp2(((double)part_m[base + c] - (double)M) * cc);
        }
        const double S = wave_sum(sl);
        if (lane == 0) {
            sM[r] = M;
            sS[r] = S;
        }
    }
    __syncthreads();

    const int32_t x = (lane < K) ? tokens[(size_t)b * K + lane] : 0;
    const bool bad = (lane < K) && (x < 0 || x >= V);
    int32_t *ot = out_tokens + (size_t)b * (K + 1);
    if (__ballot(bad) != 0) {
        if (lane <= K)
            ot[lane] = -1;
        if (lane < K && out_probs) {
            out_probs[((size_t)b * K + lane) * 2] = NAN;
            out_probs[((size_t)b * K + lane) * 2 + 1] = NAN;
        }
        if (lane == 0) {
            acc_len[b] = -1;
            SeqInfo si = {};
            si.L = -1;
            seq[b] = si;
        }
        return;
    }
    bool acc = false;
    if (lane < K) {
        const size_t it = ((size_t)b * (K + 1) + lane) * (size_t)V + x;
        float lp, lq;
        if (MODE == SAMPLING) {
            lp = Elt<DT>::one(tgt, it);
            lq = Elt<DT>::one(drf, ((size_t)b * K + lane) * (size_t)V + x);
        } else {
            const float le = Elt<DT>::one(tgt, it), la = Elt<DT>::one(drf, it);
            lp = le - la;
            lq = la;
        }
        const double P = exp(((double)lp - (double)sM[lane]) * sp.inv_t) / sS[lane];
        const double Q = exp(((double)lq - (double)sM[K + 1 + lane]) * sq.inv_t) / sS[K + 1 + lane];
        if (out_probs) {
            out_probs[((size_t)b * K + lane) * 2] = (float)P;
            out_probs[((size_t)b * K + lane) * 2 + 1] = (float)Q;
        }
        acc = (P > 0.0) && ((double)unif[(size_t)b * (K + 1) + lane] * Q <= P);
    }
    const unsigned long long am = __ballot(acc);
    const int L = __builtin_ctzll(~am);  // lanes >= K never accept, so L <= K
    if (lane < L)
        ot[lane] = x;
    else if (lane > L && lane <= K)
        ot[lane] = -1;
    if (lane == 0) {
        acc_len[b] = L;
        SeqInfo si = {};
        si.L = L;
        si.Mp = sM[L];
        si.inv_sp = 1.0 / sS[L];
        if (L < K) {
            si.Mq = sM[K + 1 + L];
            si.inv_sq = 1.0 / sS[K + 1 + L];
        }
        seq[b] = si;
    }
}

// ------------------------------------------------------------------ K4: residual / bonus draw

// The rows a sequence's draw reads: the target side (sampling: target row L; contrastive:
// expert and amateur rows L) and, when L < K, the draft side (sampling: draft row L;
// contrastive: the amateur row again).
struct DrawRows {
    const char *p0, *p1, *q;
    bool resid;
    bool al;
};

template <int DT, int MODE>
__device__ inline DrawRows draw_rows(const char *tgt, const char *drf, int b, int K, int V, int L)
{
    constexpr int BY = Elt<DT>::BYTES;
    DrawRows r;
    r.resid = L < K;
    const size_t ot = ((size_t)b * (K + 1) + L) * (size_t)V * BY;
    if (MODE == SAMPLING) {
        r.p0 = tgt + ot;
        r.p1 = nullptr;
        r.q = r.resid ? drf + ((size_t)b * K + L) * (size_t)V * BY : nullptr;
        r.al = aligned16(r.p0) && (!r.resid || aligned16(r.q));
    } else {
        r.p0 = tgt + ot;
        r.p1 = drf + ot;
        r.q = r.p1;
        r.al = aligned16(r.p0) && aligned16(r.p1);
    }
    return r;
}

// target-side and draft-side values of EPV ids from e0 (ids >= V are never used)
template <int DT, int MODE>
__device__ inline void load_draw(const DrawRows &r, int e0, int V, float (&pv)[Elt<DT>::EPV],
                                 float (&qv)[Elt<DT>::EPV])
{
    constexpr int E = Elt<DT>::EPV;
    if (MODE == SAMPLING) {
        load_elems<DT>(r.p0, r.al, e0, V, 0.0f, pv);
        if (r.resid)
            load_elems<DT>(r.q, r.al, e0, V, 0.0f, qv);
    } else {
        load_elems<DT>(r.p0, r.al, e0, V, 0.0f, pv);
        load_elems<DT>(r.p1, r.al, e0, V, 0.0f, qv);
#pragma unroll
        for (int k = 0; k < E; ++k)
            pv[k] = pv[k] - qv[k];
    }
}

// Draw weights of one id: p = target probability; w = max(0, p - q) when drawing the
// replacement (L < K), w = p for the bonus draw.  Identical in k_resid_chunks and k_draw.
__device__ inline void draw_weight(float pv, float qv, bool resid, const SeqInfo &si,
                                   const Scale &sp, const Scale &sq, double &w, double &p)
{
    p = (double)exp2s(pv - si.Mp, sp.hi, sp.lo) * si.inv_sp;
    if (resid) {
        const double q = (double)exp2s(qv - si.Mq, sq.hi, sq.lo) * si.inv_sq;
        const double d = p - q;
        w = d > 0.0 ? d : 0.0;
    } else {
        w = p;
    }
}

template <int DT, int MODE>
__global__ __launch_bounds__(WG) void k_resid_chunks(const char *__restrict__ tgt,
                                                     const char *__restrict__ drf, int K, int V,
                                                     int nch, Scale sp, Scale sq,
                                                     const SeqInfo *__restrict__ seq,
                                                     double *resid)
{
    constexpr int E = Elt<DT>::EPV;
    const int b = blockIdx.x / nch, c = blockIdx.x - b * nch;
    const SeqInfo si = seq[b];
    double ws = 0.0, ps = 0.0;
    if (si.L >= 0) {
        const DrawRows r = draw_rows<DT, MODE>(tgt, drf, b, K, V, si.L);
        const int cbase = c * CHUNK_VECS * E;
        for (int i = 0; i < NV; ++i) {
            const int e0 = cbase + (i * WG + threadIdx.x) * E;
            if (e0 >= V)
                break;
            float pv[E], qv[E];
            load_draw<DT, MODE>(r, e0, V, pv, qv);
#pragma unroll
            for (int k = 0; k < E; ++k) {
                if (e0 + k < V) {
                    double w, p;
                    draw_weight(pv[k], qv[k], r.resid, si, sp, sq, w, p);
                    ws += w;
                    ps += p;
                }
            }
        }
    }
    block_sum2(ws, ps, resid + ((size_t)b * nch + c) * 2, resid + ((size_t)b * nch + c) * 2 + 1);
}

template <int DT, int MODE>
__global__ __launch_bounds__(WG) void k_draw(const char *__restrict__ tgt,
                                             const char *__restrict__ drf,
                                             const float *__restrict__ unif, int K, int V, int nch,
                                             Scale sp, Scale sq, const SeqInfo *__restrict__ seq,
                                             const double *__restrict__ resid, int32_t *out_tokens)
{
    constexpr int E = Elt<DT>::EPV;
    const int b = blockIdx.x, t = threadIdx.x;
    const SeqInfo si = seq[b];
    if (si.L < 0)
        return;  // uniform: the whole workgroup leaves
    __shared__ int s_chunk, s_which, s_fb, s_first, s_last;
    __shared__ double s_base, s_t;
    if (t == 0) {
        const double *rb = resid + (size_t)b * nch * 2;
        double W = 0.0;
        for (int c = 0; c < nch; ++c)
            W += rb[2 * c];
        const int which = (W > 0.0) ? 0 : 1;  // 1: residual empty by rounding, use p_L
        double tot = W;
        if (which) {
            tot = 0.0;
            for (int c = 0; c < nch; ++c)
                tot += rb[2 * c + 1];
        }
        const double tt = (double)unif[(size_t)b * (K + 1) + K] * tot;
        double acc = 0.0, acc_last = 0.0;
        int cs = -1, last = -1;
        for (int c = 0; c < nch; ++c) {
            const double wc = rb[2 * c + which];
            if (wc > 0.0) {
                if (acc + wc > tt) {
                    cs = c;
                    break;
                }
                last = c;
                acc_last = acc;
            }
            acc += wc;
        }
        int fb = 0;
        if (cs < 0) {  // t at or beyond the rounded total: the last id of positive weight
            cs = last;
            acc = acc_last;
            fb = 1;
        }
        s_chunk = cs;
        s_which = which;
        s_fb = fb;
        s_base = acc;
        s_t = tt;
        s_first = WG;
        s_last = -1;
    }
    __syncthreads();
    const int cs = s_chunk;
    if (cs < 0)
        return;  // no weight anywhere: outside the contract (a row without finite logits)
    const int which = s_which;
    const DrawRows r = draw_rows<DT, MODE>(tgt, drf, b, K, V, si.L);
    const int e_begin = cs * CHUNK_VECS * E + t * NV * E;  // this thread's contiguous ids

    double T = 0.0;
    for (int i = 0; i < NV; ++i) {
        const int e0 = e_begin + i * E;
        if (e0 >= V)
            break;
        float pv[E], qv[E];
        load_draw<DT, MODE>(r, e0, V, pv, qv);
#pragma unroll
        for (int k = 0; k < E; ++k) {
            if (e0 + k < V) {
                double w, p;
                draw_weight(pv[k], qv[k], r.resid, si, sp, sq, w, p);
                T += which ? p : w;
            }
        }
    }
    const double base = s_base + block_exclusive_scan(T);
    const bool pred = !s_fb && (T > 0.0) && (base + T > s_t);
    if (pred)
        atomicMin(&s_first, t);
    if (T > 0.0)
        atomicMax(&s_last, t);
    __syncthreads();
    const bool fb = (s_first == WG);
    const int owner = fb ? s_last : s_first;
    if (t == owner) {
        // Re-walk this thread's ids with the same arithmetic as T: the running sum reaches T
        // exactly, so the predicate that chose this thread holds at one of its ids.  In the
        // fallback case keep the last id of positive weight.
        double run = 0.0;
        int y = -1;
        bool done = false;
        for (int i = 0; i < NV && !done; ++i) {
            const int e0 = e_begin + i * E;
            if (e0 >= V)
                break;
            float pv[E], qv[E];
            load_draw<DT, MODE>(r, e0, V, pv, qv);
            for (int k = 0; k < E; ++k) {
                if (e0 + k >= V)
                    break;
                double w, p;
                draw_weight(pv[k], qv[k], r.resid, si, sp, sq, w, p);
                const double wv = which ? p : w;
                run += wv;
                if (wv > 0.0) {
                    y = e0 + k;
                    if (!fb && base + run > s_t) {
                        done = true;
                        break;
                    }
                }
            }
        }
        out_tokens[(size_t)b * (K + 1) + si.L] = y;
    }
}

// ------------------------------------------------------------------ K5: greedy blockwise

template <int DT>
__global__ __launch_bounds__(WG) void k_argmax(const char *__restrict__ tgt, int V, int nch,
                                               float *part_v, int *part_i)
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    const int row = blockIdx.x / nch, c = blockIdx.x - row * nch;
    const char *rp = tgt + (size_t)row * (size_t)V * BY;
    const int cbase = c * CHUNK_VECS * E;
    const bool al = aligned16(rp);
    float x[NV][E];
    if (al && cbase + CHUNK_VECS * E <= V) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            Elt<DT>::vec(rp + (size_t)(cbase + (i * WG + threadIdx.x) * E) * BY, x[i]);
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            load_elems<DT>(rp, al, cbase + (i * WG + threadIdx.x) * E, V, -INFINITY, x[i]);
    }
    // this thread's ids ascend with (i, k); start from its first id so that an all -inf
    // run still reports the lowest id
    const int first = cbase + threadIdx.x * E;
    float bv = -INFINITY;
    int bi = (first < V) ? first : INT_MAX;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < E; ++k)
            if (x[i][k] > bv) {
                bv = x[i][k];
                bi = cbase + (i * WG + threadIdx.x) * E + k;
            }
    wave_argmax(bv, bi);
    __shared__ float sv[WG / 64];
    __shared__ int si[WG / 64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) {
        sv[w] = bv;
        si[w] = bi;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float v = sv[0];
        int id = si[0];
        for (int k = 1; k < WG / 64; ++k)
            take_better(v, id, sv[k], si[k]);
        part_v[blockIdx.x] = v;
        part_i[blockIdx.x] = id;
    }
}

__global__ __launch_bounds__(64) void k_greedy_final(const int32_t *__restrict__ props, int K,
                                                     int V, int nch,
                                                     const float *__restrict__ part_v,
                                                     const int *__restrict__ part_i,
                                                     int32_t *acc_len, int32_t *out_tokens)
{
    extern __shared__ int sg[];
    const int b = blockIdx.x, lane = threadIdx.x;
    for (int j = 0; j <= K; ++j) {
        const size_t base = ((size_t)b * (K + 1) + j) * nch;
        float v = -INFINITY;
        int id = INT_MAX;
        for (int c = lane; c < nch; c += 64)
            take_better(v, id, part_v[base + c], part_i[base + c]);
        wave_argmax(v, id);
        if (lane == 0)
            sg[j] = id;
    }
    __syncthreads();
    const int32_t x = (lane < K) ? props[(size_t)b * K + lane] : 0;
    const bool bad = (lane < K) && (x < 0 || x >= V);
    int32_t *ot = out_tokens + (size_t)b * (K + 1);
    if (__ballot(bad) != 0) {
        if (lane <= K)
            ot[lane] = -1;
        if (lane == 0)
            acc_len[b] = -1;
        return;
    }
    const unsigned long long mm = __ballot(lane < K && x != sg[lane]);
    const int L = mm ? __builtin_ctzll(mm) : K;
    if (lane <= K)
        ot[lane] = (lane <= L) ? sg[lane] : -1;
    if (lane == 0)
        acc_len[b] = L;
}

// ------------------------------------------------------------------ launchers

namespace {

struct Timer {
    const Launch &ln;
    int kind;
    Timer(const Launch &l, int k) : ln(l), kind(k)
    {
        if (ln.ev)
            hipEventRecord(ln.ev[2 * kind], ln.stream);
    }
    ~Timer()
    {
        if (ln.ev)
            hipEventRecord(ln.ev[2 * kind + 1], ln.stream);
    }
};

template <int DT, int MODE>
hipError_t sampling_impl(const Launch &ln, const Workspace &ws, int B, int K, int V,
                         const Scale &sp, const Scale &sq, const void *tgt, const void *drf,
                         const int32_t *tokens, const float *unif, int32_t *acc_len,
                         int32_t *out_tokens, float *out_probs)
{
    const int nch = num_chunks(DT, V);
    const char *t = static_cast<const char *>(tgt);
    const char *d = static_cast<const char *>(drf);
    {
        Timer tm(ln, 0);
        if (MODE == SAMPLING) {
            const unsigned grid = (unsigned)((size_t)B * (2 * K + 1) * nch);
            hipLaunchKernelGGL(k_stats_sampling<DT>, dim3(grid), dim3(WG), 0, ln.stream, t, d, K,
                               V, nch, sp, ws.part_m, ws.part_s);
        } else {
            const unsigned grid = (unsigned)((size_t)B * (K + 1) * nch);
            hipLaunchKernelGGL(k_stats_contrastive<DT>, dim3(grid), dim3(WG), 0, ln.stream, t, d,
                               K, V, nch, sp, sq, ws.part_m, ws.part_s);
        }
    }
    {
        Timer tm(ln, 1);
        const size_t lds = (size_t)(2 * K + 1) * (sizeof(double) + sizeof(float));
        hipLaunchKernelGGL((k_accept<DT, MODE>), dim3(B), dim3(64), lds, ln.stream, t, d, tokens,
                           unif, K, V, nch, sp, sq, ws.part_m, ws.part_s, acc_len, out_tokens,
                           out_probs, ws.seq);
    }
    {
        Timer tm(ln, 2);
        hipLaunchKernelGGL((k_resid_chunks<DT, MODE>), dim3((unsigned)((size_t)B * nch)), dim3(WG),
                           0, ln.stream, t, d, K, V, nch, sp, sq, ws.seq, ws.resid);
    }
    {
        Timer tm(ln, 3);
        hipLaunchKernelGGL((k_draw<DT, MODE>), dim3(B), dim3(WG), 0, ln.stream, t, d, unif, K, V,
                           nch, sp, sq, ws.seq, ws.resid, out_tokens);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t greedy_impl(const Launch &ln, const Workspace &ws, int B, int K, int V, const void *tgt,
                       const int32_t *props, int32_t *acc_len, int32_t *out_tokens)
{
    const int nch = num_chunks(DT, V);
    {
        Timer tm(ln, 4);
        const unsigned grid = (unsigned)((size_t)B * (K + 1) * nch);
        hipLaunchKernelGGL(k_argmax<DT>, dim3(grid), dim3(WG), 0, ln.stream,
                           static_cast<const char *>(tgt), V, nch, ws.part_m, ws.part_i);
    }
    {
        Timer tm(ln, 5);
        hipLaunchKernelGGL(k_greedy_final, dim3(B), dim3(64), (size_t)(K + 1) * sizeof(int),
                           ln.stream, props, K, V, nch, ws.part_m, ws.part_i, acc_len, out_tokens);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sampling(const Launch &ln, const Workspace &ws, int mode, int dtype, int B,
                           int K, int V, const Scale &sp, const Scale &sq, const void *tgt,
                           const void *drf, const int32_t *tokens, const float *unif,
                           int32_t *acc_len, int32_t *out_tokens, float *out_probs)
{
    if (mode == SAMPLING)
        return dtype == 1 ? sampling_impl<1, SAMPLING>(ln, ws, B, K, V, sp, sq, tgt, drf, tokens,
                                                       unif, acc_len, out_tokens, out_probs)
                          : sampling_impl<0, SAMPLING>(ln, ws, B, K, V, sp, sq, tgt, drf, tokens,
                                                       unif, acc_len, out_tokens, out_probs);
    return dtype == 1 ? sampling_impl<1, CONTRASTIVE>(ln, ws, B, K, V, sp, sq, tgt, drf, tokens,
                                                      unif, acc_len, out_tokens, out_probs)
                      : sampling_impl<0, CONTRASTIVE>(ln, ws, B, K, V, sp, sq, tgt, drf, tokens,
                                                      unif, acc_len, out_tokens, out_probs);
}

hipError_t launch_greedy(const Launch &ln, const Workspace &ws, int dtype, int B, int K, int V,
                         const void *tgt, const int32_t *props, int32_t *acc_len,
                         int32_t *out_tokens)
{
    return dtype == 1 ? greedy_impl<1>(ln, ws, B, K, V, tgt, props, acc_len, out_tokens)
                      : greedy_impl<0>(ln, ws, B, K, V, tgt, props, acc_len, out_tokens);
}

}  // namespace sv
