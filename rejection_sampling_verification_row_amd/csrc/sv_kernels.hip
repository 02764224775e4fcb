// gfx950 kernels for the batched verify-and-accept step of speculative decoding.
//
// A sampling or contrastive call is four launches on the caller's stream:
//   k_stats_*  one read of every logit row (nontemporal 128-bit loads).  Each 256-thread
//              workgroup reduces one chunk of a row to per-wave (max, sum exp2) partials.
//   k_accept   one workgroup per sequence merges its partials in fp64, gathers
//              p_j(x_j), q_j(x_j), accepts iff p > 0 and u * q <= p, finds the first
//              rejection L and records row L.
//   k_resid    re-read of row L (target and draft, or the target alone for the bonus
//              draw): per chunk, the sum of w = max(0, p - q) (or p).
//   k_draw     one workgroup per sequence finds the chunk holding t = u_K * W, then the
//              vector and the id inside it (block scans), and emits the first id whose
//              prefix weight exceeds t.
// A greedy blockwise call is two launches: k_argmax reduces chunks to (max, first id) and
// k_greedy_final compares each sequence's row argmaxes with its proposals.
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

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load that streams past the caches (logits are read once per pass)
__device__ inline uint4 load_stream(const char *p)
{
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ inline uint4 load_plain(const char *p) { return *reinterpret_cast<const uint4 *>(p); }

template <int DT> struct Elt;

template <> struct Elt<0> {  // float32
    static constexpr int EPV = 4;
    static constexpr int BYTES = 4;
    __device__ static inline void unpack(const uint4 v, float (&x)[4])
    {
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
    __device__ static inline void unpack(const uint4 v, float (&x)[8])
    {
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
        Elt<DT>::unpack(load_plain(row + (size_t)e0 * Elt<DT>::BYTES), x);
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k)
            x[k] = (e0 + k < V) ? Elt<DT>::one(row, (size_t)(e0 + k)) : fill;
    }
}

// 2^(d * log2(e)/T) for d <= 0 with the scale split in two floats (see Scale).
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

__device__ inline float wave_sum_f(float v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

__device__ inline double wave_sum(double v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// inclusive prefix sum over the wave's lanes (fixed order)
__device__ inline double wave_incl_scan(double v, int lane)
{
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const double n = __shfl_up(v, o);
        if (lane >= o)
            v += n;
    }
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

// exclusive prefix sum over the workgroup in thread order (fp64, fixed order)
__device__ inline double block_exclusive_scan(double v)
{
    __shared__ double wtot[WAVES];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const double inc = wave_incl_scan(v, lane);
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

// ------------------------------------------------------------------ row statistics

// Per-thread (max, sum of exp2 relative to that max) over NV vectors in registers.
// Each exponent argument is formed as fma(x, lo, fma(x, hi, -R)) with R = fl(m * hi): one
// rounding of a value of the argument's own size, like (x - m) * c, but two instructions.
// Every argument carries the same shift e = m * lo + (m * hi - R) (the second term exact
// through fma), which is removed once from the thread's sum.  Needs |x * log2(e)/T| below
// the float range.
template <int E, int NV>
__device__ inline void thread_stats(float (&x)[NV][E], const Scale &sc, float &m, float &s)
{
    m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
        for (int k = 0; k < E; ++k)
            m = fmaxf(m, x[i][k]);
    const float mr = (m == -INFINITY) ? 0.0f : m;  // an all -inf thread sums exact zeros
    const float R = mr * sc.hi;
    const float shift = __builtin_fmaf(mr, sc.lo, __builtin_fmaf(mr, sc.hi, -R));
    s = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        float t[E];
#pragma unroll
        for (int k = 0; k < E; ++k)
            t[k] = __builtin_amdgcn_exp2f(
                __builtin_fmaf(x[i][k], sc.lo, __builtin_fmaf(x[i][k], sc.hi, -R)));
        s += tree_sum<E>(t);
    }
    s *= __builtin_amdgcn_exp2f(-shift);
}

// per-wave (M, S): S = sum over lanes of s * exp2((m - M) * log2(e)/T)
__device__ inline float2 wave_stats(float m, float s, const Scale &sc)
{
    const float M = wave_max(m);
    const float e = (s > 0.0f) ? s * exp2s(m - M, sc.hi, sc.lo) : 0.0f;
    return make_float2(M, wave_sum_f(e));
}

// Store the workgroup's four per-wave partials from one thread after a barrier: a single
// 32-byte write per workgroup streams better than four single-lane writes from the waves.
__device__ inline void store_wave_partials(float2 v, float2 *dst)
{
    __shared__ float4 sp[WAVES / 2];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0)
        reinterpret_cast<float2 *>(sp)[w] = v;
    __syncthreads();
    if (threadIdx.x == 0) {
        float4 *d = reinterpret_cast<float4 *>(dst);
        d[0] = sp[0];
        d[1] = sp[1];
    }
}

// Load NV vectors per thread of chunk `cbase` of a row: streamed 16-byte loads when the
// whole chunk is inside an aligned row, element loads (ids >= V as -inf) otherwise.
template <int DT, int NV>
__device__ inline void load_chunk(const char *rp, bool al, int cbase, int V,
                                  float (&x)[NV][Elt<DT>::EPV])
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    if (al && cbase + WG * NV * E <= V) {
        uint4 raw[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i)
            raw[i] = load_stream(rp + (size_t)(cbase + (i * WG + threadIdx.x) * E) * BY);
#pragma unroll
        for (int i = 0; i < NV; ++i)
            Elt<DT>::unpack(raw[i], x[i]);
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            load_elems<DT>(rp, al, cbase + (i * WG + threadIdx.x) * E, V, -INFINITY, x[i]);
    }
}

// Sequence b after its rows' statistics: merge the per-wave partials of its 2K+1 rows (fp64),
// then wave 0 runs the accept tests and the first-rejection scan, one lane per draft
// position, and records what the residual pass needs.  The draft tokens and their logits
// are fetched first and the sequence's partials are staged in LDS in one coalesced pass,
// so the merge waits on memory once.
constexpr int ACCEPT_STAGE = 4096;  // partials staged in LDS (32 KiB), else read in place

template <int DT, int MODE>
__device__ __forceinline__ void accept_block(const char *tgt, const char *drf, const int32_t *tokens,
                             const float *unif, int b, int K, int V, int nch, const Scale &sp,
                             const Scale &sq, const float2 *part, int32_t *acc_len,
                             int32_t *out_tokens, float *out_probs, SeqInfo *seq)
{
    __shared__ float sM[MAX_ROWS];
    __shared__ double sS[MAX_ROWS];
    __shared__ float2 stage[ACCEPT_STAGE];
    const int R = 2 * K + 1, np = nch * WAVES, total = R * np;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;

    int32_t x = 0;
    float lp = 0.0f, lq = 0.0f, u = 0.0f;
    bool bad = false;
    if (w == 0 && lane < K) {
        x = tokens[(size_t)b * K + lane];
        u = unif[(size_t)b * (K + 1) + lane];
        bad = (x < 0 || x >= V);
        if (!bad) {
            const size_t it = ((size_t)b * (K + 1) + lane) * (size_t)V + x;
            if (MODE == SAMPLING) {
                lp = Elt<DT>::one(tgt, it);
                lq = Elt<DT>::one(drf, ((size_t)b * K + lane) * (size_t)V + x);
            } else {
                const float le = Elt<DT>::one(tgt, it), la = Elt<DT>::one(drf, it);
                lp = le - la;
                lq = la;
            }
        }
    }

    const float2 *pb = part + (size_t)b * total;
    const bool staged = total <= ACCEPT_STAGE;
    if (staged) {
        for (int i0 = 0; i0 < total; i0 += 4 * WG) {
            float2 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + k * WG + t;
                v[k] = (i < total) ? pb[i] : make_float2(0.0f, 0.0f);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + k * WG + t;
                if (i < total)
                    stage[i] = v[k];
            }
        }
        __syncthreads();
    }
    for (int r = w; r < R; r += WAVES) {
        const int r0 = r * np;
        const double cc = (r <= K) ? sp.c : sq.c;
        float ml = -INFINITY;
        for (int i = lane; i < np; i += 64)
            ml = fmaxf(ml, (staged ? stage[r0 + i] : pb[r0 + i]).x);
        const float M = wave_max(ml);
        double sl = 0.0;
        for (int i = lane; i < np; i += 64) {
            const float2 v = staged ? stage[r0 + i] : pb[r0 + i];
            if (v.y > 0.0f)
                sl += (double)v.y * exp2(((double)v.x - (double)M) * cc);
        }
        const double S = wave_sum(sl);
        if (lane == 0) {
            sM[r] = M;
            sS[r] = S;
        }
    }
    __syncthreads();
    if (w != 0)
        return;

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
        const double P = exp(((double)lp - (double)sM[lane]) * sp.inv_t) / sS[lane];
        const double Q = exp(((double)lq - (double)sM[K + 1 + lane]) * sq.inv_t) / sS[K + 1 + lane];
        if (out_probs) {
            out_probs[((size_t)b * K + lane) * 2] = (float)P;
            out_probs[((size_t)b * K + lane) * 2 + 1] = (float)Q;
        }
        acc = (P > 0.0) && ((double)u * Q <= P);
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
        si.isp = (float)(1.0 / sS[L]);
        if (L < K) {
            si.Mq = sM[K + 1 + L];
            si.isq = (float)(1.0 / sS[K + 1 + L]);
        }
        seq[b] = si;
    }
}

// rows b*(2K+1)+k: k <= K target row (b, k), else draft row (b, k-K-1); each wave stores its
// (max, sum) partial at part[blockIdx.x * WAVES + wave]
template <int DT>
__global__ __launch_bounds__(WG) void k_stats_sampling(const char *__restrict__ tgt,
                                                       const char *__restrict__ drf, int K, int V,
                                                       int nch, Scale sc, float2 *part)
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    const int R = 2 * K + 1;
    const int row = blockIdx.x / nch, c = blockIdx.x - row * nch;
    const int b = row / R, k = row - b * R;
    const char *rp = (k <= K) ? tgt + ((size_t)b * (K + 1) + k) * (size_t)V * BY
                              : drf + ((size_t)b * K + (k - K - 1)) * (size_t)V * BY;
    float x[NV_STATS][E];
    load_chunk<DT, NV_STATS>(rp, aligned16(rp), c * WG * NV_STATS * E, V, x);
    float m, s;
    thread_stats<E, NV_STATS>(x, sc, m, s);
    store_wave_partials(wave_stats(m, s, sc), part + (size_t)blockIdx.x * WAVES);
}

// one workgroup per (row pair (b, j), chunk): target values l_e - l_a (fp32), draft values l_a
template <int DT>
__global__ __launch_bounds__(WG) void k_stats_contrastive(const char *__restrict__ ex,
                                                          const char *__restrict__ am, int K, int V,
                                                          int nch, Scale sp, Scale sq, float2 *part)
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    const int P = K + 1, R = 2 * K + 1;
    const int pr = blockIdx.x / nch, c = blockIdx.x - pr * nch;
    const int b = pr / P, j = pr - b * P;
    const size_t off = ((size_t)b * P + j) * (size_t)V * BY;
    const char *re = ex + off, *ra = am + off;
    const int cbase = c * WG * NV_PAIR * E;
    const bool al = aligned16(re) && aligned16(ra);
    float xd[NV_PAIR][E], xa[NV_PAIR][E];
    load_chunk<DT, NV_PAIR>(re, al, cbase, V, xd);
    load_chunk<DT, NV_PAIR>(ra, al, cbase, V, xa);
    if (cbase + WG * NV_PAIR * E <= V) {
#pragma unroll
        for (int i = 0; i < NV_PAIR; ++i)
#pragma unroll
            for (int k = 0; k < E; ++k)
                xd[i][k] = xd[i][k] - xa[i][k];
    } else {  // ids past V are -inf on both sides: keep the difference at -inf
#pragma unroll
        for (int i = 0; i < NV_PAIR; ++i)
#pragma unroll
            for (int k = 0; k < E; ++k) {
                const int id = cbase + (i * WG + threadIdx.x) * E + k;
                xd[i][k] = (id < V) ? xd[i][k] - xa[i][k] : -INFINITY;
            }
    }
    float m, s;
    thread_stats<E, NV_PAIR>(xd, sp, m, s);
    store_wave_partials(wave_stats(m, s, sp), part + (((size_t)b * R + j) * nch + c) * WAVES);
    if (j < K) {  // uniform across the workgroup
        thread_stats<E, NV_PAIR>(xa, sq, m, s);
        __syncthreads();  // the LDS staging of the first store is free again
        store_wave_partials(wave_stats(m, s, sq),
                            part + (((size_t)b * R + K + 1 + j) * nch + c) * WAVES);
    }
}

// one workgroup per sequence
template <int DT, int MODE>
__global__ __launch_bounds__(WG) void k_accept(const char *__restrict__ tgt,
                                               const char *__restrict__ drf,
                                               const int32_t *__restrict__ tokens,
                                               const float *__restrict__ unif, int K, int V,
                                               int nch, Scale sp, Scale sq,
                                               const float2 *__restrict__ part, int32_t *acc_len,
                                               int32_t *out_tokens, float *out_probs, SeqInfo *seq)
{
    accept_block<DT, MODE>(tgt, drf, tokens, unif, blockIdx.x, K, V, nch, sp, sq, part, acc_len,
                           out_tokens, out_probs, seq);
}

// ------------------------------------------------------------------ residual / bonus draw

// The rows a sequence's draw reads: the target side (sampling: target row L; contrastive:
// expert and amateur rows L) and, when L < K, the draft side (sampling: draft row L;
// contrastive: the amateur row again).
struct DrawRows {
    const char *p0;   // target row L (sampling) or expert row L (contrastive)
    const char *p1;   // draft row L (sampling, L < K only) or amateur row L (contrastive)
    bool two;         // p1 is read
    bool resid;       // L < K: w = max(0, p - q); else w = p
    bool al;          // every row read is 16-byte aligned
};

template <int DT, int MODE>
__device__ inline DrawRows draw_rows(const char *tgt, const char *drf, int b, int K, int V, int L)
{
    constexpr int BY = Elt<DT>::BYTES;
    DrawRows r;
    r.resid = L < K;
    r.p0 = tgt + ((size_t)b * (K + 1) + L) * (size_t)V * BY;
    if (MODE == SAMPLING) {
        r.two = r.resid;
        r.p1 = r.resid ? drf + ((size_t)b * K + L) * (size_t)V * BY : nullptr;
    } else {
        r.two = true;
        r.p1 = drf + ((size_t)b * (K + 1) + L) * (size_t)V * BY;
    }
    r.al = aligned16(r.p0) && (!r.two || aligned16(r.p1));
    return r;
}

// Draw weight of one id from its target-side value pv and draft-side value qv (fp32):
// p = 2^((pv - Mp) log2(e)/T) / S_p; w = max(0, p - q) for a replacement, p for the bonus
// (or when `target_law` asks for p).  The same instructions run in k_resid and in the
// search, so both see identical weights.
__device__ inline float draw_weight(float pv, float qv, bool resid, bool target_law,
                                    const SeqInfo &si, const Scale &sp, const Scale &sq)
{
    const float p = exp2s(pv - si.Mp, sp.hi, sp.lo) * si.isp;
    if (!resid || target_law)
        return p;
    const float q = exp2s(qv - si.Mq, sq.hi, sq.lo) * si.isq;
    return fmaxf(p - q, 0.0f);
}

// Weights of the EPV ids from e0 (ids >= V weigh 0), element by element: the path for
// chunks that touch the end of a row or rows that are not 16-byte aligned.
template <int DT, int MODE>
__device__ inline void vec_weights_masked(const DrawRows &r, int e0, int V, bool target_law,
                                          const SeqInfo &si, const Scale &sp, const Scale &sq,
                                          float (&wv)[Elt<DT>::EPV])
{
    constexpr int E = Elt<DT>::EPV;
    float pv[E], qv[E];
    load_elems<DT>(r.p0, r.al, e0, V, 0.0f, pv);
    if (r.two)
        load_elems<DT>(r.p1, r.al, e0, V, 0.0f, qv);
#pragma unroll
    for (int k = 0; k < E; ++k) {
        if (MODE == CONTRASTIVE)
            pv[k] = pv[k] - qv[k];
        wv[k] = (e0 + k < V) ? draw_weight(pv[k], qv[k], r.resid, target_law, si, sp, sq) : 0.0f;
    }
}

// Weights of one whole 16-byte vector from its raw words.
template <int DT, int MODE>
__device__ inline void raw_weights(const DrawRows &r, const uint4 &a, const uint4 &q,
                                   bool target_law, const SeqInfo &si, const Scale &sp,
                                   const Scale &sq, float (&wv)[Elt<DT>::EPV])
{
    constexpr int E = Elt<DT>::EPV;
    float pv[E], qv[E];
    Elt<DT>::unpack(a, pv);
    if (r.two)
        Elt<DT>::unpack(q, qv);
#pragma unroll
    for (int k = 0; k < E; ++k) {
        if (MODE == CONTRASTIVE)
            pv[k] = pv[k] - qv[k];
        wv[k] = draw_weight(pv[k], qv[k], r.resid, target_law, si, sp, sq);
    }
}

// NV_RESID vectors of this thread from ids e0(i) = base + i * WG * E (the coalesced pattern
// of one chunk), both rows, all loads issued before any arithmetic.  Returns false (nothing
// loaded) when some vector is not whole or the rows are not aligned; the caller then takes
// the element path.
template <int DT, bool NT>
__device__ inline bool load_draw_vectors(const DrawRows &r, int base, int V,
                                         uint4 (&a)[NV_RESID], uint4 (&q)[NV_RESID])
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES, STRIDE = WG * Elt<DT>::EPV;
    if (!r.al || base + (NV_RESID - 1) * STRIDE + E > V)
        return false;
#pragma unroll
    for (int i = 0; i < NV_RESID; ++i) {
        const size_t o = (size_t)(base + i * STRIDE) * BY;
        a[i] = NT ? load_stream(r.p0 + o) : load_plain(r.p0 + o);
    }
    if (r.two)
#pragma unroll
        for (int i = 0; i < NV_RESID; ++i) {
            const size_t o = (size_t)(base + i * STRIDE) * BY;
            q[i] = NT ? load_stream(r.p1 + o) : load_plain(r.p1 + o);
        }
    return true;
}

// This thread's draw-weight sums over chunk c, one per vector i (fp32 tree over the
// vector's ids); vector i covers ids c*CE + (i*WG + t)*E + [0, E).  The same instructions
// run in k_resid (which sums them) and in k_draw (which searches them), so both see the
// same weights.
template <int DT, int MODE, bool NT>
__device__ inline void thread_vector_weights(const DrawRows &r, int c, int V, bool target_law,
                                             const SeqInfo &si, const Scale &sp, const Scale &sq,
                                             float (&vs)[NV_RESID], uint4 (&a)[NV_RESID],
                                             uint4 (&q)[NV_RESID], bool &whole)
{
    constexpr int E = Elt<DT>::EPV;
    const int base = c * WG * NV_RESID * E + threadIdx.x * E;
    whole = load_draw_vectors<DT, NT>(r, base, V, a, q);
#pragma unroll
    for (int i = 0; i < NV_RESID; ++i) {
        const int e0 = base + i * WG * E;
        float wv[E];
        if (whole) {
            raw_weights<DT, MODE>(r, a[i], q[i], target_law, si, sp, sq, wv);
            vs[i] = tree_sum<E>(wv);
        } else if (e0 < V) {
            vec_weights_masked<DT, MODE>(r, e0, V, target_law, si, sp, sq, wv);
            vs[i] = tree_sum<E>(wv);
        } else {
            vs[i] = 0.0f;
        }
    }
}

// Per chunk c of row L, the totals of its NV_RESID vector rows: unit (c, i) covers the
// contiguous ids c*CE + i*WG*E + [0, WG*E) and its weight sum goes to
// resid[(b * nch + c) * NV_RESID + i] (per-thread fp32 vector sums, fp64 above them).
template <int DT, int MODE>
__global__ __launch_bounds__(WG) void k_resid(const char *__restrict__ tgt,
                                              const char *__restrict__ drf, int K, int V, int nch,
                                              Scale sp, Scale sq, const SeqInfo *__restrict__ seq,
                                              double *resid)
{
    __shared__ double s_units[NV_RESID][WAVES];
    const int b = blockIdx.x / nch, c = blockIdx.x - b * nch;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const SeqInfo si = seq[b];
    if (si.L < 0)
        return;
    const DrawRows r = draw_rows<DT, MODE>(tgt, drf, b, K, V, si.L);
    float vs[NV_RESID];
    uint4 a[NV_RESID], q[NV_RESID];
    bool whole;
    thread_vector_weights<DT, MODE, true>(r, c, V, false, si, sp, sq, vs, a, q, whole);
#pragma unroll
    for (int i = 0; i < NV_RESID; ++i) {
        const double us = wave_sum((double)vs[i]);
        if (lane == 0)
            s_units[i][w] = us;
    }
    __syncthreads();
    if (threadIdx.x < NV_RESID) {
        const int i = threadIdx.x;
        resid[(size_t)blockIdx.x * NV_RESID + i] =
            ((s_units[i][0] + s_units[i][1]) + s_units[i][2]) + s_units[i][3];
    }
}

// Among `nu` units with totals unit(u) (ascending ids), wave 0 finds the first unit whose
// running total exceeds tt = u01 * W (W = the sum of all units, fixed order), or if rounding
// leaves t at or past the last one, the last unit of positive weight (*fb = 1).  Returns the
// unit (or -1 when every unit weighs 0) and writes its starting weight *base and tt.
template <typename F>
__device__ inline int find_unit(F unit, int nu, float u01, double *base, double *tt, int *fb)
{
    const int lane = threadIdx.x & 63;
    double W = 0.0;
    for (int s0 = 0; s0 < nu; s0 += 64)
        W += wave_sum((s0 + lane < nu) ? unit(s0 + lane) : 0.0);
    *tt = (double)u01 * W;
    double run = 0.0, found_base = 0.0, last_base = 0.0;
    int us = -1, last = -1;
    for (int s0 = 0; s0 < nu && us < 0; s0 += 64) {
        const double wu = (s0 + lane < nu) ? unit(s0 + lane) : 0.0;
        const double inc = wave_incl_scan(wu, lane);
        double exc = __shfl_up(inc, 1);
        if (lane == 0)
            exc = 0.0;
        const unsigned long long hit = __ballot(W > 0.0 && wu > 0.0 && run + inc > *tt);
        const unsigned long long pos = __ballot(wu > 0.0);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            us = s0 + l;
            found_base = run + __shfl(exc, l);
        } else if (pos) {
            const int l = 63 - __builtin_clzll(pos);
            last = s0 + l;
            last_base = run + __shfl(exc, l);
        }
        run += __shfl(inc, 63);
    }
    *fb = (us < 0);
    *base = (us >= 0) ? found_base : last_base;
    return (us >= 0) ? us : last;
}

// Inside unit (c, i): thread t weighs vector i*WG + t of chunk c (the same instructions as
// k_resid), a block scan of the vector sums finds the vector, and its owner emits the first
// id whose running weight exceeds tt (fb: the last id of positive weight).
template <int DT, int MODE>
__device__ __forceinline__ void search_unit(const DrawRows &r, const SeqInfo &si, int V, int unit,
                                            double base, double tt, bool fb, bool target_law,
                                            const Scale &sp, const Scale &sq, int32_t *out)
{
    constexpr int E = Elt<DT>::EPV;
    __shared__ int s_first, s_last;
    const int t = threadIdx.x;
    const int c = unit / NV_RESID, i = unit - c * NV_RESID;
    const int e0 = c * WG * NV_RESID * E + (i * WG + t) * E;
    float wv[E];
    if (e0 < V) {
        vec_weights_masked<DT, MODE>(r, e0, V, target_law, si, sp, sq, wv);
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k)
            wv[k] = 0.0f;
    }
    const float vsum = tree_sum<E>(wv);
    if (t == 0) {
        s_first = WG;
        s_last = -1;
    }
    const double bt = base + block_exclusive_scan((double)vsum);  // has a barrier
    if (!fb && vsum > 0.0f && bt + (double)vsum > tt)
        atomicMin(&s_first, t);
    if (vsum > 0.0f)
        atomicMax(&s_last, t);
    __syncthreads();
    const bool fb2 = fb || s_first == WG;
    if (t != (fb2 ? s_last : s_first))
        return;
    double run = bt;
    int y = -1, lastpos = -1;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        if (wv[k] > 0.0f) {
            run += (double)wv[k];
            lastpos = e0 + k;
            if (!fb2 && y < 0 && run > tt)
                y = e0 + k;
        }
    }
    // rounding may put t past this vector's ids: then its last id of positive weight
    *out = (y >= 0) ? y : lastpos;
}

// One workgroup per sequence: the unit holding t = u_K * W (from k_resid's unit totals),
// then the id inside it.  If rounding left the residual empty, draw from the target law p_L
// instead: its unit totals are computed here (essentially never taken).
template <int DT, int MODE>
__global__ __launch_bounds__(WG) void k_draw(const char *__restrict__ tgt,
                                             const char *__restrict__ drf,
                                             const float *__restrict__ unif, int K, int V, int nch,
                                             Scale sp, Scale sq, const SeqInfo *__restrict__ seq,
                                             const double *__restrict__ resid,
                                             int32_t *out_tokens)
{
    __shared__ int s_unit, s_fb;
    __shared__ double s_base, s_t;
    __shared__ double s_units[NV_RESID][WAVES];
    const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int nu = nch * NV_RESID;
    const double *ub = resid + (size_t)b * nu;
    const SeqInfo si = seq[b];
    if (si.L < 0)
        return;
    const float u01 = unif[(size_t)b * (K + 1) + K];
    int32_t *out = out_tokens + (size_t)b * (K + 1) + si.L;
    const DrawRows r = draw_rows<DT, MODE>(tgt, drf, b, K, V, si.L);
    if (t < 64) {
        double base, tt;
        int fb;
        const int us = find_unit([&](int k) { return ub[k]; }, nu, u01, &base, &tt, &fb);
        if (lane == 0) {
            s_unit = us;
            s_base = base;
            s_t = tt;
            s_fb = fb;
        }
    }
    __syncthreads();
    bool target_law = false;
    if (s_unit < 0) {
        // The residual is empty by rounding: draw from the target law p_L.  Its unit totals
        // are computed here chunk by chunk, twice (the total, then the scan), in LDS only.
        target_law = true;
        double run = 0.0, tt = 0.0, last_base = 0.0;
        int found = -1, last = -1;
        for (int pass = 0; pass < 2 && found < 0; ++pass) {
            run = 0.0;
            for (int c = 0; c < nch && found < 0; ++c) {
                float vs[NV_RESID];
                uint4 a[NV_RESID], q[NV_RESID];
                bool whole;
                thread_vector_weights<DT, MODE, false>(r, c, V, true, si, sp, sq, vs, a, q, whole);
                __syncthreads();  // s_units of the previous chunk have been read
#pragma unroll
                for (int i = 0; i < NV_RESID; ++i) {
                    const double v = wave_sum((double)vs[i]);
                    if (lane == 0)
                        s_units[i][w] = v;
                }
                __syncthreads();
                for (int i = 0; i < NV_RESID && found < 0; ++i) {  // every thread, same order
                    const double ui =
                        ((s_units[i][0] + s_units[i][1]) + s_units[i][2]) + s_units[i][3];
                    if (pass == 1 && ui > 0.0) {
                        if (run + ui > tt) {
                            found = c * NV_RESID + i;
                        } else {
                            last = c * NV_RESID + i;
                            last_base = run;
                        }
                    }
                    if (found < 0)
                        run += ui;
                }
            }
            if (pass == 0)
                tt = (double)u01 * run;
        }
        const int us = (found >= 0) ? found : last;
        if (us < 0) {
            if (t == 0)
                *out = -1;  // a row without finite logits: outside the contract
            return;
        }
        search_unit<DT, MODE>(r, si, V, us, (found >= 0) ? run : last_base, tt, found < 0, true,
                              sp, sq, out);
        return;
    }
    search_unit<DT, MODE>(r, si, V, s_unit, s_base, s_t, s_fb != 0, false, sp, sq, out);
}

// ------------------------------------------------------------------ greedy blockwise

// per chunk of a row: (max, first id of the max) per wave
template <int DT>
__global__ __launch_bounds__(WG) void k_argmax(const char *__restrict__ tgt, int V, int nch,
                                               float2 *part)
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    const int row = blockIdx.x / nch, c = blockIdx.x - row * nch;
    const char *rp = tgt + (size_t)row * (size_t)V * BY;
    const int cbase = c * WG * NV_ARGMAX * E;
    float x[NV_ARGMAX][E];
    load_chunk<DT, NV_ARGMAX>(rp, aligned16(rp), cbase, V, x);
    // this thread's ids ascend with (i, k); start from its first id so that an all -inf
    // run still reports the lowest id
    const int first = cbase + threadIdx.x * E;
    float bv = -INFINITY;
    int bi = (first < V) ? first : INT_MAX;
#pragma unroll
    for (int i = 0; i < NV_ARGMAX; ++i)
#pragma unroll
        for (int k = 0; k < E; ++k)
            if (x[i][k] > bv) {
                bv = x[i][k];
                bi = cbase + (i * WG + threadIdx.x) * E + k;
            }
    wave_argmax(bv, bi);
    store_wave_partials(make_float2(bv, __int_as_float(bi)), part + (size_t)blockIdx.x * WAVES);
}

// one workgroup per sequence: row argmaxes g_j, then the longest matching prefix
__global__ __launch_bounds__(WG) void k_greedy_final(const int32_t *__restrict__ props, int K,
                                                     int V, int nch,
                                                     const float2 *__restrict__ part,
                                                     int32_t *acc_len, int32_t *out_tokens)
{
    __shared__ int sg[64];
    const int b = blockIdx.x, P = K + 1;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, np = nch * WAVES;
    for (int j = w; j < P; j += WAVES) {
        const float2 *pr = part + ((size_t)b * P + j) * np;
        float v = -INFINITY;
        int id = INT_MAX;
        for (int i = lane; i < np; i += 64) {
            const float2 e = pr[i];
            take_better(v, id, e.x, __float_as_int(e.y));
        }
        wave_argmax(v, id);
        if (lane == 0)
            sg[j] = id;
    }
    __syncthreads();
    if (w != 0)
        return;
    const int32_t xp = (lane < K) ? props[(size_t)b * K + lane] : 0;
    const bool bad = (lane < K) && (xp < 0 || xp >= V);
    int32_t *ot = out_tokens + (size_t)b * (K + 1);
    if (__ballot(bad) != 0) {
        if (lane <= K)
            ot[lane] = -1;
        if (lane == 0)
            acc_len[b] = -1;
        return;
    }
    const unsigned long long mm = __ballot(lane < K && xp != sg[lane]);
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
            (void)hipEventRecord(ln.ev[2 * kind], ln.stream);
    }
    ~Timer()
    {
        if (ln.ev)
            (void)hipEventRecord(ln.ev[2 * kind + 1], ln.stream);
    }
};

template <int DT, int MODE>
hipError_t sampling_impl(const Launch &ln, const Workspace &ws, int B, int K, int V,
                         const Scale &sp, const Scale &sq, const void *tgt, const void *drf,
                         const int32_t *tokens, const float *unif, int32_t *acc_len,
                         int32_t *out_tokens, float *out_probs)
{
    const char *t = static_cast<const char *>(tgt);
    const char *d = static_cast<const char *>(drf);
    const int nch = num_chunks(MODE == SAMPLING ? NV_STATS : NV_PAIR, DT, V);
    {
        Timer tm(ln, KIND_STATS);
        if (MODE == SAMPLING) {
            const unsigned grid = (unsigned)((size_t)B * (2 * K + 1) * nch);
            hipLaunchKernelGGL(k_stats_sampling<DT>, dim3(grid), dim3(WG), 0, ln.stream, t, d, K,
                               V, nch, sp, ws.part);
        } else {
            const unsigned grid = (unsigned)((size_t)B * (K + 1) * nch);
            hipLaunchKernelGGL(k_stats_contrastive<DT>, dim3(grid), dim3(WG), 0, ln.stream, t, d,
                               K, V, nch, sp, sq, ws.part);
        }
    }
    {
        Timer tm(ln, KIND_ACCEPT);
        hipLaunchKernelGGL((k_accept<DT, MODE>), dim3(B), dim3(WG), 0, ln.stream, t, d, tokens,
                           unif, K, V, nch, sp, sq, ws.part, acc_len, out_tokens, out_probs, ws.seq);
    }
    const int ncr = num_chunks(NV_RESID, DT, V);
    {
        Timer tm(ln, KIND_RESID);
        hipLaunchKernelGGL((k_resid<DT, MODE>), dim3((unsigned)((size_t)B * ncr)), dim3(WG), 0,
                           ln.stream, t, d, K, V, ncr, sp, sq, ws.seq, ws.resid);
    }
    {
        Timer tm(ln, KIND_DRAW);
        hipLaunchKernelGGL((k_draw<DT, MODE>), dim3(B), dim3(WG), 0, ln.stream, t, d, unif, K, V,
                           ncr, sp, sq, ws.seq, ws.resid, out_tokens);
    }
    return hipGetLastError();
}

template <int DT>
hipError_t greedy_impl(const Launch &ln, const Workspace &ws, int B, int K, int V, const void *tgt,
                       const int32_t *props, int32_t *acc_len, int32_t *out_tokens)
{
    const int nch = num_chunks(NV_ARGMAX, DT, V);
    {
        Timer tm(ln, KIND_ARGMAX);
        const unsigned grid = (unsigned)((size_t)B * (K + 1) * nch);
        hipLaunchKernelGGL(k_argmax<DT>, dim3(grid), dim3(WG), 0, ln.stream,
                           static_cast<const char *>(tgt), V, nch, ws.part);
    }
    {
        Timer tm(ln, KIND_GREEDY_EMIT);
        hipLaunchKernelGGL(k_greedy_final, dim3(B), dim3(WG), 0, ln.stream, props, K, V, nch,
                           ws.part, acc_len, out_tokens);
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
