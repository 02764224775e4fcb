// gfx950 kernels for the batched verify-and-accept step of speculative decoding.
//
// A sampling or contrastive call is two launches on the caller's stream:
//   k_stats_*  one read of every logit row (nontemporal 128-bit loads).  Each 256-thread
//              workgroup reduces one chunk of a row to per-wave (max, sum exp2) partials;
//              the contrastive form reads the expert and amateur rows of a position together.
//   k_tail     one 1024-thread workgroup per sequence (or G of them sharing one draw when
//              the batch is too small to fill the chip) merges the partials in fp64,
//              gathers p_j(x_j) and q_j(x_j), accepts iff p > 0 and u * q <= p, finds the
//              first rejection L, re-reads row L into per-unit sums of w = max(0, p - q),
//              locates the unit holding t = u_K * W and emits the first id whose prefix
//              weight exceeds t.  A draw from p alone (the bonus draw, the sampler) finds
//              the chunk holding t from the statistics' chunk sums and re-reads only it.
// With early exit the statistics of the first positions come first (k_stats_prefix or
// k_pairs_prefix), k_alive lists the sequences not yet rejected there, k_stats_rest /
// k_pairs_rest read only their remaining rows, and k_tail finishes as above.
// A greedy blockwise call is k_argmax (chunk (max, first id)) and k_greedy_final, or
// k_greedy_heads when the same pass also carries the next block's proposal heads.  Its early
// exit runs k_argmax_prefix over the first positions, k_alive_greedy, then k_argmax_rest over
// the survivors' remaining rows before k_greedy_final.
// The draft-token sampler runs k_stats_sampling and k_tail with no draft (K = 0, each row
// its own sequence), and k_quantile_cut is a per-row radix select for an alpha-quantile of
// reward scores.
//
// The operations follow the speculative rejection sampling page (steps 2-4, and the
// "key guarantee" that fixes the residual law), the blockwise parallel decoding page
// (section 3.5, Verify/Accept, and the merged predict-verify step), the speculative
// contrastive decoding review (SCD) and the Speculative Rejection page (the quantile cut).
#include <float.h>
#include <math.h>
#include <hip/hip_ext.h>

#include <atomic>
#include <mutex>

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
// Butterfly reductions whose lane exchanges run on the VALU, with no LDS round trip: steps 0
// and 1 are the DPP quad permutations lane^1 and lane^2; steps 2 and 3 mirror lanes within 8
// and within 16 (once the quads are reduced, the mirrored lane holds what lane^4, lane^8
// would); step 4 swaps 16-lane rows (lane^16, v_permlane16_swap) and step 5 the wave's halves
// (lane^32, v_permlane32_swap).  Each step combines the same two operands in both lanes of a
// pair, so every lane ends with the same bits and the results are deterministic.  The whole
// wave (or, for the half-wave forms, the whole 32-lane half) must be active.

template <int S>
__device__ __forceinline__ int lane_xch(int v)
{
    const int lane = threadIdx.x & 63;
    if constexpr (S == 0)
        return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad_perm 1,0,3,2
    else if constexpr (S == 1)
        return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad_perm 2,3,0,1
    else if constexpr (S == 2)
        return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    else if constexpr (S == 3)
        return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false);  // row_mirror
    else if constexpr (S == 4) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? (int)r[0] : (int)r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (lane & 32) ? (int)r[0] : (int)r[1];
    }
}

template <int S> __device__ __forceinline__ float xch(float v)
{
    return __int_as_float(lane_xch<S>(__float_as_int(v)));
}

template <int S> __device__ __forceinline__ double xch(double v)
{
    return __hiloint2double(lane_xch<S>(__double2hiint(v)), lane_xch<S>(__double2loint(v)));
}

template <int NS, typename T> __device__ __forceinline__ T xmax(T v)
{
    v = fmaxf(v, xch<0>(v));
    v = fmaxf(v, xch<1>(v));
    v = fmaxf(v, xch<2>(v));
    v = fmaxf(v, xch<3>(v));
    v = fmaxf(v, xch<4>(v));
    if constexpr (NS == 6)
        v = fmaxf(v, xch<5>(v));
    return v;
}

template <int NS, typename T> __device__ __forceinline__ T xsum(T v)
{
    v += xch<0>(v);
    v += xch<1>(v);
    v += xch<2>(v);
    v += xch<3>(v);
    v += xch<4>(v);
    if constexpr (NS == 6)
        v += xch<5>(v);
    return v;
}

__device__ inline float wave_max(float v) { return xmax<6>(v); }
__device__ inline double wave_sum(double v) { return xsum<6>(v); }

// The same reductions with the exchanges through the LDS crossbar (ds_bpermute): a longer
// latency per call, but they leave the VALU alone, which matters where the VALU is as busy
// as the memory pipe: the row statistics kernels and the draw's row pass.
template <typename T> __device__ inline T wave_max_lds(T v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

template <typename T> __device__ inline T wave_sum_lds(T v)
{
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        v += __shfl_xor(v, o);
    return v;
}

// max and sum over each 32-lane half of the wave (the halves reduce independently)
__device__ inline float half_max(float v) { return xmax<5>(v); }
__device__ inline double half_sum(double v) { return xsum<5>(v); }

// Inclusive prefix sum of a double over the wave's lanes, with DPP moves (fixed order): row
// shifts by 1, 2, 4, 8 give each 16-lane row its own scan, then lane 15's total is added into
// rows 1 and 3 (row_bcast:15) and lane 31's into rows 2 and 3 (row_bcast:31).  Lanes with no
// source read 0.  The whole wave must be active.
template <int CTRL, int ROWS> __device__ __forceinline__ double dpp_move(double v)
{
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(v), CTRL, ROWS, 0xF, false);
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(v), CTRL, ROWS, 0xF, false);
    return __hiloint2double(hi, lo);
}

__device__ inline double wave_incl_scan(double v)
{
    v += dpp_move<0x111, 0xF>(v);  // row_shr:1
    v += dpp_move<0x112, 0xF>(v);  // row_shr:2
    v += dpp_move<0x114, 0xF>(v);  // row_shr:4
    v += dpp_move<0x118, 0xF>(v);  // row_shr:8
    v += dpp_move<0x142, 0xA>(v);  // row_bcast:15, rows 1 and 3
    v += dpp_move<0x143, 0xC>(v);  // row_bcast:31, rows 2 and 3
    return v;
}

// The exclusive prefix from the inclusive one: each lane takes its left neighbour's value
// (DPP wave_shr:1), lane 0 takes 0.
__device__ inline double wave_excl_from_incl(double inc) { return dpp_move<0x138, 0xF>(inc); }

// A lane's value read by the whole wave; the lane index must be the same in every lane.
__device__ __forceinline__ int lane_value(int v, int l) { return __builtin_amdgcn_readlane(v, l); }
__device__ __forceinline__ double lane_value(double v, int l)
{
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(v), l),
                            __builtin_amdgcn_readlane(__double2loint(v), l));
}

// lexicographic "better": larger value, then lower id
__device__ inline void take_better(float &v, int &i, float v2, int i2)
{
    if (v2 > v || (v2 == v && i2 < i)) {
        v = v2;
        i = i2;
    }
}

template <int S> __device__ __forceinline__ void argmax_step(float &v, int &i)
{
    const float v2 = xch<S>(v);
    const int i2 = lane_xch<S>(i);
    take_better(v, i, v2, i2);
}

__device__ inline void wave_argmax(float &v, int &i)
{
    argmax_step<0>(v, i);
    argmax_step<1>(v, i);
    argmax_step<2>(v, i);
    argmax_step<3>(v, i);
    argmax_step<4>(v, i);
    argmax_step<5>(v, i);
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

// thread_stats over packed words, GV vectors at a time with an online merge: the running
// (m, s) is rescaled by exp2((m - m') log2(e)/T) when a group raises the maximum to m'.  Each
// group's exponent arguments have the fma-reference form with that group's running maximum.
// Fewer values are live at once than in thread_stats, at the cost of two exps per group.
template <int DT, int NV, int GV>
__device__ inline void thread_stats_words(const uint4 (&raw)[NV], const Scale &sc, float &m,
                                          float &s)
{
    constexpr int E = Elt<DT>::EPV;
    m = -INFINITY;
    s = 0.0f;
#pragma unroll
    for (int g = 0; g < NV; g += GV) {
        float x[GV][E];
#pragma unroll
        for (int i = 0; i < GV; ++i)
            Elt<DT>::unpack(raw[g + i], x[i]);
        float mg = m;
#pragma unroll
        for (int i = 0; i < GV; ++i)
#pragma unroll
            for (int k = 0; k < E; ++k)
                mg = fmaxf(mg, x[i][k]);
        const float mr = (mg == -INFINITY) ? 0.0f : mg;  // an all -inf group sums exact zeros
        const float R = mr * sc.hi;
        const float shift = __builtin_fmaf(mr, sc.lo, __builtin_fmaf(mr, sc.hi, -R));
        float sg = 0.0f;
#pragma unroll
        for (int i = 0; i < GV; ++i) {
            float t[E];
#pragma unroll
            for (int k = 0; k < E; ++k)
                t[k] = __builtin_amdgcn_exp2f(
                    __builtin_fmaf(x[i][k], sc.lo, __builtin_fmaf(x[i][k], sc.hi, -R)));
            sg += tree_sum<E>(t);
        }
        sg *= __builtin_amdgcn_exp2f(-shift);
        s = (s > 0.0f) ? s * exp2s(m - mg, sc.hi, sc.lo) + sg : sg;
        m = mg;
    }
}

// per-wave (M, S): S = sum over lanes of s * exp2((m - M) * log2(e)/T)
__device__ inline float2 wave_stats(float m, float s, const Scale &sc)
{
    const float M = wave_max_lds(m);
    const float e = (s > 0.0f) ? s * exp2s(m - M, sc.hi, sc.lo) : 0.0f;
    return make_float2(M, wave_sum_lds(e));
}

// Store the workgroup's four per-wave partials from one thread after a barrier, as a single
// 32-byte write (the early-exit row statistics and the argmax kernels).  With one chunk per
// workgroup the contrastive statistics were 1.3 us faster per launch this way than with four
// single-lane writes; with two chunks per workgroup they store per wave, as the sampling
// statistics always have.
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

// A chunk is read by 256 threads; a workgroup of 2 * WG threads reads two chunks, one per half.
__device__ __forceinline__ int chunk_thread() { return (int)(threadIdx.x & (WG - 1)); }

// Load NV vectors per thread of chunk `cbase` of a row, ids >= V as -inf.  In an aligned row
// every vector that lies wholly below V is one streamed 16-byte load, all issued before any
// use (a chunk at the end of the row only masks some of them off); only the vector that
// straddles V, if V is not a multiple of the vector width, is read element by element.
// Unaligned rows take element loads throughout.
template <int DT, int NV>
__device__ inline void load_chunk(const char *rp, bool al, int cbase, int V,
                                  float (&x)[NV][Elt<DT>::EPV])
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    if (al && cbase + WG * NV * E <= V) {
        uint4 raw[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            raw[i] = load_stream(rp + (size_t)(cbase + (i * WG + chunk_thread()) * E) * BY);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
            Elt<DT>::unpack(raw[i], x[i]);
    } else if (al) {
        constexpr uint32_t NEG_INF_WORD = (BY == 2) ? 0xff80ff80u : 0xff800000u;
        uint4 raw[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e0 = cbase + (i * WG + chunk_thread()) * E;
            if (e0 + E <= V)
                raw[i] = load_stream(rp + (size_t)e0 * BY);
            else
                raw[i] = make_uint4(NEG_INF_WORD, NEG_INF_WORD, NEG_INF_WORD, NEG_INF_WORD);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i)
            Elt<DT>::unpack(raw[i], x[i]);
        if (V % E != 0) {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int e0 = cbase + (i * WG + chunk_thread()) * E;
                if (e0 < V && e0 + E > V)
#pragma unroll
                    for (int k = 0; k < E; ++k)
                        x[i][k] = (e0 + k < V) ? Elt<DT>::one(rp, (size_t)(e0 + k)) : -INFINITY;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            load_elems<DT>(rp, al, cbase + (i * WG + chunk_thread()) * E, V, -INFINITY, x[i]);
    }
}

// The same chunk of a bfloat16 row as load_chunk, kept as NV packed 16-byte words per thread
// (ids >= V read as -inf bits): vectors wholly below V in an aligned row are one streamed
// load each, the rest are packed element by element (element 2j in the low half of word j).
// Holding the packed words instead of NV*8 floats keeps the sampling statistics kernel at 46
// VGPRs, 8 waves per SIMD, and the contrastive one at 69 instead of 90.
__device__ inline uint4 pack_bf16(const char *rp, int e0, int V)
{
    const uint16_t *h = reinterpret_cast<const uint16_t *>(rp);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t lo = (e0 + 2 * j < V) ? (uint32_t)h[e0 + 2 * j] : 0xff80u;
        const uint32_t hi = (e0 + 2 * j + 1 < V) ? (uint32_t)h[e0 + 2 * j + 1] : 0xff80u;
        w[j] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int DT, int NV>
__device__ inline void load_chunk_words(const char *rp, bool al, int cbase, int V,
                                        uint4 (&raw)[NV])
{
    static_assert(Elt<DT>::EPV == 8, "packed words are used for bfloat16 rows only");
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    constexpr uint32_t NEG_INF_WORD = 0xff80ff80u;
    if (al && cbase + WG * NV * E <= V) {
#pragma unroll
        for (int i = 0; i < NV; ++i)
            raw[i] = load_stream(rp + (size_t)(cbase + (i * WG + chunk_thread()) * E) * BY);
    } else {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e0 = cbase + (i * WG + chunk_thread()) * E;
            if (al && e0 + E <= V)
                raw[i] = load_stream(rp + (size_t)e0 * BY);
            else if (e0 >= V)
                raw[i] = make_uint4(NEG_INF_WORD, NEG_INF_WORD, NEG_INF_WORD, NEG_INF_WORD);
            else
                raw[i] = pack_bf16(rp, e0, V);
        }
    }
}

// Per-lane inputs of the accept tests of sequence b (one wave, lane j < K): draft token x_j,
// uniform u_j and the gathered logits (the contrastive target value l_e - l_a in fp32); bad:
// x_j outside [0, V).
struct Draft {
    int32_t x;
    float lp, lq, u;
    bool bad;
};

template <int DT, int MODE>
__device__ __forceinline__ Draft gather_draft(const char *tgt, const char *drf,
                                              const int32_t *tokens, const float *unif, int b,
                                              int K, int V, int lane)
{
    Draft d = {0, 0.0f, 0.0f, 0.0f, false};
    if (lane < K) {
        d.x = tokens[(size_t)b * K + lane];
        d.u = unif[(size_t)b * (K + 1) + lane];
        d.bad = (d.x < 0 || d.x >= V);
        if (!d.bad) {
            const size_t it = ((size_t)b * (K + 1) + lane) * (size_t)V + d.x;
            if (MODE == SAMPLING) {
                d.lp = Elt<DT>::one(tgt, it);
                d.lq = Elt<DT>::one(drf, ((size_t)b * K + lane) * (size_t)V + d.x);
            } else {
                const float le = Elt<DT>::one(tgt, it), la = Elt<DT>::one(drf, it);
                d.lp = le - la;
                d.lq = la;
            }
        }
    }
    return d;
}

// Merge the per-wave partials of the rows of sequence b whose position is below npos
// (target row j and draft row j of position j) into (M, S) in fp64: M = max, S = sum of
// s * 2^((m - M) log2(e)/T).  The NT threads stage the partials in LDS in one coalesced pass
// when they fit; one wave merges each row, always with the same instructions, so every
// kernel that merges a row gets the same bits.
// nothing to do while the partials are in flight (see merge_rows)
struct NoWork {
    __device__ void operator()() const {}
};

template <int NT, class Mid = NoWork>
__device__ __forceinline__ void merge_rows(const float2 *part, int b, int K, int nch, int npos,
                                           const Scale &sp, const Scale &sq, float2 *stage,
                                           float *sM, double *sS, const Mid &mid = Mid(),
                                           bool idle_mid = false)
{
    constexpr int NW = NT / 64;
    const int R = 2 * K + 1, np = nch * WAVES, total = R * np;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const float2 *pb = part + (size_t)b * total;
    // Staged: one coalesced pass of all threads into LDS, a barrier, then the merges read LDS,
    // with mid() in the loads' shadow.  When mid() has nothing to do and every row is merged in
    // one round, the merging lanes read their partials from memory themselves: no barrier and
    // no LDS round trip (the accept phase at B=256, K=8, V=128256: 4.26 -> 3.44 us).  Either
    // way the same values are merged in the same order.
    const int per_round = (np <= 32) ? 2 * NW : NW;
    const bool staged = total <= ACCEPT_STAGE && !(idle_mid && R <= per_round);
    // mid() runs once, by every thread, while the first staging loads are in flight
    bool done_mid = false;
    if (staged) {
        for (int i0 = 0; i0 < total; i0 += 4 * NT) {
            float2 v[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + k * NT + t;
                v[k] = (i < total) ? pb[i] : make_float2(0.0f, 0.0f);
            }
            if (!done_mid) {
                mid();
                done_mid = true;
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = i0 + k * NT + t;
                if (i < total)
                    stage[i] = v[k];
            }
        }
    }
    if (!done_mid)
        mid();
    if (staged)
        __syncthreads();
    // A row with at most 32 partials is merged by half a wave, so that each wave takes two
    // rows at a time; the reductions then run over the half's 32 lanes, which gives the
    // same values as the 64-lane ones (there the other half only adds zeros and -inf).
    const bool half = np <= 32;
    const int ll = half ? (lane & 31) : lane, width = half ? 32 : 64;
    const int rstep = half ? 2 * NW : NW;
    for (int r = half ? 2 * w + (lane >> 5) : w; r < R; r += rstep) {
        const int pos = (r <= K) ? r : r - K - 1;
        if (pos >= npos)
            continue;  // not read by this call
        const int r0 = r * np;
        const double cc = (r <= K) ? sp.c : sq.c;
        float ml = -INFINITY;
        for (int i = ll; i < np; i += width)
            ml = fmaxf(ml, (staged ? stage[r0 + i] : pb[r0 + i]).x);
        const float M = half ? half_max(ml) : wave_max(ml);
        double sl = 0.0;
        for (int i = ll; i < np; i += width) {
            const float2 v = staged ? stage[r0 + i] : pb[r0 + i];
            if (v.y > 0.0f)
                sl += (double)v.y * exp2(((double)v.x - (double)M) * cc);
        }
        const double S = half ? half_sum(sl) : wave_sum(sl);
        if (ll == 0) {
            sM[r] = M;
            sS[r] = S;
        }
    }
    __syncthreads();
}

// p_j(x_j), q_j(x_j) in fp64 from the merged statistics and the accept test: kept iff
// P > 0 and u * Q <= P.
__device__ __forceinline__ bool accept_test(const Draft &d, int j, int K, const float *sM,
                                            const double *sS, const Scale &sp, const Scale &sq,
                                            double &P, double &Q)
{
    P = exp(((double)d.lp - (double)sM[j]) * sp.inv_t) / sS[j];
    Q = exp(((double)d.lq - (double)sM[K + 1 + j]) * sq.inv_t) / sS[K + 1 + j];
    return (P > 0.0) && ((double)d.u * Q <= P);
}

// Sequence b after its rows' statistics (the first phase of k_tail): merge the rows of the
// positions below npos (K+1: all of them), then the last wave runs the accept tests, one lane per
// draft position, finds the first rejection L, writes accepted_len, the kept tokens, -1
// padding and out_probs, and leaves in *info what the draw needs (L = -1 for bad ids).
// Positions at or past npos are only reached by a sequence that rejects before them.
// mask_probs: out_probs only for j <= L, NaN after (the rows after L may not have been read).
// write: whether this workgroup writes the outputs (one of the workgroups of a split draw).
// mid: work for every thread while the partials load (see merge_rows).
template <int DT, int MODE, class Mid = NoWork>
__device__ __forceinline__ void accept_phase(const char *tgt, const char *drf,
                                             const int32_t *tokens, const float *unif, int b,
                                             int K, int V, int nch, int npos, bool mask_probs,
                                             bool write, const Scale &sp, const Scale &sq,
                                             const float2 *part, float2 *stage,
                                             int32_t *acc_len, int32_t *out_tokens,
                                             float *out_probs, SeqInfo *info,
                                             const Mid &mid = Mid(), bool idle_mid = false)
{
    __shared__ float sM[MAX_ROWS];
    __shared__ double sS[MAX_ROWS];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    // The last wave gathers the draft's tokens and logits (a token load, then the logit loads
    // that depend on it) and runs the accept tests.  The partials are staged by the first
    // threads, so with a few hundred partials the last wave issues no staging load that would
    // wait behind its gather: the two round trips overlap the staging instead of delaying it.
    constexpr int GW = TAIL_WAVES - 1;
    Draft d = {0, 0.0f, 0.0f, 0.0f, false};
    if (w == GW)
        d = gather_draft<DT, MODE>(tgt, drf, tokens, unif, b, K, V, lane);
    merge_rows<TAIL_WG>(part, b, K, nch, npos, sp, sq, stage, sM, sS, mid, idle_mid);
    if (w != GW)
        return;

    int32_t *ot = out_tokens + (size_t)b * (K + 1);
    if (!write) {
        acc_len = nullptr;
        out_probs = nullptr;
    }
    if (__ballot(d.bad) != 0) {
        if (write && lane <= K)
            ot[lane] = -1;
        if (lane < K && out_probs) {
            out_probs[((size_t)b * K + lane) * 2] = NAN;
            out_probs[((size_t)b * K + lane) * 2 + 1] = NAN;
        }
        if (lane == 0) {
            if (acc_len)
                acc_len[b] = -1;
            SeqInfo si = {};
            si.L = -1;
            *info = si;
        }
        return;
    }
    bool acc = lane < K;  // lanes >= K never accept; positions >= npos are never reached
    double P = NAN, Q = NAN;
    if (lane < K && lane < npos)
        acc = accept_test(d, lane, K, sM, sS, sp, sq, P, Q);
    const unsigned long long am = __ballot(acc);
    const int L = __builtin_ctzll(~am);  // L <= K
    if (lane < K && out_probs) {
        const bool show = !mask_probs || lane <= L;
        out_probs[((size_t)b * K + lane) * 2] = show ? (float)P : NAN;
        out_probs[((size_t)b * K + lane) * 2 + 1] = show ? (float)Q : NAN;
    }
    if (write && lane < L)
        ot[lane] = d.x;
    else if (write && lane > L && lane <= K)
        ot[lane] = -1;
    // What the draw needs.  Its fp64 chains run as one exp2 and one division over the lanes
    // (lane 0: 2^-e_p / S_p, lane 1: 2^-e_q / S_q, lane 2: kappa = 2^(M_p c_p - M_q c_q) times
    // S_p / S_q, the residual draw's draft-side scale for terms without the rows' maxima).
    const float Mp = sM[L];
    const bool dr = L < K;
    const float Mq = dr ? sM[K + 1 + L] : 0.0f;
    const double Sp = sS[L], Sq = dr ? sS[K + 1 + L] : 0.0;
    const float Rp = Mp * sp.hi, Rq = Mq * sq.hi;
    const float ep = __builtin_fmaf(Mp, sp.lo, __builtin_fmaf(Mp, sp.hi, -Rp));
    const float eq = __builtin_fmaf(Mq, sq.lo, __builtin_fmaf(Mq, sq.hi, -Rq));
    const double kd = (double)Mp * sp.c - (double)Mq * sq.c;
    const bool kok = dr && fabs(kd) <= 900.0;
    double arg = 0.0, num = 1.0, den = 1.0;
    if (lane == 0) {
        arg = -(double)ep;
        den = Sp;
    } else if (lane == 1 && dr) {
        arg = -(double)eq;
        den = Sq;
    } else if (lane == 2 && kok) {
        arg = kd;
        den = Sq;
    }
    const double e = exp2(arg);
    if (lane == 2)
        num = Sp;
    else
        num = e;
    const double q = num / den;
    if (lane == 0) {
        if (acc_len)
            acc_len[b] = L;
        info->L = L;
        info->Mp = Mp;
        info->Sp = Sp;
        info->Rp = Rp;
        info->isp = (float)q;
    } else if (lane == 1) {
        info->Mq = Mq;
        info->Sq = Sq;
        info->Rq = dr ? Rq : 0.0f;
        info->isq = dr ? (float)q : 0.0f;
    } else if (lane == 2) {
        info->kappa = kok ? e * q : 0.0;
    }
}

// Per-thread (max, sum) of one chunk of a sampling row.  bfloat16 keeps the chunk as packed
// words and reduces it two vectors at a time (46 VGPRs, 8 waves per SIMD: 1-2 us faster per
// launch at B=256, K=8, V=128256 than 64 unpacked floats at 79 VGPRs, 6 waves); float32 keeps
// the unpacked values (its 32 per thread are no burden, and it ran slower as packed words).
// The full-read and the early-exit statistics both use this, so they agree bit for bit.
template <int DT>
__device__ __forceinline__ void sampling_chunk_stats(const char *rp, int V, int c, const Scale &sc,
                                                     float &m, float &s)
{
    constexpr int E = Elt<DT>::EPV;
    const int cbase = c * WG * NV_STATS * E;
    if constexpr (E == 8) {
        uint4 raw[NV_STATS];
        load_chunk_words<DT, NV_STATS>(rp, aligned16(rp), cbase, V, raw);
        thread_stats_words<DT, NV_STATS, 2>(raw, sc, m, s);
    } else {
        float x[NV_STATS][E];
        load_chunk<DT, NV_STATS>(rp, aligned16(rp), cbase, V, x);
        thread_stats<E, NV_STATS>(x, sc, m, s);
    }
}

// The per-call tables of the residual draw (see the draw below): slot k < GTAB_DOUBLES is table
// k / TAB_DOUBLES (0: the target law's c, 1: the draft law's), sign block and slot i of the LDS
// layout; i in 1..TAB_HALF holds 2^(v c) in fp64 for the bfloat16 value v of magnitude pattern
// TAB_LO + i - 1, the sentinel slots 0 and TAB_HALF + 1 hold NaN, the rest 0.  The first
// workgroups of a statistics launch write them, one slot per thread, before their chunk.
__device__ inline void global_tables(const TabJob &tj)
{
    if (tj.gtab == nullptr)
        return;
    const int k = (int)(blockIdx.x * blockDim.x + threadIdx.x);
    if (k >= GTAB_DOUBLES)
        return;
    const int tb = k / TAB_DOUBLES, r = k - tb * TAB_DOUBLES;
    const int sg = r / TAB_SIGN, i = r - sg * TAB_SIGN;
    double v = 0.0;
    if (i == 0 || i == TAB_HALF + 1) {
        v = __builtin_nan("");
    } else if (i <= TAB_HALF) {
        const uint32_t bits = ((uint32_t)(TAB_LO + i - 1) << 16) | (sg ? 0x80000000u : 0u);
        v = exp2((double)__uint_as_float(bits) * (tb ? tj.cq : tj.cp));
    }
    tj.gtab[k] = v;
}

// rows b*(2K+1)+r: r <= K target row (b, r), else draft row (b, r-K-1).  A workgroup of Q * WG
// threads reads Q consecutive chunks of one row (quarter, or half, q of the workgroup reads chunk
// Q g + q); each wave stores its (max, sum) partial at part[(row * nch + chunk) * WAVES + wave].
// Two chunks per 512-thread workgroup: 205.3-205.6 us per call at B=256, K=8, V=128256 against
// 210.2-211.2 with one chunk per 256-thread workgroup and 212.7-213.9 with four per 1024 (the
// same partials, bit for bit).
template <int DT, int Q>
__global__ __launch_bounds__(WG * Q) void k_stats_sampling(const char *__restrict__ tgt,
                                                           const char *__restrict__ drf, int K,
                                                           int V, int nch, Scale sc, float2 *part,
                                                           TabJob tj)
{
    constexpr int BY = Elt<DT>::BYTES;
    const int R = 2 * K + 1;
    global_tables(tj);
    // The grid walks the target tensor's rows, then the draft tensor's, each in memory order
    // (about 1 us faster per launch at B=256, K=8, V=128256 than each sequence's 2K+1 rows in
    // turn); the partials keep the sequence's row order.
    const int ngrp = (nch + Q - 1) / Q;
    const int grow = blockIdx.x / ngrp;
    const int c = (blockIdx.x - grow * ngrp) * Q + (int)(threadIdx.x / WG);
    if (c >= nch)
        return;  // the row's last group has fewer than Q chunks (whole waves leave)
    const int Bn = (int)(gridDim.x / ngrp) / R;  // sequences
    int b, r;
    if (grow < Bn * (K + 1)) {
        b = grow / (K + 1);
        r = grow - b * (K + 1);
    } else {
        const int i2 = grow - Bn * (K + 1);
        b = i2 / K;
        r = K + 1 + (i2 - b * K);
    }
    const int row = b * R + r;
    const char *rp = (r <= K) ? tgt + ((size_t)b * (K + 1) + r) * (size_t)V * BY
                              : drf + ((size_t)b * K + (r - K - 1)) * (size_t)V * BY;
    float m, s;
    sampling_chunk_stats<DT>(rp, V, c, sc, m, s);
    // each wave stores its own partial: no barrier holds the workgroup at its end (measured
    // 1-2.5 us faster per launch at B=256, K=8, V=128256 than one 32-byte store after a barrier)
    const float2 ws = wave_stats(m, s, sc);
    if ((threadIdx.x & 63) == 0)
        part[((size_t)row * nch + c) * WAVES + ((threadIdx.x >> 6) & (WAVES - 1))] = ws;
}

// One chunk of the row pair (b, j): target values l_e - l_a (fp32), draft values l_a.  The
// pair's expert row gives p_j's partials (row j of the sequence), its amateur row q_j's (row
// K+1+j, j < K).
template <int DT>
__device__ __forceinline__ void pair_chunk_stats(const char *ex, const char *am, int b, int j,
                                                 int c, int K, int V, int nch, const Scale &sp,
                                                 const Scale &sq, float2 *part)
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    const int P = K + 1, R = 2 * K + 1;
    const size_t off = ((size_t)b * P + j) * (size_t)V * BY;
    const char *re = ex + off, *ra = am + off;
    const int cbase = c * WG * NV_PAIR * E;
    const bool al = aligned16(re) && aligned16(ra);
    float xd[NV_PAIR][E], xa[NV_PAIR][E];
    if constexpr (E == 8) {
        // bfloat16: both rows as packed words first (one load path for every case), then
        // unpacked: 69 VGPRs instead of 90 (7 waves per SIMD instead of 5), 1 us faster per
        // launch at B=128, K=4, V=152064, with the same values
        uint4 we[NV_PAIR], wa[NV_PAIR];
        load_chunk_words<DT, NV_PAIR>(re, al, cbase, V, we);
        load_chunk_words<DT, NV_PAIR>(ra, al, cbase, V, wa);
#pragma unroll
        for (int i = 0; i < NV_PAIR; ++i) {
            Elt<DT>::unpack(we[i], xd[i]);
            Elt<DT>::unpack(wa[i], xa[i]);
        }
    } else {
        load_chunk<DT, NV_PAIR>(re, al, cbase, V, xd);
        load_chunk<DT, NV_PAIR>(ra, al, cbase, V, xa);
    }
    // ids past V are -inf on both sides: keep the difference at -inf (one select, no branch)
    const bool whole = cbase + WG * NV_PAIR * E <= V;
#pragma unroll
    for (int i = 0; i < NV_PAIR; ++i)
#pragma unroll
        for (int k = 0; k < E; ++k) {
            const int id = cbase + (i * WG + chunk_thread()) * E + k;
            xd[i][k] = (whole || id < V) ? xd[i][k] - xa[i][k] : -INFINITY;
        }
    float m, s, ma, sa;
    thread_stats<E, NV_PAIR>(xd, sp, m, s);
    thread_stats<E, NV_PAIR>(xa, sq, ma, sa);
    // each wave stores its own partials, as the sampling statistics do: no barrier, so a
    // workgroup may hold two chunks (or one, the other half having returned)
    const int wv = (threadIdx.x >> 6) & (WAVES - 1);
    const float2 wp = wave_stats(m, s, sp);
    if ((threadIdx.x & 63) == 0)
        part[(((size_t)b * R + j) * nch + c) * WAVES + wv] = wp;
    if (j < K) {
        const float2 wa = wave_stats(ma, sa, sq);
        if ((threadIdx.x & 63) == 0)
            part[(((size_t)b * R + K + 1 + j) * nch + c) * WAVES + wv] = wa;
    }
}

// Q consecutive chunks of one row pair (b, j) per workgroup of Q * WG threads, one per WG-thread
// part: two chunks per workgroup read c5's 389 MB faster than one (as for the sampling rows)
template <int DT, int Q>
__global__ __launch_bounds__(WG *Q) void k_stats_contrastive(const char *__restrict__ ex,
                                                             const char *__restrict__ am, int K,
                                                             int V, int nch, Scale sp, Scale sq,
                                                             float2 *part, TabJob tj)
{
    global_tables(tj);
    const int ngrp = (nch + Q - 1) / Q;
    const int pr = blockIdx.x / ngrp;
    const int c = (blockIdx.x - pr * ngrp) * Q + (int)(threadIdx.x / WG);
    if (c >= nch)
        return;
    const int b = pr / (K + 1), j = pr - b * (K + 1);
    pair_chunk_stats<DT>(ex, am, b, j, c, K, V, nch, sp, sq, part);
}

// ------------------------------------------------------------------ residual / bonus draw

// The rows a sequence's draw reads: the target side (sampling: target row L; contrastive:
// expert and amateur rows L) and, when L < K, the draft side (sampling: draft row L;
// contrastive: the amateur row again).
struct DrawRows {
    const char *p0;   // target row L (sampling) or expert row L (contrastive)
    const char *p1;   // draft row L (sampling, L < K only) or amateur row L (contrastive)
    // the same rows as buffer resources over their V * BYTES bytes, for the row pass: each of
    // its loads then takes one 32-bit byte offset register instead of a 64-bit address (reads
    // past the end of the row return zeros)
    __amdgpu_buffer_rsrc_t b0, b1;
    bool two;         // p1 is read
    bool resid;       // L < K: w = max(0, p - q); else w = p
    bool al;          // every row read is 16-byte aligned
};

// Raw buffer resource for `bytes` bytes from p (gfx9 descriptor word 3: 32-bit data format).
__device__ inline __amdgpu_buffer_rsrc_t row_resource(const char *p, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(p), (short)0, bytes, 0x00020000);
}

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
    r.b0 = row_resource(r.p0, V * BY);
    r.b1 = row_resource(r.two ? r.p1 : r.p0, V * BY);
    return r;
}

// Draw weight of one id from its target-side value pv and draft-side value qv (fp32):
// p = 2^((pv - Mp) log2(e)/T) / S_p in the fma-reference form of the row statistics (see
// SeqInfo); w = max(0, p - q) for a replacement, p for the bonus (or when `target_law` asks
// for p).  The same instructions run in the unit pass and in the search, so both see
// identical weights.
__device__ inline float draw_weight(float pv, float qv, bool resid, bool target_law,
                                    const SeqInfo &si, const Scale &sp, const Scale &sq)
{
    const float p =
        __builtin_amdgcn_exp2f(__builtin_fmaf(pv, sp.lo, __builtin_fmaf(pv, sp.hi, -si.Rp))) *
        si.isp;
    if (!resid || target_law)
        return p;
    // p - q with q = e_q * is_q in one fma: one rounding, one instruction fewer per id
    const float eq =
        __builtin_amdgcn_exp2f(__builtin_fmaf(qv, sq.lo, __builtin_fmaf(qv, sq.hi, -si.Rq)));
    return fmaxf(__builtin_fmaf(-eq, si.isq, p), 0.0f);
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

// Weights of one whole 16-byte vector from its raw words; TWO: a draft-side vector q is
// read too (the residual, or the contrastive target's amateur half), else the target law p.
template <int DT, int MODE, bool TWO>
__device__ inline void raw_weights(const DrawRows &r, const uint4 &a, const uint4 &q,
                                   bool target_law, const SeqInfo &si, const Scale &sp,
                                   const Scale &sq, float (&wv)[Elt<DT>::EPV])
{
    constexpr int E = Elt<DT>::EPV;
    float pv[E], qv[E];
    Elt<DT>::unpack(a, pv);
    if constexpr (TWO) {
        Elt<DT>::unpack(q, qv);
#pragma unroll
        for (int k = 0; k < E; ++k) {
            if (MODE == CONTRASTIVE)
                pv[k] = pv[k] - qv[k];
            wv[k] = draw_weight(pv[k], qv[k], r.resid, target_law, si, sp, sq);
        }
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k)
            wv[k] = draw_weight(pv[k], 0.0f, false, true, si, sp, sq);
    }
}

// A k_tail iteration with NV vectors per thread covers CE = TAIL_WG * NV * E contiguous ids;
// thread t holds the NV vectors base + i*TAIL_WG*E + [0, E), base = the iteration's first id
// + t*E, so a wave's loads are 1 KiB contiguous.  NV = NV_TAIL when a draft-side row is read
// as well (TWO), 2 * NV_TAIL when only the target row is: the same bytes in flight either
// way.  In an aligned row every vector is one streamed 16-byte buffer load per row read.
// The whole byte offset goes in the VGPR operand, the part the range check covers (the SGPR
// offset is outside it), so the ones at or past V read zeros from the V-element resource and
// never touch memory past the row; they are not used either (tail_weigh weighs the vector
// that straddles V element by element and gives the ones past it weight 0).
template <int DT, int NV, bool TWO>
__device__ inline void tail_load(const DrawRows &r, int it_first, int V, uint4 (&a)[NV],
                                 uint4 (&q)[NV])
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES, STRIDE = TAIL_WG * Elt<DT>::EPV;
    if (!r.al)
        return;
    const int vo = ((int)threadIdx.x * E + it_first) * BY;   // this thread's first vector
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const u32x4 v =
            __builtin_amdgcn_raw_buffer_load_b128(r.b0, vo + i * STRIDE * BY, 0, 2);  // 2: nontemporal
        a[i] = make_uint4(v.x, v.y, v.z, v.w);
    }
    if constexpr (TWO) {
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r.b1, vo + i * STRIDE * BY, 0, 2);
            q[i] = make_uint4(v.x, v.y, v.z, v.w);
        }
    }
}

// The draw-weight sums of this thread's vectors from tail_load (fp32 tree over each vector's
// ids).  Vectors past V weigh 0; the one that straddles V (V not a multiple of the vector
// width), and every vector of an unaligned row, is weighed element by element through
// vec_weights_masked, which the unit search also uses: every id gets the same weight, bit
// for bit, in both places.
template <int DT, int MODE, int NV, bool TWO>
__device__ inline void tail_weigh(const DrawRows &r, int base, int V, bool target_law,
                                  const SeqInfo &si, const Scale &sp, const Scale &sq,
                                  const uint4 (&a)[NV], const uint4 (&q)[NV], float (&vs)[NV])
{
    constexpr int E = Elt<DT>::EPV, STRIDE = TAIL_WG * Elt<DT>::EPV;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e0 = base + i * STRIDE;
        float wv[E];
        if (r.al && e0 + E <= V) {
            raw_weights<DT, MODE, TWO>(r, a[i], q[i], target_law, si, sp, sq, wv);
            vs[i] = tree_sum<E>(wv);
        } else if (e0 < V) {
            vec_weights_masked<DT, MODE>(r, e0, V, target_law, si, sp, sq, wv);
            vs[i] = tree_sum<E>(wv);
        } else {
            vs[i] = 0.0f;
        }
    }
}

template <int NV>
__device__ __forceinline__ void tail_store_units(int it, const float (&vs)[NV], double *units)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const double s = wave_sum_lds((double)vs[i]);
        if (lane == 0)
            units[(it * NV + i) * TAIL_WAVES + w] = s;
    }
}

// A pass over row L (and the draft row L when TWO) for the iterations first, first + step, ...
// below nit: unit u = (it*NV + i)*TAIL_WAVES + w holds the fp64 sum of wave w's draw weights
// at vector slot i of iteration it, i.e. the 64*E contiguous ids it*CE + i*TAIL_WG*E + w*64*E
// + [0, 64*E); unit order is id order.  Two register buffers alternate; each is reloaded
// with the iteration after next as soon as it has been weighed, before the unit sums (a
// chain of lane exchanges) are formed, so that two iterations' loads are in flight while
// one is weighed and summed.
template <int DT, int MODE, int NV, bool TWO>
__device__ __forceinline__ void tail_unit_sums(const DrawRows &r, int V, int nit, int first,
                                               int step, bool target_law, const SeqInfo &si,
                                               const Scale &sp, const Scale &sq, double *units)
{
    constexpr int E = Elt<DT>::EPV, CE = TAIL_WG * NV * Elt<DT>::EPV;
    const int t0 = threadIdx.x * E;
    uint4 a0[NV], q0[NV], a1[NV], q1[NV];
    float vs[NV];
    if (first >= nit)
        return;
    tail_load<DT, NV, TWO>(r, first * CE, V, a0, q0);
    if (first + step < nit)
        tail_load<DT, NV, TWO>(r, (first + step) * CE, V, a1, q1);
    for (int it = first; it < nit; it += 2 * step) {
        const int it1 = it + step;
        tail_weigh<DT, MODE, NV, TWO>(r, it * CE + t0, V, target_law, si, sp, sq, a0, q0, vs);
        if (it + 2 * step < nit)
            tail_load<DT, NV, TWO>(r, (it + 2 * step) * CE, V, a0, q0);
        tail_store_units<NV>(it, vs, units);
        if (it1 < nit) {
            tail_weigh<DT, MODE, NV, TWO>(r, it1 * CE + t0, V, target_law, si, sp, sq, a1, q1,
                                          vs);
            if (it1 + 2 * step < nit)
                tail_load<DT, NV, TWO>(r, (it1 + 2 * step) * CE, V, a1, q1);
            tail_store_units<NV>(it1, vs, units);
        }
    }
}

// Among the `nu` unit totals in LDS (ascending ids) the whole workgroup finds the first unit
// whose running total exceeds tt = u01 * W (W = the sum of all units), or, if rounding leaves
// t at or past the last one, the last unit of positive weight (fb = 1); -1 when every unit
// weighs 0.  Thread t owns the units [t*U, t*U + U): it sums them in order, a wave scan and a
// scan of the 16 wave totals (the same order in every thread, so every thread holds the same
// W) give each thread's starting total, and each thread tests its own units.  The unit, its
// starting total, tt, fb and W go to LDS, readable after the next barrier.
__device__ inline void find_unit_block(const double *units, int nu, float u01, int *s_unit,
                                       double *s_base, double *s_t, int *s_fb, double *s_W)
{
    __shared__ double sw[TAIL_WAVES], shb[TAIL_WAVES], slb[TAIL_WAVES];
    __shared__ int sh[TAIL_WAVES], sl[TAIL_WAVES];
    // the thread index passes through an empty asm so that nothing derived from it is
    // hoisted out of the caller's loop and kept live across the row pass before it
    int t;
    asm volatile("" : "=v"(t) : "0"((int)threadIdx.x));
    const int lane = t & 63, w = t >> 6;
    const int U = (nu + TAIL_WG - 1) / TAIL_WG;
    const int k0 = t * U, k1 = (k0 + U < nu) ? k0 + U : nu;
    double ts = 0.0;
    for (int k = k0; k < k1; ++k)
        ts += units[k];
    const double inc = wave_incl_scan(ts);
    const double exc = wave_excl_from_incl(inc);
    if (lane == 63)
        sw[w] = inc;
    __syncthreads();
    double W = 0.0, wb = 0.0;
#pragma unroll
    for (int v = 0; v < TAIL_WAVES; ++v) {
        if (v == w)
            wb = W;
        W += sw[v];
    }
    const double tt = (double)u01 * W;
    double run = wb + exc, hb = 0.0, lb = 0.0;
    int hit = -1, last = -1;
    for (int k = k0; k < k1; ++k) {
        const double wu = units[k];
        if (hit < 0 && W > 0.0 && wu > 0.0 && run + wu > tt) {
            hit = k;
            hb = run;
        }
        if (wu > 0.0) {
            last = k;
            lb = run;
        }
        run += wu;
    }
    // the wave's first hit is in its lowest hitting lane, its last positive unit in the
    // highest lane that has one
    const unsigned long long hm = __ballot(hit >= 0), pm = __ballot(last >= 0);
    const int lh = hm ? __builtin_ctzll(hm) : 0, lp = pm ? 63 - __builtin_clzll(pm) : 0;
    const int wh = lane_value(hit, lh), wl = lane_value(last, lp);
    const double whb = lane_value(hb, lh), wlb = lane_value(lb, lp);
    if (lane == 0) {
        sh[w] = hm ? wh : -1;
        shb[w] = whb;
        sl[w] = pm ? wl : -1;
        slb[w] = wlb;
    }
    __syncthreads();
    if (w == 0) {  // lane v < 16 holds wave v's candidates: the first hit, else the last positive
        const bool in = lane < TAIL_WAVES;
        const int hv = in ? sh[lane] : -1, lv = in ? sl[lane] : -1;
        const double hbv = in ? shb[lane] : 0.0, lbv = in ? slb[lane] : 0.0;
        const unsigned long long hmk = __ballot(hv >= 0), lmk = __ballot(lv >= 0);
        const int fh = hmk ? __builtin_ctzll(hmk) : 0, fl = lmk ? 63 - __builtin_clzll(lmk) : 0;
        const int uh = lane_value(hv, fh), ul = lane_value(lv, fl);
        const double bh = lane_value(hbv, fh), bl = lane_value(lbv, fl);
        if (lane == 0) {
            *s_unit = hmk ? uh : (lmk ? ul : -1);
            *s_base = hmk ? bh : (lmk ? bl : 0.0);
            *s_t = tt;
            *s_fb = hmk ? 0 : 1;
            *s_W = W;
        }
    }
}

// p(x) = exp((x - M) / T) / S in fp64, the drawn id's probability.  Out of line: its fp64 exp
// would otherwise keep constants in registers across the whole row pass of k_tail.
__device__ __noinline__ float drawn_prob(float x, float M, double inv_t, double S)
{
    return (float)(exp(((double)x - (double)M) * inv_t) / S);
}

// Inside unit `unit` (one wave): lane l weighs the unit's vector l with the instructions of
// the unit pass, a wave scan of the vector sums from `base` finds the vector, and its lane
// emits the first id whose running weight exceeds tt (fb: the last id of positive weight).
template <int DT, int MODE>
__device__ __forceinline__ void search_unit(const DrawRows &r, const SeqInfo &si, int V, int nv,
                                            int unit, double base, double tt, bool fb,
                                            bool target_law, const Scale &sp, const Scale &sq,
                                            int32_t *out, float *out_prob)
{
    constexpr int E = Elt<DT>::EPV;
    const int lane = threadIdx.x & 63;
    const int it = unit / (nv * TAIL_WAVES), rem = unit - it * (nv * TAIL_WAVES);
    const int i = rem / TAIL_WAVES, ww = rem - i * TAIL_WAVES;
    const int e0 = it * (TAIL_WG * nv * E) + i * TAIL_WG * E + (ww * 64 + lane) * E;
    float wv[E];
    if (e0 < V) {
        vec_weights_masked<DT, MODE>(r, e0, V, target_law, si, sp, sq, wv);
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k)
            wv[k] = 0.0f;
    }
    const float vsum = tree_sum<E>(wv);
    const double inc = wave_incl_scan((double)vsum);
    const double exc = wave_excl_from_incl(inc);
    const double bt = base + exc;
    const unsigned long long hit = __ballot(!fb && vsum > 0.0f && bt + (double)vsum > tt);
    const unsigned long long pos = __ballot(vsum > 0.0f);
    if (pos == 0) {  // the unit's total is a sum of these vector sums, so this is not reached
        if (lane == 0) {
            *out = -1;
            if (out_prob)
                *out_prob = NAN;
        }
        return;
    }
    const bool fb2 = fb || hit == 0;
    const int owner = fb2 ? 63 - __builtin_clzll(pos) : __builtin_ctzll(hit);
    if (lane != owner)
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
    const int id = (y >= 0) ? y : lastpos;
    *out = id;
    if (MODE == SAMPLING && out_prob)  // p_L(id) in fp64 from the row's merged statistics
        *out_prob = drawn_prob(Elt<DT>::one(r.p0, (size_t)id), si.Mp, sp.inv_t, si.Sp);
}

// ------------------------------------------------------------------ fp64 residual draw
//
// The residual draw compares cumulative weights of w = max(0, p - q) with t = u * W, W the
// residual mass, so an error in the weights enters the decision as (error) / W.  fp32 weights
// carry about 1e-7 of p each, and the fp32 row statistics put a common error of the same order
// on every p (or q) of a row, which max(0, p - q) does not cancel; at W of 1e-3 that is far
// above the 1e-6 decision margins.  So the residual draw is computed in fp64 from the logits of
// row L.  Per id v it forms a(v) = 2^((z_p(v) - M_p) log2(e)/T_p) * r and
// b(v) = 2^((x_q(v) - M_q) log2(e)/T_q) (z_p the target-side logit, or the expert-minus-amateur
// difference formed exactly in fp64; r a scale), and the sums S_a = sum a, S_b = sum b, so
// that p(v) = a(v) / S_a and q(v) = b(v) / S_b.  Which side of the residual an id is on,
// a / S_a > b / S_b, is needed before the sums are known; with r = S~_q / S~_p from the
// statistics' approximate sums the pass sorts an id to the positive side when a > b, keeps
// per unit A = sum a and B = sum b over its positive-side ids, and afterwards takes the unit's
// weight A / S_a - B / S_b with the exact sums.  The exact side test is a > b * theta,
// theta = S_a / S_b, so an id can be sorted differently only if a / b lies between 1 and
// theta; each such id moves the weights by at most rel (1 + rel) b / S_b, rel = |theta - 1|.
// The pass sums the draft mass b of the ids whose a and b agree to about 2^-18 (their upper
// 32 bits differ by at most NEAR_HI), which holds every such id while rel <= 2^-19; when that
// bound is not far below the decision scale (2^-24 W) the pass is repeated with r from the
// exact sums.
//
// The row is cut into 16 G contiguous segments, one per wave of the G workgroups that share
// the draw; a wave streams its segment (1 KiB per load) and keeps its sums in registers, so a
// unit is a segment.  The draw then finds the segment holding t, weighs its vectors one per
// wave to find the vector, and one wave finds the lane and the id in it.
//
// For bfloat16 rows a and b come from LDS tables: a bfloat16 value is one of 65536 bit
// patterns, and the 7168 with 2^-20 <= |x| < 2^8 cover the logits of a language model's head.
// A slot is found from the bit pattern with packed 16-bit integer operations, two ids at a
// time; values outside the tables read a NaN sentinel (or +0.0 for values below -2^8 whose
// term is negligible), which spoils the lane's sums for that step; the lane weighs the step
// again after its segment, the tables' terms for the other ids and fp64 exp2 for those ids.

// The ids whose a and b have upper words at most NEAR_HI apart count as near the threshold.
// Two positive doubles within a ratio 1 + d have upper words (sign, exponent, 20 mantissa
// bits, monotone in the value) at most d 2^21 + 1 apart, so NEAR_HI = 8 holds every id within
// 7 2^-21 (3.3e-6) of the threshold; NEAR_REL keeps rel below that.  The statistics' sums put rel
// near 1e-7.  (A window of 32 had taken in the ids whose target and draft values are equal,
// hundreds in some rows when kappa is close to 1, and their steps' near mass cost one wave up to
// 5 us at B=256, K=8, V=128256.)
constexpr uint32_t NEAR_HI = 8;
constexpr double NEAR_REL = 0x1p-19;      // the largest rel for which NEAR_HI holds every such id

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// byte offset of the slot of one bfloat16 pattern b (16 bits) within a table: the magnitude's
// 15 bits less TAB_LO - 1, clamped to [0, TAB_HALF + 1], times 8, and the sign in bit 15
__device__ __forceinline__ uint32_t tab_offset(uint32_t b)
{
    const int d = (int)(b & 0x7fffu) - (TAB_LO - 1);
    const int s = min(max(d, 0), TAB_HALF + 1);
    return (uint32_t)(s * 8) | (b & 0x8000u);
}

// the same for the two patterns of a 32-bit word, in its two halves (packed 16-bit operations:
// a saturating subtract takes magnitudes below TAB_LO - 1 to slot 0, a minimum the rest)
__device__ __forceinline__ uint32_t tab_offsets2(uint32_t w)
{
    const u16x2 m = __builtin_bit_cast(u16x2, w & 0x7fff7fffu);
    const u16x2 d = __builtin_elementwise_sub_sat(m, (u16x2)(unsigned short)(TAB_LO - 1));
    const u16x2 c = __builtin_elementwise_min(d, (u16x2)(unsigned short)(TAB_HALF + 1));
    const u16x2 o = c << (u16x2)(unsigned short)3;
    return __builtin_bit_cast(uint32_t, o) | (w & 0x80008000u);
}

// The tables live at LDS address 0 (the kernel's first LDS variable, see k_tail), so a slot's
// byte offset is its address and the loads need no base register.
__device__ __forceinline__ double tab_at(const char *tab, uint32_t off)
{
    return *reinterpret_cast<const double *>(tab + off);
}
// table 0 (the target side) and table 1 (the draft side) at the low or high half's offset of a
// packed pair (one byte permute each)
__device__ __forceinline__ uint32_t t0_lo(uint32_t o2) { return __builtin_amdgcn_perm(0u, o2, 0x0c0c0100u); }
__device__ __forceinline__ uint32_t t0_hi(uint32_t o2) { return __builtin_amdgcn_perm(0u, o2, 0x0c0c0302u); }
__device__ __forceinline__ uint32_t t1_lo(uint32_t o2) { return __builtin_amdgcn_perm(0x10000u, o2, 0x0c060100u); }
__device__ __forceinline__ uint32_t t1_hi(uint32_t o2) { return __builtin_amdgcn_perm(0x10000u, o2, 0x0c060302u); }

// |x - y| of two 32-bit words (v_sad_u32)
__device__ __forceinline__ uint32_t absdiff(uint32_t x, uint32_t y)
{
    uint32_t d;
    asm("v_sad_u32 %0, %1, %2, 0" : "=v"(d) : "v"(x), "v"(y));
    return d;
}

// fp64 exp2 for the ids outside the tables: out of line, so that its constants do not take
// registers from the table path
__device__ __noinline__ double exp2_cold(double a) { return exp2(a); }

// What the fp64 pass needs about the two rows.  An id's terms are
// a = 2^((z - ea) c_p) ra and b = 2^((x_q - eb) c_q) rb (z the target-side value): either
// unscaled (ea = eb = 0, ra = 1, rb = kappa, the tables copied from the per-call tables) or
// relative to the rows' maxima (ea = M_p, eb = M_q, ra = r, rb = 1, tables built for the row).
struct ExactRows {
    const char *p0, *p1;     // target (expert) row L, draft (amateur) row L
    __amdgpu_buffer_rsrc_t b0, b1;  // the same rows as buffer resources (see DrawRows)
    bool al;                 // both rows 16-byte aligned
    bool tabled;             // bfloat16 rows with tables built
    float Mp, Mq;            // the rows' maxima from the statistics
    double cp, cq;           // log2(e) / T of each law
    double ea, eb;           // the exps' reference points
    double ra, rb;           // the terms' scales
    const char *tab;         // LDS: table 0 at +0, table 1 at +64 KiB
};

// Whether the tables serve this row pair.  Sampling: while one group's span of 16 mantissa
// steps, at most 2^4 c in the exponent, keeps its largest value finite (c <= 60).  Contrastive:
// the target-side table holds factors 2^(v c_p) * sqrt(2^(-M_p c_p) r) with a = f(z_e) f(-z_a);
// both factors and their product stay inside the fp64 range while 512 c_p <= 1000 and
// |M_p| <= 512.
template <int MODE>
__device__ __forceinline__ bool exact_tabled(float Mp, double cp, double cq)
{
    if (MODE == SAMPLING)
        return cp <= 60.0 && cq <= 60.0;
    return 512.0 * cp <= 1000.0 && fabsf(Mp) <= 512.0f && cq <= 60.0;
}

// The LDS tables (bfloat16), by the whole workgroup.  Table 0: sampling a = 2^((x - ea) c_p) ra;
// contrastive the factors 2^(x c_p) sqrt(2^(-ea c_p) ra).  Table 1: b = 2^((x - eb) c_q) rb.
// which: 1 table 0, 2 table 1, 3 both.  A slot's value v = +-(128 + 16 jb + j) 2^(E - 134)
// (exponent field E = TAB_E0 + e, mantissa 16 jb + j) is the product of its group's largest
// value (j = 15 for +, j = 0 for -) and 2^(-d c 2^(E - 134)), d its mantissa steps below it,
// each by fp64 exp2 (a few ulps for the product).  Phase 1 computes those group values and
// step powers into the unused slots past TAB_HALF + 1 (group (s, e, jb) at TAB_SPARE0 +
// 8 e + jb of sign block s; power (e, d) at TAB_SPARE0 + 224 + 8 e + d % 8 of sign block
// d / 8); phase 2 writes every slot, consecutive threads consecutive slots.  The caller's
// barrier (LDS only suffices) follows.
constexpr int TAB_SPARE0 = TAB_HALF + 2;      // the first unused slot of a sign block
constexpr int TAB_GRP = TAB_NE * 8;           // groups per sign
static_assert(TAB_SPARE0 + 2 * TAB_GRP <= TAB_SIGN, "the phase-1 values fit in the unused slots");

// A workgroup barrier that orders LDS only: unlike __syncthreads() it does not wait for the
// wave's global loads, so loads issued before it stay in flight across it.
__device__ __forceinline__ void lds_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 2^(E - 134) for exponent field E = TAB_E0 + e: one mantissa step of that binade
__device__ __forceinline__ double tab_unit(int e)
{
    return __hiloint2double((TAB_E0 + e - 134 + 1023) << 20, 0);
}

// Sentinel k (0..7: table k / 4, sign (k / 2) % 2, below or above) of the tables in `which`:
// NaN (the id takes exp2), or +0.0 above in magnitude for negative values (below -2^8) when
// such a term is at most 2^TAB_TINY_LOG2 of the row's largest, (-2^8 - M) c <= TAB_TINY_LOG2
// (not for contrastive factors).
template <int MODE>
__device__ inline void tab_sentinel(const ExactRows &x, double *tab, int which, int k)
{
    const int tb = k >> 2, s = (k >> 1) & 1, above = k & 1;
    if (!((which >> tb) & 1))
        return;
    double v = __builtin_nan("");
    if (above && s == 1 && !(MODE == CONTRASTIVE && tb == 0)) {
        const double top = (double)(1 << (TAB_E0 + TAB_NE - 127));
        const float M = tb ? x.Mq : x.Mp;
        const double c = tb ? x.cq : x.cp;
        if ((-top - (double)M) * c <= TAB_TINY_LOG2)
            v = 0.0;
    }
    tab[tb * TAB_DOUBLES + s * TAB_SIGN + (above ? TAB_HALF + 1 : 0)] = v;
}

template <int MODE>
__device__ inline void exact_tables(const ExactRows &x, double *tab, int which)
{
    const int t = threadIdx.x;
    // phase 1: per table 2 * TAB_GRP group values and TAB_NE * 16 step powers (as many); then
    // the sentinels (below and above, per sign and table)
    constexpr int P1 = 4 * TAB_GRP;
    for (int k1 = t; k1 < 2 * P1 + 8; k1 += TAIL_WG) {
        if (k1 >= 2 * P1) {
            tab_sentinel<MODE>(x, tab, which, k1 - 2 * P1);
            continue;
        }
        const int tb = k1 >= P1 ? 1 : 0, r = k1 - tb * P1;
        if (!((which >> tb) & 1))
            continue;
        const double c = tb ? x.cq : x.cp;
        double *T = tab + tb * TAB_DOUBLES;
        if (r < 2 * TAB_GRP) {  // group value: sign s, exponent e, mantissas 16 jb ..
            const int s = r >= TAB_GRP ? 1 : 0, g = r - s * TAB_GRP, e = g >> 3, jb = g & 7;
            const double xv = (s ? -1.0 : 1.0) * (double)(128 + 16 * jb + (s ? 0 : 15)) *
                              tab_unit(e);
            double v;
            if (tb == 0 && MODE == CONTRASTIVE)
                v = exp2(xv * c) * (exp2(-x.ea * c * 0.5) * sqrt(x.ra));
            else
                v = exp2((xv - (tb ? x.eb : x.ea)) * c) * (tb ? x.rb : x.ra);
            T[s * TAB_SIGN + TAB_SPARE0 + g] = v;
        } else {  // step power: exponent e, d steps
            const int q = r - 2 * TAB_GRP, e = q >> 4, d = q & 15;
            T[(d >> 3) * TAB_SIGN + TAB_SPARE0 + TAB_GRP + 8 * e + (d & 7)] =
                exp2(-(double)d * tab_unit(e) * c);
        }
    }
    lds_barrier();
    // phase 2: slot 1 + m of sign s, m = 128 e + 16 jb + j
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
        const int tb = ts >> 1, s = ts & 1;
        if (!((which >> tb) & 1))
            continue;
        double *T = tab + tb * TAB_DOUBLES;
        for (int m = t; m < TAB_HALF; m += TAIL_WG) {
            const int e = m >> 7, jb = (m >> 4) & 7, j = m & 15, d = s ? j : 15 - j;
            const double gv = T[s * TAB_SIGN + TAB_SPARE0 + 8 * e + jb];
            const double pw = T[(d >> 3) * TAB_SIGN + TAB_SPARE0 + TAB_GRP + 8 * e + (d & 7)];
            T[s * TAB_SIGN + 1 + m] = gv * pw;
        }
    }
}

// Whether tables of 2^(x c) alone (no row maximum, no scale) stay inside the fp64 range, so
// that they can be built before the accept tests have named row L: |x| < 2^8 with 256 c <= 1000
// (contrastive factors: their products reach 512 c_p).
template <int MODE> __device__ __forceinline__ bool tables_before_rows(double cp, double cq)
{
    return (MODE == SAMPLING ? 256.0 * cp : 512.0 * cp) <= 1000.0 && 256.0 * cq <= 1000.0;
}

// Every slot of table 0 times k0 and of table 1 times k1 (the tables in `which`), and their
// sentinels for the rows' maxima: table 1 takes the draft side's scale kappa when the tables
// were built without one, and the exact scale when the side test is redone.  The caller's
// barrier (LDS only suffices) follows.
template <int MODE>
__device__ inline void exact_rescale(const ExactRows &x, double *tab, double k0, double k1,
                                     int which)
{
    const int t = threadIdx.x;
#pragma unroll
    for (int ts = 0; ts < 4; ++ts) {
        const int tb = ts >> 1, s = ts & 1;
        if (!((which >> tb) & 1))
            continue;
        double *T = tab + tb * TAB_DOUBLES + s * TAB_SIGN + 1;
        const double k = tb ? k1 : k0;
        for (int m = t; m < TAB_HALF; m += TAIL_WG)
            T[m] *= k;
    }
}

// Table 1's tabulated slots (1..TAB_HALF of each sign) times k, from table 1 itself or (from0)
// from table 0, two slots per 16-byte LDS operation: the slot pairs (2 p, 2 p + 1),
// p = 1 .. TAB_HALF / 2 - 1, hold slots 2 .. TAB_HALF - 1, and slots 1 and TAB_HALF (which share
// their pairs with the sentinels 0 and TAB_HALF + 1) are taken singly.  The caller's barrier
// (LDS only suffices) follows.
__device__ inline void scale_table1(double *tab, double k, bool from0)
{
    static_assert(TAB_HALF % 2 == 0 && TAB_SIGN % 2 == 0, "slot pairs");
    const int t = threadIdx.x;
    constexpr int NP = TAB_HALF / 2 - 1;
    const int src = from0 ? 0 : TAB_DOUBLES;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const double2 *F = reinterpret_cast<const double2 *>(tab + src + s * TAB_SIGN);
        double2 *T = reinterpret_cast<double2 *>(tab + TAB_DOUBLES + s * TAB_SIGN);
        for (int p = 1 + t; p <= NP; p += TAIL_WG) {
            const double2 v = F[p];
            T[p] = make_double2(v.x * k, v.y * k);
        }
        if (t == TAIL_WG - 9 - s) {  // slots 1 and TAB_HALF
            const double *G = tab + src + s * TAB_SIGN;
            double *S = tab + TAB_DOUBLES + s * TAB_SIGN;
            S[1] = G[1] * k;
            S[TAB_HALF] = G[TAB_HALF] * k;
        }
    }
}

// One id's a and b from its bit patterns (bfloat16: bp, bq; float32: the float bits): the
// tables where they hold its values, else fp64 exp2.  The pass's slow path and the search use
// this; the pass's fast path reads the same table entries with the same products.
template <int DT, int MODE>
__device__ __forceinline__ void exact_terms(uint32_t bp, uint32_t bq, const ExactRows &x,
                                            double &a, double &b)
{
    bool da = true, db = true;
    if (DT == 1 && x.tabled) {
        const uint32_t op = tab_offset(bp), oq = tab_offset(bq);
        b = tab_at(x.tab, 0x10000u | oq);
        a = tab_at(x.tab, op);
        if (MODE == CONTRASTIVE)
            a *= tab_at(x.tab, oq ^ 0x8000u);
        da = __builtin_isnan(a);
        db = __builtin_isnan(b);
    }
    const double pv = (DT == 1) ? (double)__uint_as_float(bp << 16) : (double)__uint_as_float(bp);
    const double qv = (DT == 1) ? (double)__uint_as_float(bq << 16) : (double)__uint_as_float(bq);
    const double ap = ((MODE == SAMPLING ? pv : pv - qv) - x.ea) * x.cp;
    const double aq = (qv - x.eb) * x.cq;
    if (DT == 1) {
        if (da)
            a = exp2_cold(ap) * x.ra;
        if (db)
            b = exp2_cold(aq) * x.rb;
    } else {
        a = exp2(ap) * x.ra;
        b = exp2(aq) * x.rb;
    }
}

// A lane's sums over one step of its segment: A, B over the positive side (a > b), the totals
// of a and b, and the draft mass of the ids near the threshold.  The table path only flags a
// step with a near id (nf) and leaves its near mass to near_mass_vec, after the segment.
struct ExactLoc {
    double A, B, tp, tq, near;
    bool nf;
};

// whether a and b are near the threshold: upper 32 bits at most NEAR_HI apart
__device__ __forceinline__ bool exact_near(double a, double b)
{
    return absdiff((uint32_t)__double2hiint(a), (uint32_t)__double2hiint(b)) <= NEAR_HI;
}

// the sums of one id, its near flag in l.nf (the table path) or its near mass in l.near (ids
// weighed one by one)
template <bool FLAG>
__device__ __forceinline__ void exact_acc(double a, double b, ExactLoc &l)
{
    const double mv = (a > b) ? 1.0 : 0.0;
    l.A = __builtin_fma(a, mv, l.A);
    l.B = __builtin_fma(b, mv, l.B);
    l.tp += a;
    l.tq += b;
    if (FLAG)
        l.nf = l.nf | exact_near(a, b);
    else
        l.near = __builtin_fma(b, exact_near(a, b) ? 1.0 : 0.0, l.near);
}

// The terms of one 16-byte vector of each row (bfloat16, tables): eight ids, two per word, in
// id order; f(k, a, b) takes each.
template <int MODE, class F>
__device__ __forceinline__ void exact_vec_terms(const uint4 &vp, const uint4 &vq, const char *tab,
                                                const F &f)
{
    const uint32_t P[4] = {vp.x, vp.y, vp.z, vp.w}, Q[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t op = tab_offsets2(P[k]), oq = tab_offsets2(Q[k]);
        const double b0 = tab_at(tab, t1_lo(oq)), b1 = tab_at(tab, t1_hi(oq));
        double a0 = tab_at(tab, t0_lo(op)), a1 = tab_at(tab, t0_hi(op));
        if (MODE == CONTRASTIVE) {
            const uint32_t on = oq ^ 0x80008000u;  // the amateur value negated
            a0 *= tab_at(tab, t0_lo(on));
            a1 *= tab_at(tab, t0_hi(on));
        }
        f(2 * k, a0, b0);
        f(2 * k + 1, a1, b1);
    }
}

template <int MODE>
__device__ __forceinline__ void exact_fast_vec(const uint4 &vp, const uint4 &vq, const char *tab,
                                               ExactLoc &l)
{
    exact_vec_terms<MODE>(vp, vq, tab, [&](int, double a, double b) { exact_acc<true>(a, b, l); });
}

// the draft mass of the near ids of one vector pair (a flagged step, weighed again)
template <int MODE>
__device__ __forceinline__ double near_mass_vec(const uint4 &vp, const uint4 &vq, const char *tab)
{
    double n = 0.0;
    exact_vec_terms<MODE>(vp, vq, tab, [&](int, double a, double b) {
        n = __builtin_fma(b, exact_near(a, b) ? 1.0 : 0.0, n);
    });
    return n;
}

// Geometry of the fp64 pass: the row's wave vectors (64 lanes x one 16-byte vector, WV ids)
// go to nseg = 16 G segments of nsub = nst * NV_EXACT consecutive wave vectors; a wave takes
// NV_EXACT of them per step.
struct ExactGeom {
    int nst, nsub, nseg;
};

template <int DT> __device__ __forceinline__ ExactGeom exact_geom(int V, int G)
{
    constexpr int WV = 64 * Elt<DT>::EPV;
    const int nwv = (V + WV - 1) / WV, per = TAIL_WAVES * G * NV_EXACT;
    ExactGeom gm;
    gm.nst = (nwv + per - 1) / per;
    gm.nsub = gm.nst * NV_EXACT;
    gm.nseg = TAIL_WAVES * G;
    return gm;
}

// Wave vector vw of the two rows, this lane's 16 bytes, loaded nontemporally through the
// rows' buffer resources (past V they read zeros, which the caller does not use).
template <int DT>
__device__ __forceinline__ void exact_fetch(const ExactRows &x, int vw0, uint4 (&rp)[NV_EXACT],
                                            uint4 (&rq)[NV_EXACT])
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES, WV = 64 * E;
    const int vo = (vw0 * WV + (int)(threadIdx.x & 63) * E) * BY;
#pragma unroll
    for (int i = 0; i < NV_EXACT; ++i) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(x.b0, vo + i * WV * BY, 0, 2);
        const u32x4 u = __builtin_amdgcn_raw_buffer_load_b128(x.b1, vo + i * WV * BY, 0, 2);
        rp[i] = make_uint4(v.x, v.y, v.z, v.w);
        rq[i] = make_uint4(u.x, u.y, u.z, u.w);
    }
}

// the lane's E ids of wave vector vw as raw words: the fetched words when the vector is whole
// and the rows aligned, else element loads (bfloat16: two ids per word, the lower in the low
// half; ids >= V are filled with anything and never used)
template <int DT>
__device__ __forceinline__ uint4 exact_words(const char *row, bool al, int e0, int V)
{
    constexpr int E = Elt<DT>::EPV;
    uint4 raw[1];
    if (al && e0 + E <= V) {
        raw[0] = load_plain(row + (size_t)e0 * Elt<DT>::BYTES);
    } else if constexpr (E == 8) {
        raw[0] = pack_bf16(row, e0, V);
    } else {
        uint32_t wd[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            wd[k] = (e0 + k < V) ? __float_as_uint(Elt<DT>::one(row, (size_t)(e0 + k))) : 0u;
        raw[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    }
    return raw[0];
}

// 32-bit word q (0..3) of a 16-byte vector
__device__ __forceinline__ uint32_t word_of(const uint4 &v, int q)
{
    return q == 0 ? v.x : q == 1 ? v.y : q == 2 ? v.z : v.w;
}

// id k (0..E-1) of a vector: its bit pattern (bfloat16 16 bits, float32 32 bits)
template <int DT> __device__ __forceinline__ uint32_t id_bits(const uint4 &v, int k)
{
    if constexpr (Elt<DT>::EPV == 8) {
        const uint32_t wd = word_of(v, k >> 1);
        return (k & 1) ? (wd >> 16) : (wd & 0xffffu);
    } else {
        return word_of(v, k);
    }
}

// One id of the lane by the general path (ids >= V add nothing).
template <int DT, int MODE>
__device__ __forceinline__ void exact_slow_vec(const ExactRows &x, int V, int e0, const uint4 &vp,
                                               const uint4 &vq, ExactLoc &l)
{
    constexpr int E = Elt<DT>::EPV;
    constexpr int KU = (E == 4) ? 4 : 1;  // float32 unrolled: its word index would come from memory
#pragma unroll KU
    for (int k = 0; k < E; ++k) {
        if (e0 + k < V) {
            double a, b;
            exact_terms<DT, MODE>(id_bits<DT>(vp, k), id_bits<DT>(vq, k), x, a, b);
            exact_acc<false>(a, b, l);
        }
    }
}

// One vector of a whole step that read a sentinel: the ids whose two table entries are numbers
// are weighed from them at once, as in the pass (their lookups in flight together), and only the
// others one by one with exp2.  Weighing all sixteen one by one would wait for one table lookup
// at a time while every other wave of the workgroup keeps the LDS busy.
template <int MODE>
__device__ __forceinline__ void exact_fix_vec(const ExactRows &x, const uint4 &vp, const uint4 &vq,
                                              ExactLoc &l)
{
    uint32_t bad = 0;
    exact_vec_terms<MODE>(vp, vq, x.tab, [&](int k, double a, double b) {
        const bool sent = __builtin_isnan(a) || __builtin_isnan(b);
        bad |= (sent ? 1u : 0u) << k;
        exact_acc<false>(sent ? 0.0 : a, sent ? 0.0 : b, l);  // 0 and 0 add nothing
    });
    while (bad) {
        const int k = __builtin_ctz(bad);
        bad &= bad - 1;
        double a, b;
        exact_terms<1, MODE>(id_bits<1>(vp, k), id_bits<1>(vq, k), x, a, b);
        exact_acc<false>(a, b, l);
    }
}

// A step weighed id by id, for one lane: the wave vectors vw0 .. vw0 + NV_EXACT - 1 (ids >= V
// add nothing), from the fetched words when the step is whole, else by element loads.  Out of
// line for bfloat16 rows, where only a step with a value outside the tables (or the row's end,
// or an unaligned row) takes it: the fast path then keeps its registers.
template <int DT, int MODE>
__device__ __forceinline__ ExactLoc exact_step_ids(const ExactRows &x, int V, int vw0, bool whole,
                                                   const uint4 (&rp)[NV_EXACT],
                                                   const uint4 (&rq)[NV_EXACT])
{
    constexpr int E = Elt<DT>::EPV, WV = 64 * E;
    const int lane = threadIdx.x & 63;
    ExactLoc l = {0.0, 0.0, 0.0, 0.0, 0.0, false};
#pragma unroll
    for (int i = 0; i < NV_EXACT; ++i) {
        const int e0 = (vw0 + i) * WV + lane * E;
        if (e0 >= V)
            continue;
        const uint4 vp = whole ? rp[i] : exact_words<DT>(x.p0, x.al, e0, V);
        const uint4 vq = whole ? rq[i] : exact_words<DT>(x.p1, x.al, e0, V);
        exact_slow_vec<DT, MODE>(x, V, e0, vp, vq, l);
    }
    return l;
}

__device__ __forceinline__ void exact_merge(const ExactLoc &l, double &A, double &B, ExactLoc &tot)
{
    A += l.A;
    B += l.B;
    tot.tp += l.tp;
    tot.tq += l.tq;
    tot.near += l.near;
}

// steps of a segment whose words are in registers at once: EXACT_BUFS - 1 in flight while one
// is weighed (float32 rows, whose exp2 needs more registers per id, keep one in flight)
template <int DT> constexpr int exact_bufs() { return 2; }
static_assert((MAX_VOCAB + 64 * 8 - 1) / (64 * 8) <= 64 * TAIL_WAVES * NV_EXACT,
              "a bfloat16 segment has at most 64 steps (one bit each)");

// One segment s by one wave: the lane's positive-side sums (A, B) of the segment, and its
// totals added to tot.  float32 rows weigh every id with exp2.  For bfloat16 rows with tables a
// whole step runs without branches; a step in which the lane read a sentinel (its sums turned
// NaN), and the steps at the row's end or of an unaligned row, only set the step's bit, and
// after the segment the lane weighs those steps again (out of the loop, so that the loop keeps
// its registers for words in flight): a whole step of an aligned row from the tables with
// exp2 for its sentinel ids only, the others id by id.  The buffers rotate through an unrolled
// loop.
template <int DT, int MODE>
__device__ inline void exact_segment(const ExactRows &x, int V, const ExactGeom &gm, int s,
                                     double &A, double &B, ExactLoc &tot,
                                     const uint4 (&p0)[NV_EXACT], const uint4 (&q0)[NV_EXACT],
                                     bool pre)
{
    constexpr int WV = 64 * Elt<DT>::EPV;
    const int vbase = s * gm.nsub, nst = gm.nst;
    A = 0.0;
    B = 0.0;
    uint64_t redo = 0;  // bfloat16: steps to weigh again
    uint64_t nearm = 0; // bfloat16: steps weighed by the tables that hold a near id
    constexpr int EXACT_BUFS = exact_bufs<DT>();
    uint4 bp[EXACT_BUFS][NV_EXACT], bq[EXACT_BUFS][NV_EXACT];
    if (x.al) {
#pragma unroll
        for (int k = 0; k < EXACT_BUFS - 1; ++k) {
            if (k == 0 && pre) {  // the caller's early fetch of step 0
#pragma unroll
                for (int i = 0; i < NV_EXACT; ++i) {
                    bp[0][i] = p0[i];
                    bq[0][i] = q0[i];
                }
            } else if (k < nst) {
                exact_fetch<DT>(x, vbase + k * NV_EXACT, bp[k], bq[k]);
            }
        }
    }
    for (int j0 = 0; j0 < nst; j0 += EXACT_BUFS) {
#pragma unroll
        for (int k = 0; k < EXACT_BUFS; ++k) {
            const int j = j0 + k;
            if (j < nst) {
                // step j + EXACT_BUFS - 1 goes to the buffer that step j - 1 has freed
                const int kf = (k + EXACT_BUFS - 1) % EXACT_BUFS;  // constant once unrolled
                if (j + EXACT_BUFS - 1 < nst && x.al)
                    exact_fetch<DT>(x, vbase + (j + EXACT_BUFS - 1) * NV_EXACT, bp[kf], bq[kf]);
                const int vw0 = vbase + j * NV_EXACT;
                const bool whole = x.al && (vw0 + NV_EXACT) * WV <= V;
                if constexpr (DT == 1) {
                    bool ok = false;
                    if (x.tabled && whole) {
                        ExactLoc l = {0.0, 0.0, 0.0, 0.0, 0.0, false};
#pragma unroll
                        for (int i = 0; i < NV_EXACT; ++i)
                            exact_fast_vec<MODE>(bp[k][i], bq[k][i], x.tab, l);
                        ok = !__builtin_isnan(l.tp) && !__builtin_isnan(l.tq);
                        // selects, not a branch: a branch would let the compiler defer the
                        // sums it guards and keep every looked-up term live until the test
                        A = ok ? A + l.A : A;
                        B = ok ? B + l.B : B;
                        tot.tp = ok ? tot.tp + l.tp : tot.tp;
                        tot.tq = ok ? tot.tq + l.tq : tot.tq;
                        if (ok && l.nf)
                            nearm |= 1ull << j;
                    }
                    if (!ok)
                        redo |= 1ull << j;
                } else {
                    exact_merge(exact_step_ids<DT, MODE>(x, V, vw0, whole, bp[k], bq[k]), A, B,
                                tot);
                }
            }
        }
    }
    if constexpr (DT == 1) {
        // The near mass of the steps with a near id, read and looked up again: a near id is rare
        // (a and b within ~2^-15 of each other), and keeping it out of the loop saves two
        // instructions per id there (24.1-24.8 us against 26.0-26.2 for the pass at B=256,
        // K=8, V=128256).
        while (nearm) {
            const int j = __builtin_ctzll(nearm);
            nearm &= nearm - 1;
            uint4 rp[NV_EXACT], rq[NV_EXACT];
            exact_fetch<DT>(x, vbase + j * NV_EXACT, rp, rq);
            double n = 0.0;
#pragma unroll
            for (int i = 0; i < NV_EXACT; ++i)
                n += near_mass_vec<MODE>(rp[i], rq[i], x.tab);
            tot.near += n;
        }
        while (redo) {  // rare: values outside the tables, the row's end, an unaligned row
            const int j = __builtin_ctzll(redo);
            redo &= redo - 1;
            const int vw0 = vbase + j * NV_EXACT;
            if (x.tabled && x.al && (vw0 + NV_EXACT) * WV <= V) {
                uint4 rp[NV_EXACT], rq[NV_EXACT];
                exact_fetch<DT>(x, vw0, rp, rq);
                ExactLoc l = {0.0, 0.0, 0.0, 0.0, 0.0, false};
#pragma unroll
                for (int i = 0; i < NV_EXACT; ++i)
                    exact_fix_vec<MODE>(x, rp[i], rq[i], l);
                exact_merge(l, A, B, tot);
            } else {
                const uint4 none[NV_EXACT] = {};
                exact_merge(exact_step_ids<DT, MODE>(x, V, vw0, false, none, none), A, B, tot);
            }
        }
    }
}

// The fp64 pass over segments s_first + w, s_first + w + 16, ... below s_end (w the wave):
// units[2 s] = A, units[2 s + 1] = B of each, and the thread's totals in tot.  pre: p0, q0
// hold the first segment's step 0, fetched by the caller.
template <int DT, int MODE>
__device__ inline void exact_pass(const ExactRows &x, int V, const ExactGeom &gm, int s_first,
                                  int s_end, double *units, ExactLoc &tot,
                                  const uint4 (&p0)[NV_EXACT], const uint4 (&q0)[NV_EXACT],
                                  bool pre)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    tot = {0.0, 0.0, 0.0, 0.0, 0.0, false};
    for (int s = s_first + w; s < s_end; s += TAIL_WAVES) {
        double A, B;
        exact_segment<DT, MODE>(x, V, gm, s, A, B, tot, p0, q0, pre && s == s_first + w);
        A = wave_sum(A);
        B = wave_sum(B);
        if (lane == 0) {
            units[2 * s] = A;
            units[2 * s + 1] = B;
        }
    }
}

// The draw weights of the lane's E ids of wave vector vw: max(0, a / S_a - b / S_b) for ids
// on the positive side of the pass's side test (a > b), else 0; ids >= V weigh 0.
template <int DT, int MODE>
__device__ __forceinline__ void exact_vec_weights(const ExactRows &x, int V, int vw, double ia,
                                                  double ib, double (&wv)[Elt<DT>::EPV])
{
    constexpr int E = Elt<DT>::EPV;
    const int e0 = vw * 64 * E + (int)(threadIdx.x & 63) * E;
    const uint4 vp = exact_words<DT>(x.p0, x.al, e0, V), vq = exact_words<DT>(x.p1, x.al, e0, V);
    if constexpr (DT == 1) {
        if (x.tabled && e0 + E <= V) {
            // the eight ids' table entries looked up at once (as in the pass), then exp2 for
            // the ids that read a sentinel: the same terms, products and weights as one by one
            uint32_t bad = 0;
            exact_vec_terms<MODE>(vp, vq, x.tab, [&](int k, double a, double b) {
                const bool sent = __builtin_isnan(a) || __builtin_isnan(b);
                bad |= (sent ? 1u : 0u) << k;
                const double d = a * ia - b * ib;
                wv[k] = (!sent && a > b && d > 0.0) ? d : 0.0;
            });
            if (bad) {
#pragma unroll
                for (int k = 0; k < E; ++k) {
                    if ((bad >> k) & 1u) {
                        double a, b;
                        exact_terms<DT, MODE>(id_bits<DT>(vp, k), id_bits<DT>(vq, k), x, a, b);
                        const double d = a * ia - b * ib;
                        wv[k] = (a > b && d > 0.0) ? d : 0.0;
                    }
                }
            }
            return;
        }
    }
#pragma unroll
    for (int k = 0; k < E; ++k) {
        wv[k] = 0.0;
        if (e0 + k < V) {
            double a, b;
            exact_terms<DT, MODE>(id_bits<DT>(vp, k), id_bits<DT>(vq, k), x, a, b);
            const double d = a * ia - b * ib;
            wv[k] = (a > b && d > 0.0) ? d : 0.0;
        }
    }
}

// The weights of the wave vectors of segment s, by the waves in turn: sub[j] = the sum over
// wave vector s * nsub + j.  Wave w keeps its lanes' id weights of vector w in wv.
template <int DT, int MODE>
__device__ inline void exact_sub_sums(const ExactRows &x, int V, const ExactGeom &gm, int s,
                                      double ia, double ib, double *sub,
                                      double (&wv)[Elt<DT>::EPV])
{
    constexpr int E = Elt<DT>::EPV;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int k = 0; k < E; ++k)
        wv[k] = 0.0;
    for (int j = w; j < gm.nsub; j += TAIL_WAVES) {
        double wt[E];
        exact_vec_weights<DT, MODE>(x, V, s * gm.nsub + j, ia, ib, wt);
        double vs = 0.0;
#pragma unroll
        for (int k = 0; k < E; ++k) {
            vs += wt[k];
            if (j == w)
                wv[k] = wt[k];
        }
        vs = wave_sum(vs);
        if (lane == 0)
            sub[j] = vs;
    }
}

// One wave, for at most 64 segments: the weights A / S_a - B / S_b (clamped at 0) from the
// unit sums, their running totals, W, tt = u01 * W and the first segment whose running total
// exceeds tt (else, rounding at u near 1, the last of positive weight: fb = 1; -1 if W = 0),
// as find_unit_block leaves them; readable after the next barrier.
__device__ inline void find_segment_wave(const double *units, int nseg, double ia, double ib,
                                         float u01, int *s_unit, double *s_base, double *s_t,
                                         int *s_fb, double *s_W)
{
    const int lane = threadIdx.x & 63;
    double wk = 0.0;
    if (lane < nseg) {
        const double d = units[2 * lane] * ia - units[2 * lane + 1] * ib;
        wk = d > 0.0 ? d : 0.0;
    }
    const double inc = wave_incl_scan(wk);
    const double exc = wave_excl_from_incl(inc);
    const double W = lane_value(inc, 63), tt = (double)u01 * W;
    const unsigned long long hm = __ballot(W > 0.0 && wk > 0.0 && exc + wk > tt);
    const unsigned long long pm = __ballot(wk > 0.0);
    const int lh = hm ? __builtin_ctzll(hm) : 0, lp = pm ? 63 - __builtin_clzll(pm) : 0;
    const double bh = lane_value(exc, lh), bl = lane_value(exc, lp);
    if (lane == 0) {
        *s_unit = hm ? lh : (pm ? lp : -1);
        *s_base = hm ? bh : (pm ? bl : 0.0);
        *s_t = tt;
        *s_fb = hm ? 0 : 1;
        *s_W = W;
    }
}

// Wave 0: among the nsub vector weights of the chosen segment (from `base`), the first whose
// running total exceeds tt (unless fb), else the last of positive weight: its index, starting
// total and whether it is a fallback go to s_pick (-1: no vector of the segment has weight, a
// segment whose weight is rounding alone, misclassified ids only, about 1e-16 of W).
__device__ inline void exact_pick_vector(const double *sub, int nsub, double base, double tt,
                                         bool fb, int *s_j, double *s_b, int *s_f)
{
    const int lane = threadIdx.x & 63;
    double carry = base, hb = 0.0, lb = 0.0;
    int hit = -1, lastp = -1;
    for (int j0 = 0; j0 < nsub; j0 += 64) {
        const int j = j0 + lane;
        const double wj = (j < nsub) ? sub[j] : 0.0;
        const double sc = wave_incl_scan(wj);
        const double inc = sc + carry, exc = wave_excl_from_incl(sc) + carry;
        const unsigned long long hm = __ballot(!fb && wj > 0.0 && inc > tt);
        const unsigned long long pm = __ballot(wj > 0.0);
        if (hit < 0 && hm) {
            const int l = __builtin_ctzll(hm);
            hit = j0 + l;
            hb = lane_value(exc, l);
        }
        if (pm) {
            const int l = 63 - __builtin_clzll(pm);
            lastp = j0 + l;
            lb = lane_value(exc, l);
        }
        carry = lane_value(inc, 63);
    }
    if (lane == 0) {
        const bool f = fb || hit < 0;
        *s_j = f ? lastp : hit;
        *s_b = f ? lb : hb;
        *s_f = f ? 1 : 0;
    }
}

// One wave inside wave vector vw with its lanes' id weights wv: the lane by a wave scan from
// `base`, and the id by the lane's walk (the first id whose running weight exceeds tt; fb: the
// last id of positive weight).
template <int DT>
__device__ inline void exact_pick_id(const double (&wv)[Elt<DT>::EPV], int vw, double base,
                                     double tt, bool fb, int32_t *out)
{
    constexpr int E = Elt<DT>::EPV;
    const int lane = threadIdx.x & 63;
    double vs = 0.0;
#pragma unroll
    for (int k = 0; k < E; ++k)
        vs += wv[k];
    const double inc = wave_incl_scan(vs);
    const double bt = base + wave_excl_from_incl(inc);
    const unsigned long long hl = __ballot(!fb && vs > 0.0 && bt + vs > tt);
    const unsigned long long pl = __ballot(vs > 0.0);
    const bool fb3 = fb || hl == 0;
    // the vector's weight is the sum of these lane sums, so some lane has weight
    const int owner = fb3 ? (pl ? 63 - __builtin_clzll(pl) : 63) : __builtin_ctzll(hl);
    if (lane != owner)
        return;
    const int e0 = vw * 64 * E + lane * E;
    double run = bt;
    int y = -1, lastid = -1;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        if (wv[k] > 0.0) {
            run += wv[k];
            lastid = e0 + k;
            if (!fb3 && y < 0 && run > tt)
                y = e0 + k;
        }
    }
    *out = (y >= 0) ? y : lastid;
}

// The block's sums of three per-thread values, in a fixed order (wave sums, then the waves in
// order), into s_out[0..2] after the next barrier.
__device__ inline void block_sum3(double a, double b, double c, double *s_out)
{
    __shared__ double s_red[3][TAIL_WAVES];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    a = wave_sum_lds(a);
    b = wave_sum_lds(b);
    c = wave_sum_lds(c);
    if (lane == 0) {
        s_red[0][w] = a;
        s_red[1][w] = b;
        s_red[2][w] = c;
    }
    __syncthreads();
    if (t == 0) {
        double x = 0.0, y = 0.0, z = 0.0;
        for (int v = 0; v < TAIL_WAVES; ++v) {
            x += s_red[0][v];
            y += s_red[1][v];
            z += s_red[2][v];
        }
        s_out[0] = x;
        s_out[1] = y;
        s_out[2] = z;
    }
}

// Arguments of k_tail.
struct TailArgs {
    const char *tgt, *drf;
    const int32_t *tokens;
    const float *unif;
    const float2 *part;
    int32_t *acc_len, *out_tokens;
    float *out_probs, *draw_probs;
    const int *alive;   // early exit: alive[b] = 1 if every row was read, else the first
                        // `prefix` positions were; NULL: every row was read
    double *gunits;     // split > 1: [B][nu_stride] the unit sums of each sequence's row pass
    int *gcount;        // split > 1: [B] workgroups done with their share; 0 between calls
    const double *gtab; // the per-call tables of 2^(x c) the statistics kernel wrote, or NULL
    Scale sp, sq;
    int K, V, nch, prefix, mask_probs, split, nu_stride;
    unsigned flags;     // TestFlag bits
};

// The draw when its weights are the target law p_L alone (the bonus draw at L = K, which is
// every draw of the sampler).  The row statistics left every chunk's per-wave partials (m, s)
// of p_L, so the chunk sums S_c = sum over the chunk's waves of s * 2^((m - M_p) log2(e)/T) /
// S_p (fp64, in chunk order) locate the chunk that holds t = u * W, W = sum_c S_c, and only
// that chunk is read again (contrastive: the chunk of the expert and of the amateur row).  A
// statistics chunk is NVC vectors per thread of this workgroup (two for sampling rows, one
// for contrastive row pairs), so it is weighed exactly as an iteration of the whole-row pass
// with NVC vectors, into NVC * 16 unit sums; one wave finds the unit holding t and the id
// inside it as that pass does.  The chunk sums carry the fp32 rounding of the statistics
// (about 1e-7 relative each), the same order as the whole-row pass's unit sums.  Returns
// false, having written nothing, if every chunk weighs 0 or rounding leaves the chosen
// chunk's ids without weight; the caller then makes the draw from a pass over the whole row.
template <int DT, int MODE>
__device__ __forceinline__ bool chunk_draw(const TailArgs &a, const DrawRows &r,
                                           const SeqInfo &si, int b, float u01, double *units,
                                           int32_t *out, float *out_prob)
{
    __shared__ int s_c, s_fb, s_u;
    __shared__ double s_base, s_t;
    constexpr bool TWO = (MODE == CONTRASTIVE);
    constexpr int E = Elt<DT>::EPV, NVC = TWO ? 1 : 2, CH = TAIL_WG * NVC * E;
    static_assert(CH == WG * (TWO ? NV_PAIR : NV_STATS) * E,
                  "a statistics chunk is NVC vectors per tail thread");
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, nch = a.nch;
    if (w == 0) {
        const float2 *pr = a.part + ((size_t)b * (2 * a.K + 1) + si.L) * (size_t)nch * WAVES;
        double carry = 0.0;
        for (int c0 = 0; c0 < nch; c0 += 64) {  // units[c] = running total through chunk c
            const int c = c0 + lane;
            double sc = 0.0;
            if (c < nch) {
#pragma unroll
                for (int k = 0; k < WAVES; ++k) {
                    const float2 v = pr[c * WAVES + k];
                    if (v.y > 0.0f)
                        sc += (double)v.y * exp2(((double)v.x - (double)si.Mp) * a.sp.c);
                }
                sc /= si.Sp;
            }
            const double inc = wave_incl_scan(sc) + carry;
            if (c < nch)
                units[c] = inc;
            carry = lane_value(inc, 63);
        }
        // lanes read their neighbours' totals next: keep those reads after the writes
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const double tt = (double)u01 * carry;
        // the first chunk whose running total exceeds tt, else (rounding at u near 1) the
        // last chunk that adds weight
        int hit = -1, lastp = -1;
        for (int c0 = 0; c0 < nch; c0 += 64) {
            const int c = c0 + lane;
            const double inc = (c < nch) ? units[c] : 0.0;
            const double prev = (c < nch && c > 0) ? units[c - 1] : 0.0;
            const unsigned long long hm = __ballot(c < nch && inc > tt);
            const unsigned long long pm = __ballot(c < nch && inc > prev);
            if (hit < 0 && hm)
                hit = c0 + __builtin_ctzll(hm);
            if (pm)
                lastp = c0 + 63 - __builtin_clzll(pm);
        }
        const int ck = (hit >= 0) ? hit : lastp;
        if (lane == 0) {
            s_c = ck;
            s_fb = (hit >= 0) ? 0 : 1;
            s_base = (ck > 0) ? units[ck - 1] : 0.0;
            s_t = tt;
        }
    }
    __syncthreads();
    const int ck = s_c;
    if (ck < 0)
        return false;
    uint4 av[NVC], qv[NVC];
    float vs[NVC];
    tail_load<DT, NVC, TWO>(r, ck * CH, a.V, av, qv);
    tail_weigh<DT, MODE, NVC, TWO>(r, ck * CH + t * E, a.V, false, si, a.sp, a.sq, av, qv, vs);
    tail_store_units<NVC>(0, vs, units);  // the chunk totals were read before the barrier
    __syncthreads();
    if (w == 0) {
        const bool fb = s_fb != 0;
        const double base = s_base, tt = s_t;
        constexpr int NU = NVC * TAIL_WAVES;  // 32 units, in id order
        const double uv = (lane < NU) ? units[lane] : 0.0;
        const double inc = wave_incl_scan(uv);
        const double exc = wave_excl_from_incl(inc);
        const unsigned long long hm = __ballot(!fb && uv > 0.0 && base + inc > tt);
        const unsigned long long pm = __ballot(uv > 0.0);
        const bool fb2 = fb || hm == 0;
        const int un = pm == 0 ? -1 : (fb2 ? 63 - __builtin_clzll(pm) : __builtin_ctzll(hm));
        if (un >= 0)
            search_unit<DT, MODE>(r, si, a.V, NVC, ck * NU + un,
                                      base + lane_value(exc, un), tt, fb2, false, a.sp, a.sq,
                                      out, out_prob);
        if (lane == 0)
            s_u = un;
    }
    __syncthreads();
    return s_u >= 0;
}

// The draw from p_L over the whole row L by one workgroup (the fp32 row pass with the target law):
// after a one-chunk draw that found no weight, or when the residual is empty in fp64 as well.
// Writes -1 (and a NaN probability) for a row without finite logits.
template <int DT, int MODE>
__device__ inline void target_law_draw(const DrawRows &r, const SeqInfo &si, int V, float u01,
                                       const Scale &sp, const Scale &sq, double *units,
                                       int32_t *out, float *out_prob)
{
    __shared__ int s_unit, s_fb;
    __shared__ double s_base, s_t, s_W;
    constexpr int E = Elt<DT>::EPV;
    // a draft-side row read as well: NV_TAIL vectors per row per iteration, else twice as many
    const bool two = (MODE == CONTRASTIVE) || r.two;
    const int nv = two ? NV_TAIL : 2 * NV_TAIL, ce = TAIL_WG * nv * E;
    const int nit = (V + ce - 1) / ce, nu = nit * nv * TAIL_WAVES;
    if (two)
        tail_unit_sums<DT, MODE, NV_TAIL, true>(r, V, nit, 0, 1, true, si, sp, sq, units);
    else if constexpr (MODE == SAMPLING)
        tail_unit_sums<DT, MODE, 2 * NV_TAIL, false>(r, V, nit, 0, 1, true, si, sp, sq, units);
    __syncthreads();
    find_unit_block(units, nu, u01, &s_unit, &s_base, &s_t, &s_fb, &s_W);
    __syncthreads();
    if (s_unit >= 0) {
        if ((threadIdx.x >> 6) == 0)
            search_unit<DT, MODE>(r, si, V, nv, s_unit, s_base, s_t, s_fb != 0, true, sp, sq, out,
                                  out_prob);
    } else if (threadIdx.x == 0) {  // a row without finite logits: outside the contract
        *out = -1;
        if (out_prob)
            *out_prob = NAN;
    }
}

// `split` workgroups of 1024 threads per sequence, after the row statistics.  Each runs the
// accept phase (merge, gather, accept tests, L: the same decisions in every one; the first
// writes the outputs).  A draw from p_L alone (L = K, and the sampler) is made by the first
// workgroup from one chunk of the row (chunk_draw).  A residual draw (L < K) runs the fp64 pass
// over row L and the draft row L, workgroup g's waves taking segments 16 g .. 16 g + 15, into
// per-segment fp64 sums.  With one workgroup it then forms the sums S_a, S_b and the segment
// weights, finds the segment holding t = u_K * W, the wave vector in it and the id.  With
// several, each copies its segment sums to the workspace (device-coherent stores, waited for)
// and counts itself in; the last to arrive reads the others' sums (device-coherent loads),
// resets the count and draws.  If the residual is empty in fp64, that workgroup draws from p_L
// over the whole row.  LDS: the fp64 tables (bfloat16, static, at address 0); dynamic: the
// staged partials during the accept phase, then the unit sums of a draw from p_L or the
// segment sums of the residual draw.
template <int DT, int MODE, bool SPLIT>
__global__ __launch_bounds__(TAIL_WG) void k_tail(const TailArgs a)
{
    // the fp64 tables first, at LDS address 0 (see tab_at); then the dynamic LDS
    constexpr int NTAB = (DT == 1) ? 2 * TAB_DOUBLES : 1;
    __shared__ __attribute__((aligned(65536))) double s_tab[NTAB];
    extern __shared__ double dyn[];
    __shared__ SeqInfo s_info;
    __shared__ int s_unit, s_fb, s_last;
    __shared__ double s_base, s_t, s_W, s_S[3];
    // SPLIT: a.split workgroups share each sequence; else one, and this compiles to the plain
    // single-workgroup pass
    const int G = SPLIT ? a.split : 1, K = a.K, V = a.V;
    const int b = SPLIT ? blockIdx.x / G : blockIdx.x, g = SPLIT ? blockIdx.x - b * G : 0;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    // rows read by this call: every position, or with early exit the first `prefix` ones for
    // a sequence that was not alive after them
    const int npos = (a.alive == nullptr || a.alive[b]) ? K + 1 : a.prefix;
    // bfloat16 verify: the tables of 2^(x c), which depend on the temperatures alone, are read
    // from the per-call tables the statistics kernel wrote (or built, without them, while the
    // partials load); once L is known, table 1 takes the draft side's scale
    const bool pre_tab = DT == 1 && K > 0 && tables_before_rows<MODE>(a.sp.c, a.sq.c);
    const bool copy_tab = pre_tab && a.gtab != nullptr;
    // one law's table serves both when the two laws have the same scale (sampling verify):
    // table 1 is then table 0 times kappa
    const bool one_tab = a.sp.c == a.sq.c;
    if (copy_tab) {
        // 64 or 128 KiB straight from memory into LDS (LDS DMA, no registers), issued first:
        // the tables are cache-resident and arrive with the partials, which any wait for the
        // partials then also covers.  Each wave's load places its lanes' 16-byte pieces at
        // consecutive addresses from the wave's base, so piece i * TAIL_WG + t of the per-call
        // tables lands in slot pair i * TAIL_WG + t.
        const int npiece = one_tab ? 4 : 8;
        for (int i = 0; i < npiece; ++i) {
            const int piece = i * TAIL_WG + w * 64;  // the wave's first piece
            __builtin_amdgcn_global_load_lds(
                reinterpret_cast<const void *>(a.gtab + 2 * (piece + lane)),
                (__attribute__((address_space(3))) void *)(s_tab + 2 * piece), 16, 0, 0);
        }
    }
    struct {
        bool build;
        ExactRows x0;
        double *tab;
        __device__ void operator()() const  // while the partials load
        {
            if (build)
                exact_tables<MODE>(x0, tab, 3);
        }
    } prep;
    prep.build = pre_tab && !copy_tab;
    prep.x0 = {};
    prep.x0.cp = a.sp.c;
    prep.x0.cq = a.sq.c;
    prep.x0.ra = 1.0;
    prep.x0.rb = 1.0;
    prep.tab = s_tab;
    accept_phase<DT, MODE>(a.tgt, a.drf, a.tokens, a.unif, b, K, V, a.nch, npos,
                           a.mask_probs != 0, g == 0, a.sp, a.sq, a.part,
                           reinterpret_cast<float2 *>(dyn), a.acc_len, a.out_tokens, a.out_probs,
                           &s_info, prep, !prep.build);
    if (copy_tab)  // the tables' LDS DMA (not tracked by the compiler's waits on LDS reads)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const SeqInfo si = s_info;
    if (si.L < 0)
        return;
    const DrawRows r = draw_rows<DT, MODE>(a.tgt, a.drf, b, K, V, si.L);
    const float u01 = a.unif[(size_t)b * (K + 1) + K];
    int32_t *out = a.out_tokens + (size_t)b * (K + 1) + si.L;
    float *out_prob = a.draw_probs ? a.draw_probs + b : nullptr;
    if (!r.resid) {  // w = p_L: one chunk of the row is read again, not the whole row
        if (SPLIT && g != 0)
            return;
        if ((a.flags & TEST_CHUNK_FALLBACK) ||
            !chunk_draw<DT, MODE>(a, r, si, b, u01, dyn, out, out_prob))
            target_law_draw<DT, MODE>(r, si, V, u01, a.sp, a.sq, dyn, out, out_prob);
        return;
    }

    // ---- the residual draw, in fp64
    const ExactGeom gm = exact_geom<DT>(V, G);
    // LDS (dynamic): 2 nseg unit sums, then nsub vector weights
    double *units = dyn;
    ExactRows x;
    x.p0 = r.p0;
    x.p1 = r.p1;
    x.b0 = r.b0;
    x.b1 = r.b1;
    x.al = r.al;
    x.Mp = si.Mp;
    x.Mq = si.Mq;
    x.cp = a.sp.c;
    x.cq = a.sq.c;
    x.tabled = (DT == 1) && exact_tabled<MODE>(si.Mp, x.cp, x.cq);
    x.tab = reinterpret_cast<const char *>(s_tab);
    // Unscaled terms when the tables were made before L and every term, and the scale kappa of
    // the draft side, stay inside the fp64 range (|M c| <= 900 on both rows, and their
    // difference, else kappa = 0); else terms relative to the rows' maxima, with tables built
    // for the row.  Either way an id is sorted with the statistics' approximate sums: kappa =
    // 2^(M_p c_p - M_q c_q) S~_p / S~_q (the accept phase's), or r = S~_q / S~_p.
    const double dp = (double)si.Mp * x.cp, dq = (double)si.Mq * x.cq;
    const bool unscaled = DT == 1 && x.tabled && pre_tab && fabs(dp) <= 900.0 &&
                          fabs(dq) <= 900.0 && si.kappa > 0.0;
    if (unscaled) {
        x.ea = 0.0;
        x.eb = 0.0;
        x.ra = 1.0;
        x.rb = si.kappa;
    } else {
        x.ea = si.Mp;
        x.eb = si.Mq;
        x.ra = si.Sq / si.Sp;
        x.rb = 1.0;
    }
    // this wave's first step, loaded while the tables are made
    uint4 p0[NV_EXACT], q0[NV_EXACT];
    const bool pre = x.al && g * TAIL_WAVES + w < gm.nseg;
    if (pre)
        exact_fetch<DT>(x, (g * TAIL_WAVES + w) * gm.nsub, p0, q0);
    if (DT == 1 && x.tabled) {
        if (unscaled) {
            scale_table1(s_tab, x.rb, copy_tab && one_tab);  // table 1 times kappa
            // the sentinels for the rows' maxima (other slots than the scaling's)
            if (t >= TAIL_WG - 8)
                tab_sentinel<MODE>(x, s_tab, 3, t - (TAIL_WG - 8));
        } else {
            exact_tables<MODE>(x, s_tab, 3);
        }
        lds_barrier();
    }
    ExactLoc tot;
    exact_pass<DT, MODE>(x, V, gm, g * TAIL_WAVES, (g + 1) * TAIL_WAVES, units, tot, p0, q0,
                         pre);
    block_sum3(tot.tp, tot.tq, tot.near, s_S);
    __syncthreads();
    const int nseg = gm.nseg;
    if (SPLIT) {
        // gunits of sequence b: 2 sums per segment, then 3 totals per workgroup
        double *gu = a.gunits + (size_t)b * a.nu_stride;
        constexpr int OWN = 2 * TAIL_WAVES;  // this workgroup's segment sums
        if (w == 0) {
            // The sums go out as device-coherent stores, and the wave waits until they are
            // acknowledged before it counts in, so a workgroup that sees the count complete
            // reads every share with device-coherent loads.  (A device fence would also write
            // back the whole L2, which costs more than the draw.)
            if (lane < OWN)
                __hip_atomic_store(gu + g * OWN + lane, units[g * OWN + lane], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            if (lane < 3)
                __hip_atomic_store(gu + 2 * nseg + 3 * g + lane, s_S[lane], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            int last = 0;
            if (lane == 0)
                last = (__hip_atomic_fetch_add(a.gcount + b, 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT) == G - 1);
            last = __shfl(last, 0);
            if (last && lane == 0)  // every share is in: ready for the next call
                __hip_atomic_store(a.gcount + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (lane == 0)
                s_last = last;
        }
        __syncthreads();
        if (!s_last)
            return;
        for (int k = t; k < 2 * nseg; k += TAIL_WG)
            if (k / OWN != g)
                units[k] = __hip_atomic_load(gu + k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (t == 0) {  // the totals of every workgroup, in workgroup order
            double tt3[3] = {0.0, 0.0, 0.0};
            for (int v = 0; v < G; ++v)
                for (int k = 0; k < 3; ++k)
                    tt3[k] += (v == g) ? s_S[k]
                                       : __hip_atomic_load(gu + 2 * nseg + 3 * v + k,
                                                           __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
            s_S[0] = tt3[0];
            s_S[1] = tt3[1];
            s_S[2] = tt3[2];
        }
        __syncthreads();
    }
    double Sa = s_S[0], Sb = s_S[1];
    const double near_b = s_S[2];
    if (!(Sa > 0.0) || !(Sb > 0.0)) {  // a row without finite logits: outside the contract
        __syncthreads();
        target_law_draw<DT, MODE>(r, si, V, u01, a.sp, a.sq, dyn, out, out_prob);
        return;
    }
    static_assert(16 * TAIL_MAX_SPLIT <= TAIL_WG, "one thread per segment");
    double ia = 1.0 / Sa, ib = 1.0 / Sb;
    for (int pass = 0; pass < 2; ++pass) {
        // the segment weights A / S_a - B / S_b and the segment holding t
        if (nseg <= 64) {
            if (w == 0)
                find_segment_wave(units, nseg, ia, ib, u01, &s_unit, &s_base, &s_t, &s_fb, &s_W);
        } else {  // compacted to one double per segment, then the whole workgroup's search
            double wk = 0.0;
            if (t < nseg) {
                const double d = units[2 * t] * ia - units[2 * t + 1] * ib;
                wk = d > 0.0 ? d : 0.0;
            }
            __syncthreads();
            if (t < nseg)
                units[t] = wk;
            __syncthreads();
            find_unit_block(units, nseg, u01, &s_unit, &s_base, &s_t, &s_fb, &s_W);
        }
        __syncthreads();
        // An id may be sorted differently by the exact sums only if a / b lies between 1 and
        // theta = S_a / S_b; each such id moves the weights by at most rel (1 + rel) b / S_b.
        // Keep the draw when the near ids' draft mass bounds that far below the decision scale,
        // else sort again with the draft side scaled by theta (b' = b S_a / S_b against a).
        // theta is a division, not S_a times a rounded 1 / S_b: equal sums (equal rows, an empty
        // residual) must give exactly 1, or every tied id would cross to one side.
        const double theta = Sa / Sb;  // the draft side's new scale over the old one
        const double rel = fabs(theta - 1.0);
        const bool sure = pass == 1 || (rel <= NEAR_REL &&
                                        rel * (1.0 + rel) * near_b * ib <= 0x1p-24 * s_W &&
                                        !(a.flags & TEST_EXACT_TWO_PASS));
        if (sure)
            break;
        x.rb *= theta;
        if (DT == 1 && x.tabled) {
            exact_rescale<MODE>(x, s_tab, 1.0, theta, 2);
            __syncthreads();
        }
        exact_pass<DT, MODE>(x, V, gm, 0, nseg, units, tot, p0, q0, false);
        block_sum3(tot.tp, tot.tq, tot.near, s_S);
        __syncthreads();
        Sa = s_S[0];
        Sb = s_S[1];
        ia = 1.0 / Sa;
        ib = 1.0 / Sb;
    }
    if (s_unit >= 0) {
        // the segment holding t, then its wave vector (each wave weighs one and keeps its
        // lanes' id weights), then the lane and the id
        const int s = s_unit;
        const double tt = s_t;
        double *sub = units + 2 * nseg;
        double wv[Elt<DT>::EPV];
        exact_sub_sums<DT, MODE>(x, V, gm, s, ia, ib, sub, wv);
        __syncthreads();
        if (w == 0)
            exact_pick_vector(sub, gm.nsub, s_base, tt, s_fb != 0, &s_unit, &s_base, &s_fb);
        __syncthreads();
        const int jv = s_unit;
        if (jv < 0) {  // see exact_pick_vector: the segment's first id
            if (t == 0)
                *out = min(s * gm.nsub * 64 * Elt<DT>::EPV, V - 1);
            return;
        }
        if (w == (jv < TAIL_WAVES ? jv : 0)) {
            if (jv >= TAIL_WAVES)  // a vector no wave kept: weigh it again
                exact_vec_weights<DT, MODE>(x, V, s * gm.nsub + jv, ia, ib, wv);
            exact_pick_id<DT>(wv, s * gm.nsub + jv, s_base, tt, s_fb != 0, out);
        }
        return;
    }
    // every weight is 0 in fp64 as well: the residual is empty; draw from p_L
    __syncthreads();
    target_law_draw<DT, MODE>(r, si, V, u01, a.sp, a.sq, dyn, out, out_prob);
}


// ------------------------------------------------------------------ early-exit verify
//
// Rows after a sequence's first rejection are not needed for its tokens.  Early exit reads
// the first `prefix` positions of every sequence (k_stats_prefix), runs their accept tests
// (k_alive: the sequences that accept all of them are listed), reads the remaining rows of
// the listed sequences only (k_stats_rest), and k_tail finishes every sequence from the rows
// it has.  The statistics and the accept tests are the same instructions as the full pass,
// so the decisions are the same.

// the partials of one chunk of one row, as k_stats_sampling computes them
template <int DT>
__device__ __forceinline__ void row_chunk_stats(const char *rp, int V, int c, const Scale &sc,
                                                float2 *dst)
{
    float m, s;
    sampling_chunk_stats<DT>(rp, V, c, sc, m, s);  // as k_stats_sampling: the same bits
    store_wave_partials(wave_stats(m, s, sc), dst);
}

// target rows 0..prefix-1 and draft rows 0..prefix-1 of every sequence (prefix <= K); workgroup
// 0 also clears the survivor count for k_alive
template <int DT>
__global__ __launch_bounds__(WG) void k_stats_prefix(const char *__restrict__ tgt,
                                                     const char *__restrict__ drf, int K, int V,
                                                     int nch, int prefix, Scale sc, float2 *part,
                                                     int *count, TabJob tj)
{
    constexpr int BY = Elt<DT>::BYTES;
    global_tables(tj);
    const int per = 2 * prefix * nch;
    const int b = blockIdx.x / per, rem = blockIdx.x - b * per;
    const int lr = rem / nch, c = rem - lr * nch;
    const bool draft = lr >= prefix;
    const int j = draft ? lr - prefix : lr;
    const char *rp = draft ? drf + ((size_t)b * K + j) * (size_t)V * BY
                           : tgt + ((size_t)b * (K + 1) + j) * (size_t)V * BY;
    const int r = draft ? K + 1 + j : j;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *count = 0;
    row_chunk_stats<DT>(rp, V, c, sc, part + (((size_t)b * (2 * K + 1) + r) * nch + c) * WAVES);
}

// One 256-thread workgroup per sequence: the accept tests at positions 0..prefix-1 on the same
// merged statistics as k_tail.  A sequence with valid ids that accepts all of them is alive:
// alive[b] = 1 and it is appended to list (count = list length); else alive[b] = 0.
template <int DT, int MODE>
__global__ __launch_bounds__(WG) void k_alive(const char *__restrict__ tgt,
                                              const char *__restrict__ drf,
                                              const int32_t *__restrict__ tokens,
                                              const float *__restrict__ unif, int K, int V,
                                              int nch, int prefix, Scale sp, Scale sq,
                                              const float2 *__restrict__ part, int *alive,
                                              int *list, int *count)
{
    __shared__ float2 stage[ACCEPT_STAGE];
    __shared__ float sM[MAX_ROWS];
    __shared__ double sS[MAX_ROWS];
    const int b = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    Draft d = {0, 0.0f, 0.0f, 0.0f, false};
    if (w == 0)
        d = gather_draft<DT, MODE>(tgt, drf, tokens, unif, b, K, V, lane);
    merge_rows<WG>(part, b, K, nch, prefix, sp, sq, stage, sM, sS);
    if (w != 0)
        return;
    bool acc = true;
    if (lane < prefix) {
        double P, Q;
        acc = accept_test(d, lane, K, sM, sS, sp, sq, P, Q);
    }
    const bool live = __ballot(d.bad) == 0 && __ballot(!acc) == 0;
    if (lane == 0) {
        alive[b] = live ? 1 : 0;
        if (live)
            list[atomicAdd(count, 1)] = b;
    }
}

// The rows of positions prefix..K of the listed sequences: item i of count * rows * nch
// (rows = 2K + 1 - 2 prefix per sequence: target rows prefix..K, draft rows prefix..K-1) is one
// chunk of one row, taken by workgroup i mod gridDim in turn; the loop bound is read from the
// count k_alive left, so every workgroup ends.
template <int DT>
__global__ __launch_bounds__(WG) void k_stats_rest(const char *__restrict__ tgt,
                                                   const char *__restrict__ drf, int K, int V,
                                                   int nch, int prefix, Scale sc, float2 *part,
                                                   const int *__restrict__ list,
                                                   const int *__restrict__ count)
{
    constexpr int BY = Elt<DT>::BYTES;
    const int nt = K + 1 - prefix;                       // target rows per sequence
    const int per = (2 * K + 1 - 2 * prefix) * nch;
    const long total = (long)(*count) * per;
    for (long item = blockIdx.x; item < total; item += gridDim.x) {
        const int a = (int)(item / per), rem = (int)(item - (long)a * per);
        const int lr = rem / nch, c = rem - lr * nch;
        const int b = list[a];
        const bool draft = lr >= nt;
        const int j = prefix + (draft ? lr - nt : lr);
        const char *rp = draft ? drf + ((size_t)b * K + j) * (size_t)V * BY
                               : tgt + ((size_t)b * (K + 1) + j) * (size_t)V * BY;
        const int r = draft ? K + 1 + j : j;
        row_chunk_stats<DT>(rp, V, c, sc, part + (((size_t)b * (2 * K + 1) + r) * nch + c) * WAVES);
        __syncthreads();  // the LDS of store_wave_partials is reused by the next item
    }
}

// contrastive: the row pairs of positions 0..prefix-1 of every sequence (prefix <= K);
// workgroup 0 also clears the survivor count for k_alive
template <int DT>
__global__ __launch_bounds__(WG) void k_pairs_prefix(const char *__restrict__ ex,
                                                     const char *__restrict__ am, int K, int V,
                                                     int nch, int prefix, Scale sp, Scale sq,
                                                     float2 *part, int *count, TabJob tj)
{
    global_tables(tj);
    const int pr = blockIdx.x / nch, c = blockIdx.x - pr * nch;
    const int b = pr / prefix, j = pr - b * prefix;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *count = 0;
    pair_chunk_stats<DT>(ex, am, b, j, c, K, V, nch, sp, sq, part);
}

// contrastive: the row pairs of positions prefix..K of the listed sequences, item i of
// count * (K+1-prefix) * nch taken by workgroup i mod gridDim (as k_stats_rest)
template <int DT>
__global__ __launch_bounds__(WG) void k_pairs_rest(const char *__restrict__ ex,
                                                   const char *__restrict__ am, int K, int V,
                                                   int nch, int prefix, Scale sp, Scale sq,
                                                   float2 *part, const int *__restrict__ list,
                                                   const int *__restrict__ count)
{
    const int per = (K + 1 - prefix) * nch;
    const long total = (long)(*count) * per;
    for (long item = blockIdx.x; item < total; item += gridDim.x) {
        const int a = (int)(item / per), rem = (int)(item - (long)a * per);
        const int lr = rem / nch, c = rem - lr * nch;
        pair_chunk_stats<DT>(ex, am, list[a], prefix + lr, c, K, V, nch, sp, sq, part);
    }
}

// ------------------------------------------------------------------ greedy blockwise

// One chunk of a row (rp, V ids): per wave, the max and the first id of the max, stored at
// dst[0..WAVES).  Every greedy pass (the full one and the early-exit prefix and rest) computes a
// chunk with this, so they agree bit for bit.
template <int DT>
__device__ __forceinline__ void chunk_argmax(const char *rp, int V, int c, float2 *dst)
{
    constexpr int E = Elt<DT>::EPV;
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
    store_wave_partials(make_float2(bv, __int_as_float(bi)), dst);
}

// per chunk of a row: (max, first id of the max) per wave.  Logical row r is stored at row
// r * row_stride of the input (1 for [B][K+1][V]; H to take head 0 of [B][K+1][H][V]).
template <int DT>
__global__ __launch_bounds__(WG) void k_argmax(const char *__restrict__ tgt, int V, int nch,
                                               int row_stride, float2 *part)
{
    constexpr int BY = Elt<DT>::BYTES;
    const int row = blockIdx.x / nch, c = blockIdx.x - row * nch;
    chunk_argmax<DT>(tgt + (size_t)row * row_stride * (size_t)V * BY, V, c,
                     part + (size_t)blockIdx.x * WAVES);
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

// ------------------------------------------------------------------ greedy with early exit
//
// A sequence's emitted tokens stop at its first mismatch, so rows after it are not needed.
// k_argmax_prefix takes positions 0..prefix-1 of every sequence, k_alive_greedy lists the
// sequences whose (valid) proposals match the argmax at all of them, k_argmax_rest takes the
// remaining rows of the listed ones, and k_greedy_final finishes every sequence as in the full
// pass: a sequence not listed mismatches inside the prefix (or has a bad id), so the rows it
// did not read are never emitted.

// rows (b, j) for j < prefix, chunk by chunk; workgroup 0 also clears the survivor count
template <int DT>
__global__ __launch_bounds__(WG) void k_argmax_prefix(const char *__restrict__ tgt, int K, int V,
                                                      int nch, int prefix, float2 *part,
                                                      int *count)
{
    constexpr int BY = Elt<DT>::BYTES;
    const int per = prefix * nch;
    const int b = blockIdx.x / per, rem = blockIdx.x - b * per;
    const int j = rem / nch, c = rem - j * nch;
    const size_t row = (size_t)b * (K + 1) + j;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        *count = 0;
    chunk_argmax<DT>(tgt + row * (size_t)V * BY, V, c, part + (row * nch + c) * WAVES);
}

// One 256-thread workgroup per sequence: the argmaxes g_j of rows j < prefix (merged as
// k_greedy_final merges them), then alive iff every proposal id is in [0, V) and x_j == g_j
// for every j < prefix; an alive sequence is appended to list (count = list length).
__global__ __launch_bounds__(WG) void k_alive_greedy(const int32_t *__restrict__ props, int K,
                                                     int V, int nch, int prefix,
                                                     const float2 *__restrict__ part,
                                                     int *list, int *count)
{
    __shared__ int sg[64];
    const int b = blockIdx.x, P = K + 1;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, np = nch * WAVES;
    for (int j = w; j < prefix; j += WAVES) {
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
    const bool miss = (lane < prefix) && xp != sg[lane];
    const bool live = __ballot(bad) == 0 && __ballot(miss) == 0;
    if (lane == 0 && live)
        list[atomicAdd(count, 1)] = b;
}

// The rows of positions prefix..K of the listed sequences: item i of count * rows * nch is one
// chunk of one row, taken by workgroup i mod gridDim in turn; the loop bound is read from the
// count k_alive_greedy left, so every workgroup ends.
template <int DT>
__global__ __launch_bounds__(WG) void k_argmax_rest(const char *__restrict__ tgt, int K, int V,
                                                    int nch, int prefix, float2 *part,
                                                    const int *__restrict__ list,
                                                    const int *__restrict__ count)
{
    constexpr int BY = Elt<DT>::BYTES;
    const int per = (K + 1 - prefix) * nch;
    const long total = (long)(*count) * per;
    for (long item = blockIdx.x; item < total; item += gridDim.x) {
        const int a = (int)(item / per), rem = (int)(item - (long)a * per);
        const int lr = rem / nch, c = rem - lr * nch;
        const size_t row = (size_t)list[a] * (K + 1) + prefix + lr;
        chunk_argmax<DT>(tgt + row * (size_t)V * BY, V, c, part + (row * nch + c) * WAVES);
        __syncthreads();  // the LDS of store_wave_partials is reused by the next item
    }
}

// Greedy blockwise verify with the next block's proposals: one 256-thread workgroup per
// (sequence b, head h = 1..H-1; one per sequence when H = 1).  Each merges head 0's argmax
// partials into g_j for every position (the same merge as k_greedy_final), compares them with
// the proposals and finds L; the head-1 workgroup writes accepted_len and g_0..g_L.  Then each
// takes the first argmax of its head at position L (row ((b*(K+1) + L)*H + h) of the input),
// the next block's proposal from that head: chunk by chunk, the row kept as packed words and
// each value widened as it is compared, so a thread's ids ascend and a strict '>' keeps the
// first maximum; the waves merge by value, then lowest id.  Spreading the heads over
// workgroups (1536 at B=512, H=4) keeps more loads in flight than one workgroup walking a
// sequence's three rows: 46.2 against 48.5 us per call at B=512 K=4 H=4 V=32000 bf16.
template <int DT>
__global__ __launch_bounds__(WG) void k_greedy_heads(const char *__restrict__ logits,
                                                     const int32_t *__restrict__ props, int K,
                                                     int H, int V, int nch,
                                                     const float2 *__restrict__ part,
                                                     int32_t *acc_len, int32_t *out_tokens,
                                                     int32_t *next_props)
{
    constexpr int E = Elt<DT>::EPV, BY = Elt<DT>::BYTES;
    __shared__ int sg[64];
    __shared__ int s_L;
    __shared__ float s_v[WAVES];
    __shared__ int s_i[WAVES];
    const int G = H > 1 ? H - 1 : 1;
    const int b = blockIdx.x / G, h = 1 + (int)(blockIdx.x - b * G);
    const int P = K + 1;
    const int t = threadIdx.x, lane = t & 63, w = t >> 6, np = nch * WAVES;
    // the proposals do not depend on the partials: their load goes out first
    const int32_t xp = (w == 0 && lane < K) ? props[(size_t)b * K + lane] : 0;
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
    const bool writer = (h == 1);  // one workgroup per sequence writes the verify outputs
    if (w == 0) {
        const bool bad = (lane < K) && (xp < 0 || xp >= V);
        int32_t *ot = out_tokens + (size_t)b * (K + 1);
        if (__ballot(bad) != 0) {
            if (writer && lane <= K)
                ot[lane] = -1;
            if (lane == 0) {
                if (writer)
                    acc_len[b] = -1;
                s_L = -1;
            }
        } else {
            const unsigned long long mm = __ballot(lane < K && xp != sg[lane]);
            const int L = mm ? __builtin_ctzll(mm) : K;
            if (writer && lane <= K)
                ot[lane] = (lane <= L) ? sg[lane] : -1;
            if (lane == 0) {
                if (writer)
                    acc_len[b] = L;
                s_L = L;
            }
        }
    }
    __syncthreads();
    const int L = s_L;
    if (H < 2)
        return;
    int32_t *nx = next_props + (size_t)b * (H - 1) + (h - 1);
    if (L < 0) {
        if (t == 0)
            *nx = -1;
        return;
    }
    const char *rp = logits + (((size_t)b * P + L) * H + h) * (size_t)V * BY;
    float bv = -INFINITY;
    int bi = (t * E < V) ? t * E : INT_MAX;  // an all -inf row still reports its lowest id
    for (int c = 0; c < nch; ++c) {
        const int cbase = c * WG * NV_ARGMAX * E;
        if constexpr (E == 8) {
            uint4 raw[NV_ARGMAX];
            load_chunk_words<DT, NV_ARGMAX>(rp, aligned16(rp), cbase, V, raw);
#pragma unroll
            for (int i = 0; i < NV_ARGMAX; ++i) {
                const uint32_t wd[4] = {raw[i].x, raw[i].y, raw[i].z, raw[i].w};
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t hw = wd[k >> 1];
                    const float x = __uint_as_float((k & 1) ? (hw & 0xffff0000u) : (hw << 16));
                    if (x > bv) {
                        bv = x;
                        bi = cbase + (i * WG + t) * E + k;
                    }
                }
            }
        } else {
            float x[NV_ARGMAX][E];
            load_chunk<DT, NV_ARGMAX>(rp, aligned16(rp), cbase, V, x);
#pragma unroll
            for (int i = 0; i < NV_ARGMAX; ++i)
#pragma unroll
                for (int k = 0; k < E; ++k)
                    if (x[i][k] > bv) {
                        bv = x[i][k];
                        bi = cbase + (i * WG + t) * E + k;
                    }
        }
    }
    wave_argmax(bv, bi);
    if (lane == 0) {
        s_v[w] = bv;
        s_i[w] = bi;
    }
    __syncthreads();
    if (t == 0) {
        float v = s_v[0];
        int id = s_i[0];
        for (int k = 1; k < WAVES; ++k)
            take_better(v, id, s_v[k], s_i[k]);
        *nx = id;
    }
}

// ------------------------------------------------------------------ alpha-quantile cut

// float -> uint32 with the same order (negative floats flipped, positive ones offset)
__device__ inline uint32_t order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline float key_to_float(uint32_t k)
{
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// One 1024-thread workgroup per prompt: r_cut = the (k+1)-th smallest of its N scores
// (radix selection on order keys in LDS, one byte per pass from the top), keep[i] =
// (score_i >= r_cut), n_keep = the count.  Comparisons only, so exact.
__global__ __launch_bounds__(TAIL_WG) void k_quantile_cut(const float *__restrict__ scores, int N,
                                                          int k, float *r_cut, uint8_t *keep,
                                                          int32_t *n_keep)
{
    extern __shared__ uint32_t keys[];
    // two histograms and two (prefix, rank) slots alternate between passes, so that a pass
    // needs two barriers: the next pass's bins are cleared while wave 0 scans this pass's
    __shared__ uint32_t hist[2][256];
    __shared__ uint32_t s_prefix[2], s_rank[2];
    __shared__ int s_cnt[TAIL_WAVES];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const float *row = scores + (size_t)blockIdx.x * N;
    for (int i = t; i < N; i += TAIL_WG)
        keys[i] = order_key(row[i]);
    if (t < 256)
        hist[0][t] = 0;
    __syncthreads();
    uint32_t prefix = 0, mask = 0, rank = (uint32_t)k;
    int pb = 0;
    for (int shift = 24; shift >= 0; shift -= 8, pb ^= 1) {
        for (int i = t; i < N; i += TAIL_WG) {
            const uint32_t key = keys[i];
            if ((key & mask) == prefix)
                atomicAdd(&hist[pb][(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (t >= 64 && t < 64 + 256)  // waves 1-4 clear the next pass's bins
            hist[pb ^ 1][t - 64] = 0;
        if (w == 0) {  // lane l owns bins 4l..4l+3: find the bin holding the rank-th key
            uint32_t c[4], sum = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                c[q] = hist[pb][4 * lane + q];
                sum += c[q];
            }
            uint32_t inc = sum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const uint32_t n = __shfl_up(inc, o);
                if (lane >= o)
                    inc += n;
            }
            const uint32_t exc = inc - sum;
            const unsigned long long hit = __ballot(inc > rank);
            const int l = __builtin_ctzll(hit);  // the keys left hold rank, so some lane hits
            if (lane == l) {
                uint32_t below = exc;
                int q = 0;
                while (q < 3 && below + c[q] <= rank) {
                    below += c[q];
                    ++q;
                }
                s_rank[pb] = rank - below;
                s_prefix[pb] = prefix | ((uint32_t)(4 * l + q) << shift);
            }
        }
        __syncthreads();
        rank = s_rank[pb];
        prefix = s_prefix[pb];
        mask |= 0xffu << shift;
    }
    const float cut = key_to_float(prefix);
    int cnt = 0;
    for (int i = t; i < N; i += TAIL_WG) {
        // the score's own bits, back from its order key: compared as floats (-0 == +0)
        const bool kk = key_to_float(keys[i]) >= cut;
        keep[(size_t)blockIdx.x * N + i] = kk ? 1 : 0;
        cnt += kk;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
        cnt += __shfl_xor(cnt, o);
    if (lane == 0)
        s_cnt[w] = cnt;
    __syncthreads();
    if (t == 0) {
        int total = 0;
        for (int q = 0; q < TAIL_WAVES; ++q)
            total += s_cnt[q];
        n_keep[blockIdx.x] = total;
        r_cut[blockIdx.x] = cut;
    }
}

// ------------------------------------------------------------------ launchers

namespace {

// Workgroups per sequence for the tail: enough to give every compute unit a share of the
// draws when the batch is small (at most TAIL_MAX_SPLIT, at most one per step of the fp64
// pass, and only for batches the workspace's unit-sum buffer holds).
int tail_split(const Workspace &ws, int dtype, int B, int V)
{
    if (B < 1 || B > ws.split_batch)
        return 1;
    // steps of NV_EXACT wave vectors of a workgroup's 16 waves in the fp64 pass
    const int wv = 64 * elems_per_vec(dtype), per = TAIL_WAVES * NV_EXACT;
    const int nst = ((V + wv - 1) / wv + per - 1) / per;
    int g = ws.num_cus / B;
    g = g < TAIL_MAX_SPLIT ? g : TAIL_MAX_SPLIT;
    g = g < nst ? g : nst;
    return g > 1 ? g : 1;
}

TailArgs tail_args(const Workspace &ws, int dtype, int B, int K, int V, int nch, const Scale &sp,
                   const Scale &sq, const void *tgt, const void *drf, const int32_t *tokens,
                   const float *unif, int32_t *acc_len, int32_t *out_tokens, float *out_probs,
                   float *draw_probs, const int *alive, int prefix, int mask_probs,
                   const double *gtab)
{
    TailArgs a;
    a.gtab = gtab;
    a.tgt = static_cast<const char *>(tgt);
    a.drf = static_cast<const char *>(drf);
    a.tokens = tokens;
    a.unif = unif;
    a.part = ws.part;
    a.acc_len = acc_len;
    a.out_tokens = out_tokens;
    a.out_probs = out_probs;
    a.draw_probs = draw_probs;
    a.alive = alive;
    a.gunits = ws.gunits;
    a.gcount = ws.gcount;
    a.sp = sp;
    a.sq = sq;
    a.K = K;
    a.V = V;
    a.nch = nch;
    a.prefix = prefix;
    a.mask_probs = mask_probs;
    a.split = tail_split(ws, dtype, B, V);
    a.nu_stride = ws.nu_stride;
    a.flags = ws.test_flags;
    return a;
}

// Launches one kernel on the call's stream.  When its kind is being timed, the kind's start
// and stop events are handed to the dispatch itself (hipExtLaunchKernel stamps them with the
// kernel's own begin and end), so timing puts no marker packets, and no extra gaps, between
// dependent kernels.  Untimed launches are ordinary launches (capturable in a HIP graph).
inline bool timed(const Launch &ln, int kind) { return ln.ev && ((ln.mask >> kind) & 1u); }

#define SV_LAUNCH(ln, kind, kernel, grid, block, lds, ...)                                        \
    do {                                                                                          \
        if (timed((ln), (kind)))                                                                  \
            hipExtLaunchKernelGGL(kernel, (grid), (block), (std::uint32_t)(lds), (ln).stream,     \
                                  (ln).ev[2 * (kind)], (ln).ev[2 * (kind) + 1], 0u, __VA_ARGS__); \
        else                                                                                      \
            hipLaunchKernelGGL(kernel, (grid), (block), (lds), (ln).stream, __VA_ARGS__);         \
    } while (0)

// The sampling statistics over every row of B sequences (2K+1 rows each): two chunks per
// 512-thread workgroup when a row has more than one.
// The draw's per-call tables (bfloat16 verify, K > 0) ride on a statistics launch of `threads`
// work-items when it has one per slot; else NULL and the draw builds them itself.
inline TabJob tab_job(const Workspace &ws, int dtype, int K, const Scale &sp, const Scale &sq,
                      size_t threads)
{
    TabJob tj;
    tj.gtab = (dtype == 1 && K > 0 && threads >= (size_t)GTAB_DOUBLES) ? ws.gtab : nullptr;
    tj.cp = sp.c;
    tj.cq = sq.c;
    return tj;
}

template <int DT>
TabJob launch_stats_sampling(const Launch &ln, const Workspace &ws, int B, int K, int V, int nch,
                             const Scale &sc, const char *t, const char *d)
{
    const size_t rows = (size_t)B * (2 * K + 1);
    if (nch >= 2) {
        const size_t grid = rows * (size_t)((nch + 1) / 2);
        const TabJob tj = tab_job(ws, DT, K, sc, sc, grid * 2 * WG);
        SV_LAUNCH(ln, KIND_STATS, (k_stats_sampling<DT, 2>), dim3((unsigned)grid), dim3(2 * WG),
                  0, t, d, K, V, nch, sc, ws.part, tj);
        return tj;
    }
    const TabJob tj = tab_job(ws, DT, K, sc, sc, rows * WG);
    SV_LAUNCH(ln, KIND_STATS, (k_stats_sampling<DT, 1>), dim3((unsigned)rows), dim3(WG), 0, t, d,
              K, V, nch, sc, ws.part, tj);
    return tj;
}

template <int DT>
TabJob launch_stats_contrastive(const Launch &ln, const Workspace &ws, int B, int K, int V,
                                int nch, const Scale &sp, const Scale &sq, const char *t,
                                const char *d)
{
    const size_t pairs = (size_t)B * (K + 1);
    if (nch >= 2) {
        const size_t grid = pairs * (size_t)((nch + 1) / 2);
        const TabJob tj = tab_job(ws, DT, K, sp, sq, grid * 2 * WG);
        SV_LAUNCH(ln, KIND_STATS, (k_stats_contrastive<DT, 2>), dim3((unsigned)grid),
                  dim3(2 * WG), 0, t, d, K, V, nch, sp, sq, ws.part, tj);
        return tj;
    }
    const TabJob tj = tab_job(ws, DT, K, sp, sq, pairs * WG);
    SV_LAUNCH(ln, KIND_STATS, (k_stats_contrastive<DT, 1>), dim3((unsigned)pairs), dim3(WG), 0,
              t, d, K, V, nch, sp, sq, ws.part, tj);
    return tj;
}

template <int DT, int MODE>
void launch_tail(const Launch &ln, const TailArgs &a, int B, size_t lds)
{
    if (a.split > 1)
        SV_LAUNCH(ln, KIND_TAIL, (k_tail<DT, MODE, true>), dim3((unsigned)(B * a.split)),
                  dim3(TAIL_WG), lds, a);
    else
        SV_LAUNCH(ln, KIND_TAIL, (k_tail<DT, MODE, false>), dim3((unsigned)B), dim3(TAIL_WG), lds,
                  a);
}

template <int DT, int MODE>
hipError_t sampling_impl(const Launch &ln, const Workspace &ws, int B, int K, int V,
                         const Scale &sp, const Scale &sq, const void *tgt, const void *drf,
                         const int32_t *tokens, const float *unif, int32_t *acc_len,
                         int32_t *out_tokens, float *out_probs, float *draw_probs)
{
    const char *t = static_cast<const char *>(tgt);
    const char *d = static_cast<const char *>(drf);
    const int nch = num_chunks(MODE == SAMPLING ? NV_STATS : NV_PAIR, DT, V);
    TabJob tj;
    if (MODE == SAMPLING) {
        tj = launch_stats_sampling<DT>(ln, ws, B, K, V, nch, sp, t, d);
    } else {
        tj = launch_stats_contrastive<DT>(ln, ws, B, K, V, nch, sp, sq, t, d);
    }
    const TailArgs a = tail_args(ws, DT, B, K, V, nch, sp, sq, tgt, drf, tokens, unif, acc_len,
                                 out_tokens, out_probs, draw_probs, nullptr, K + 1, 0, tj.gtab);
    launch_tail<DT, MODE>(ln, a, B, tail_lds_bytes(DT, K, V, nch));
    return hipGetLastError();
}

template <int DT>
hipError_t greedy_early_impl(const Launch &ln, const Workspace &ws, int B, int K, int V,
                             const void *tgt, const int32_t *props, int32_t *acc_len,
                             int32_t *out_tokens, int rest_grid)
{
    const int nch = num_chunks(NV_ARGMAX, DT, V);
    const char *t = static_cast<const char *>(tgt);
    const int prefix = EARLY_PREFIX_GREEDY < K + 1 ? EARLY_PREFIX_GREEDY : K + 1;
    if (prefix == K + 1) {  // every position is in the prefix: one full pass
        SV_LAUNCH(ln, KIND_ARGMAX, k_argmax<DT>, dim3((unsigned)((size_t)B * (K + 1) * nch)),
                  dim3(WG), 0, t, V, nch, 1, ws.part);
    } else {
        SV_LAUNCH(ln, KIND_ARGMAX, k_argmax_prefix<DT>, dim3((unsigned)((size_t)B * prefix * nch)),
                  dim3(WG), 0, t, K, V, nch, prefix, ws.part, ws.count);
        SV_LAUNCH(ln, KIND_EARLY_ACCEPT, k_alive_greedy, dim3(B), dim3(WG), 0, props, K, V, nch,
                  prefix, ws.part, ws.list, ws.count);
        const size_t items = (size_t)B * (K + 1 - prefix) * nch;
        const unsigned grid = (unsigned)(items < (size_t)rest_grid ? items : rest_grid);
        SV_LAUNCH(ln, KIND_EARLY_REST, k_argmax_rest<DT>, dim3(grid), dim3(WG), 0, t, K, V, nch,
                  prefix, ws.part, ws.list, ws.count);
    }
    SV_LAUNCH(ln, KIND_GREEDY_EMIT, k_greedy_final, dim3(B), dim3(WG), 0, props, K, V, nch, ws.part,
              acc_len, out_tokens);
    return hipGetLastError();
}

template <int DT>
hipError_t greedy_impl(const Launch &ln, const Workspace &ws, int B, int K, int V, const void *tgt,
                       const int32_t *props, int32_t *acc_len, int32_t *out_tokens)
{
    const int nch = num_chunks(NV_ARGMAX, DT, V);
    const unsigned grid = (unsigned)((size_t)B * (K + 1) * nch);
    SV_LAUNCH(ln, KIND_ARGMAX, k_argmax<DT>, dim3(grid), dim3(WG), 0,
              static_cast<const char *>(tgt), V, nch, 1, ws.part);
    SV_LAUNCH(ln, KIND_GREEDY_EMIT, k_greedy_final, dim3(B), dim3(WG), 0, props, K, V, nch, ws.part,
              acc_len, out_tokens);
    return hipGetLastError();
}

template <int DT, int MODE>
hipError_t early_exit_impl(const Launch &ln, const Workspace &ws, int B, int K, int V,
                           const Scale &sp, const Scale &sq, const void *tgt, const void *drf,
                           const int32_t *tokens, const float *unif, int32_t *acc_len,
                           int32_t *out_tokens, float *out_probs, int rest_grid)
{
    const char *t = static_cast<const char *>(tgt);
    const char *d = static_cast<const char *>(drf);
    const int nch = num_chunks(MODE == SAMPLING ? NV_STATS : NV_PAIR, DT, V);
    const int prefix = EARLY_PREFIX < K + 1 ? EARLY_PREFIX : K + 1;
    const int *alive = nullptr;
    TabJob tj;
    if (prefix == K + 1) {  // every position is in the prefix: one full pass
        if (MODE == SAMPLING) {
            tj = launch_stats_sampling<DT>(ln, ws, B, K, V, nch, sp, t, d);
        } else {
            tj = launch_stats_contrastive<DT>(ln, ws, B, K, V, nch, sp, sq, t, d);
        }
    } else {
        if (MODE == SAMPLING) {
            const size_t grid = (size_t)B * 2 * prefix * nch;
            tj = tab_job(ws, DT, K, sp, sq, grid * WG);
            SV_LAUNCH(ln, KIND_STATS, k_stats_prefix<DT>, dim3((unsigned)grid), dim3(WG), 0, t, d,
                      K, V, nch, prefix, sp, ws.part, ws.count, tj);
        } else {
            const size_t grid = (size_t)B * prefix * nch;
            tj = tab_job(ws, DT, K, sp, sq, grid * WG);
            SV_LAUNCH(ln, KIND_STATS, k_pairs_prefix<DT>, dim3((unsigned)grid), dim3(WG), 0, t, d,
                      K, V, nch, prefix, sp, sq, ws.part, ws.count, tj);
        }
        SV_LAUNCH(ln, KIND_EARLY_ACCEPT, (k_alive<DT, MODE>), dim3(B), dim3(WG), 0, t, d, tokens,
                  unif, K, V, nch, prefix, sp, sq, ws.part, ws.alive, ws.list, ws.count);
        const size_t rows = (MODE == SAMPLING) ? (size_t)(2 * K + 1 - 2 * prefix)
                                               : (size_t)(K + 1 - prefix);
        const size_t items = (size_t)B * rows * nch;
        const unsigned grid = (unsigned)(items < (size_t)rest_grid ? items : rest_grid);
        if (MODE == SAMPLING)
            SV_LAUNCH(ln, KIND_EARLY_REST, k_stats_rest<DT>, dim3(grid), dim3(WG), 0, t, d, K, V,
                      nch, prefix, sp, ws.part, ws.list, ws.count);
        else
            SV_LAUNCH(ln, KIND_EARLY_REST, k_pairs_rest<DT>, dim3(grid), dim3(WG), 0, t, d, K, V,
                      nch, prefix, sp, sq, ws.part, ws.list, ws.count);
        alive = ws.alive;
    }
    const TailArgs a = tail_args(ws, DT, B, K, V, nch, sp, sq, tgt, drf, tokens, unif, acc_len,
                                 out_tokens, out_probs, nullptr, alive, prefix, 1, tj.gtab);
    launch_tail<DT, MODE>(ln, a, B, tail_lds_bytes(DT, K, V, nch));
    return hipGetLastError();
}

template <int DT>
hipError_t greedy_heads_impl(const Launch &ln, const Workspace &ws, int B, int K, int H, int V,
                             const void *logits, const int32_t *props, int32_t *acc_len,
                             int32_t *out_tokens, int32_t *next_props)
{
    const int nch = num_chunks(NV_ARGMAX, DT, V);
    const char *lg = static_cast<const char *>(logits);
    const unsigned grid = (unsigned)((size_t)B * (K + 1) * nch);
    SV_LAUNCH(ln, KIND_ARGMAX, k_argmax<DT>, dim3(grid), dim3(WG), 0, lg, V, nch, H, ws.part);
    const int G = H > 1 ? H - 1 : 1;  // workgroups per sequence: one per proposal head
    SV_LAUNCH(ln, KIND_GREEDY_EMIT, k_greedy_heads<DT>, dim3((unsigned)((size_t)B * G)), dim3(WG),
              0, lg, props, K, H, V, nch, ws.part, acc_len, out_tokens, next_props);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_early_exit(const Launch &ln, const Workspace &ws, int mode, int dtype, int B,
                             int K, int V, const Scale &sp, const Scale &sq, const void *tgt,
                             const void *drf, const int32_t *tokens, const float *unif,
                             int32_t *acc_len, int32_t *out_tokens, float *out_probs,
                             int rest_grid)
{
    auto f = (mode == SAMPLING)
                 ? (dtype == 1 ? early_exit_impl<1, SAMPLING> : early_exit_impl<0, SAMPLING>)
                 : (dtype == 1 ? early_exit_impl<1, CONTRASTIVE> : early_exit_impl<0, CONTRASTIVE>);
    return f(ln, ws, B, K, V, sp, sq, tgt, drf, tokens, unif, acc_len, out_tokens, out_probs,
             rest_grid);
}

hipError_t launch_greedy_heads(const Launch &ln, const Workspace &ws, int dtype, int B, int K,
                               int H, int V, const void *logits, const int32_t *props,
                               int32_t *acc_len, int32_t *out_tokens, int32_t *next_props)
{
    auto f = dtype == 1 ? greedy_heads_impl<1> : greedy_heads_impl<0>;
    return f(ln, ws, B, K, H, V, logits, props, acc_len, out_tokens, next_props);
}

hipError_t launch_quantile_cut(const Launch &ln, int P, int N, int k, const float *scores,
                               float *r_cut, uint8_t *keep, int32_t *n_keep)
{
    SV_LAUNCH(ln, KIND_CUT, k_quantile_cut, dim3(P), dim3(TAIL_WG), (size_t)N * sizeof(uint32_t),
              scores, N, k, r_cut, keep, n_keep);
    return hipGetLastError();
}

// ------------------------------------------------------------------ static scratch
//
// The workspace of specverify_run_sampling_static, for callers that cannot allocate: one
// array per device, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory, so host code uses only the address hipGetSymbolAddress returns
// for the current device, taken once per device and kept.
static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];

namespace {
std::mutex scratch_mu;
std::atomic<void *> scratch_at[STATIC_SCRATCH_DEVICES];
}  // namespace

hipError_t static_scratch(int device, void **ptr)
{
    if (device < 0 || device >= STATIC_SCRATCH_DEVICES)
        return hipErrorInvalidDevice;
    void *p = scratch_at[device].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(scratch_mu);
        p = scratch_at[device].load(std::memory_order_relaxed);
        if (!p) {
            const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess)
                return e;
            if (!p)
                return hipErrorInvalidSymbol;
            scratch_at[device].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return hipSuccess;
}

__global__ __launch_bounds__(WG) void k_zero_ints(int *p, int n)
{
    for (int i = threadIdx.x; i < n; i += WG)
        p[i] = 0;
}

hipError_t launch_zero_ints(hipStream_t stream, int *p, int n)
{
    if (n > 0)
        hipLaunchKernelGGL(k_zero_ints, dim3(1), dim3(WG), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_sampling(const Launch &ln, const Workspace &ws, int mode, int dtype, int B,
                           int K, int V, const Scale &sp, const Scale &sq, const void *tgt,
                           const void *drf, const int32_t *tokens, const float *unif,
                           int32_t *acc_len, int32_t *out_tokens, float *out_probs,
                           float *draw_probs)
{
    auto f = (mode == SAMPLING) ? (dtype == 1 ? sampling_impl<1, SAMPLING> : sampling_impl<0, SAMPLING>)
                                : (dtype == 1 ? sampling_impl<1, CONTRASTIVE>
                                              : sampling_impl<0, CONTRASTIVE>);
    return f(ln, ws, B, K, V, sp, sq, tgt, drf, tokens, unif, acc_len, out_tokens, out_probs,
             draw_probs);
}

hipError_t launch_greedy(const Launch &ln, const Workspace &ws, int dtype, int B, int K, int V,
                         const void *tgt, const int32_t *props, int32_t *acc_len,
                         int32_t *out_tokens)
{
    return dtype == 1 ? greedy_impl<1>(ln, ws, B, K, V, tgt, props, acc_len, out_tokens)
                      : greedy_impl<0>(ln, ws, B, K, V, tgt, props, acc_len, out_tokens);
}

hipError_t launch_greedy_early_exit(const Launch &ln, const Workspace &ws, int dtype, int B, int K,
                                    int V, const void *tgt, const int32_t *props,
                                    int32_t *acc_len, int32_t *out_tokens, int rest_grid)
{
    return dtype == 1
               ? greedy_early_impl<1>(ln, ws, B, K, V, tgt, props, acc_len, out_tokens, rest_grid)
               : greedy_early_impl<0>(ln, ws, B, K, V, tgt, props, acc_len, out_tokens, rest_grid);
}

}  // namespace sv
