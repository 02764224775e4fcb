// Internal interface between the C-ABI runtime (specverify.cpp) and the gfx950 kernels
// (sv_kernels.hip).  Not installed; the public interface is include/specverify.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// Work geometry.  A row of V logits is cut into chunks aligned to element ids: chunk c of a
// pass with NV vectors per thread covers ids [c*CE, (c+1)*CE), CE = WG * NV * (16 / bytes).
// One 256-thread workgroup handles one chunk; thread t loads vectors i*WG + t, i < NV, so a
// wave's loads are 1 KiB contiguous.
constexpr int WG = 256;               // threads per workgroup (4 wave64)
constexpr int WAVES = WG / 64;
constexpr int NV_STATS = 8;           // sampling row statistics: 32 KiB per workgroup
constexpr int NV_PAIR = 4;            // contrastive row pairs: 2 x 16 KiB per workgroup
constexpr int NV_RESID = 8;           // residual / bonus weights
constexpr int NV_ARGMAX = 8;          // greedy argmax
constexpr int MAX_ROWS = 2 * 63 + 1;  // rows per sequence at the largest K

inline int elems_per_vec(int dtype) { return dtype == 1 ? 8 : 4; }
inline int chunk_elems(int nv, int dtype) { return WG * nv * elems_per_vec(dtype); }
inline int num_chunks(int nv, int dtype, int V)
{
    return (V + chunk_elems(nv, dtype) - 1) / chunk_elems(nv, dtype);
}
// the most chunks any pass needs for a row of V ids (float32 pairs have the smallest chunks)
inline int max_chunks(int V) { return num_chunks(NV_PAIR, 0, V); }

// log2(e) / T split into two floats so that d * hi + d * lo carries ~48 bits of the
// product: the exponent argument of every term then loses only one fp32 rounding.
// lo is kept strictly positive so that d = -inf yields -inf rather than NaN.
struct Scale {
    float hi, lo;
    double c;        // log2(e) / T in double, for the fp64 combination steps
    double inv_t;    // 1 / T in double, for the exact gathered probabilities
};
Scale make_scale(double temperature);

// What the residual / bonus pass needs to know about one sequence after the accept scan.
struct SeqInfo {
    int L;           // first rejected position, K if none, -1 for bad ids
    float Mp, Mq;    // row maxima of the target row L and of the draft row L (L < K)
    float isp, isq;  // 1 / S of those rows
    int pad[3];
};

enum Mode { SAMPLING = 0, CONTRASTIVE = 1 };

struct Workspace {
    float2 *part;       // [rows][nch][WAVES] per-wave (max, sum of exp2) or (max, id) partials
    SeqInfo *seq;       // [B]
    double *resid;      // [B][nch][NV_RESID] draw-weight totals of each chunk's vector rows
};

struct Launch {
    hipStream_t stream;
    hipEvent_t *ev;     // NULL, or 2 events per kernel kind to time (start, stop)
};

// kernel kinds for timing
enum Kind {
    KIND_STATS = 0,
    KIND_ACCEPT = 1,
    KIND_RESID = 2,
    KIND_DRAW = 3,
    KIND_ARGMAX = 4,
    KIND_GREEDY_EMIT = 5,
    NUM_KINDS = 6
};

hipError_t launch_sampling(const Launch &ln, const Workspace &ws, int mode, int dtype, int B,
                           int K, int V, const Scale &sp, const Scale &sq, const void *tgt,
                           const void *drf, const int32_t *tokens, const float *unif,
                           int32_t *acc_len, int32_t *out_tokens, float *out_probs);

hipError_t launch_greedy(const Launch &ln, const Workspace &ws, int dtype, int B, int K, int V,
                         const void *tgt, const int32_t *props, int32_t *acc_len,
                         int32_t *out_tokens);

}  // namespace sv
