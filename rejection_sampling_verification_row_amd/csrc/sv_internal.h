// Internal interface between the C-ABI runtime (specverify.cpp) and the gfx950 kernels
// (sv_kernels.hip).  Not installed; the public interface is include/specverify.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sv {

// Work geometry shared by every streaming kernel.  A row of V logits is cut into chunks of
// CHUNK_VECS 16-byte vectors; one 256-thread workgroup handles one chunk, each thread NV
// vectors.  Chunks are aligned to element indices (chunk c covers ids [c*CE, (c+1)*CE)).
constexpr int WG = 256;               // threads per workgroup (4 wave64)
constexpr int NV = 8;                 // 16-byte vectors per thread per chunk
constexpr int CHUNK_VECS = WG * NV;   // 2048 vectors = 32 KiB of logits per chunk

inline int elems_per_vec(int dtype) { return dtype == 1 ? 8 : 4; }
inline int chunk_elems(int dtype) { return CHUNK_VECS * elems_per_vec(dtype); }
inline int num_chunks(int dtype, int V) { return (V + chunk_elems(dtype) - 1) / chunk_elems(dtype); }
// the most chunks any dtype needs for a row of V ids (float32 rows have the smaller chunks)
inline int max_chunks(int V) { return num_chunks(0, V); }

// log2(e) / T split into two floats so that d * hi + d * lo carries ~48 bits of the
// product: the exponent argument of every term then loses only one fp32 rounding.
// lo is kept strictly positive so that d = -inf yields -inf rather than NaN.
struct Scale {
    float hi, lo;
    double c;        // log2(e) / T in double, for the fp64 combination steps
    double inv_t;    // 1 / T in double, for the exact gathered probabilities
};
Scale make_scale(double temperature);

// What the draw kernels need to know about one sequence after the accept scan.
struct SeqInfo {
    int L;           // first rejected position, K if none, -1 for bad ids
    int pad;
    float Mp, Mq;    // row maxima of the target row L and of the draft row L (L < K)
    double inv_sp;   // 1 / S of target row L
    double inv_sq;   // 1 / S of draft row L (L < K)
};

enum Mode { SAMPLING = 0, CONTRASTIVE = 1 };

struct Workspace {
    float *part_m;      // [rows][nch] chunk maxima (also argmax values in greedy mode)
    double *part_s;     // [rows][nch] chunk sums of exp2((l - m) * c), relative to part_m
    int *part_i;        // [rows][nch] chunk argmax ids (greedy)
    SeqInfo *seq;       // [B]
    double *resid;      // [B][nch][2] chunk sums of the draw weights: residual, target law
};

struct Launch {
    hipStream_t stream;
    hipEvent_t *ev;     // NULL, or 2 events per kernel to time (start, stop)
};

hipError_t launch_sampling(const Launch &ln, const Workspace &ws, int mode, int dtype, int B,
                           int K, int V, const Scale &sp, const Scale &sq, const void *tgt,
                           const void *drf, const int32_t *tokens, const float *unif,
                           int32_t *acc_len, int32_t *out_tokens, float *out_probs);

hipError_t launch_greedy(const Launch &ln, const Workspace &ws, int dtype, int B, int K, int V,
                         const void *tgt, const int32_t *props, int32_t *acc_len,
                         int32_t *out_tokens);

}  // namespace sv
