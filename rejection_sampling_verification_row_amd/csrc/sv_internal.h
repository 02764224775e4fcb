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
constexpr int NV_ARGMAX = 8;          // greedy argmax
constexpr int MAX_ROWS = 2 * 63 + 1;  // rows per sequence at the largest K

// The per-sequence tail (accept scan + draw) runs one 1024-thread workgroup per sequence;
// its pass over row L loads NV_TAIL vectors per thread per row and iteration when the draft
// row L is read too, 2 * NV_TAIL when only the target row is (64 KiB per iteration either
// way, the next iteration's loads in flight while the current one is weighed), and keeps one
// fp64 weight sum per wave and vector slot ("unit") in LDS.
constexpr int TAIL_WG = 1024;
constexpr int TAIL_WAVES = TAIL_WG / 64;
constexpr int NV_TAIL = 2;
constexpr int ACCEPT_STAGE = 3072;    // float2 partials staged in LDS by the accept phase
constexpr int MAX_VOCAB = 1 << 20;    // keeps the unit sums within 32 KiB of LDS
constexpr int MAX_CUT_N = 8192;       // scores per prompt of the quantile cut (32 KiB of LDS)
constexpr int EARLY_PREFIX = 2;       // positions every sequence reads before early exit
constexpr int EARLY_PREFIX_GREEDY = 3; // the same for greedy verify (B=512 K=8 V=32000, proposals
                                      // matching w.p. 0.7: 39.1 us against 41.2 with 2 and 39.5 with 4)
constexpr int TAIL_MAX_SPLIT = 8;     // most workgroups that share one sequence's draw

// The residual draw (L < K) is made in fp64 from the logits of row L (see exact_pass in the
// kernels): the row's wave vectors (64 lanes x 16 bytes) go to 16 contiguous segments per
// workgroup sharing the draw, a wave streams its segment NV_EXACT wave vectors per step, and a
// segment's unit sums are two fp64 values.  bfloat16 kernels also hold two 64 KiB tables in LDS.
constexpr int NV_EXACT = 2;

// The bfloat16 tables of the residual draw: one slot per bit pattern with 2^-20 <= |x| < 2^8.
constexpr int TAB_E0 = 107;               // bfloat16 exponent field of 2^-20
constexpr int TAB_NE = 28;                // fields 107..134: 2^-20 <= |x| < 2^8
constexpr int TAB_LO = TAB_E0 << 7;       // the smallest tabulated magnitude's 15 low bits
constexpr int TAB_HALF = TAB_NE * 128;    // tabulated magnitudes per sign
// Each sign's block is 4096 doubles: slot 0 takes magnitudes below the tabulated ones, slots
// 1..TAB_HALF the tabulated ones, slot TAB_HALF + 1 those above; the sign is bit 15 of the
// slot's byte offset and table 1 lies 64 KiB after table 0.
constexpr int TAB_SIGN = 4096;
constexpr int TAB_DOUBLES = 2 * TAB_SIGN;  // one table: 64 KiB
static_assert(TAB_HALF + 2 <= TAB_SIGN && TAB_SIGN * 8 == 0x8000, "slot byte offsets are 15 bits");
constexpr double TAB_TINY_LOG2 = -80.0;   // a term 2^-80 or less of the row's largest counts as 0
// The per-call tables of 2^(x c) (no row maximum, no scale) that the statistics kernels write for
// the draw: table 0 for the target law's c, table 1 for the draft law's, in the LDS layout.
constexpr int GTAB_DOUBLES = 2 * TAB_DOUBLES;
struct TabJob {
    double *gtab;   // NULL: no tables this call
    double cp, cq;  // log2(e) / T of the two laws
};

// test-only switches (specverify_set_test_flags): reach draw paths that data rarely reaches
enum TestFlag : unsigned {
    TEST_CHUNK_FALLBACK = 1u,   // a draw from p_L alone skips the chunk draw: whole-row pass
    TEST_EXACT_TWO_PASS = 2u,   // the fp64 residual pass always runs its exact second pass
    TEST_FLAGS_ALL = 3u
};

inline int elems_per_vec(int dtype) { return dtype == 1 ? 8 : 4; }
inline int chunk_elems(int nv, int dtype) { return WG * nv * elems_per_vec(dtype); }
inline int num_chunks(int nv, int dtype, int V)
{
    return (V + chunk_elems(nv, dtype) - 1) / chunk_elems(nv, dtype);
}
// the most chunks any pass needs for a row of V ids (float32 pairs have the smallest chunks)
inline int max_chunks(int V) { return num_chunks(NV_PAIR, 0, V); }
// unit sums of one row pass: NV_TAIL vectors per thread and iteration when two rows are read,
// 2 * NV_TAIL when one is; the LDS holds the larger count
inline int tail_units(int dtype, int V)
{
    int most = 0;
    for (int nv = NV_TAIL; nv <= 2 * NV_TAIL; nv += NV_TAIL) {
        const int ce = TAIL_WG * nv * elems_per_vec(dtype);
        const int n = (V + ce - 1) / ce * nv * TAIL_WAVES;
        most = n > most ? n : most;
    }
    return most;
}
// segments of the fp64 residual pass of one sequence (16 per workgroup sharing the draw)
constexpr int EXACT_MAX_SEGS = TAIL_WAVES * TAIL_MAX_SPLIT;
// wave vectors per segment of the fp64 residual pass with one workgroup (the most)
inline int exact_seg_vectors(int dtype, int V)
{
    const int wv = 64 * elems_per_vec(dtype), nwv = (V + wv - 1) / wv;
    const int per = TAIL_WAVES * NV_EXACT;
    return (nwv + per - 1) / per * NV_EXACT;
}
// dynamic LDS of the tail kernel: the staged partials, then (reusing it) the unit sums of the
// fp32 pass of a draw from p_L, or the residual pass's two fp64 sums per segment and one
// weight per wave vector of a segment
inline size_t tail_lds_bytes(int dtype, int K, int V, int nch)
{
    const size_t parts = (size_t)(2 * K + 1) * nch * WAVES;
    const size_t stage = parts <= (size_t)ACCEPT_STAGE ? parts * 8 : 0;
    const size_t units = (size_t)tail_units(dtype, V) * 8;
    const size_t exact = (size_t)(2 * EXACT_MAX_SEGS + exact_seg_vectors(dtype, V)) * 8;
    size_t m = stage > units ? stage : units;
    return m > exact ? m : exact;
}

// log2(e) / T split into two floats so that d * hi + d * lo carries ~48 bits of the
// product: the exponent argument of every term then loses only one fp32 rounding.
// lo is kept strictly positive so that d = -inf yields -inf rather than NaN.
struct Scale {
    float hi, lo;
    double c;        // log2(e) / T in double, for the fp64 combination steps
    double inv_t;    // 1 / T in double, for the exact gathered probabilities
};
Scale make_scale(double temperature);

// What the draw needs to know about one sequence after the accept scan.
// For the target row L (p) and the draft row L (q, L < K) with maximum M and sum S:
// R = fl(M * hi) and is = 2^-e / S, e = fma(M, lo, fma(M, hi, -R)), so that a probability is
// exp2(fma(x, lo, fma(x, hi, -R))) * is, the same form as the row statistics.
struct SeqInfo {
    int L;           // first rejected position, K if none, -1 for bad ids
    float Rp, Rq;
    float isp, isq;
    float Mp, Mq;    // maximum and merged sum (fp64) of the target row L and the draft row L
    double Sp, Sq;
    double kappa;    // L < K: 2^(M_p c_p - M_q c_q) S_p / S_q, the residual draw's draft-side
                     // scale for terms without the rows' maxima (0 if out of range)
};

enum Mode { SAMPLING = 0, CONTRASTIVE = 1 };

struct Workspace {
    float2 *part;       // [rows][nch][WAVES] per-wave (max, sum of exp2) or (max, id) partials
    int *alive;         // [B] early exit: 1 if the sequence accepted its first positions
    int *list;          // [B] early exit: the alive sequences, in no particular order
    int *count;         // early exit: the number of alive sequences
    double *gunits;     // [split_batch][nu_stride] fp64 unit sums and per-workgroup totals of a
                        // residual draw shared by workgroups
    int *gcount;        // [split_batch] arrival counts of those workgroups, 0 between calls
    double *gtab;       // [GTAB_DOUBLES] the draw's tables of 2^(x c), written by the statistics
                        // kernels of each call (NULL: the draw builds them itself)
    int split_batch;    // largest batch whose draws may be shared (0: never)
    int nu_stride;      // doubles per sequence in gunits
    int num_cus;        // compute units of the device
    unsigned test_flags; // TestFlag bits (0 in normal use)
};

struct Launch {
    hipStream_t stream;
    hipEvent_t *ev;     // NULL, or 2 events per kernel kind (start, stop)
    unsigned mask;      // kernel kinds whose events are recorded
};

// kernel kinds for timing
enum Kind {
    KIND_STATS = 0,
    KIND_TAIL = 1,
    KIND_ARGMAX = 2,
    KIND_GREEDY_EMIT = 3,
    KIND_CUT = 4,
    KIND_EARLY_ACCEPT = 5,
    KIND_EARLY_REST = 6,
    NUM_KINDS = 7
};

// Sampling or contrastive verify (mode), or, with K = 0, acc_len = NULL and draw_probs set,
// one draw per row (the draft-token sampler).  draw_probs [B]: the drawn token's probability
// under the target law p_L (sampling mode only; may be NULL).
hipError_t launch_sampling(const Launch &ln, const Workspace &ws, int mode, int dtype, int B,
                           int K, int V, const Scale &sp, const Scale &sq, const void *tgt,
                           const void *drf, const int32_t *tokens, const float *unif,
                           int32_t *acc_len, int32_t *out_tokens, float *out_probs,
                           float *draw_probs);

// Sampling or contrastive verify (mode) reading rows only up to each sequence's first
// rejection: the first EARLY_PREFIX positions of every sequence, then the rest of the
// sequences that accepted them (the rest pass runs rest_grid workgroups over that work).
// Tokens and accepted_len as launch_sampling; out_probs for j <= L only (NaN after).
hipError_t launch_early_exit(const Launch &ln, const Workspace &ws, int mode, int dtype, int B,
                             int K, int V, const Scale &sp, const Scale &sq, const void *tgt,
                             const void *drf, const int32_t *tokens, const float *unif,
                             int32_t *acc_len, int32_t *out_tokens, float *out_probs,
                             int rest_grid);

// greedy verify over [B][K+1][H][V] head logits (head 0 verifies) plus next_props [B][H-1],
// the first argmaxes of heads 1..H-1 at the emitted position
hipError_t launch_greedy_heads(const Launch &ln, const Workspace &ws, int dtype, int B, int K,
                               int H, int V, const void *logits, const int32_t *props,
                               int32_t *acc_len, int32_t *out_tokens, int32_t *next_props);

// per prompt of N scores: r_cut = the (k+1)-th smallest, keep = score >= r_cut, n_keep
hipError_t launch_quantile_cut(const Launch &ln, int P, int N, int k, const float *scores,
                               float *r_cut, uint8_t *keep, int32_t *n_keep);

// The workspace of the entry point that allocates nothing: a file-scope device array of
// STATIC_SCRATCH_BYTES per device (see static_scratch in the kernels' source).
constexpr size_t STATIC_SCRATCH_BYTES = size_t(4) << 20;
constexpr int STATIC_SCRATCH_DEVICES = 64;
// The device address of the current device's scratch array, taken once per device with
// hipGetSymbolAddress (device: the current device's index).
hipError_t static_scratch(int device, void **ptr);
// n ints from p set to 0 by a small kernel (capturable in a HIP graph, unlike a memset node)
hipError_t launch_zero_ints(hipStream_t stream, int *p, int n);

hipError_t launch_greedy(const Launch &ln, const Workspace &ws, int dtype, int B, int K, int V,
                         const void *tgt, const int32_t *props, int32_t *acc_len,
                         int32_t *out_tokens);

// greedy verify reading rows only up to each sequence's first mismatch: the first
// EARLY_PREFIX_GREEDY positions of every sequence, then the rest of the sequences that matched
// them (rest_grid workgroups); accepted_len and out_tokens exactly as launch_greedy
hipError_t launch_greedy_early_exit(const Launch &ln, const Workspace &ws, int dtype, int B, int K,
                                    int V, const void *tgt, const int32_t *props,
                                    int32_t *acc_len, int32_t *out_tokens, int rest_grid);

}  // namespace sv
