"""Residual draws at a small residual mass, and the draw paths that data rarely reaches, through
the C-ABI against the oracle (needs an MI355X).

A draft that is the target plus very little noise rejects with a residual max(0, p - q) of mass
W between about 1e-6 and 1e-2 (and exactly 0 where the rows are equal).  A weight's error enters
the draw as (error) / W, so the library computes the residual draw in fp64 from the logits; every
sequence must satisfy the parity rule, whatever W is.  Test flags then force the fp64 draw's
exact second pass and the whole-row fallback of a draw from p alone, each against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import compare, compare_sample, oracle_whole_batch, run, run_sample
from rejection_sampling_verification_row_amd import binding as sv
from rejection_sampling_verification_row_amd import synth
from rejection_sampling_verification_row_amd.synth import BF16, F32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    h = sv.specverify_create(0, 256, 8, 160000)
    yield h
    sv.specverify_destroy(h)


class flags:
    """Test flags on a context for the duration of a with-block."""

    def __init__(self, ctx, bits):
        self.ctx, self.bits = ctx, bits

    def __enter__(self):
        sv.specverify_set_test_flags(self.ctx, self.bits)

    def __exit__(self, *exc):
        sv.specverify_set_test_flags(self.ctx, 0)


def residual_mass(w, j=0):
    """W = sum max(0, p_j - q_j) per sequence, from the oracle's fp64 softmax."""
    t = synth.decode(w.target[:, j], w.dtype).astype(np.float64)
    d = synth.decode(w.draft[:, j], w.dtype).astype(np.float64)
    out = np.empty(w.B)
    for b in range(w.B):
        if w.mode == synth.CONTRASTIVE:
            p = oracle.softmax((t[b] - d[b]) / w.temperature)
            q = oracle.softmax(d[b])
        else:
            p = oracle.softmax(t[b] / w.temperature)
            q = oracle.softmax(d[b] / w.temperature)
        out[b] = np.maximum(p - q, 0.0).sum()
    return out


def _report(name, rep, extra=""):
    print("\n[%s] %s%s" % (name, rep, extra), flush=True)


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_small_residual_mass_at_full_vocabulary(ctx, dtype):
    """B = 256, V = 128256: position 0 rejects with W spread over 1e-6..1e-2; at least 60
    sequences draw at W in [1e-4, 2e-3], and every sequence meets the parity rule."""
    w = synth.make_small_residual(256, 128256, dtype, 0.7, seed=7101 + dtype)
    print("\n[small residual %s] generated" % synth.DTYPE_NAMES[dtype], flush=True)
    g = run(ctx, w)
    o = oracle_whole_batch(w)
    rep = compare(w, g, o)
    W = residual_mass(w)
    rej = o.accepted_len == 0
    band = rej & (W >= 1e-4) & (W <= 2e-3)
    _report("small residual %s" % synth.DTYPE_NAMES[dtype], rep,
            "; %d rejections at position 0, %d with W in [1e-4, 2e-3], smallest W %.3g"
            % (rej.sum(), band.sum(), W[rej].min()))
    assert band.sum() >= 60
    assert (rej & (W < 1e-4)).sum() >= 5          # and some below the range as well


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_small_residual_mass_contrastive(ctx, dtype):
    """Contrastive verify with the amateur at half the expert plus little noise, so that the two
    laws nearly coincide, and an accept uniform just under 1: rejections at small W."""
    w = synth.make_contrastive(128, 2, 152064, dtype, 1.0, seed=7201 + dtype,
                               amateur_scale=0.5, amateur_sigma=0.01)
    w.uniforms[:, :2] = np.float32(1.0 - 2.0 ** -13)
    g = run(ctx, w)
    o = oracle_whole_batch(w)
    rep = compare(w, g, o)
    W = residual_mass(w)
    rej = o.accepted_len == 0
    _report("contrastive small residual %s" % synth.DTYPE_NAMES[dtype], rep,
            "; %d rejections at position 0, W from %.3g to %.3g"
            % (rej.sum(), W[rej].min() if rej.any() else np.nan,
               W[rej].max() if rej.any() else np.nan))
    assert rej.sum() >= 20 and W[rej].max() < 0.05


@pytest.mark.parametrize("two_pass", [False, True])
@pytest.mark.parametrize("dtype", [BF16, F32])
def test_empty_residual_draws_from_the_target(ctx, dtype, two_pass):
    """Equal target and draft rows at position 0 with the draft token at an id whose logit is
    -inf in both: P = 0 rejects it, the residual is empty (W = 0 exactly), and the replacement
    is drawn from p_0, as the oracle does.  With the exact second pass forced as well: the two
    rows' equal sums give the draft side a scale of exactly 1 (a ratio formed with a rounded
    reciprocal had pushed every tied id to the positive side, a residual of about 1e-17)."""
    w = synth.make_small_residual(24, 50000, dtype, 0.9, seed=7301 + dtype)
    ninf = synth.f32_to_bf16_bits(np.float32([-np.inf]))[0] if dtype == BF16 else np.float32(-np.inf)
    for b in range(w.B):
        w.draft[b, 0] = w.target[b, 0]
        x = int(w.tokens[b, 0])
        w.target[b, 0, x] = ninf
        w.draft[b, 0, x] = ninf
    if two_pass:
        with flags(ctx, sv.SPECVERIFY_TEST_EXACT_TWO_PASS):
            g = run(ctx, w)
    else:
        g = run(ctx, w)
    o = oracle.run_workload(w)
    rep = compare(w, g, o)
    _report("empty residual %s" % synth.DTYPE_NAMES[dtype], rep)
    assert np.all(o.accepted_len == 0) and np.all(g.accepted_len == 0)
    assert np.all(residual_mass(w) == 0.0)


@pytest.mark.parametrize("cfg", ["c2", "c3", "c5"])
def test_fp64_second_pass_at_full_size(ctx, cfg):
    """The fp64 draw's exact second pass forced for every residual draw of the full-size
    sampling and contrastive workloads, against the oracle for every sequence, and bit-equal to
    the one-pass draw wherever the oracle's margins are clear."""
    w = synth.CONFIGS[cfg]()
    h = sv.specverify_create(0, w.B, w.K, w.V)
    try:
        one = run(h, w)
        with flags(h, sv.SPECVERIFY_TEST_EXACT_TWO_PASS):
            g = run(h, w)
    finally:
        sv.specverify_destroy(h)
    o = oracle_whole_batch(w)
    rep = compare(w, g, o)
    _report("%s fp64 second pass" % w.name, rep)
    clear = (o.margin_accept >= oracle.LOW_MARGIN) & (o.margin_sample >= oracle.LOW_MARGIN)
    assert np.array_equal(one.out_tokens[clear], g.out_tokens[clear])


SHAPES = [
    ("sampling", BF16, 9, 3, 1001),
    ("sampling", F32, 7, 2, 16385),
    ("sampling", BF16, 5, 4, 70001),
    ("sampling", F32, 3, 1, 2),
    ("contrastive", BF16, 6, 2, 33000),
    ("contrastive", F32, 5, 3, 4099),
]


def _shape(mode, dtype, B, K, V, seed):
    if mode == "sampling":
        return synth.make_sampling(B, K, V, dtype, 0.85, seed, target_sigma=2.5, draft_sigma=1.0)
    return synth.make_contrastive(B, K, V, dtype, 1.3, seed)


@pytest.mark.parametrize("mode,dtype,B,K,V", SHAPES)
@pytest.mark.parametrize("misalign", [0, 1])
@pytest.mark.parametrize("bits", [0, 2], ids=["fp64", "fp64-two-pass"])
def test_fp64_residual_draw_small_shapes(ctx, mode, dtype, B, K, V, misalign, bits):
    """The fp64 draw (and its exact second pass) on ragged and unaligned rows of both types."""
    w = _shape(mode, dtype, B, K, V, seed=7400 + B * 5 + K + V % 97)
    with flags(ctx, bits):
        g = run(ctx, w, misalign=misalign)
    rep = compare(w, g, oracle.run_workload(w))
    _report("%s %s B=%d K=%d V=%d misalign=%d flags=%d" % (mode, synth.DTYPE_NAMES[dtype], B, K,
                                                           V, misalign, bits), rep)


def test_fp64_two_pass_at_small_residual_mass(ctx):
    w = synth.make_small_residual(96, 128256, BF16, 0.7, seed=7501)
    with flags(ctx, sv.SPECVERIFY_TEST_EXACT_TWO_PASS):
        g = run(ctx, w)
    rep = compare(w, g, oracle_whole_batch(w))
    _report("small residual, fp64 second pass", rep)


@pytest.mark.parametrize("dtype,B,K,V", [(BF16, 6, 3, 16384 * 3 + 5), (F32, 150, 2, 8192 * 4),
                                         (BF16, 160, 1, 40000)])
@pytest.mark.parametrize("misalign", [0, 1])
def test_whole_row_fallback_of_the_bonus_draw(ctx, dtype, B, K, V, misalign):
    """An identical draft accepts every token; with the chunk draw switched off the bonus draw
    from p_K weighs the whole row (the path taken when rounding leaves the chosen chunk empty)."""
    w = synth.make_sampling(B, K, V, dtype, 0.9, seed=7600 + B + V, target_sigma=2.5,
                            draft_sigma=0.0)
    with flags(ctx, sv.SPECVERIFY_TEST_CHUNK_FALLBACK):
        g = run(ctx, w, misalign=misalign)
    o = oracle.run_workload(w)
    rep = compare(w, g, o)
    _report("bonus draws by the whole-row pass %s B=%d" % (synth.DTYPE_NAMES[dtype], B), rep)
    assert np.all(g.accepted_len == K)


@pytest.mark.parametrize("dtype,N,V", [(BF16, 256, 128256), (F32, 40, 30001)])
def test_whole_row_fallback_of_the_sampler(ctx, dtype, N, V):
    w = synth.make_sampler(N, V, dtype, 0.7, seed=7700 + N, sigma=4.0, n_peaks=20)
    with flags(ctx, sv.SPECVERIFY_TEST_CHUNK_FALLBACK):
        tok, pr = run_sample(ctx, w)
    o = oracle.sample_rows(w.dtype, N, V, w.temperature, w.target, w.uniforms.reshape(N))
    rep = compare_sample(w, tok, pr, o)
    _report("sampler by the whole-row pass %s N=%d" % (synth.DTYPE_NAMES[dtype], N), rep)


def test_test_flags_are_checked(ctx):
    with pytest.raises(sv.SpecVerifyError) as ei:
        sv.specverify_set_test_flags(ctx, 4)
    assert ei.value.status == sv.SPECVERIFY_EINVAL
    sv.specverify_set_test_flags(ctx, 0)
