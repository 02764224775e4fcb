"""GPU parity of the operations next to the verify step (needs an MI355X): the draft-token
sampler, greedy verify with the next block's proposals, and the alpha-quantile cut, each
through the C-ABI against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import compare_sample, dev, run_cut, run_heads, run_sample
from rejection_sampling_verification_row_amd import binding as sv
from rejection_sampling_verification_row_amd import synth
from rejection_sampling_verification_row_amd.synth import BF16, F32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    h = sv.specverify_create(0, 1024, 16, 160000)
    yield h
    sv.specverify_destroy(h)


# ----------------------------------------------------------------- draft-token sampler

def test_sampler_full_size(ctx):
    w = synth.sampler_draft_rows()
    tok, pr = run_sample(ctx, w)
    rep = compare_sample(w, tok, pr, oracle.run_workload(w))
    print("\n[%s] %s" % (w.name, rep), flush=True)


@pytest.mark.parametrize("dtype,N,V", [(F32, 3, 1), (F32, 17, 7), (BF16, 9, 2), (BF16, 33, 1001),
                                       (F32, 5, 32769), (BF16, 6, 65537), (BF16, 4, 131072)])
@pytest.mark.parametrize("misalign", [0, 1])
def test_sampler_small_shapes(ctx, dtype, N, V, misalign):
    w = synth.make_sampler(N, V, dtype, 0.9, seed=300 + N + V, sigma=2.0)
    tok, pr = run_sample(ctx, w, misalign=misalign)
    compare_sample(w, tok, pr, oracle.run_workload(w))


U_LO, U_HI = 0.5 * 2.0 ** -23, 1.0 - 2.0 ** -24   # the two ends of the uniforms' lattice


@pytest.mark.parametrize("dtype", [F32, BF16])
@pytest.mark.parametrize("misalign", [0, 1])
def test_sampler_sparse_rows_and_extreme_uniforms(ctx, dtype, misalign):
    """All weight in a few ids of a few chunks (every other logit -inf), in some rows only in
    the ragged last chunk, with uniforms at the two ends of their lattice and in the middle:
    the draw finds its chunk from the row statistics' chunk sums, and at u near 1 rounding
    can leave t at the end of the row (the last id of positive weight is then drawn)."""
    N, V = 30, 3 * 16384 + 777
    w = synth.make_sampler(N, V, dtype, 1.0, seed=4242, sigma=2.0)
    rng = np.random.default_rng(4243)
    x = np.full((N, V), -np.inf, np.float32)
    for n in range(N):
        ids = (np.array([V - 1 - n]) if n % 3 == 0
               else rng.choice(V, size=1 + n % 5, replace=False))
        x[n, ids] = rng.normal(0.0, 1.5, ids.size).astype(np.float32)
    w.target = synth.f32_to_bf16_bits(x) if dtype == BF16 else x
    w.uniforms = np.array([[U_LO], [U_HI], [0.5]] * (N // 3), np.float32)
    tok, pr = run_sample(ctx, w, misalign=misalign)
    compare_sample(w, tok, pr, oracle.run_workload(w))
    finite = np.isfinite(x)
    assert all(finite[n, tok[n]] for n in range(N))


@pytest.mark.parametrize("dtype,V", [(F32, 8192 * 5 + 3), (BF16, 16384 * 7 + 1), (BF16, 16384 * 2),
                                     (F32, 8192 * 100 + 7), (F32, 1 << 20), (BF16, (1 << 20) - 3)])
def test_sampler_uniforms_across_the_lattice(ctx, dtype, V):
    """Uniforms spread over the whole lattice on dense rows of several chunks (so that t falls
    in every chunk in turn), whole and ragged last chunks; float32 rows of more than 64 chunks
    carry the chunks' running total from one 64-chunk block to the next."""
    N = 64
    w = synth.make_sampler(N, V, dtype, 0.8, seed=77 + V, sigma=1.0)
    w.uniforms = ((np.arange(N, dtype=np.float64) + 0.5) / N).astype(np.float32).reshape(N, 1)
    big = V > 160000   # beyond the module context's vocabulary: a context of its own
    h = sv.specverify_create(0, N, 0, V) if big else ctx
    try:
        tok, pr = run_sample(h, w)
    finally:
        if big:
            sv.specverify_destroy(h)
    compare_sample(w, tok, pr, oracle.run_workload(w))


def test_sampler_matches_verify_with_no_draft(ctx):
    """The sampler is the K = 0 case of sampling verify: same ids for the same rows."""
    w = synth.make_sampler(64, 5000, BF16, 0.7, seed=17, sigma=3.0)
    tok, _ = run_sample(ctx, w, with_probs=False)
    acc = torch.empty(64, dtype=torch.int32, device="cuda")
    out = torch.empty((64, 1), dtype=torch.int32, device="cuda")
    sv.specverify_run_sampling(ctx, None, BF16, 64, 0, w.V, w.temperature, dev(w.target), None,
                               None, dev(w.uniforms), acc, out)
    torch.cuda.synchronize()
    assert np.array_equal(tok, out.cpu().numpy()[:, 0])


def _raw(*xs):
    """Device addresses as plain integers: the binding passes them unchecked, so these tests
    reach the library's own host-side checks (they refuse before any launch)."""
    return tuple(x if x is None or isinstance(x, int) else x.data_ptr() for x in xs)


def test_sampler_errors(ctx):
    w = synth.make_sampler(2, 10, F32, 1.0, seed=1)
    lg, u = dev(w.target), dev(w.uniforms.reshape(2))
    tok = torch.full((2,), 9, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="logits"):   # the binding: N x V beyond the tensor
        sv.specverify_sample(ctx, None, F32, 2000, 10, 1.0, lg, u, tok)
    lg, u, tok_p = _raw(lg, u, tok)
    E = sv.SpecVerifyError
    for args, want in [((F32, 2, 10, 0.0, lg, u, tok), sv.SPECVERIFY_EINVAL),
                       ((F32, 2, 10, 1.0, None, u, tok), sv.SPECVERIFY_EINVAL),
                       ((F32, 2000, 10, 1.0, lg, u, tok), sv.SPECVERIFY_ECAPACITY),
                       ((F32, 2, 200000, 1.0, lg, u, tok), sv.SPECVERIFY_ECAPACITY),
                       ((5, 2, 10, 1.0, lg, u, tok), sv.SPECVERIFY_EUNSUPPORTED)]:
        args = args[:-1] + (tok_p,)
        with pytest.raises(E) as ei:
            sv.specverify_sample(ctx, None, *args)
        assert ei.value.status == want
    sv.specverify_sample(ctx, None, F32, 0, 10, 1.0, None, None, None)  # N = 0: no-op
    torch.cuda.synchronize()
    assert torch.all(tok == 9)


# ----------------------------------------------------------------- greedy with next proposals

def _check_heads(w, acc, tok, nxt):
    o = oracle.run_workload(w)
    assert np.array_equal(acc, o.accepted_len)
    assert np.array_equal(tok, o.out_tokens)
    assert np.array_equal(nxt, o.next_proposals)


def test_heads_full_size(ctx):
    w = synth.greedy_heads_blockwise()
    _check_heads(w, *run_heads(ctx, w))


@pytest.mark.parametrize("dtype,B,K,H,V", [(BF16, 7, 3, 1, 50), (F32, 9, 0, 3, 33),
                                           (BF16, 12, 4, 2, 1001), (F32, 5, 6, 5, 16400),
                                           (BF16, 6, 15, 4, 40003), (BF16, 3, 2, 3, 1)])
@pytest.mark.parametrize("misalign", [0, 1])
def test_heads_small_shapes(ctx, dtype, B, K, H, V, misalign):
    # coarse values so that ties (first occurrence) are frequent
    w = synth.make_greedy_heads(B, K, H, V, dtype, seed=500 + B + K + H + V, sigma=1.0)
    _check_heads(w, *run_heads(ctx, w, misalign=misalign))


def test_heads_bad_ids(ctx):
    w = synth.make_greedy_heads(4, 3, 3, 100, BF16, seed=9)
    w.tokens[2, 1] = 100
    acc, tok, nxt = run_heads(ctx, w)
    assert acc[2] == -1 and np.all(tok[2] == -1) and np.all(nxt[2] == -1)
    _check_heads(w, acc, tok, nxt)


def test_heads_with_one_head_equals_greedy(ctx):
    w = synth.make_greedy_heads(16, 5, 1, 3000, BF16, seed=4)
    acc, tok, _ = run_heads(ctx, w)
    a2 = torch.empty(16, dtype=torch.int32, device="cuda")
    t2 = torch.empty((16, 6), dtype=torch.int32, device="cuda")
    sv.specverify_run_greedy(ctx, None, BF16, 16, 5, w.V, dev(w.target.reshape(16, 6, w.V)),
                             dev(w.tokens), a2, t2)
    torch.cuda.synchronize()
    assert np.array_equal(acc, a2.cpu().numpy()) and np.array_equal(tok, t2.cpu().numpy())


def test_heads_errors(ctx):
    w = synth.make_greedy_heads(2, 2, 3, 10, F32, seed=1)
    lg, x = dev(w.target), dev(w.tokens)
    acc = torch.empty(2, dtype=torch.int32, device="cuda")
    tok = torch.empty((2, 3), dtype=torch.int32, device="cuda")
    nxt = torch.empty((2, 2), dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="logits"):   # the binding: 17 positions beyond the tensor
        sv.specverify_run_greedy_heads(ctx, None, F32, 2, 17, 3, 10, lg, x, acc, tok, nxt)
    lg, x, acc, tok, nxt = _raw(lg, x, acc, tok, nxt)
    E = sv.SpecVerifyError
    for args, want in [((F32, 2, 2, 0, 10, lg, x, acc, tok, nxt), sv.SPECVERIFY_EINVAL),
                       ((F32, 2, 2, 3, 10, lg, x, acc, tok, None), sv.SPECVERIFY_EINVAL),
                       ((F32, 2, 17, 3, 10, lg, x, acc, tok, nxt), sv.SPECVERIFY_ECAPACITY),
                       # B * (H - 1) workgroups of 256 threads would pass 2^32 - 1 work-items;
                       # refused on the host before any launch
                       ((F32, 2, 2, (1 << 23) + 1, 10, lg, x, acc, tok, nxt),
                        sv.SPECVERIFY_ECAPACITY)]:
        with pytest.raises(E) as ei:
            sv.specverify_run_greedy_heads(ctx, None, *args)
        assert ei.value.status == want


# ----------------------------------------------------------------- alpha-quantile cut

def _check_cut(P, N, alpha, scores, misalign=0, ctx=None):
    cut, keep, n = run_cut(ctx, P, N, alpha, scores, misalign)
    o = oracle.quantile_cut(P, N, alpha, scores)
    assert np.array_equal(cut, o.r_cut)     # as floats: -0 == +0
    assert np.array_equal(keep, o.keep)
    assert np.array_equal(n, o.n_keep)


def test_cut_full_size(ctx):
    w = synth.cut_best_of_n()
    _check_cut(w.P, w.N, w.alpha, w.scores, ctx=ctx)


@pytest.mark.parametrize("N", [1, 2, 7, 255, 256, 1000, 1025, 8192])
@pytest.mark.parametrize("alpha", [0.0, 0.3, 0.5, 0.9, 1.0])
def test_cut_shapes(ctx, N, alpha):
    w = synth.make_cut(5, N, alpha, seed=N)
    _check_cut(5, N, w.alpha, w.scores, misalign=N % 2, ctx=ctx)


def test_cut_special_values(ctx):
    rng = np.random.default_rng(3)
    s = rng.standard_normal((6, 64)).astype(np.float32)
    s[0] = 1.25                                        # all equal
    s[1, :32] = 0.0
    s[1, 32:] = -0.0                                   # signed zeros
    s[2] = np.float32(3.0e38) * np.sign(s[2])         # extremes
    s[3, ::2] = np.float32(1e-45)                      # denormals
    s[4] = np.inf
    s[4, 10] = -np.inf                                 # infinities are ordered too
    for alpha in (0.0, 0.25, 0.5, 1.0):
        _check_cut(6, 64, alpha, s, ctx=ctx)


def test_cut_errors(ctx):
    s = dev(np.zeros((2, 8), np.float32))
    cut = torch.empty(2, dtype=torch.float32, device="cuda")
    keep = torch.empty((2, 8), dtype=torch.uint8, device="cuda")
    n = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="scores"):   # the binding: P x N beyond the tensor
        sv.specverify_quantile_cut(ctx, None, 1 << 22, 8, 0.5, s, cut, keep, n)
    s, cut, keep, n = _raw(s, cut, keep, n)
    E = sv.SpecVerifyError
    for args, want in [((2, 8, 1.5, s, cut, keep, n), sv.SPECVERIFY_EINVAL),
                       ((2, 8, float("nan"), s, cut, keep, n), sv.SPECVERIFY_EINVAL),
                       ((2, 0, 0.5, s, cut, keep, n), sv.SPECVERIFY_EINVAL),
                       ((2, 8, 0.5, None, cut, keep, n), sv.SPECVERIFY_EINVAL),
                       ((2, sv.SPECVERIFY_MAX_CUT_N + 1, 0.5, s, cut, keep, n),
                        sv.SPECVERIFY_ECAPACITY),
                       # 2^22 prompts of one 1024-thread workgroup each: 2^32 work-items
                       ((1 << 22, 8, 0.5, s, cut, keep, n), sv.SPECVERIFY_ECAPACITY)]:
        with pytest.raises(E) as ei:
            sv.specverify_quantile_cut(ctx, None, *args)
        assert ei.value.status == want
    sv.specverify_quantile_cut(ctx, None, 0, 8, 0.5, None, None, None, None)  # P = 0: no-op


def test_profile_kinds_of_the_next_operations(ctx):
    w = synth.make_cut(4, 100, 0.5, seed=1)
    sv.specverify_profile_begin(ctx, 2)
    run_cut(ctx, 4, 100, w.alpha, w.scores)
    ws = synth.make_sampler(4, 100, F32, 1.0, seed=2)
    run_sample(ctx, ws)
    ms, n = sv.specverify_profile_end(ctx)
    assert n["quantile_cut"] == 1 and n["row_stats"] == 1 and n["accept_draw"] == 1
