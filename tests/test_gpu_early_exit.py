"""GPU parity of sampling and contrastive verify with early exit (needs an MI355X): the same
tokens and accepted lengths as the oracle and as the full-read entry points, out_probs up
to L."""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import compare, compare_early, oracle_whole_batch, run, run_early
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


def _same_as_full(ctx, w, g):
    f = run(ctx, w)
    assert np.array_equal(g.accepted_len, f.accepted_len)
    assert np.array_equal(g.out_tokens, f.out_tokens)
    for b in range(w.B):
        L = int(f.accepted_len[b])
        if L >= 0:
            assert np.array_equal(g.out_probs[b, :L + 1], f.out_probs[b, :L + 1])


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3", "c5"])
def test_early_exit_full_size(ctx, cfg):
    """Every sequence of the full-size sampling and contrastive workloads."""
    w = synth.CONFIGS[cfg]()
    g = run_early(ctx, w)
    o = oracle_whole_batch(w)
    rep = compare_early(w, g, o)
    print("\n[early exit %s] %s" % (w.name, rep), flush=True)
    _same_as_full(ctx, w, g)


@pytest.mark.parametrize("dtype,B,K,V", [(F32, 6, 0, 100), (BF16, 7, 1, 300), (F32, 9, 2, 1001),
                                         (BF16, 11, 3, 16385), (BF16, 5, 12, 50001),
                                         (F32, 4, 7, 40000)])
@pytest.mark.parametrize("misalign", [0, 1])
def test_early_exit_small_shapes(ctx, dtype, B, K, V, misalign):
    w = synth.make_sampling(B, K, V, dtype, 0.85, seed=700 + B + K + V, target_sigma=2.5,
                            draft_sigma=1.0)
    g = run_early(ctx, w, misalign=misalign)
    compare_early(w, g, oracle.run_workload(w))
    _same_as_full(ctx, w, g)


@pytest.mark.parametrize("draft_sigma", [0.0, 6.0])
def test_early_exit_all_alive_and_none_alive(ctx, draft_sigma):
    """An identical draft accepts everything (every sequence reads every row); a far draft
    rejects almost at once (nothing left after the first positions)."""
    w = synth.make_sampling(24, 6, 3000, BF16, 1.0, seed=5, target_sigma=2.0,
                            draft_sigma=draft_sigma)
    g = run_early(ctx, w)
    compare_early(w, g, oracle.run_workload(w))
    _same_as_full(ctx, w, g)
    if draft_sigma == 0.0:
        assert np.all(g.accepted_len == 6)


def test_early_exit_bad_id_after_an_early_rejection(ctx):
    """A bad id anywhere marks the sequence, even past the rows early exit reads."""
    w = synth.make_sampling(6, 5, 500, F32, 1.0, seed=8, target_sigma=2.0, draft_sigma=4.0)
    w.tokens[3, 4] = 500
    g = run_early(ctx, w)
    assert g.accepted_len[3] == -1 and np.all(g.out_tokens[3] == -1)
    assert np.all(np.isnan(g.out_probs[3]))
    compare_early(w, g, oracle.run_workload(w))


def test_early_exit_is_deterministic(ctx):
    w = synth.make_sampling(64, 6, 20000, BF16, 0.8, seed=12, target_sigma=3.0, draft_sigma=1.2)
    a, b = run_early(ctx, w), run_early(ctx, w)
    assert np.array_equal(a.out_tokens, b.out_tokens)
    assert np.array_equal(a.out_probs, b.out_probs, equal_nan=True)


@pytest.mark.parametrize("dtype,B,K,V", [(BF16, 5, 0, 999), (F32, 6, 1, 3000), (BF16, 13, 3, 40003),
                                         (F32, 4, 6, 20001)])
@pytest.mark.parametrize("misalign", [0, 1])
def test_contrastive_early_exit_small_shapes(ctx, dtype, B, K, V, misalign):
    w = synth.make_contrastive(B, K, V, dtype, 1.3, seed=900 + B + K + V)
    g = run_early(ctx, w, misalign=misalign)
    compare_early(w, g, oracle.run_workload(w))
    _same_as_full(ctx, w, g)


def test_contrastive_early_exit_with_survivors(ctx):
    """With l_a close to l_e / 2 and tau = 1 the contrastive target is close to the amateur's
    law, so most sequences stay alive past the prefix and the rest pass runs too."""
    w = synth.make_contrastive(20, 6, 5000, BF16, 1.0, seed=31, amateur_scale=0.5,
                               amateur_sigma=0.1)
    g = run_early(ctx, w)
    compare_early(w, g, oracle.run_workload(w))
    _same_as_full(ctx, w, g)
    assert np.mean(g.accepted_len >= 2) > 0.5


# ----------------------------------------------------------------- greedy with early exit

def _greedy_same_as_full(ctx, w, g):
    f = run(ctx, w)
    assert np.array_equal(g.accepted_len, f.accepted_len)
    assert np.array_equal(g.out_tokens, f.out_tokens)


def test_greedy_early_exit_full_size(ctx):
    """Every sequence of the full-size greedy workload: the oracle's tokens exactly, and the
    full-read entry point's."""
    w = synth.CONFIGS["c4"]()
    g = run_early(ctx, w)
    rep = compare(w, g, oracle_whole_batch(w))
    print("\n[early exit %s] %s" % (w.name, rep), flush=True)
    _greedy_same_as_full(ctx, w, g)


@pytest.mark.parametrize("dtype,B,K,V", [(BF16, 7, 0, 100), (F32, 9, 1, 300), (BF16, 11, 2, 16385),
                                         (F32, 6, 5, 8193), (BF16, 13, 8, 32000),
                                         (BF16, 3, 16, 5000), (F32, 5, 12, 40001)])
@pytest.mark.parametrize("misalign", [0, 1])
def test_greedy_early_exit_small_shapes(ctx, dtype, B, K, V, misalign):
    w = synth.make_greedy(B, K, V, dtype, seed=1700 + B + K + V,
                          sigma=1.0 if dtype == BF16 else 3.0)
    g = run_early(ctx, w, misalign=misalign)
    compare(w, g, oracle.run_workload(w))
    _greedy_same_as_full(ctx, w, g)


@pytest.mark.parametrize("match", [1.0, 0.0])
def test_greedy_early_exit_all_and_none_matching(ctx, match):
    """Proposals equal to the argmax everywhere (every sequence reads every row) or nowhere
    (no sequence reads past the prefix)."""
    w = synth.make_greedy(40, 6, 20000, BF16, seed=1801, match_prob=match)
    g = run_early(ctx, w)
    compare(w, g, oracle.run_workload(w))
    _greedy_same_as_full(ctx, w, g)
    assert np.all(g.accepted_len == (6 if match == 1.0 else 0))


def test_greedy_early_exit_bad_id_past_the_prefix(ctx):
    w = synth.make_greedy(8, 6, 3000, F32, seed=1802, match_prob=1.0)
    w.tokens[5, 4] = 3000
    g = run_early(ctx, w)
    assert g.accepted_len[5] == -1 and np.all(g.out_tokens[5] == -1)
    compare(w, g, oracle.run_workload(w))


def test_greedy_early_exit_ignores_rows_left_from_an_earlier_call(ctx):
    """Rows a sequence does not read keep the previous call's partials in the workspace; they
    must never reach the output."""
    first = synth.make_greedy(32, 8, 30000, BF16, seed=1803, match_prob=0.95)
    second = synth.make_greedy(32, 8, 30000, BF16, seed=1804, match_prob=0.5)
    run(ctx, first)
    g = run_early(ctx, second)
    compare(second, g, oracle.run_workload(second))
    _greedy_same_as_full(ctx, second, g)
