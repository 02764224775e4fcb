"""A seeded sweep of random shapes through every verify mode, the early-exit entry points and
the sampler, each against the oracle under the parity rule (needs an MI355X).  The cases mix
tiny and ragged vocabularies with ones of many chunks, K from 0 to 63, both logit types,
16-byte aligned and unaligned rows, and drafts close to the target (long accepted runs, so
bonus draws) with ordinary ones."""
import numpy as np
import pytest
import torch

import oracle
from gpu_support import compare, compare_early, compare_sample, run, run_early, run_sample
from rejection_sampling_verification_row_amd import binding as sv
from rejection_sampling_verification_row_amd import synth
from rejection_sampling_verification_row_amd.synth import BF16, F32

pytestmark = pytest.mark.gpu

MAX_B, MAX_K, MAX_V = 96, 63, 200000
LOGITS_CAP = 12_000_000      # logits per case, so that the oracle takes well under a second
MODES = ("sampling", "contrastive", "greedy", "sample", "early")
VOCABS = (1, 2, 7, 100, 999, 4096, 8191, 16385, 32000, 50001, 131072, 200000)


def _cases(n=40, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        mode = MODES[i % len(MODES)]
        dtype = BF16 if rng.random() < 0.6 else F32
        K = 0 if mode == "sample" else int(rng.choice([0, 1, 2, 3, 5, 8, 13, 31, 63]))
        V = int(rng.choice(VOCABS))
        rows = 1 if mode == "sample" else 2 * K + 1
        B = int(min(rng.integers(1, MAX_B + 1), max(1, LOGITS_CAP // (rows * V))))
        misalign = int(rng.random() < 0.3)
        near = bool(rng.random() < 0.25)
        out.append((i, mode, dtype, B, K, V, misalign, near))
    return out


CASES = _cases()


def _workload(i, mode, dtype, B, K, V, near):
    seed = 31000 + i
    if mode == "sample":
        return synth.make_sampler(B, V, dtype, 0.8, seed, sigma=2.0)
    contrastive = mode == "contrastive" or (mode == "early" and i % 2 == 1)
    if contrastive:
        return synth.make_contrastive(B, K, V, dtype, 1.0 if near else 1.2, seed,
                                      amateur_scale=0.5 if near else 0.6,
                                      amateur_sigma=0.02 if near else 2.0)
    if mode == "greedy":
        return synth.make_greedy(B, K, V, dtype, seed, sigma=1.0 if dtype == BF16 else 3.0,
                                 match_prob=0.95 if near else 0.7)
    return synth.make_sampling(B, K, V, dtype, 0.9, seed, target_sigma=2.5,
                               draft_sigma=0.05 if near else 1.0)


@pytest.fixture(scope="module")
def ctx():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    h = sv.specverify_create(0, MAX_B, MAX_K, MAX_V)
    yield h
    sv.specverify_destroy(h)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%d-%s-%s-B%d-K%d-V%d-m%d%s" % (
    c[0], c[1], synth.DTYPE_NAMES[c[2]], c[3], c[4], c[5], c[6], "-near" if c[7] else ""))
def test_random_shape(ctx, case):
    i, mode, dtype, B, K, V, misalign, near = case
    w = _workload(i, mode, dtype, B, K, V, near)
    o = oracle.run_workload(w)
    if mode == "sample":
        tok, pr = run_sample(ctx, w, misalign=misalign)
        compare_sample(w, tok, pr, o)
    elif mode == "early":
        compare_early(w, run_early(ctx, w, misalign=misalign), o)
    else:
        compare(w, run(ctx, w, misalign=misalign), o)


def test_the_sweep_reaches_its_corners():
    """The seeded cases include what they are meant to: every mode, both types, K = 0 and a
    long draft, a one-id and a many-chunk vocabulary, unaligned rows and near drafts."""
    assert {c[1] for c in CASES} == set(MODES)
    assert {c[2] for c in CASES} == {BF16, F32}
    assert any(c[4] == 0 for c in CASES if c[1] != "sample") and max(c[4] for c in CASES) >= 31
    assert min(c[5] for c in CASES) <= 7 and max(c[5] for c in CASES) >= 131072
    assert any(c[6] for c in CASES) and any(c[7] for c in CASES)
