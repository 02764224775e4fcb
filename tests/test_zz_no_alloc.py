"""The sampling verify that allocates nothing (specverify_run_sampling_static) against the
context entry point specverify_run_sampling, through the C-ABI (needs an MI355X).

Both run the same kernels; the static one keeps its workspace in a device array that every
call on the device shares, so two calls in a row, the second smaller (and with a draw shared
by several workgroups, whose arrival counts it clears), must each give the context path's
outputs bit for bit.
"""
import numpy as np
import pytest
import torch

from gpu_support import dev
from rejection_sampling_verification_row_amd import binding as sv
from rejection_sampling_verification_row_amd import synth

pytestmark = pytest.mark.gpu


def _outputs(w, static, ctx=None):
    B, K = w.B, w.K
    acc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    tok = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
    probs = torch.full((B, K, 2), -7.0, dtype=torch.float32, device="cuda")
    args = (w.dtype, B, K, w.V, w.temperature, dev(w.target), dev(w.draft), dev(w.tokens),
            dev(w.uniforms), acc, tok, probs)
    if static:
        sv.specverify_run_sampling_static(None, *args)
    else:
        sv.specverify_run_sampling(ctx, None, *args)
    torch.cuda.synchronize()
    return acc.cpu().numpy(), tok.cpu().numpy(), probs.cpu().numpy()


def test_static_scratch_matches_the_context_path():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    # the full-size large-vocabulary workload, then a smaller one whose draws are shared by
    # several workgroups per sequence (B = 64)
    for name in ("c3", "c2"):
        w = synth.CONFIGS[name]()
        print("\n[no-alloc] %s: %s" % (name, w.name), flush=True)
        h = sv.specverify_create(0, w.B, w.K, w.V)
        try:
            want = _outputs(w, False, h)
        finally:
            sv.specverify_destroy(h)
        got = _outputs(w, True)
        for g, e, what in zip(got, want, ("accepted_len", "out_tokens", "out_probs")):
            assert np.array_equal(g.view(np.uint32) if g.dtype == np.float32 else g,
                                  e.view(np.uint32) if e.dtype == np.float32 else e), what
        assert (got[0] >= 0).all()


def test_static_scratch_rejects_what_does_not_fit():
    # B * (2K+1) * chunks * 32 bytes of partials above the array: refused before any GPU work
    with pytest.raises(sv.SpecVerifyError) as ei:
        sv.specverify_run_sampling_static(None, sv.SPECVERIFY_BF16, 4096, 8, 128256, 1.0, 16, 16,
                                          16, 16, 16, 16, None)
    assert ei.value.status == sv.SPECVERIFY_ECAPACITY
