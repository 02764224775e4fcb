"""Batched speculative-decoding verify-and-accept on MI355X (gfx950).

The computation lives in libspecverify.so (hand-written HIP kernels behind the C-ABI in
include/specverify.h); ``binding`` exposes its entry points to Python under the same names.
"""
from .binding import (  # noqa: F401
    SPECVERIFY_BF16, SPECVERIFY_F32, SpecVerifyError, specverify_create, specverify_destroy,
    specverify_profile_begin, specverify_profile_end, specverify_run_contrastive,
    specverify_run_greedy, specverify_run_sampling, specverify_strerror,
    specverify_workspace_bytes)
