"""Python binding of libspecverify.so: the C-ABI's entry points under the same names.

Argument marshalling only.  Array arguments are torch CUDA tensors (contiguous; their
device pointers are passed) or raw device addresses as ints; ``stream`` is a torch stream,
a raw hipStream_t as an int, or None for torch's current stream.  A non-zero status from
the library raises SpecVerifyError.  All computation happens in the library's kernels;
there is no fallback: if the library cannot be built or loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

from . import build as _build

SPECVERIFY_F32 = 0
SPECVERIFY_BF16 = 1

SPECVERIFY_OK = 0
SPECVERIFY_EINVAL = -1
SPECVERIFY_EUNSUPPORTED = -2
SPECVERIFY_ENOMEM = -3
SPECVERIFY_EHIP = -4
SPECVERIFY_ECAPACITY = -5

SPECVERIFY_MAX_K = 63
SPECVERIFY_MAX_VOCAB = 1 << 20
SPECVERIFY_STATIC_SCRATCH_BYTES = 4 << 20
SPECVERIFY_MAX_CUT_N = 8192
SPECVERIFY_NUM_KERNELS = 7
SPECVERIFY_TEST_CHUNK_FALLBACK = 1
SPECVERIFY_TEST_EXACT_TWO_PASS = 2
KERNEL_NAMES = ("row_stats", "accept_draw", "row_argmax", "greedy_emit", "quantile_cut",
                "early_accept", "early_rest_stats")

_lib = None
_lock = threading.Lock()


class SpecVerifyError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, specverify_strerror(status), status))


def library_path() -> str:
    return _build.LIB


def load():
    """Load libspecverify.so, building it first only if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_build.LIB):
            _build.build(force=True)
        lib = ctypes.CDLL(_build.LIB)
        vp, i, f, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64
        lib.specverify_create.argtypes = [ctypes.POINTER(vp), i, i, i, i]
        lib.specverify_create.restype = i
        lib.specverify_workspace_bytes.argtypes = [vp]
        lib.specverify_workspace_bytes.restype = i64
        lib.specverify_run_sampling.argtypes = [vp, vp, i, i, i, i, f, vp, vp, vp, vp, vp, vp, vp]
        lib.specverify_run_sampling.restype = i
        lib.specverify_run_sampling_early_exit.argtypes = lib.specverify_run_sampling.argtypes
        lib.specverify_run_sampling_early_exit.restype = i
        lib.specverify_run_sampling_static.argtypes = [vp, i, i, i, i, f, vp, vp, vp, vp, vp, vp,
                                                       vp]
        lib.specverify_run_sampling_static.restype = i
        lib.specverify_run_contrastive.argtypes = [vp, vp, i, i, i, i, f, vp, vp, vp, vp, vp, vp,
                                                   vp]
        lib.specverify_run_contrastive.restype = i
        lib.specverify_run_contrastive_early_exit.argtypes = lib.specverify_run_contrastive.argtypes
        lib.specverify_run_contrastive_early_exit.restype = i
        lib.specverify_run_greedy.argtypes = [vp, vp, i, i, i, i, vp, vp, vp, vp]
        lib.specverify_run_greedy.restype = i
        lib.specverify_run_greedy_early_exit.argtypes = lib.specverify_run_greedy.argtypes
        lib.specverify_run_greedy_early_exit.restype = i
        lib.specverify_sample.argtypes = [vp, vp, i, i, i, f, vp, vp, vp, vp]
        lib.specverify_sample.restype = i
        lib.specverify_run_greedy_heads.argtypes = [vp, vp, i, i, i, i, i, vp, vp, vp, vp, vp]
        lib.specverify_run_greedy_heads.restype = i
        lib.specverify_quantile_cut.argtypes = [vp, vp, i, i, f, vp, vp, vp, vp]
        lib.specverify_quantile_cut.restype = i
        lib.specverify_set_test_flags.argtypes = [vp, ctypes.c_uint]
        lib.specverify_set_test_flags.restype = i
        lib.specverify_destroy.argtypes = [vp]
        lib.specverify_destroy.restype = i
        lib.specverify_strerror.argtypes = [i]
        lib.specverify_strerror.restype = ctypes.c_char_p
        lib.specverify_profile_begin.argtypes = [vp, i, ctypes.c_uint, i]
        lib.specverify_profile_begin.restype = i
        lib.specverify_profile_launches.argtypes = [vp, i, ctypes.POINTER(ctypes.c_float), i]
        lib.specverify_profile_launches.restype = i
        lib.specverify_profile_end.argtypes = [vp, ctypes.POINTER(ctypes.c_double),
                                               ctypes.POINTER(ctypes.c_int)]
        lib.specverify_profile_end.restype = i
        _lib = lib
        return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if not x.is_cuda:
            raise ValueError("expected a device tensor, got one on %s" % x.device)
        if not x.is_contiguous():
            raise ValueError("expected a contiguous tensor")
        return x.data_ptr()
    raise TypeError("expected a torch tensor, an int device address or None, got %r" % type(x))


def _stream(s):
    if isinstance(s, int):
        return s
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return s.cuda_stream


def _check(status: int, where: str):
    if status != SPECVERIFY_OK:
        raise SpecVerifyError(status, where)


def specverify_strerror(status: int) -> str:
    return load().specverify_strerror(int(status)).decode()


def specverify_create(device: int, max_batch: int, max_k: int, max_vocab: int) -> int:
    """Returns the context handle (an int)."""
    h = ctypes.c_void_p()
    _check(load().specverify_create(ctypes.byref(h), device, max_batch, max_k, max_vocab),
           "specverify_create")
    return h.value


def specverify_workspace_bytes(ctx: int) -> int:
    return int(load().specverify_workspace_bytes(ctx))


def specverify_run_sampling(ctx, stream, dtype, B, K, V, temperature, target_logits,
                            draft_logits, draft_tokens, uniforms, accepted_len, out_tokens,
                            out_probs=None) -> None:
    _check(load().specverify_run_sampling(
        ctx, _stream(stream), dtype, B, K, V, float(temperature), _ptr(target_logits),
        _ptr(draft_logits), _ptr(draft_tokens), _ptr(uniforms), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(out_probs)), "specverify_run_sampling")


def specverify_run_sampling_static(stream, dtype, B, K, V, temperature, target_logits,
                                   draft_logits, draft_tokens, uniforms, accepted_len, out_tokens,
                                   out_probs=None) -> None:
    _check(load().specverify_run_sampling_static(
        _stream(stream), dtype, B, K, V, float(temperature), _ptr(target_logits),
        _ptr(draft_logits), _ptr(draft_tokens), _ptr(uniforms), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(out_probs)), "specverify_run_sampling_static")


def specverify_run_sampling_early_exit(ctx, stream, dtype, B, K, V, temperature, target_logits,
                                       draft_logits, draft_tokens, uniforms, accepted_len,
                                       out_tokens, out_probs=None) -> None:
    _check(load().specverify_run_sampling_early_exit(
        ctx, _stream(stream), dtype, B, K, V, float(temperature), _ptr(target_logits),
        _ptr(draft_logits), _ptr(draft_tokens), _ptr(uniforms), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(out_probs)), "specverify_run_sampling_early_exit")


def specverify_run_contrastive(ctx, stream, dtype, B, K, V, tau, expert_logits, amateur_logits,
                               draft_tokens, uniforms, accepted_len, out_tokens,
                               out_probs=None) -> None:
    _check(load().specverify_run_contrastive(
        ctx, _stream(stream), dtype, B, K, V, float(tau), _ptr(expert_logits),
        _ptr(amateur_logits), _ptr(draft_tokens), _ptr(uniforms), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(out_probs)), "specverify_run_contrastive")


def specverify_run_contrastive_early_exit(ctx, stream, dtype, B, K, V, tau, expert_logits,
                                          amateur_logits, draft_tokens, uniforms, accepted_len,
                                          out_tokens, out_probs=None) -> None:
    _check(load().specverify_run_contrastive_early_exit(
        ctx, _stream(stream), dtype, B, K, V, float(tau), _ptr(expert_logits),
        _ptr(amateur_logits), _ptr(draft_tokens), _ptr(uniforms), _ptr(accepted_len),
        _ptr(out_tokens), _ptr(out_probs)), "specverify_run_contrastive_early_exit")


def specverify_run_greedy(ctx, stream, dtype, B, K, V, target_logits, proposals, accepted_len,
                          out_tokens) -> None:
    _check(load().specverify_run_greedy(
        ctx, _stream(stream), dtype, B, K, V, _ptr(target_logits), _ptr(proposals),
        _ptr(accepted_len), _ptr(out_tokens)), "specverify_run_greedy")


def specverify_run_greedy_early_exit(ctx, stream, dtype, B, K, V, target_logits, proposals,
                                     accepted_len, out_tokens) -> None:
    _check(load().specverify_run_greedy_early_exit(
        ctx, _stream(stream), dtype, B, K, V, _ptr(target_logits), _ptr(proposals),
        _ptr(accepted_len), _ptr(out_tokens)), "specverify_run_greedy_early_exit")


def specverify_sample(ctx, stream, dtype, N, V, temperature, logits, uniforms, out_tokens,
                      out_probs=None) -> None:
    _check(load().specverify_sample(
        ctx, _stream(stream), dtype, N, V, float(temperature), _ptr(logits), _ptr(uniforms),
        _ptr(out_tokens), _ptr(out_probs)), "specverify_sample")


def specverify_run_greedy_heads(ctx, stream, dtype, B, K, H, V, logits, proposals, accepted_len,
                                out_tokens, next_proposals=None) -> None:
    _check(load().specverify_run_greedy_heads(
        ctx, _stream(stream), dtype, B, K, H, V, _ptr(logits), _ptr(proposals),
        _ptr(accepted_len), _ptr(out_tokens), _ptr(next_proposals)),
        "specverify_run_greedy_heads")


def specverify_quantile_cut(ctx, stream, P, N, alpha, scores, r_cut, keep, n_keep) -> None:
    _check(load().specverify_quantile_cut(
        ctx, _stream(stream), P, N, float(alpha), _ptr(scores), _ptr(r_cut), _ptr(keep),
        _ptr(n_keep)), "specverify_quantile_cut")


def specverify_set_test_flags(ctx, flags: int) -> None:
    """Test hook: SPECVERIFY_TEST_* bits forcing rarely reached draw paths (0 = normal)."""
    _check(load().specverify_set_test_flags(ctx, int(flags)), "specverify_set_test_flags")


def specverify_destroy(ctx) -> None:
    _check(load().specverify_destroy(ctx), "specverify_destroy")


def specverify_profile_begin(ctx, max_calls: int, kinds=None, stride: int = 1) -> None:
    """kinds: kernel names (from KERNEL_NAMES) to time, or None for all of them; stride: time
    every stride-th call (the first, then every stride-th after it)."""
    mask = 0
    for k in kinds or ():
        mask |= 1 << KERNEL_NAMES.index(k)
    _check(load().specverify_profile_begin(ctx, max_calls, mask, stride),
           "specverify_profile_begin")


def specverify_profile_launches(ctx, kind: str) -> list:
    """Durations in ms of the timed launches of kernel `kind` (a KERNEL_NAMES entry) since
    specverify_profile_begin, in call order."""
    lib = load()
    k = KERNEL_NAMES.index(kind)
    n = lib.specverify_profile_launches(ctx, k, None, 0)
    _check(min(n, 0), "specverify_profile_launches")
    ms = (ctypes.c_float * max(n, 1))()
    got = lib.specverify_profile_launches(ctx, k, ms, n)
    _check(min(got, 0), "specverify_profile_launches")
    return list(ms)[:min(n, got)]


def specverify_profile_end(ctx):
    """Returns ({kernel name: summed ms}, {kernel name: launches})."""
    ms = (ctypes.c_double * SPECVERIFY_NUM_KERNELS)()
    n = (ctypes.c_int * SPECVERIFY_NUM_KERNELS)()
    _check(load().specverify_profile_end(ctx, ms, n), "specverify_profile_end")
    return (dict(zip(KERNEL_NAMES, list(ms))), dict(zip(KERNEL_NAMES, list(n))))
