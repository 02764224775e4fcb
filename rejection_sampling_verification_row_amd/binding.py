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


# Another build of the same sources may be loaded instead (the sanitizer run of the CPU tests
# builds the host code with AddressSanitizer and UndefinedBehaviorSanitizer).
_LIB_OVERRIDE = os.environ.get("SPECVERIFY_LIB")


def library_path() -> str:
    return _LIB_OVERRIDE or _build.LIB


def load():
    """Load libspecverify.so, building it first only if it is missing."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not _LIB_OVERRIDE and not os.path.exists(_build.LIB):
            _build.build(force=True)
        lib = ctypes.CDLL(library_path())
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


_ITEMSIZE = {"i32": 4, "f32": 4, "u8": 1}


def _ptrs(*specs):
    """The pointers of a call's array arguments, each spec (x, count, kind, name): every tensor
    is first checked against the call's shape (_arr), then converted (_ptr)."""
    for x, count, kind, name in specs:
        _arr(x, count, kind, name)
    return tuple(_ptr(x) for x, _, _, _ in specs)


def _arr(x, count: int, kind, name: str):
    """Check a tensor argument against the call's shape: its element type (kind: "i32", "f32",
    "u8", or a logits dtype SPECVERIFY_F32 / SPECVERIFY_BF16) and at least `count` elements,
    so that no kernel reads or writes past it.  Plain integer addresses are not checked: their
    extent is the caller's to guarantee."""
    if x is None or isinstance(x, int) or not hasattr(x, "data_ptr"):
        return
    import torch
    if kind in (SPECVERIFY_F32, SPECVERIFY_BF16):
        ok = ({torch.float32} if kind == SPECVERIFY_F32
              else {torch.bfloat16, torch.int16, torch.uint16})
        what = "float32" if kind == SPECVERIFY_F32 else "bfloat16 (or its 16-bit patterns)"
    else:
        ok = {"i32": {torch.int32}, "f32": {torch.float32}, "u8": {torch.uint8, torch.bool}}[kind]
        what = {"i32": "int32", "f32": "float32", "u8": "uint8"}[kind]
    if x.dtype not in ok:
        raise ValueError("%s: expected %s elements, got %s" % (name, what, x.dtype))
    if x.numel() < max(int(count), 0):
        raise ValueError("%s: needs at least %d elements for this call, has %d"
                         % (name, count, x.numel()))


def _verify_args(dtype, B, K, V, target, draft, tokens, uniforms, acc, out, probs, draft_rows):
    """The pointers of a sampling or contrastive verify call, checked against B, K and V
    (draft_rows: K for sampling, K + 1 for contrastive)."""
    return _ptrs((target, B * (K + 1) * V, dtype, "target/expert logits"),
                 (draft, B * draft_rows * V, dtype, "draft/amateur logits"),
                 (tokens, B * K, "i32", "draft_tokens"),
                 (uniforms, B * (K + 1), "f32", "uniforms"),
                 (acc, B, "i32", "accepted_len"),
                 (out, B * (K + 1), "i32", "out_tokens"),
                 (probs, B * K * 2, "f32", "out_probs"))


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
    ptrs = _verify_args(dtype, B, K, V, target_logits, draft_logits, draft_tokens, uniforms,
                        accepted_len, out_tokens, out_probs, K)
    _check(load().specverify_run_sampling(ctx, _stream(stream), dtype, B, K, V,
                                          float(temperature), *ptrs), "specverify_run_sampling")


def specverify_run_sampling_static(stream, dtype, B, K, V, temperature, target_logits,
                                   draft_logits, draft_tokens, uniforms, accepted_len, out_tokens,
                                   out_probs=None) -> None:
    ptrs = _verify_args(dtype, B, K, V, target_logits, draft_logits, draft_tokens, uniforms,
                        accepted_len, out_tokens, out_probs, K)
    _check(load().specverify_run_sampling_static(_stream(stream), dtype, B, K, V,
                                                 float(temperature), *ptrs),
           "specverify_run_sampling_static")


def specverify_run_sampling_early_exit(ctx, stream, dtype, B, K, V, temperature, target_logits,
                                       draft_logits, draft_tokens, uniforms, accepted_len,
                                       out_tokens, out_probs=None) -> None:
    ptrs = _verify_args(dtype, B, K, V, target_logits, draft_logits, draft_tokens, uniforms,
                        accepted_len, out_tokens, out_probs, K)
    _check(load().specverify_run_sampling_early_exit(ctx, _stream(stream), dtype, B, K, V,
                                                     float(temperature), *ptrs),
           "specverify_run_sampling_early_exit")


def specverify_run_contrastive(ctx, stream, dtype, B, K, V, tau, expert_logits, amateur_logits,
                               draft_tokens, uniforms, accepted_len, out_tokens,
                               out_probs=None) -> None:
    ptrs = _verify_args(dtype, B, K, V, expert_logits, amateur_logits, draft_tokens, uniforms,
                        accepted_len, out_tokens, out_probs, K + 1)
    _check(load().specverify_run_contrastive(ctx, _stream(stream), dtype, B, K, V, float(tau),
                                             *ptrs), "specverify_run_contrastive")


def specverify_run_contrastive_early_exit(ctx, stream, dtype, B, K, V, tau, expert_logits,
                                          amateur_logits, draft_tokens, uniforms, accepted_len,
                                          out_tokens, out_probs=None) -> None:
    ptrs = _verify_args(dtype, B, K, V, expert_logits, amateur_logits, draft_tokens, uniforms,
                        accepted_len, out_tokens, out_probs, K + 1)
    _check(load().specverify_run_contrastive_early_exit(ctx, _stream(stream), dtype, B, K, V,
                                                        float(tau), *ptrs),
           "specverify_run_contrastive_early_exit")


def specverify_run_greedy(ctx, stream, dtype, B, K, V, target_logits, proposals, accepted_len,
                          out_tokens) -> None:
    _check(load().specverify_run_greedy(
        ctx, _stream(stream), dtype, B, K, V,
        *_ptrs((target_logits, B * (K + 1) * V, dtype, "target_logits"),
               (proposals, B * K, "i32", "proposals"), (accepted_len, B, "i32", "accepted_len"),
               (out_tokens, B * (K + 1), "i32", "out_tokens"))), "specverify_run_greedy")


def specverify_run_greedy_early_exit(ctx, stream, dtype, B, K, V, target_logits, proposals,
                                     accepted_len, out_tokens) -> None:
    _check(load().specverify_run_greedy_early_exit(
        ctx, _stream(stream), dtype, B, K, V,
        *_ptrs((target_logits, B * (K + 1) * V, dtype, "target_logits"),
               (proposals, B * K, "i32", "proposals"), (accepted_len, B, "i32", "accepted_len"),
               (out_tokens, B * (K + 1), "i32", "out_tokens"))),
        "specverify_run_greedy_early_exit")


def specverify_sample(ctx, stream, dtype, N, V, temperature, logits, uniforms, out_tokens,
                      out_probs=None) -> None:
    _check(load().specverify_sample(
        ctx, _stream(stream), dtype, N, V, float(temperature),
        *_ptrs((logits, N * V, dtype, "logits"), (uniforms, N, "f32", "uniforms"),
               (out_tokens, N, "i32", "out_tokens"), (out_probs, N, "f32", "out_probs"))),
        "specverify_sample")


def specverify_run_greedy_heads(ctx, stream, dtype, B, K, H, V, logits, proposals, accepted_len,
                                out_tokens, next_proposals=None) -> None:
    _check(load().specverify_run_greedy_heads(
        ctx, _stream(stream), dtype, B, K, H, V,
        *_ptrs((logits, B * (K + 1) * max(H, 0) * V, dtype, "logits"),
               (proposals, B * K, "i32", "proposals"), (accepted_len, B, "i32", "accepted_len"),
               (out_tokens, B * (K + 1), "i32", "out_tokens"),
               (next_proposals, B * max(H - 1, 0), "i32", "next_proposals"))),
        "specverify_run_greedy_heads")


def specverify_quantile_cut(ctx, stream, P, N, alpha, scores, r_cut, keep, n_keep) -> None:
    _check(load().specverify_quantile_cut(
        ctx, _stream(stream), P, N, float(alpha),
        *_ptrs((scores, P * N, "f32", "scores"), (r_cut, P, "f32", "r_cut"),
               (keep, P * N, "u8", "keep"), (n_keep, P, "i32", "n_keep"))),
        "specverify_quantile_cut")


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
