"""CPU oracle for the speculative-decoding verify-and-accept step (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg may
import this package.  The GPU product path never calls it and shares no code with it.

The arithmetic lives in ``specverify_oracle.c`` (plain C, fp64, ascending loops); this
module builds it with gcc when the shared object is missing and marshals numpy arrays.
Every function here is pinned by ``tests/test_oracle_pins.py`` against what the pages
and the mathematics fix (library softmax/argmax, exact distribution invariance by
enumeration, closed-form acceptance rates, the pages' worked examples).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "specverify_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A test may point the wrapper at another build of the same source (the mutation tests
# load deliberately broken copies to show that the pins catch them).
_LIB_OVERRIDE = os.environ.get("SPECVERIFY_ORACLE_LIB")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math, no contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or _LIB
        if not _LIB_OVERRIDE and not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(path)
        vp, i32p, f32p, f64p = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p
        lib.oracle_run_sampling.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_double, vp, vp, i32p, f32p, i32p, i32p, f64p,
                                            f64p, i32p]
        lib.oracle_run_sampling.restype = ctypes.c_int
        lib.oracle_run_contrastive.argtypes = lib.oracle_run_sampling.argtypes
        lib.oracle_run_contrastive.restype = ctypes.c_int
        lib.oracle_run_greedy.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          vp, i32p, i32p, i32p]
        lib.oracle_run_greedy.restype = ctypes.c_int
        lib.oracle_softmax.argtypes = [f64p, ctypes.c_int, f64p]
        lib.oracle_softmax.restype = None
        lib.oracle_sample_rows.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_double, vp, f32p, i32p, f64p, f64p, i32p]
        lib.oracle_sample_rows.restype = ctypes.c_int
        lib.oracle_run_greedy_heads.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                ctypes.c_int, ctypes.c_int, vp, i32p, i32p, i32p,
                                                i32p]
        lib.oracle_run_greedy_heads.restype = ctypes.c_int
        lib.oracle_quantile_cut.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_double, f32p,
                                            f32p, vp, i32p]
        lib.oracle_quantile_cut.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


@dataclass
class Result:
    accepted_len: np.ndarray                  # int32 [B]
    out_tokens: np.ndarray                    # int32 [B][K+1]
    out_probs: Optional[np.ndarray] = None    # float64 [B][K][2]: (P_j, Q_j) at the draft tokens
    margin_accept: Optional[np.ndarray] = None  # float64 [B]: min |u_j - min(1, P/Q)| over j <= L
    margin_sample: Optional[np.ndarray] = None  # float64 [B]: distance of t to the drawn interval's
                                                # nearer edge, over W
    alt_token: Optional[np.ndarray] = None    # int32 [B]: positive-weight id across that edge

    @property
    def margin(self) -> Optional[np.ndarray]:
        """Smallest decision margin per sequence (None for greedy, which has none)."""
        if self.margin_accept is None:
            return None
        return np.minimum(self.margin_accept, self.margin_sample)


def _logits(a: np.ndarray, dtype: int) -> np.ndarray:
    want = np.uint16 if dtype == BF16 else np.float32
    if a.dtype != want:
        raise TypeError("logits must be %s for dtype %d, got %s" % (want, dtype, a.dtype))
    return np.ascontiguousarray(a)


def softmax(z: np.ndarray) -> np.ndarray:
    """The oracle's row softmax on float64 scaled logits z."""
    z = np.ascontiguousarray(z, dtype=np.float64)
    out = np.empty_like(z)
    _load().oracle_softmax(_ptr(z), int(z.shape[0]), _ptr(out))
    return out


def run_sampling(dtype: int, B: int, K: int, V: int, T: float, target, draft, draft_tokens,
                 uniforms) -> Result:
    lib = _load()
    target = _logits(target, dtype)
    draft = _logits(draft, dtype) if K > 0 else np.zeros(1, dtype=target.dtype)
    assert target.size == B * (K + 1) * V and (K == 0 or draft.size == B * K * V)
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, K)
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, K + 1)
    L = np.empty(B, np.int32)
    tok = np.empty((B, K + 1), np.int32)
    pr = np.empty((B, K, 2), np.float64)
    mg = np.empty((B, 2), np.float64)
    alt = np.empty(B, np.int32)
    rc = lib.oracle_run_sampling(dtype, B, K, V, float(T), _ptr(target), _ptr(draft), _ptr(x),
                                 _ptr(u), _ptr(L), _ptr(tok), _ptr(pr), _ptr(mg), _ptr(alt))
    if rc != 0:
        raise ValueError("oracle_run_sampling failed: %d" % rc)
    return Result(L, tok, pr, mg[:, 0].copy(), mg[:, 1].copy(), alt)


def run_contrastive(dtype: int, B: int, K: int, V: int, tau: float, expert, amateur,
                    draft_tokens, uniforms) -> Result:
    lib = _load()
    expert = _logits(expert, dtype)
    amateur = _logits(amateur, dtype)
    assert expert.size == B * (K + 1) * V and amateur.size == B * (K + 1) * V
    x = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(B, K)
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(B, K + 1)
    L = np.empty(B, np.int32)
    tok = np.empty((B, K + 1), np.int32)
    pr = np.empty((B, K, 2), np.float64)
    mg = np.empty((B, 2), np.float64)
    alt = np.empty(B, np.int32)
    rc = lib.oracle_run_contrastive(dtype, B, K, V, float(tau), _ptr(expert), _ptr(amateur),
                                    _ptr(x), _ptr(u), _ptr(L), _ptr(tok), _ptr(pr), _ptr(mg),
                                    _ptr(alt))
    if rc != 0:
        raise ValueError("oracle_run_contrastive failed: %d" % rc)
    return Result(L, tok, pr, mg[:, 0].copy(), mg[:, 1].copy(), alt)


def run_greedy(dtype: int, B: int, K: int, V: int, target, proposals) -> Result:
    lib = _load()
    target = _logits(target, dtype)
    assert target.size == B * (K + 1) * V
    x = np.ascontiguousarray(proposals, dtype=np.int32).reshape(B, K)
    L = np.empty(B, np.int32)
    tok = np.empty((B, K + 1), np.int32)
    rc = lib.oracle_run_greedy(dtype, B, K, V, _ptr(target), _ptr(x), _ptr(L), _ptr(tok))
    if rc != 0:
        raise ValueError("oracle_run_greedy failed: %d" % rc)
    return Result(L, tok)


@dataclass
class SampleResult:
    tokens: np.ndarray        # int32 [N]
    probs: np.ndarray         # float64 [N]: the drawn token's probability
    margin: np.ndarray        # float64 [N]: distance of t to the drawn interval's nearer edge, / W
    alt_token: np.ndarray     # int32 [N]: the id across that edge


def sample_rows(dtype: int, N: int, V: int, T: float, logits, uniforms) -> SampleResult:
    """One inverse-CDF draw per row from softmax(logits / T) (the draft-token sampler)."""
    lib = _load()
    logits = _logits(logits, dtype)
    assert logits.size == N * V
    u = np.ascontiguousarray(uniforms, dtype=np.float32).reshape(N)
    tok = np.empty(N, np.int32)
    pr = np.empty(N, np.float64)
    mg = np.empty(N, np.float64)
    alt = np.empty(N, np.int32)
    rc = lib.oracle_sample_rows(dtype, N, V, float(T), _ptr(logits), _ptr(u), _ptr(tok), _ptr(pr),
                                _ptr(mg), _ptr(alt))
    if rc != 0:
        raise ValueError("oracle_sample_rows failed: %d" % rc)
    return SampleResult(tok, pr, mg, alt)


@dataclass
class HeadsResult:
    accepted_len: np.ndarray    # int32 [B]
    out_tokens: np.ndarray      # int32 [B][K+1]
    next_proposals: np.ndarray  # int32 [B][H-1]


def run_greedy_heads(dtype: int, B: int, K: int, H: int, V: int, logits, proposals) -> HeadsResult:
    """Greedy blockwise verify over [B][K+1][H][V] head logits, with the next block's
    proposals from heads 1..H-1 at the emitted position."""
    lib = _load()
    logits = _logits(logits, dtype)
    assert logits.size == B * (K + 1) * H * V
    x = np.ascontiguousarray(proposals, dtype=np.int32).reshape(B, K)
    L = np.empty(B, np.int32)
    tok = np.empty((B, K + 1), np.int32)
    nxt = np.empty((B, max(H - 1, 0)), np.int32)
    rc = lib.oracle_run_greedy_heads(dtype, B, K, H, V, _ptr(logits), _ptr(x), _ptr(L), _ptr(tok),
                                     _ptr(nxt))
    if rc != 0:
        raise ValueError("oracle_run_greedy_heads failed: %d" % rc)
    return HeadsResult(L, tok, nxt)


@dataclass
class CutResult:
    r_cut: np.ndarray   # float32 [P]
    keep: np.ndarray    # bool [P][N]
    n_keep: np.ndarray  # int32 [P]


def quantile_cut(P: int, N: int, alpha: float, scores) -> CutResult:
    """Per prompt: r_cut = the (min(floor(alpha N), N-1) + 1)-th smallest score; keep the
    responses scoring >= r_cut."""
    lib = _load()
    s = np.ascontiguousarray(scores, dtype=np.float32).reshape(P, N)
    cut = np.empty(P, np.float32)
    keep = np.empty((P, N), np.uint8)
    n = np.empty(P, np.int32)
    rc = lib.oracle_quantile_cut(P, N, float(alpha), _ptr(s), _ptr(cut), _ptr(keep), _ptr(n))
    if rc != 0:
        raise ValueError("oracle_quantile_cut failed: %d" % rc)
    return CutResult(cut, keep.astype(bool), n)


def run_workload(w) -> Result:
    """Run the oracle on a ``synth.Workload``."""
    if w.mode == "sampling":
        return run_sampling(w.dtype, w.B, w.K, w.V, w.temperature, w.target, w.draft, w.tokens,
                            w.uniforms)
    if w.mode == "contrastive":
        return run_contrastive(w.dtype, w.B, w.K, w.V, w.temperature, w.target, w.draft,
                               w.tokens, w.uniforms)
    if w.mode == "greedy":
        return run_greedy(w.dtype, w.B, w.K, w.V, w.target, w.tokens)
    if w.mode == "sample":
        return sample_rows(w.dtype, w.B, w.V, w.temperature, w.target, w.uniforms)
    if w.mode == "greedy_heads":
        return run_greedy_heads(w.dtype, w.B, w.K, w.meta["H"], w.V, w.target, w.tokens)
    raise ValueError(w.mode)


LOW_MARGIN = 1e-6
"""Sequences whose smallest decision margin is below this are excluded from the
bit-exact comparison of ids and lengths (and counted)."""
