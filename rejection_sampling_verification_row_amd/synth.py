"""Seeded synthetic workloads for the speculative-decoding verify-and-accept step.

This module only *draws* inputs: logits, draft tokens, proposals and uniforms.
It holds none of the verification arithmetic (no softmax, no accept test, no
residual, no inverse CDF), so the GPU path and the CPU oracle can both be fed
from it without sharing any of the method.

* Draft tokens are drawn from the draft distribution softmax(l_d / T) by the
  Gumbel-max trick (argmax of l_d / T plus standard Gumbel noise), an exact
  sampler that is a different algorithm from the inverse-CDF sampling the
  verify step performs.
* Greedy proposals need the position of each row's maximum so that a chosen
  fraction of them match it; that position is taken with ``numpy.argmax``
  (first occurrence), used here only to shape the workload.
* Uniforms sit on the lattice u = (k + 1/2) * 2**-23, k in [0, 2**23): every
  value is an exact float32 strictly inside (0, 1) (the finer half-offset lattice
  (k + 1/2) * 2**-24 is not representable above 1/2, where float32 spacing is 2**-24).

The five named workloads follow the shapes and value distributions of the
batched verify step as the pages describe it (speculative rejection sampling,
blockwise greedy verification, speculative contrastive decoding); the draw
order within each is fixed: target/expert logits, noise, peaks, draft tokens
or proposals, uniforms.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F32 = 0
BF16 = 1
DTYPE_NAMES = {F32: "f32", BF16: "bf16"}

SAMPLING = "sampling"
GREEDY = "greedy"
CONTRASTIVE = "contrastive"
SAMPLE = "sample"              # draft-token sampler: one draw per row
GREEDY_HEADS = "greedy_heads"  # greedy verify over [B][K+1][H][V] head logits

_U_BITS = 23
_U_SCALE = 2.0 ** -_U_BITS


_ROWS_PER_BLOCK = 8
_THREADS = max(1, min(8, os.cpu_count() or 1))


def _blocks(rows: int):
    return [(s, min(rows, s + _ROWS_PER_BLOCK)) for s in range(0, rows, _ROWS_PER_BLOCK)]


def _parallel(fn, items):
    if len(items) <= 1 or _THREADS == 1:
        for it in items:
            fn(it)
        return
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fn, items))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. Inputs must be finite or +-inf.
    """
    src = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.empty(src.shape, dtype=np.uint16)
    step = 1 << 20

    def one(s):
        b = src[s:s + step].view(np.uint32)
        t = b >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += b
        t >>= np.uint32(16)
        out[s:s + step] = t

    _parallel(one, list(range(0, src.size, step)))
    return out.reshape(np.shape(x))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def decode(arr: np.ndarray, dtype: int) -> np.ndarray:
    """float32 view of logits stored as float32 or as bfloat16 bits."""
    return bf16_bits_to_f32(arr) if dtype == BF16 else np.asarray(arr, dtype=np.float32)


def lattice_uniforms(rng: np.random.Generator, shape) -> np.ndarray:
    """float32 uniforms (k + 0.5) * 2**-23, k uniform in [0, 2**23)."""
    k = rng.integers(0, 1 << _U_BITS, size=shape, dtype=np.int64)
    return ((k.astype(np.float64) + 0.5) * _U_SCALE).astype(np.float32)


def normal_rows(ss: np.random.SeedSequence, rows: int, V: int, sigma: float) -> np.ndarray:
    """float32 [rows][V] of N(0, sigma^2); row block i draws from its own child stream of
    ``ss`` so the result does not depend on the number of threads."""
    out = np.empty((rows, V), dtype=np.float32)
    blocks = _blocks(rows)
    kids = ss.spawn(len(blocks))
    s32 = np.float32(sigma)

    def one(i):
        a, b = blocks[i]
        g = np.random.Generator(np.random.PCG64(kids[i]))
        g.standard_normal(out=out[a:b], dtype=np.float32)
        out[a:b] *= s32

    _parallel(one, list(range(len(blocks))))
    return out


def gumbel_max_tokens(ss: np.random.SeedSequence, logits: np.ndarray,
                      temperature: float) -> np.ndarray:
    """One draw per row from softmax(logits / temperature) via the Gumbel-max trick.

    ``logits`` is float32 of shape [..., V]; returns int32 of shape [...].
    """
    flat = logits.reshape(-1, logits.shape[-1])
    out = np.empty(flat.shape[0], dtype=np.int32)
    inv_t = np.float32(1.0 / temperature)
    blocks = _blocks(flat.shape[0])
    kids = ss.spawn(len(blocks))

    def one(i):
        a, b = blocks[i]
        g = np.random.Generator(np.random.PCG64(kids[i]))
        u = g.random((b - a, flat.shape[1]), dtype=np.float32)
        # -log(-log(u)); u == 0 gives -inf, which simply never wins.
        with np.errstate(divide="ignore"):
            np.log(u, out=u)
            np.negative(u, out=u)
            np.log(u, out=u)
        u *= np.float32(-1.0)
        u += flat[a:b] * inv_t
        out[a:b] = np.argmax(u, axis=1)

    _parallel(one, list(range(len(blocks))))
    return out.reshape(logits.shape[:-1])


def _distinct_positions(rng: np.random.Generator, rows: int, count: int, V: int) -> np.ndarray:
    """``count`` distinct uniform positions in [0, V) for each of ``rows`` rows."""
    pos = rng.integers(0, V, size=(rows, count), dtype=np.int64)
    while True:
        srt = np.sort(pos, axis=1)
        dup = np.any(srt[:, 1:] == srt[:, :-1], axis=1)
        if not dup.any():
            return pos
        idx = np.nonzero(dup)[0]
        pos[idx] = rng.integers(0, V, size=(idx.size, count), dtype=np.int64)


@dataclass
class Workload:
    """One batch of verify-step inputs.

    sampling:    target [B][K+1][V], draft [B][K][V], tokens = draft tokens [B][K],
                 uniforms [B][K+1] (u[0..K-1] accept tests, u[K] residual/bonus draw).
    greedy:      target [B][K+1][V], tokens = proposals [B][K]; no draft, no uniforms.
    contrastive: target = expert [B][K+1][V], draft = amateur [B][K+1][V],
                 tokens = draft tokens [B][K], uniforms [B][K+1].
    Logit arrays are float32 (dtype F32) or uint16 bfloat16 bit patterns (dtype BF16).
    """
    name: str
    mode: str
    dtype: int
    B: int
    K: int
    V: int
    temperature: float
    target: np.ndarray
    draft: Optional[np.ndarray]
    tokens: np.ndarray
    uniforms: Optional[np.ndarray]
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def logit_bytes(self) -> int:
        """Bytes of logits one pass over every row reads."""
        n = self.target.nbytes + (self.draft.nbytes if self.draft is not None else 0)
        return int(n)

    def subset(self, idx) -> "Workload":
        """The same workload restricted to the sequences ``idx`` (a list of batch indices)."""
        idx = np.asarray(idx, dtype=np.int64)
        return Workload(
            name=f"{self.name}[subset {idx.size}]", mode=self.mode, dtype=self.dtype,
            B=int(idx.size), K=self.K, V=self.V, temperature=self.temperature,
            target=np.ascontiguousarray(self.target[idx]),
            draft=None if self.draft is None else np.ascontiguousarray(self.draft[idx]),
            tokens=np.ascontiguousarray(self.tokens[idx]),
            uniforms=None if self.uniforms is None else np.ascontiguousarray(self.uniforms[idx]),
            seed=self.seed, meta=dict(self.meta))


def _f32(t: float) -> float:
    """Temperatures cross the C-ABI as float32; keep the float32 value everywhere."""
    return float(np.float32(t))


def _store(x: np.ndarray, dtype: int) -> np.ndarray:
    return f32_to_bf16_bits(x) if dtype == BF16 else np.ascontiguousarray(x, dtype=np.float32)


def _streams(seed: int):
    """Independent child streams, in draw order: logits, noise, peaks, tokens, uniforms."""
    return np.random.SeedSequence(seed).spawn(5)


def make_sampling(B: int, K: int, V: int, dtype: int, temperature: float, seed: int, *,
                  target_sigma: float, draft_scale: float = 1.0, draft_sigma: float = 1.0,
                  n_peaks: int = 0, peak_height: float = 8.0, name: str = "sampling") -> Workload:
    """Sampling-verify workload.

    target l_t ~ N(0, target_sigma^2) per entry, plus ``peak_height`` added at ``n_peaks``
    distinct uniform positions of every target row; draft rows j < K are
    draft_scale * l_t[j] + N(0, draft_sigma^2), formed in float32 before any bf16 rounding.
    Draft tokens are drawn from softmax(l_d / T) of the stored (rounded) draft logits.
    """
    s_logits, s_noise, s_peaks, s_tokens, s_unif = _streams(seed)
    t = normal_rows(s_logits, B * (K + 1), V, target_sigma).reshape(B, K + 1, V)
    noise = normal_rows(s_noise, B * K, V, draft_sigma).reshape(B, K, V)
    if n_peaks:
        rng = np.random.Generator(np.random.PCG64(s_peaks))
        pos = _distinct_positions(rng, B * (K + 1), n_peaks, V)
        flat = t.reshape(B * (K + 1), V)
        rows = np.repeat(np.arange(B * (K + 1)), n_peaks)
        flat[rows, pos.reshape(-1)] += np.float32(peak_height)
    if draft_scale != 1.0:
        noise += t[:, :K, :] * np.float32(draft_scale)
    else:
        noise += t[:, :K, :]
    target = _store(t, dtype)
    del t
    draft = _store(noise, dtype)
    del noise
    tokens = gumbel_max_tokens(s_tokens, decode(draft, dtype), temperature).astype(np.int32)
    uniforms = lattice_uniforms(np.random.Generator(np.random.PCG64(s_unif)), (B, K + 1))
    return Workload(name=name, mode=SAMPLING, dtype=dtype, B=B, K=K, V=V,
                    temperature=_f32(temperature), target=target, draft=draft,
                    tokens=np.ascontiguousarray(tokens.reshape(B, K)), uniforms=uniforms, seed=seed)


def make_small_residual(B: int, V: int, dtype: int, temperature: float, seed: int, *,
                        target_sigma: float = 4.0, n_peaks: int = 20, peak_height: float = 8.0,
                        noise_lo: float = 1e-4, noise_hi: float = 3e-2, top: int = 100,
                        name: str = "small residual") -> Workload:
    """Sampling-verify workload (K = 1) shaped so that position 0 rejects with a small residual
    mass: a draft that is the target plus very little noise.

    Target rows are N(0, target_sigma^2) plus ``peak_height`` at ``n_peaks`` distinct positions,
    as in the large-vocabulary workload.  The draft row of position 0 is the float32 target row
    plus N(0, s_b^2) noise, s_b log-uniform in [noise_lo, noise_hi] per sequence, then stored in
    the logit type (a bfloat16 draft differs from its target only where the noise crosses a
    rounding boundary, by one bfloat16 step).  The draft token is, among the ``top`` largest
    target logits of the row (by value, with numpy's sort), the id whose stored draft logit rose
    the most over its stored target logit, so that the draft favours it; the accept uniform is
    1 - 2^-13 and the draw uniform a lattice value.  Nothing here evaluates a probability: the
    workload only shapes logits.
    """
    s_logits, s_noise, s_peaks, _s_tokens, s_unif = _streams(seed)
    t = normal_rows(s_logits, B * 2, V, target_sigma).reshape(B, 2, V)
    if n_peaks:
        rng = np.random.Generator(np.random.PCG64(s_peaks))
        pos = _distinct_positions(rng, B * 2, n_peaks, V)
        flat = t.reshape(B * 2, V)
        flat[np.repeat(np.arange(B * 2), n_peaks), pos.reshape(-1)] += np.float32(peak_height)
    noise = normal_rows(s_noise, B, V, 1.0)
    rng = np.random.Generator(np.random.PCG64(s_unif))
    sb = np.exp(rng.uniform(np.log(noise_lo), np.log(noise_hi), size=B)).astype(np.float32)
    noise *= sb[:, None]
    noise += t[:, 0, :]
    target = _store(t, dtype)
    draft = _store(noise.reshape(B, 1, V), dtype)
    del t, noise
    tv = decode(target[:, 0, :], dtype)
    dv = decode(draft[:, 0, :], dtype)
    idx = np.argsort(-tv, axis=1, kind="stable")[:, :top]
    rise = np.take_along_axis(dv, idx, 1) - np.take_along_axis(tv, idx, 1)
    tokens = np.take_along_axis(idx, np.argmax(rise, axis=1)[:, None], 1).astype(np.int32)
    k_acc = (1 << _U_BITS) - (1 << (_U_BITS - 13))
    u_acc = np.full((B, 1), (k_acc + 0.5) * _U_SCALE, dtype=np.float32)
    uniforms = np.concatenate([u_acc, lattice_uniforms(rng, (B, 1))], axis=1)
    return Workload(name=name, mode=SAMPLING, dtype=dtype, B=B, K=1, V=V,
                    temperature=_f32(temperature), target=target, draft=draft,
                    tokens=np.ascontiguousarray(tokens), uniforms=uniforms, seed=seed)


def make_greedy(B: int, K: int, V: int, dtype: int, seed: int, *, sigma: float = 4.0,
                match_prob: float = 0.7, name: str = "greedy") -> Workload:
    """Greedy blockwise workload: l ~ N(0, sigma^2); proposal j equals the row's first
    maximum with probability ``match_prob``, else a uniformly chosen other id."""
    s_logits, _s_noise, _s_peaks, s_tokens, _s_unif = _streams(seed)
    t = normal_rows(s_logits, B * (K + 1), V, sigma).reshape(B, K + 1, V)
    target = _store(t, dtype)
    del t
    top = np.argmax(decode(target[:, :K, :], dtype), axis=2)  # first occurrence
    rng = np.random.Generator(np.random.PCG64(s_tokens))
    match = rng.random((B, K)) < match_prob
    r = rng.integers(0, max(V - 1, 1), size=(B, K), dtype=np.int64)
    other = top if V == 1 else r + (r >= top)
    props = np.where(match, top, other).astype(np.int32)
    return Workload(name=name, mode=GREEDY, dtype=dtype, B=B, K=K, V=V, temperature=1.0,
                    target=target, draft=None, tokens=np.ascontiguousarray(props),
                    uniforms=None, seed=seed)


def make_contrastive(B: int, K: int, V: int, dtype: int, tau: float, seed: int, *,
                     expert_sigma: float = 4.0, amateur_scale: float = 0.6,
                     amateur_sigma: float = 2.0, name: str = "contrastive") -> Workload:
    """Contrastive-target workload: l_e ~ N(0, expert_sigma^2);
    l_a = amateur_scale * stored(l_e) + N(0, amateur_sigma^2); draft tokens from softmax(l_a)."""
    s_logits, s_noise, _s_peaks, s_tokens, s_unif = _streams(seed)
    e = normal_rows(s_logits, B * (K + 1), V, expert_sigma).reshape(B, K + 1, V)
    expert = _store(e, dtype)
    del e
    a = normal_rows(s_noise, B * (K + 1), V, amateur_sigma).reshape(B, K + 1, V)
    a += decode(expert, dtype) * np.float32(amateur_scale)
    amateur = _store(a, dtype)
    del a
    tokens = gumbel_max_tokens(s_tokens, decode(amateur[:, :K, :], dtype), 1.0).astype(np.int32)
    uniforms = lattice_uniforms(np.random.Generator(np.random.PCG64(s_unif)), (B, K + 1))
    return Workload(name=name, mode=CONTRASTIVE, dtype=dtype, B=B, K=K, V=V,
                    temperature=_f32(tau), target=expert, draft=amateur,
                    tokens=np.ascontiguousarray(tokens.reshape(B, K)), uniforms=uniforms, seed=seed)


def make_sampler(N: int, V: int, dtype: int, temperature: float, seed: int, *,
                 sigma: float = 4.0, n_peaks: int = 0, peak_height: float = 8.0,
                 name: str = "sample") -> Workload:
    """Draft-token sampler workload: N rows l ~ N(0, sigma^2) plus ``peak_height`` at
    ``n_peaks`` distinct positions per row, one lattice uniform per row.  Stored as a
    Workload with K = 0 (``target`` holds the rows, ``uniforms`` is [N][1])."""
    s_logits, _s_noise, s_peaks, _s_tokens, s_unif = _streams(seed)
    t = normal_rows(s_logits, N, V, sigma)
    if n_peaks:
        rng = np.random.Generator(np.random.PCG64(s_peaks))
        pos = _distinct_positions(rng, N, n_peaks, V)
        t[np.repeat(np.arange(N), n_peaks), pos.reshape(-1)] += np.float32(peak_height)
    logits = _store(t, dtype)
    del t
    uniforms = lattice_uniforms(np.random.Generator(np.random.PCG64(s_unif)), (N, 1))
    return Workload(name=name, mode=SAMPLE, dtype=dtype, B=N, K=0, V=V,
                    temperature=_f32(temperature), target=logits, draft=None,
                    tokens=np.zeros((N, 0), np.int32), uniforms=uniforms, seed=seed)


def make_greedy_heads(B: int, K: int, H: int, V: int, dtype: int, seed: int, *,
                      sigma: float = 4.0, match_prob: float = 0.7,
                      name: str = "greedy_heads") -> Workload:
    """Greedy verify with H heads: logits [B][K+1][H][V] ~ N(0, sigma^2); proposal j equals
    head 0's first maximum at position j with probability ``match_prob``, else a uniformly
    chosen other id.  ``meta["H"]`` holds H."""
    s_logits, _s_noise, _s_peaks, s_tokens, _s_unif = _streams(seed)
    t = normal_rows(s_logits, B * (K + 1) * H, V, sigma).reshape(B, K + 1, H, V)
    logits = _store(t, dtype)
    del t
    top = np.argmax(decode(logits[:, :K, 0, :], dtype), axis=2)  # first occurrence
    rng = np.random.Generator(np.random.PCG64(s_tokens))
    match = rng.random((B, K)) < match_prob
    r = rng.integers(0, max(V - 1, 1), size=(B, K), dtype=np.int64)
    other = top if V == 1 else r + (r >= top)
    props = np.where(match, top, other).astype(np.int32)
    return Workload(name=name, mode=GREEDY_HEADS, dtype=dtype, B=B, K=K, V=V, temperature=1.0,
                    target=logits, draft=None, tokens=np.ascontiguousarray(props),
                    uniforms=None, seed=seed, meta={"H": H})


@dataclass
class CutWorkload:
    """P prompts with N partial-reward scores each, and the cut fraction alpha."""
    name: str
    P: int
    N: int
    alpha: float
    scores: np.ndarray  # float32 [P][N]
    seed: int = 0


def make_cut(P: int, N: int, alpha: float, seed: int, *, grid: float = 2.0 ** -8,
             name: str = "cut") -> CutWorkload:
    """Scores ~ N(0, 1) rounded to multiples of ``grid`` (reward scores with ties)."""
    s_scores = _streams(seed)[0]
    x = np.random.Generator(np.random.PCG64(s_scores)).standard_normal((P, N))
    scores = (np.round(x / grid) * grid).astype(np.float32)
    return CutWorkload(name=name, P=P, N=N, alpha=float(np.float32(alpha)), scores=scores,
                       seed=seed)


# The five named workloads. Each takes an optional batch override so that tests can
# run the same distributions at a smaller B; the default is the full size.
def c1_sampling_tiny(B: int = 1, seed: int = 1001) -> Workload:
    """B=1, K=4, V=1000 fp32; target ~N(0,2^2), draft = target + N(0,0.5^2), T=1."""
    return make_sampling(B, 4, 1000, F32, 1.0, seed, target_sigma=2.0, draft_sigma=0.5,
                         name="sampling-tiny B=%d K=4 V=1000 f32" % B)


def c2_sampling_mid(B: int = 64, seed: int = 1002) -> Workload:
    """B=64, K=5, V=32000 fp32; target ~N(0,3^2), draft = 0.8*target + N(0,1), T=1."""
    return make_sampling(B, 5, 32000, F32, 1.0, seed, target_sigma=3.0, draft_scale=0.8,
                         draft_sigma=1.0, name="sampling-mid B=%d K=5 V=32000 f32" % B)


def c3_sampling_large_vocab(B: int = 256, seed: int = 1003) -> Workload:
    """B=256, K=8, V=128256 bf16; target ~N(0,4^2) + 8 at 20 distinct positions per row,
    draft = target + N(0,1.5^2), T=0.7 for both."""
    return make_sampling(B, 8, 128256, BF16, 0.7, seed, target_sigma=4.0, draft_sigma=1.5,
                         n_peaks=20, peak_height=8.0,
                         name="sampling-large-vocab B=%d K=8 V=128256 bf16 T=0.7" % B)


def c4_greedy_blockwise(B: int = 512, seed: int = 1004) -> Workload:
    """B=512, K=8, V=32000 bf16; l ~N(0,4^2); proposals match the argmax w.p. 0.7."""
    return make_greedy(B, 8, 32000, BF16, seed, sigma=4.0, match_prob=0.7,
                       name="greedy-blockwise B=%d K=8 V=32000 bf16" % B)


def c5_contrastive(B: int = 128, seed: int = 1005) -> Workload:
    """B=128, K=4, V=152064 bf16; expert ~N(0,4^2), amateur = 0.6*expert + N(0,2^2), tau=1."""
    return make_contrastive(B, 4, 152064, BF16, 1.0, seed,
                            name="contrastive B=%d K=4 V=152064 bf16 tau=1" % B)


CONFIGS = {
    "c1": c1_sampling_tiny,
    "c2": c2_sampling_mid,
    "c3": c3_sampling_large_vocab,
    "c4": c4_greedy_blockwise,
    "c5": c5_contrastive,
}


# Workloads of the operations next to the verify step, at the shapes of their neighbours.
def sampler_draft_rows(N: int = 256, seed: int = 1006) -> Workload:
    """One drafting step of 256 sequences: N=256 rows, V=128256 bf16, T=0.7, rows shaped
    like the large-vocabulary target rows (N(0,4^2) + 8 at 20 positions)."""
    return make_sampler(N, 128256, BF16, 0.7, seed, sigma=4.0, n_peaks=20,
                        name="sampler N=%d V=128256 bf16 T=0.7" % N)


def greedy_heads_blockwise(B: int = 512, seed: int = 1007) -> Workload:
    """Blockwise decoding with merged predict/verify: B=512, K=4 proposals, H=4 heads,
    V=32000 bf16, l ~N(0,4^2), proposals match head 0's argmax w.p. 0.7."""
    return make_greedy_heads(B, 4, 4, 32000, BF16, seed, sigma=4.0, match_prob=0.7,
                             name="greedy-heads B=%d K=4 H=4 V=32000 bf16" % B)


def cut_best_of_n(P: int = 128, seed: int = 1008) -> CutWorkload:
    """P=128 prompts with N=1000 partial-reward scores each, alpha=0.5."""
    return make_cut(P, 1000, 0.5, seed, name="cut P=%d N=1000 alpha=0.5" % P)


NEXT_CONFIGS = {
    "sample": sampler_draft_rows,
    "heads": greedy_heads_blockwise,
    "cut": cut_best_of_n,
}
