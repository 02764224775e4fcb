"""The oracle pins must catch plausible mistakes (CPU only).

Each case compiles a copy of the oracle's C source with one deliberate slip, points the
oracle wrapper at it through SPECVERIFY_ORACLE_LIB, runs the pin suite in a child
process and requires that it fails.  The unmodified source must pass the same run.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "specverify_oracle.c")

# (name, exact text in the source, replacement)
MUTANTS = [
    ("replacement drawn from p, not the residual",
     "double d = pL[v] - qL[v];", "double d = pL[v];"),
    ("accept ratio inverted (q/p)",
     "int accept = (P > 0.0) && (uj * Q <= P);", "int accept = (Q > 0.0) && (uj * P <= Q);"),
    ("replacement reuses the rejected position's uniform",
     "int y = inverse_cdf(w, V, (double)u[K], &mu_y, &alt);",
     "int y = inverse_cdf(w, V, (double)u[L], &mu_y, &alt);"),
    ("temperature left off the draft",
     "z[v] = logit_at(dtype, draft, off + v) / T;", "z[v] = logit_at(dtype, draft, off + v);"),
    ("draft law read one position late",
     "double Q = q[(size_t)j * V + x[j]];",
     "double Q = q[(size_t)(j + 1 < K ? j + 1 : j) * V + x[j]];"),
    ("bonus drawn from the last draft position",
     "const double *pL = p + (size_t)L * V;",
     "const double *pL = p + (size_t)(L < K ? L : (K > 0 ? K - 1 : 0)) * V;"),
    ("no truncation after the first rejection",
     "        if (L < K)\n            continue; /* already rejected: later tokens are discarded */\n",
     ""),
    ("argmax ties go to the highest id", "if (x > bv) {", "if (x >= bv) {"),
    ("inverse CDF with >= instead of >", "if (c > t) {", "if (c >= t) {"),
    ("softmax without the max shift", "S += exp(z[v] - m);", "S += exp(z[v]);"),
    ("contrastive difference reversed",
     "z[v] = (logit_at(dtype, expert, off + v) - logit_at(dtype, amateur, off + v)) / tau;",
     "z[v] = (logit_at(dtype, amateur, off + v) - logit_at(dtype, expert, off + v)) / tau;"),
    ("contrastive draft law tempered by tau",
     "z[v] = logit_at(dtype, amateur, off + v);", "z[v] = logit_at(dtype, amateur, off + v) / tau;"),
    ("greedy emits the proposal at the mismatch",
     "            tok[j] = g;\n", "            tok[j] = (j < K) ? x[j] : g;\n"),
    ("next proposals from the last accepted position instead of L",
     "size_t rowL = ((size_t)b * (K + 1) + L) * H;",
     "size_t rowL = ((size_t)b * (K + 1) + (L > 0 ? L - 1 : 0)) * H;"),
    ("next proposals from the head before",
     "nxt[h - 1] = first_argmax(dtype, logits, (rowL + h) * V, V);",
     "nxt[h - 1] = first_argmax(dtype, logits, (rowL + h - 1) * V, V);"),
    ("sampler without the temperature",
     "            z[v] = logit_at(dtype, logits, off + v) / T;\n        oracle_softmax(z, V, p);",
     "            z[v] = logit_at(dtype, logits, off + v);\n        oracle_softmax(z, V, p);"),
    ("quantile index rounded up", "long k = (long)floor(alpha * (double)N);",
     "long k = (long)ceil(alpha * (double)N);"),
    ("cut keeps only scores strictly above it", "uint8_t kk = row[i] >= cut;",
     "uint8_t kk = row[i] > cut;"),
]

# the quick pins (the z-tests at the larger sizes add nothing for these slips)
PIN_SELECTION = "not (mean_accepted_length and (c2 or c3 or c5))"


def _build(src_text, out):
    cpath = out + ".c"
    with open(cpath, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", out, cpath, "-lm"])


def _run_pins(lib):
    env = dict(os.environ, SPECVERIFY_ORACLE_LIB=lib)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
           os.path.join(ROOT, "tests", "test_oracle_pins.py"),
           os.path.join(ROOT, "tests", "test_oracle_pins_next.py"), "-k", PIN_SELECTION]
    return subprocess.run(cmd, env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)


def test_unmodified_oracle_passes(tmp_path):
    lib = str(tmp_path / "liboracle_ok.so")
    _build(open(SRC).read(), lib)
    res = _run_pins(lib)
    assert res.returncode == 0, res.stdout[-3000:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor vanished: " + name
    lib = str(tmp_path / "liboracle_mut.so")
    _build(src.replace(old, new), lib)
    res = _run_pins(lib)
    assert res.returncode != 0, "pins did not catch: " + name
