"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle -- a dropped term, a
wrong sign, index or exponent, a transposed operand -- and runs the pin suite
(tests/test_oracle_pins.py) against it in a fresh interpreter: some pin must
fail with an assertion (pytest exit status 1).  The unmodified oracle must
pass the same run, so a broken runner cannot pass for a caught mistake.

C mistakes are planted in a copy of oracle/la_oracle.c built into a temporary
library; the numpy parts (the gated group RMSNorm epilogue, the packed-batch
driver) are replaced by mistaken versions in the child interpreter only.
Nothing here touches the GPU or the HIP library.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "la_oracle.c")

# (name, text to replace, replacement, which occurrence of the text)
C_MUTANTS = [
    ("forward decay sign", "lam = exp(-(double)slope[h]);", "lam = exp((double)slope[h]);", 0),
    ("forward outer product transposed", "kt[i] * vt[j];", "kt[j] * vt[i];", 0),
    ("forward output reads the wrong q entry",
     "ot[j] += qt[i] * S[(size_t)i * d + j]", "ot[j] += qt[j] * S[(size_t)i * d + j]", 0),
    ("forward drops the initial state",
     "memcpy(S, S0 + sb, sizeof(double) * (size_t)d * d);",
     "memset(S, 0, sizeof(double) * (size_t)d * d);", 0),
    ("forward decays the current token",
     "lam * S[(size_t)i * d + j] + kt[i] * vt[j]", "lam * (S[(size_t)i * d + j] + kt[i] * vt[j])", 0),
    ("decode reads o with k", "ob[j] += qb[i] * S", "ob[j] += kb[i] * S", 0),
    ("decode without decay", "lam = exp(-(double)slope[h]);", "lam = 1.0;", 1),
    ("backward dq with the state transposed",
     "acc += S[(size_t)i * d + j] * gt[j];", "acc += S[(size_t)j * d + i] * gt[j];", 0),
    ("backward adjoint state built from k", "qt[i] * gt[j];", "kt[i] * gt[j];", 0),
    ("backward dk with the adjoint transposed",
     "acc += G[(size_t)i * d + j] * vt[j];", "acc += G[(size_t)j * d + i] * vt[j];", 0),
    ("backward dv sign", "dvt[j] += G[(size_t)i * d + j] * kt[i];",
     "dvt[j] -= G[(size_t)i * d + j] * kt[i];", 0),
    ("backward decays the current token",
     "lam * G[(size_t)i * d + j] + qt[i] * gt[j]", "lam * (G[(size_t)i * d + j] + qt[i] * gt[j])", 0),
    ("backward decay sign", "lam = exp(-(double)slope[h]);", "lam = exp((double)slope[h]);", 2),
    ("chunked intra-chunk mask exponent", "exp(-s * (double)(i - j))",
     "exp(-s * (double)(i - j + 1))", 0),
    ("chunked inter-chunk row decay", "exp(-s * (double)(i + 1))", "exp(-s * (double)(i))", 0),
    ("chunked state decay", "exp(-s * (double)n)", "exp(-s * (double)(n - 1))", 0),
    ("chunked state update weights", "exp(-s * (double)(n - 1 - j))", "exp(-s * (double)(n - j))", 0),
    ("chunked drops the initial state",
     "memcpy(S, S0 + sb, sizeof(double) * (size_t)d * d);",
     "memset(S, 0, sizeof(double) * (size_t)d * d);", 2),
]

PY_MUTANTS = [
    "gated norm: eps outside the square root",
    "gated norm: gate sign",
    "gated norm: mean over tokens",
    "gated norm: no weight",
    "packed batch: state carried into the next sequence",
]

# The child: plant the mistake, then run the pin suite in-process.
RUNNER = r"""
import os, sys
root, kind, arg = sys.argv[1], sys.argv[2], sys.argv[3]
sys.path.insert(0, root)
import numpy as np
import oracle
import oracle.core as core

def patch(name, f):
    setattr(core, name, f)
    setattr(oracle, name, f)

def gated(o, gate, weight, eps, eps_in=True, sign=1.0, axis=-1, use_w=True):
    o = np.asarray(o, dtype=np.float64); g = np.asarray(gate, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    ms = np.mean(o * o, axis=axis, keepdims=True)
    r = np.sqrt(ms + eps) if eps_in else np.sqrt(ms) + eps
    y = o / r / (1.0 + np.exp(-sign * g))
    return y * w[:, None, :] if use_w else y

if kind == "lib":
    core._LIB = arg
    core._lib = None
elif kind == "py":
    if arg == "gated norm: eps outside the square root":
        patch("gated_group_rmsnorm", lambda o, g, w, e: gated(o, g, w, e, eps_in=False))
    elif arg == "gated norm: gate sign":
        patch("gated_group_rmsnorm", lambda o, g, w, e: gated(o, g, w, e, sign=-1.0))
    elif arg == "gated norm: mean over tokens":
        patch("gated_group_rmsnorm", lambda o, g, w, e: gated(o, g, w, e, axis=-2))
    elif arg == "gated norm: no weight":
        patch("gated_group_rmsnorm", lambda o, g, w, e: gated(o, g, w, e, use_w=False))
    elif arg == "packed batch: state carried into the next sequence":
        def fwd_varlen(q, k, v, slope, cu, S0=None):
            q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
            H, T, d = q.shape
            cu = [int(x) for x in cu]
            o = np.empty_like(q)
            S = np.empty((len(cu) - 1, H, d, d))
            prev = None
            for s in range(len(cu) - 1):
                a, b = cu[s], cu[s + 1]
                init = prev if prev is not None else (None if S0 is None else np.asarray(S0)[s][None])
                o_s, S_s = core.fwd(q[None, :, a:b], k[None, :, a:b], v[None, :, a:b], slope, init)
                o[:, a:b] = o_s[0]
                S[s] = S_s[0]
                prev = S_s
            return o, S
        patch("fwd_varlen", fwd_varlen)
    else:
        raise SystemExit("unknown mutant " + arg)

import pytest
sys.exit(pytest.main(["-x", "-q", "-p", "no:cacheprovider",
                      os.path.join(root, "tests", "test_oracle_pins.py")]))
"""


def run_pins(kind, arg):
    r = subprocess.run([sys.executable, "-c", RUNNER, ROOT, kind, arg], cwd=ROOT,
                       capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-3000:]


def plant(src, old, new, occurrence):
    at = -1
    for _ in range(occurrence + 1):
        at = src.find(old, at + 1)
        assert at >= 0, "mutation site not found: %r #%d" % (old, occurrence)
    return src[:at] + new + src[at + len(old):]


def test_unmodified_oracle_passes_the_pins():
    code, out = run_pins("none", "-")
    assert code == 0, out


@pytest.mark.parametrize("name,old,new,occurrence", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_mistake_fails_a_pin(tmp_path, name, old, new, occurrence):
    src = open(SRC).read()
    mutated = plant(src, old, new, occurrence)
    assert mutated != src
    c = tmp_path / "mutant.c"
    so = tmp_path / "libmutant.so"
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(c),
                           "-o", str(so), "-lm"])
    code, out = run_pins("lib", str(so))
    assert code == 1, "%s: pins exit status %d (1 = a pin failed)\n%s" % (name, code, out)


@pytest.mark.parametrize("name", PY_MUTANTS)
def test_numpy_mistake_fails_a_pin(name):
    code, out = run_pins("py", name)
    assert code == 1, "%s: pins exit status %d (1 = a pin failed)\n%s" % (name, code, out)
