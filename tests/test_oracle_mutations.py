"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one typical mistake in a scratch copy of
oracle/uly_oracle.c, builds it, and runs the oracle's pin tests against that
build in a child process (ULY_ORACLE_LIB points the oracle at it).  Every
mutant must fail at least one pin; the unmodified source, built the same
way, must pass them all.  The mistakes are the kind a port of the pages'
formulas could make: a dropped term, a flipped sign, a wrong index or map,
a transposed operand.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "uly_oracle.c")
PINS = [os.path.join(ROOT, "tests", f) for f in
        ("test_oracle_relayout.py", "test_oracle_norm_rope.py", "test_oracle_proj.py")]

# (name, text in uly_oracle.c, replacement); each replacement keeps every access in bounds
MUTANTS = [
    ("eps dropped", "1.0 / sqrt(ss / (double)D + eps)", "1.0 / sqrt(ss / (double)D)"),
    ("mean over D-1", "1.0 / sqrt(ss / (double)D + eps)", "1.0 / sqrt(ss / (double)(D - 1) + eps)"),
    ("|x| for x^2", "ss += xr[i] * xr[i];", "ss += fabs(xr[i]);"),
    ("weight index", "double n1 = xr[2 * j + 1] * inv * w[2 * j + 1];", "double n1 = xr[2 * j + 1] * inv * w[2 * j];"),
    ("sign of y_2j", "yr[2 * j] = n0 * c - n1 * s;", "yr[2 * j] = n0 * c + n1 * s;"),
    ("sign of y_2j+1", "yr[2 * j + 1] = n0 * s + n1 * c;", "yr[2 * j + 1] = -n0 * s + n1 * c;"),
    ("rotate-half pairing", "double n1 = xr[2 * j + 1] * inv * w[2 * j + 1];",
     "double n1 = xr[(2 * j + half) % D] * inv * w[(2 * j + half) % D];"),
    ("frequency exponent halved", "double freq = pow(theta, -2.0 * (double)j / (double)D);",
     "double freq = pow(theta, -1.0 * (double)j / (double)D);"),
    ("3-D table: w axis for the h band", "pos_a = h; k = j - n_t; width = 2 * n_h;",
     "pos_a = w; k = j - n_t; width = 2 * n_h;"),
    ("round-robin heads", "int64_t src = ((((r * B + b) * S_l + s) * H) + (q * Hl + j)) * D + d;",
     "int64_t src = ((((r * B + b) * S_l + s) * H) + (j * P + q)) * D + d;"),
    ("transposed sequence map", "int64_t dst = ((((q * B + b) * S + (r * S_l + s)) * Hl) + j) * D + d;",
     "int64_t dst = ((((q * B + b) * S + (s * P + r)) * Hl) + j) * D + d;"),
    ("gather head band", "int64_t dst = ((((r * B + b) * S_l + s) * H) + (q * Hl + j)) * D + d;",
     "int64_t dst = ((((r * B + b) * S_l + s) * H) + (j * P + q)) * D + d;"),
    ("chunk exchange not transposed", "memcpy(y + (q * P + r) * chunk_bytes, x + (r * P + q) * chunk_bytes",
     "memcpy(y + (r * P + q) * chunk_bytes, x + (r * P + q) * chunk_bytes"),
    ("projection operand transposed", "acc += x[m * K + k] * w[n * K + k];", "acc += x[m * K + k] * w[k * N + n];"),
    ("pad shard map", "int64_t g = r * S_l + s;\n                    unsigned char *dst", "int64_t g = s * P + r;\n                    unsigned char *dst"),
    ("halo bound dropped", "if (i < h[r] + 2 * halo && src_row >= 0 && src_row < Hh)", "if (src_row >= 0 && src_row < Hh)"),
    ("stacked gather keeps the halo", "sh + ((((r * N) + n) * rows + (halo + i)) * W + c) * es",
     "sh + ((((r * N) + n) * rows + i) * W + c) * es"),
]


def _run_pins(src_text: str, tmp: str, tag: str) -> int:
    c_path = os.path.join(tmp, "m_%s.c" % tag)
    so_path = os.path.join(tmp, "m_%s.so" % tag)
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-o", so_path, c_path, "-lm"])
    env = dict(os.environ, ULY_ORACLE_LIB=so_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, timeout=600)
    return r.returncode


def test_pins_catch_planted_mistakes():
    text = open(SRC).read()
    for name, old, new in MUTANTS:
        assert text.count(old) == 1, "mutation site for %r not found exactly once" % name
    with tempfile.TemporaryDirectory() as tmp:
        jobs = [("control", text)] + [(name, text.replace(old, new)) for name, old, new in MUTANTS]
        with ThreadPoolExecutor(max_workers=4) as ex:
            codes = list(ex.map(lambda j: _run_pins(j[1], tmp, "%02d" % jobs.index(j)), jobs))
    assert codes[0] == 0, "the unmodified oracle must pass its pins (exit %d)" % codes[0]
    missed = [name for (name, _), code in zip(jobs[1:], codes[1:]) if code == 0]
    assert not missed, "mutants no pin caught: %s" % missed
