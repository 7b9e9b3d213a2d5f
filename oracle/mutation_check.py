"""Check that the oracle's pins catch plausible mistakes (CPU only).

For each planted mistake below, a copy of ``oracle/``, ``synth/`` and the pin
tests is made in a temporary directory, the mistake is written into the
copy's ``moe_oracle.c``, and ``tests/test_oracle_pins.py`` is run there.  A
mistake the pins do not catch is reported as MISSED.  The repository's own
sources are never modified.

    python oracle/mutation_check.py
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, original text, planted text).  "clamp at 128" is an equivalent
# mutant: with s = amax/127 no |x/s| rounds above 127, so no pin can catch it.
MUTANTS = [
    ("tie-break keeps higher index", "z[e] > z[best]", "z[e] >= z[best]"),
    ("int4 nibble order", "(idx & 1) ? (byte >> 4) : (byte & 15)", "(idx & 1) ? (byte & 15) : (byte >> 4)"),
    ("int4 zero point 7", "return u - 8;", "return u - 7;"),
    ("silu sign", "z / (1.0 + exp(-z))", "z / (1.0 + exp(z))"),
    ("round half away from zero", "rintf(x[b * 32 + i] / sc)", "roundf(x[b * 32 + i] / sc)"),
    ("router bias sign", "if (bias) acc += (double)bias[e];", "if (bias) acc -= (double)bias[e];"),
    ("activation scale amax/128", "amax / 127.0f", "amax / 128.0f"),
    ("gate and up swapped (float)", "h[n] = silu(g[n]) * u[n];", "h[n] = silu(u[n]) * g[n];"),
    ("gate and up swapped (int8)", "hf[n] = (float)(silu(g[n]) * u[n]);", "hf[n] = (float)(silu(u[n]) * g[n]);"),
    ("scale block index off by one", "r * nb + c / 32", "r * nb + (c / 32 + 1) % nb"),
    ("gates applied in reverse slot order", "gates[(size_t)t * k + j] * ysel",
     "gates[(size_t)t * k + (k - 1 - j)] * ysel"),
    ("softmax term perturbed", "p[j] = exp(z[ids[j]] - m);", "p[j] = exp(z[ids[j]] - m) * (j == 0 ? 1.0 : 1.0001);"),
    ("permutation not stable", "int32_t p = cursor[ids[f]]++;",
     "int32_t p = offsets[ids[f] + 1] - 1 - (cursor[ids[f]]++ - offsets[ids[f]]);"),
    ("rmsnorm eps outside the root", "sqrt(ss / (double)d + eps)", "(sqrt(ss / (double)d) + 1e-2)"),
    ("residual dropped", "double acc = residual ? (double)residual[(size_t)t * d + o] : 0.0;", "double acc = 0.0;"),
    ("shared expert dropped", "if (ysh) acc += ysh[(size_t)i * d + o];", "if (ysh) acc += 0.0;"),
    ("binary16 subnormal exponent", "ldexp((double)m, -24)", "ldexp((double)m, -25)"),
    ("down matrix transposed", "X->wd[(size_t)o * f + n]", "X->wd[(size_t)(n % d) * f + (o % f)]"),
    ("clamp at 128 (equivalent)", "if (r > 127.0f) r = 127.0f;", "if (r > 128.0f) r = 128.0f;"),
    # the int8-activation second half: requantised h and the int8 down projection
    ("h block scales 0.2% high", "quant8_row(hf, f, hq, hs);",
     "quant8_row(hf, f, hq, hs); for (int b_ = 0; b_ < f / 32; ++b_) hs[b_] *= 1.002f;"),
    ("g and u rounded to fp32 before SwiGLU", "hf[n] = (float)(silu(g[n]) * u[n]);",
     "hf[n] = (float)(silu((double)(float)g[n]) * (double)(float)u[n]);"),
    ("int8 down scaled by the x block scales", "y[o] = q8_dot(hq, hs,", "y[o] = q8_dot(hq, xs,"),
    ("int8 block sum drops its last element", "for (int i = 0; i < 32; ++i) blk +=",
     "for (int i = 0; i < 31; ++i) blk +="),
    ("h code off by one at the top", "q[b * 32 + i] = (int8_t)v;",
     "q[b * 32 + i] = (int8_t)(v == 127 ? 126 : v);"),
]


def run() -> int:
    src = open(os.path.join(ROOT, "oracle", "moe_oracle.c")).read()
    missed = []
    with tempfile.TemporaryDirectory() as tmp:
        for sub in ("oracle", "synth", "tests"):
            shutil.copytree(os.path.join(ROOT, sub), os.path.join(tmp, sub),
                            ignore=shutil.ignore_patterns("*.so", "__pycache__", "golden"))
        shutil.copy(os.path.join(ROOT, "pytest.ini"), tmp)
        for name, a, b in MUTANTS:
            if a not in src:
                print("%-40s SITE NOT FOUND" % name, flush=True)
                missed.append(name)
                continue
            with open(os.path.join(tmp, "oracle", "moe_oracle.c"), "w") as fh:
                fh.write(src.replace(a, b, 1))
            lib = os.path.join(tmp, "oracle", "liboracle.so")
            if os.path.exists(lib):
                os.remove(lib)
            r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                                "tests/test_oracle_pins.py"], cwd=tmp, capture_output=True, text=True)
            failed = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
            if r.returncode == 0:
                print("%-40s MISSED" % name, flush=True)
                missed.append(name)
            else:
                print("%-40s caught by %s" % (name, failed[0].split(" ")[1] if failed else "(error)"), flush=True)
    expected = {"clamp at 128 (equivalent)"}
    return 0 if set(missed) <= expected else 1


if __name__ == "__main__":
    sys.exit(run())
