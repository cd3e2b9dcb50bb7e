"""The oracle's pins must catch plausible mistakes.

Each case below plants one mistake in a copy of the oracle's C source (in a
temporary directory; the real oracle is untouched), builds it, and runs the
oracle's pin tests against that build in a child process: they must fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sage_oracle.c")
PINS = ["tests/test_oracle_codecs.py", "tests/test_oracle_quant.py", "tests/test_oracle_attention.py"]

MUTATIONS = {
    "online softmax: running sum not rescaled": ("l *= alpha;", ""),
    "online softmax: accumulator not rescaled": ("for (int c = 0; c < dp; ++c) acc[c] *= alpha;", ""),
    # the reference maximum kept until a tile exceeds it by 3 (a lazy update)
    "online softmax: lazy maximum (threshold 3)": ("float mn = mt > m ? mt : m;",
                                                   "float mn = (m == -INFINITY || mt > m + 3.0f) ? mt : m;"),
    # the exponent formed as (B + S) f + (-B f - m') with a large integer bias B
    "exponent: biased fused form": ("volatile float x = s[j] - m;",
                                    "volatile float x = fmaf(10680707.0f + (float)S[j], kscale[j] * ci2, "
                                    "fmaf(-10680707.0f, kscale[j] * ci2, -m));"),
    "row sum over unrounded P": ("l += pq;", "l += (double)pp;"),
    "dequant: wrong key-group scale": ("volatile float t = (float)S[j] * kscale[j];",
                                       "volatile float t = (float)S[j] * kscale[j + 1 < nk ? j + 1 : j];"),
    "P scale 256 instead of 448": ("const double pscale = p_mode == 0 ? E4M3_MAX : 1.0;",
                                   "const double pscale = p_mode == 0 ? 256.0 : 1.0;"),
    "lse: smoothing correction sign": ("lse[ri] = ((double)m - log2(pscale) + log2(l)) * M_LN2 + corr;",
                                       "lse[ri] = ((double)m - log2(pscale) + log2(l)) * M_LN2 - corr;"),
    "causal: diagonal masked": ("long lim = (long)i + causal_shift;\n            if (lim < last) last = (int)lim;",
                                "long lim = (long)i + causal_shift - 1;\n            if (lim < last) last = (int)lim;"),
    "epilogue: V scale dropped": ("double sc = p_mode == 0 ? (double)vscale[c] : 1.0;",
                                  "double sc = p_mode == 0 ? 1.0 / 448.0 : 1.0;"),
    "epilogue: V mean not added back": ("out[(size_t)ri * dp + c] = o * sc + (vmean ? (double)vmean[c] : 0.0);",
                                        "out[(size_t)ri * dp + c] = o * sc;"),
    "allowance: exponent band ignored": ("if (delta > 0.0) {", "if (delta < 0.0) {"),
    "INT8: truncation instead of rounding": ("float q = nearbyintf(t);", "float q = truncf(t);"),
    "INT8: scale amax/128": ("volatile float scale = amax / 127.0f;", "volatile float scale = amax / 128.0f;"),
    "tile max over one key": ("for (int j = t0; j <= t1; ++j) if (s[j] > mt) mt = s[j];",
                              "for (int j = t0; j <= t1 && j < t0 + 1; ++j) if (s[j] > mt) mt = s[j];"),
    "E4M3 without subnormals": ("static double e4m3_value(double x) {               /* x already in [-448, 448] */\n    return fmt_rne(x, 3, -6);",
                                "static double e4m3_value(double x) {\n    return fmt_rne(x, 3, -7);"),
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    a, b = MUTATIONS[name]
    assert a in src, "mutation anchor not found; update the case"
    mutated = tmp_path / "mutated.c"
    mutated.write_text(src.replace(a, b))
    so = tmp_path / "libmutated.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", str(mutated),
                           "-o", str(so), "-lm"])
    env = dict(os.environ, SAGE_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
