"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
its pins catch every one.  Each mutant is compiled to a temporary library and
run by tests/mutation_battery.py in a subprocess."""
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")

# (name, text in oracle.c, replacement): each is a mistake someone could make.
MUTANTS = [
    ("1d pad side swapped", "long pL = causal ? K - 1 : (K - 1) / 2;", "long pL = causal ? 0 : (K - 1) / 2;"),
    ("1d symmetric pad off by one", "long pL = causal ? K - 1 : (K - 1) / 2;", "long pL = causal ? K - 1 : K / 2;"),
    ("1d weights read as [C][K]", "acc += xp[t + k] * (double)w[k * C + c];", "acc += xp[t + k] * (double)w[c * K + k];"),
    ("1d kernel flipped", "acc += xp[t + k] * (double)w[k * C + c];", "acc += xp[t + k] * (double)w[(K - 1 - k) * C + c];"),
    ("1d input mask one frame late", "xp[s] = (t >= 0 && t < len)", "xp[s] = (t >= 0 && t <= len && t < T)"),
    ("1d input not masked", "xp[s] = (t >= 0 && t < len)", "xp[s] = (t >= 0 && t < T)"),
    ("1d output mask dropped", "                if (t < len) {\n                    for (long k = 0; k < K; ++k)",
     "                if (1) {\n                    for (long k = 0; k < K; ++k)"),
    ("1d bias dropped", "                    acc += bias ? (double)bias[c] : 0.0;\n                }\n                y[(b * T + t) * C + c] = acc;",
     "                }\n                y[(b * T + t) * C + c] = acc;"),
    ("1d batch axis scrambled", "xp[s] = (t >= 0 && t < len) ? (double)x[(b * T + t) * C + c] : 0.0;",
     "xp[s] = (t >= 0 && t < len) ? (double)x[(((B - 1 - b)) * T + t) * C + c] : 0.0;"),
    ("length not clamped", "    if (l > T) l = T;\n", "\n"),
    ("2d stride ignored in time", "long t = s * to + i - pt0;\n                            if (t < 0 || t >= len) continue; /* padding or pre-masked */",
     "long t = to + i - pt0;\n                            if (t < 0 || t >= len) continue; /* padding or pre-masked */"),
    ("2d time pad taken from the wrong side", "long t = s * to + i - pt0;\n                            if (t < 0 || t >= len) continue; /* padding or pre-masked */",
     "long t = s * to + i - pt1;\n                            if (t < 0 || t >= len) continue; /* padding or pre-masked */"),
    ("2d frequency pad taken from time", "                                long f = s * fo + j - pf0;",
     "                                long f = s * fo + j - pt0;"),
    ("2d bwd frequency pad from the wrong side", "                            long f = s * fo + j - pf0;\n                            if (f < 0 || f >= F) continue;\n                            size_t xi",
     "                            long f = s * fo + j - pf1;\n                            if (f < 0 || f >= F) continue;\n                            size_t xi"),
    ("output length doubles the pad before", "long o = floor_div(n + pl + ph - k, s) + 1;", "long o = floor_div(n + 2 * pl - k, s) + 1;"),
    ("2d empty item not masked", "        if (leno > To) leno = To;\n        if (len == 0) leno = 0;\n        for (long to = 0; to < To; ++to)",
     "        if (leno > To) leno = To;\n        for (long to = 0; to < To; ++to)"),
    ("front causal mode pads symmetrically", "    long pl = causal ? 2 : 1;\n    long T1 = conv_out_len(T, 3, 2, pl, 1), F1 = conv_out_len(F, 3, 2, pl, 1);\n    long T2 = conv_out_len(T1, 3, 2, pl, 1), F2 = conv_out_len(F1, 3, 2, pl, 1);\n    size_t hn = (size_t)(T1 * F1 * C);\n    double *h",
     "    long pl = 1;\n    long T1 = conv_out_len(T, 3, 2, pl, 1), F1 = conv_out_len(F, 3, 2, pl, 1);\n    long T2 = conv_out_len(T1, 3, 2, pl, 1), F2 = conv_out_len(F1, 3, 2, pl, 1);\n    size_t hn = (size_t)(T1 * F1 * C);\n    double *h"),
    ("front causal mask ceil(len/2)", "long L1 = len > 0 ? conv_out_len(len, 3, 2, pl, 1) : 0;", "long L1 = (len + 1) / 2;"),
    ("front empty item not masked", "long L1 = len > 0 ? conv_out_len(len, 3, 2, pl, 1) : 0;", "long L1 = conv_out_len(len, 3, 2, pl, 1);"),
    ("front bwd causal pads symmetric", "    long pl = causal ? 2 : 1;\n    long T1 = conv_out_len(T, 3, 2, pl, 1), F1 = conv_out_len(F, 3, 2, pl, 1);\n    long T2 = conv_out_len(T1, 3, 2, pl, 1), F2 = conv_out_len(F1, 3, 2, pl, 1);\n    size_t hn = (size_t)(T1 * F1 * C);\n    double *z",
     "    long pl = 1;\n    long T1 = conv_out_len(T, 3, 2, pl, 1), F1 = conv_out_len(F, 3, 2, pl, 1);\n    long T2 = conv_out_len(T1, 3, 2, pl, 1), F2 = conv_out_len(F1, 3, 2, pl, 1);\n    size_t hn = (size_t)(T1 * F1 * C);\n    double *z"),
    ("2d pre-mask dropped", "if (t < 0 || t >= len) continue; /* padding or pre-masked */",
     "if (t < 0 || t >= T) continue; /* padding or pre-masked */"),
    ("2d post-mask length floor", "        long leno = conv_out_len(len, KH, s, pt0, pt1);\n        if (leno > To) leno = To;\n        if (len == 0) leno = 0;\n        for (long to = 0; to < To; ++to)",
     "        long leno = len / 2;\n        if (leno > To) leno = To;\n        if (len == 0) leno = 0;\n        for (long to = 0; to < To; ++to)"),
    ("2d taps transposed", "                                       (double)w[(i * KW + j) * C + c];",
     "                                       (double)w[(j * KH + i) * C + c];"),
    ("2d bias after mask", "                        acc += bias ? (double)bias[c] : 0.0;\n                    }\n                    y[((b * To + to) * Fo + fo) * C + c] = acc;",
     "                    }\n                    acc += bias ? (double)bias[c] : 0.0;\n                    y[((b * To + to) * Fo + fo) * C + c] = acc;"),
    ("bwd dy beyond the mask used", "        for (long to = 0; to < leno; ++to)\n            for (long fo = 0; fo < Fo; ++fo)\n                for (long c = 0; c < C; ++c) {\n                    double g",
     "        for (long to = 0; to < To; ++to)\n            for (long fo = 0; fo < Fo; ++fo)\n                for (long c = 0; c < C; ++c) {\n                    double g"),
    ("bwd dx uses flipped taps", "if (dx) dx[xi] += g * (double)w[wi];",
     "if (dx) dx[xi] += g * (double)w[((KH - 1 - i) * KW + (KW - 1 - j)) * C + c];"),
    ("bwd db counted per tap", "                    if (db) db[c] += g;\n                    for (long i = 0; i < KH; ++i) {",
     "                    for (long i = 0; i < KH; ++i) {\n                        if (db) db[c] += g;"),
    ("bwd dw misses the pre-mask", "                        long t = s * to + i - pt0;\n                        if (t < 0 || t >= len) continue;\n                        for (long j = 0; j < KW; ++j) {\n                            long f = s * fo + j - pf0;\n                            if (f < 0 || f >= F) continue;\n                            size_t xi",
     "                        long t = s * to + i - pt0;\n                        if (t < 0 || t >= T) continue;\n                        for (long j = 0; j < KW; ++j) {\n                            long f = s * fo + j - pf0;\n                            if (f < 0 || f >= F) continue;\n                            size_t xi"),
    ("front ReLU dropped", "v = acc > 0.0 ? acc : 0.0;", "v = acc;"),
    ("front mask floor(len/2)", "long L1 = len > 0 ? conv_out_len(len, 3, 2, pl, 1) : 0;", "long L1 = len / 2;"),
    ("front mask dropped", "if (t1 < L1) {", "if (1) {"),
    ("front input length-masked", "                            if (t < 0 || t >= T) continue;\n                            for (long j = 0; j < 3; ++j) {\n                                long f = 2 * f1 + j - pl;",
     "                            if (t < 0 || t >= len) continue;\n                            for (long j = 0; j < 3; ++j) {\n                                long f = 2 * f1 + j - pl;"),
    ("front output bias dropped", "                    acc += b1 ? (double)b1[c] : 0.0;\n", "\n"),
    ("front conv0 bias after ReLU", "                        acc += b0 ? (double)b0[c] : 0.0;\n                        v = acc > 0.0 ? acc : 0.0;",
     "                        v = acc > 0.0 ? acc : 0.0;\n                        v += b0 ? (double)b0[c] : 0.0;"),
    ("front stage-2 stride 1", "long t1 = 2 * t2 + i - pl;", "long t1 = t2 + i - pl;"),
    ("front bwd ReLU derivative ignored", "double dz = z[q] > 0.0 ? dh[q] : 0.0;", "double dz = dh[q];"),
    ("front bwd time mask ignored", "if (t1 >= L1) continue; /* masked", "if (0) continue; /* masked"),
    ("front bwd dh with flipped taps", "dh[q] += g * (double)w1[(i * 3 + j) * C + c];",
     "dh[q] += g * (double)w1[((2 - i) * 3 + (2 - j)) * C + c];"),
    ("front bwd dw1 from pre-ReLU z", "if (dw1) dw1[(i * 3 + j) * C + c] += g * h[q];",
     "if (dw1) dw1[(i * 3 + j) * C + c] += g * z[q];"),
    ("front bwd dw0 taps transposed", "dw0[(i * 3 + j) * C + c] += dz * (double)x[(b * T + t) * F + f];",
     "dw0[(j * 3 + i) * C + c] += dz * (double)x[(b * T + t) * F + f];"),
    ("1d bwd dx with unflipped taps", "if (dx) dx[(b * T + u) * C + c] += g * (double)w[k * C + c];",
     "if (dx) dx[(b * T + u) * C + c] += g * (double)w[(K - 1 - k) * C + c];"),
    ("1d bwd dy beyond the length used", "        for (long t = 0; t < len; ++t)\n            for (long c = 0; c < C; ++c) {\n                double g = (double)dy[(b * T + t) * C + c];",
     "        for (long t = 0; t < T; ++t)\n            for (long c = 0; c < C; ++c) {\n                double g = (double)dy[(b * T + t) * C + c];"),
    ("1d bwd x beyond the length used", "if (u < 0 || u >= len) continue;\n                    if (dx) dx[(b * T + u) * C + c]",
     "if (u < 0 || u >= T) continue;\n                    if (dx) dx[(b * T + u) * C + c]"),
    ("1d bwd pad side swapped", "    long pL = causal ? K - 1 : (K - 1) / 2;\n    if (dx) memset(dx, 0, sizeof(double) * (size_t)(B * T * C));",
     "    long pL = causal ? 0 : (K - 1) / 2;\n    if (dx) memset(dx, 0, sizeof(double) * (size_t)(B * T * C));"),
    ("stream cache taken from the chunk end", "cache_out[(b * (K - 1) + j) * C + c] = sq[len + j];",
     "cache_out[(b * (K - 1) + j) * C + c] = sq[Tc + j];"),
    ("stream cache not shifted", "cache_out[(b * (K - 1) + j) * C + c] = sq[len + j];",
     "cache_out[(b * (K - 1) + j) * C + c] = sq[j];"),
    ("stream chunk placed before the cache", "for (long u = 0; u < len; ++u) sq[K - 1 + u] = (double)x[(b * Tc + u) * C + c];",
     "for (long u = 0; u < len; ++u) sq[u] = (double)x[(b * Tc + u) * C + c];"),
    ("stream output mask dropped", "                if (t < len) {\n                    for (long k = 0; k < K; ++k)\n                        acc += sq[t + k]",
     "                if (t < Tc) {\n                    for (long k = 0; k < K; ++k)\n                        acc += sq[t + k]"),
    ("stream kernel flipped", "acc += sq[t + k] * (double)w[k * C + c];", "acc += sq[t + k] * (double)w[(K - 1 - k) * C + c];"),
    ("front bwd b0 left out of the recompute", "acc += b0 ? (double)b0[c] : 0.0;\n                    size_t q",
     "size_t q"),
]


def run_battery(src_text, tmpdir, tag):
    src = os.path.join(tmpdir, f"{tag}.c")
    lib = os.path.join(tmpdir, f"{tag}.so")
    with open(src, "w") as f:
        f.write(src_text)
    oracle.compile_c(src, lib)
    r = subprocess.run([sys.executable, os.path.join(HERE, "mutation_battery.py"), lib],
                       capture_output=True, text=True, timeout=300)
    return r


@pytest.fixture(scope="module")
def tmpdir():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.fixture(scope="module")
def original():
    with open(SRC) as f:
        return f.read()


def test_unmutated_oracle_passes_the_battery(original, tmpdir):
    r = run_battery(original, tmpdir, "control")
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, original, tmpdir):
    assert original.count(old) >= 1, f"mutation site not found: {name}"
    mutated = original.replace(old, new, 1)
    assert mutated != original
    r = run_battery(mutated, tmpdir, name.replace(" ", "_").replace("/", "_"))
    assert r.returncode != 0, f"mutant '{name}' survived every pin:\n{r.stdout}\n{r.stderr}"
