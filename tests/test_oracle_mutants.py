"""Planted mistakes in the oracle, on the CPU: each must make a pin fail.

Each mutant is oracle.c with one plausible slip (a dropped term, a wrong sign, a wrong
pairing or table row, a missing scale, a misaligned mask, a wrong head grouping).  It
is compiled to a temporary library and the pin suite is run against it in a child
process; the suite has to fail.  This shows the pins are not blind to the slip.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "eps outside the root": ("sqrt(ms + eps)", "(sqrt(ms) + eps)"),
    "eps dropped": ("sqrt(ms + eps)", "sqrt(ms)"),
    "weight dropped": ("x[e] / root * w[e]", "x[e] / root"),
    "sum not divided by d": ("ms /= (double)d;", ";"),
    "wrong turn sign": ("x[e + half] = b * c + a * s;", "x[e + half] = b * c - a * s;"),
    "turn the other way": ("x[e] = a * c - b * s;\n        x[e + half] = b * c + a * s;",
                           "x[e] = a * c + b * s;\n        x[e + half] = b * c - a * s;"),
    "adjacent pairs": ("const double a = x[e], b = x[e + half];",
                       "const double a = x[e], b = x[e + 1];"),
    "table row off by one": ("cos_t + pos[r] * half", "cos_t + (pos[r] ? pos[r] - 1 : 0) * half"),
    "cos and sin swapped": ("const double c = cos_row[e], s = sin_row[e];",
                            "const double c = sin_row[e], s = cos_row[e];"),
    "scale dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "top-left causal mask": ("if (causal && i + n - tq < last)\n        last = i + n - tq;",
                             "if (causal && i < last)\n        last = i;"),
    "interleaved head groups": ("const int64_t g = h / (hq / hkv);",
                                "const int64_t g = h % hkv;"),
    "max not subtracted consistently": ("const double wj = exp(s[j] - m);",
                                        "const double wj = exp(s[j] - m) * (j == 0 ? 2.0 : 1.0);"),
    "pairs: wrong turn sign": ("x[2 * i + 1] = b * c + a * s;", "x[2 * i + 1] = b * c - a * s;"),
    "pairs: wrong table entry": ("const double c = cos_row[i], s = sin_row[i];",
                                 "const double c = cos_row[i / 2], s = sin_row[i / 2];"),
    "pairs: partner half away": ("const double a = x[2 * i], b = x[2 * i + 1];",
                                 "const double a = x[2 * i], b = x[i + half];"),
    "row norm over one head": ("acc /= (double)width;", "acc /= (double)head;"),
    "row rotary: same angles for every head": ("t = h * half + j;", "t = j;"),
    "kv: codes truncated, not rounded": ("float t = rintf((x - lo) * inv);", "float t = truncf((x - lo) * inv);"),
    "kv: codes not clamped at the top": ("if (t > (float)top) t = (float)top;", ";"),
    "kv: step over 2^bits levels": ("*st = (hw + hw) / (float)top;", "*st = (hw + hw) / (float)(top + 1);"),
    "kv: range starts at the minimum": ("*lo = centre - hw;", "*lo = centre - r;"),
    "kv: the largest error wins": ("if (sse < best) {", "if (sse > best || best == INFINITY) {"),
    "int8: scale over 128": ("const float s = amax > 0.0f ? amax / 127.0f : 1.0f;",
                             "const float s = amax > 0.0f ? amax / 128.0f : 1.0f;"),
    "int8: codes truncated": ("float t = rintf(xu[i] * inv);", "float t = truncf(xu[i] * inv);"),
    "e4m3: two fraction bits": ("step = ldexpf(1.0f, e - 1 - 3);", "step = ldexpf(1.0f, e - 1 - 2);"),
    "e4m3: ties away from zero": ("const float q = rintf(m / step) * step;", "const float q = roundf(m / step) * step;"),
    "value of wrong key": ("const double *vj = v + ((b * tk + j) * hkv + g) * dv;",
                           "const double *vj = v + ((b * tk + (j ? j - 1 : 0)) * hkv + g) * dv;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found: " + name
    mutant = tmp_path / "oracle_mutant.c"
    mutant.write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99",
                    "-I", os.path.join(ROOT, "oracle"), str(mutant), "-o", str(lib), "-lm"],
                   check=True)
    env = dict(os.environ, ATTN_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "no pin caught the mutant '%s':\n%s" % (name, r.stdout[-2000:])
