"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of oracle/oracle.c (a wrong exponent bias, a
dropped sign or scale, truncation in place of round-to-nearest-even, a wrong or
transposed index, an operand used twice, a group stride ignored, an off-by-one row
bound), builds the copy with the oracle's own compile command and runs the pin suite
(tests/test_oracle_pins.py) against it in a child process with ORC_LIB pointing at
the copy.  The suite must fail for every planted mistake and pass for the unmodified
copy.  Everything here runs on the CPU; nothing touches the HIP library.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

E4M3_RNE = "n = nearbyint(a / q);       /* exact division by a power of two; RNE (default mode) */\n" \
           "    if (n < 8.0)"
BF16_RNE = "n = nearbyint(a / q);\n    if (n < 128.0)"

# (name, text in oracle.c, replacement, occurrences of the text in the source; the first is replaced)
MUTANTS = [
    ("e4m3 exponent bias", "(int)e - 10)", "(int)e - 9)", 1),
    ("e4m3 subnormal step", "mag = ldexp((double)f, -9);", "mag = ldexp((double)f, -10);", 1),
    ("e4m3 decode drops the sign",
     "(int)e - 10);\n    return s ? -mag : mag;", "(int)e - 10);\n    return mag;", 1),
    ("e4m3 encode truncates", E4M3_RNE, E4M3_RNE.replace("nearbyint", "trunc"), 1),
    ("e4m3 encode saturates to NaN", "if (a >= 448.0) return (uint8_t)(sign | 0x7Eu);",
     "if (a >= 448.0) return (uint8_t)(sign | 0x7Fu);", 1),
    ("e4m3 encode drops the sign", "sign = signbit(x) ? 0x80u : 0u;", "sign = 0u;", 2),
    ("e5m2 exponent bias", "(int)e - 17)", "(int)e - 16)", 1),
    ("bf16 encode truncates", BF16_RNE, BF16_RNE.replace("nearbyint", "trunc"), 1),
    ("cast scale uses another FP8 maximum", "(fmt ? 57344.0f : 448.0f)", "(fmt ? 57344.0f : 240.0f)", 1),
    ("all-zero block gets scale 0", "return amax == 0.0f ? 1.0f : s;", "return s;", 1),
    ("B-side cast stores its scales transposed", "sb[(long)nb * kbn + kb] = s;",
     "sb[(long)kb * nbn + nb] = s;", 1),
    ("A scale read without its leading dimension", "sa_col[(long)kb * ld_sa]", "sa_col[kb]", 1),
    ("B scale row ignores the N block", "sbg + (long)(j / ORC_KBLOCK) * kbn", "sbg", 1),
    ("B scale K blocks reversed", "(double)sb_row[kb];", "(double)sb_row[kbn - 1 - kb];", 1),
    ("scales dropped from the sum", "acc += s * p;", "acc += p;", 1),
    ("block dot uses A twice", "p += DEC[a[t]] * DEC[b[t]];", "p += DEC[a[t]] * DEC[a[t]];", 1),
    ("block dot swaps the operand formats", "MANT[fa][a[t]] * (__int128)MANT[fb][b[t]]",
     "MANT[fb][a[t]] * (__int128)MANT[fa][b[t]]", 1),
    ("contiguous padding rows computed", "if (g < 0) return;", "if (g < 0) g = 0;", 1),
    ("masked row bound off by one", "if (local >= mm) return;", "if (local > mm) return;", 1),
    ("grouped B ignores the group", "bg = J->b + (long)g * J->b_group_stride;", "bg = J->b;", 1),
    ("masked A scales ignore the group", "sa_col = J->sa + (long)g * J->sa_group_stride + local;",
     "sa_col = J->sa + local;", 1),
]


def plant(src_text, old, new, count):
    assert src_text.count(old) == count, f"{old!r} occurs {src_text.count(old)} times, expected {count}"
    return src_text.replace(old, new, 1)


def run_pins(lib):
    env = dict(os.environ, ORC_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-3000:] + r.stderr[-2000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants")
    with open(oracle._SRC) as f:
        text = f.read()
    cases = [("unmodified", text)] + [(name, plant(text, old, new, n)) for name, old, new, n in MUTANTS]
    libs = {}
    for i, (name, body) in enumerate(cases):
        src = os.path.join(d, f"m{i}.c")
        with open(src, "w") as f:
            f.write(body)
        libs[name] = os.path.join(d, f"m{i}.so")
        oracle.compile_library(src, libs[name])
    workers = max(1, min(4, (os.cpu_count() or 2) // 2))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = dict(zip(libs, ex.map(run_pins, libs.values())))
    return results


def test_unmodified_copy_passes_the_pins(outcomes):
    rc, log = outcomes["unmodified"]
    assert rc == 0, log


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(outcomes, name):
    rc, log = outcomes[name]
    assert rc == 1, f"pins did not catch '{name}' (exit {rc}):\n{log}"
    assert "failed" in log
