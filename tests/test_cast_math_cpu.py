"""CPU evidence for the FP8 casts' fast arithmetic (no GPU needed).

The cast kernels compute each block's scale fp32(amax / FMAX) on their fast path
with a constant reciprocal and one correction step instead of a division.
``host_models/block_scale_check.c`` replays those steps in IEEE single precision
for every fp32 amax the fast path admits and compares them with the IEEE quotient;
here it must find no difference, for E4M3 (FMAX 448) and E5M2 (FMAX 57344).  The
same program without the correction step must find differences, so the comparison
is shown to notice a merely faithful quotient.
"""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host_models", "block_scale_check.c")


def _has_fma() -> bool:
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if not _has_fma():
        pytest.skip("host CPU has no FMA instructions to replay the kernels' fused multiply-adds")
    exe = str(tmp_path_factory.mktemp("castmath") / "block_scale_check")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-fno-fast-math", "-pthread", SRC, "-o", exe,
                    "-lm"], check=True)
    return exe


def _run(exe, *args):
    threads = str(min(16, os.cpu_count() or 1))
    r = subprocess.run([exe, args[0], threads, *args[1:]], capture_output=True, text=True, timeout=600)
    fields = r.stdout.split()
    return r.returncode, int(fields[1]), int(fields[3])


@pytest.mark.parametrize("fmax", ["448", "57344"])
def test_block_scale_exact_for_every_amax(checker, fmax):
    rc, checked, bad = _run(checker, fmax)
    assert checked > 1_900_000_000            # every fp32 value of the fast path's range
    assert bad == 0 and rc == 0


@pytest.mark.parametrize("fmax", ["448", "57344"])
def test_block_scale_check_notices_an_uncorrected_quotient(checker, fmax):
    rc, checked, bad = _run(checker, fmax, "uncorrected")
    assert checked == 1 << 24
    assert bad > 0 and rc == 1
