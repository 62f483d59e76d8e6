"""AddressSanitizer + UndefinedBehaviorSanitizer builds of the host code, run on the CPU.

* The C ABI's validation and planning: fp8_block_scaled_e4m3_amd/csrc/dg_api.cpp,
  compiled unchanged with g++, linked with host_models/dg_host_stub.cpp (the library's
  own configuration table with recording launchers, one fake 256-CU device) and driven
  by host_models/dg_host_check.cpp: documented statuses, planned launches for the
  workloads, hostile sizes, the per-thread configuration pin, the layout checker.
* The oracle: oracle/oracle.c with host_models/oracle_check.c, every export on small
  edge-heavy inputs plus a few closed forms.
Any sanitizer report aborts the program (no recovery), so each test passes only when
the driver's own checks pass and the sanitizers stay silent.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
MODELS = os.path.join(HERE, "host_models")
SAN = ["-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ROCM_INCLUDE = "/opt/rocm/include"


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, f"{os.path.basename(exe)} rc={r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "0 failures" in r.stdout


def test_dispatcher_under_sanitizers(tmp_path):
    if not shutil.which("g++") or not os.path.isdir(os.path.join(ROCM_INCLUDE, "hip")):
        pytest.skip("needs g++ and the HIP headers")
    exe = str(tmp_path / "dg_host_check")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I" + ROCM_INCLUDE,
                    os.path.join(ROOT, "fp8_block_scaled_e4m3_amd", "csrc", "dg_api.cpp"),
                    os.path.join(MODELS, "dg_host_stub.cpp"), os.path.join(MODELS, "dg_host_check.cpp"),
                    "-o", exe, "-pthread"], check=True)
    _run(exe)


def test_oracle_under_sanitizers(tmp_path):
    if not shutil.which("gcc"):
        pytest.skip("needs gcc")
    exe = str(tmp_path / "oracle_check")
    subprocess.run(["gcc", "-std=gnu11", *SAN, "-ffp-contract=off", "-pthread",
                    os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(MODELS, "oracle_check.c"),
                    "-o", exe, "-lm"], check=True)
    _run(exe)
