"""The ahead-of-time build's options (CPU, no GPU): the per-kernel resource remarks that
stand in for the JIT's verbose register report, and the compiler output shown when a
compile fails."""
import os
import shutil
import subprocess

import pytest

from fp8_block_scaled_e4m3_amd import build as B


pytestmark = pytest.mark.skipif(not shutil.which(B.hipcc()) and not os.path.exists(B.hipcc()),
                                reason="needs hipcc")


def test_resource_remarks_name_every_kernel(tmp_path):
    out = B.compile_source("dg_quant.hip", str(tmp_path / "q.o"), resource_usage=True)
    rem = B.resource_remarks(out)
    kernels = [r for r in rem if r.startswith("Function Name:")]
    assert any("quant_1x128_kernel" in k for k in kernels)
    assert any("quant_128x128_kernel" in k for k in kernels)
    assert any("sa_mn_major_kernel" in k for k in kernels)
    for key in ("VGPRs:", "AGPRs:", "ScratchSize", "Occupancy", "LDS Size"):
        assert sum(r.startswith(key) for r in rem) == len(kernels), key
    # the casts keep everything in registers
    assert all(r.endswith(": 0") for r in rem if r.startswith("ScratchSize") or r.startswith("VGPRs Spill"))


def test_failed_compile_shows_the_compiler_output(tmp_path, capsys):
    bad = tmp_path / "bad.hip"
    bad.write_text("this is not C++\n")
    with pytest.raises(subprocess.CalledProcessError):
        B.run_tool([B.hipcc(), "--offload-arch=gfx950", "-c", str(bad), "-o", str(tmp_path / "bad.o")], False)
    assert "error" in capsys.readouterr().err
