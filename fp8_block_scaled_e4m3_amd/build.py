"""Ahead-of-time build of libdg.so (gfx950 HIP kernels + C ABI) with hipcc.

Every kernel configuration is a template instance compiled here, once; nothing
is compiled at run time.  The library lands next to this file so that it
travels with the source tree.

Environment (the build-time counterparts of the JIT settings the library's README
lists; there is no kernel cache because nothing is compiled at run time):
  DG_HIPCC (or HIPCC)        the hipcc to use (default /opt/rocm/bin/hipcc)
  DG_PRINT_HIPCC_COMMAND=1   print every compile and link command
  DG_RESOURCE_USAGE=1        print the compiler's per-kernel resource remarks
                             (VGPRs, AGPRs, SGPRs, scratch, LDS, occupancy)
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdg.so")
BUILD_DIR = os.path.join(HERE, "_build")
SOURCES = ["dg_gemm.hip", "dg_quant.hip", "dg_api.cpp"]
ARCH = "gfx950"

# Packed-fp32 VALU forms stay disabled; the compiler would otherwise fuse float
# pairs into them on its own.
# MFMA results go to architectural VGPRs.  A kernel of four waves (one per SIMD) may
# use 512 registers, and with that budget the compiler otherwise writes each MFMA
# result into accumulation registers and copies it back with four
# V_ACCVGPR_READ per 16x16 result before the promotion's FMAs can read it: one
# more vector instruction per FMA.  With the results in VGPRs the 64x64, 64x112 and
# 128x128 tiles run 7-17% faster at K = 7168 and no kernel needs more than 256
# VGPRs.  The eight-wave kernels are limited to 256 registers and already used
# VGPRs; their code is unchanged.
CODEGEN_FLAGS = [
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", *CODEGEN_FLAGS,
    "-Wall", "-Wno-unused-function", "-I" + INCLUDE,
]
RESOURCE_FLAG = "-Rpass-analysis=kernel-resource-usage"


def env_flag(name: str) -> bool:
    return os.environ.get(name, "0") not in ("", "0")


def hipcc() -> str:
    for cand in (os.environ.get("DG_HIPCC"), os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def run_tool(cmd: list, verbose: bool) -> str:
    """Run a compiler command; its output comes back, and is shown in full on failure."""
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode:
        print(r.stdout[-20000:], file=sys.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd, r.stdout)
    return r.stdout


def resource_remarks(compiler_output: str) -> list:
    """The kernel-resource-usage remarks of a compile (one "Function Name: ..." line per
    kernel, then its VGPRs, AGPRs, SGPRs, scratch, occupancy, spills and LDS size),
    without source positions and the option tag."""
    out = []
    tag = "[" + RESOURCE_FLAG + "]"
    for line in compiler_output.splitlines():
        if "remark:" in line and tag in line:
            out.append(line.split("remark:", 1)[1].replace(tag, "").strip())
    return out


def compile_source(src: str, obj: str, verbose: bool = False, resource_usage: bool = False) -> str:
    """Compile one source of csrc/ to an object; returns the compiler's output."""
    cmd = [hipcc(), *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if resource_usage and src.endswith(".hip"):
        cmd.append(RESOURCE_FLAG)
    return run_tool(cmd, verbose)


def build(verbose: bool = False) -> str:
    verbose = verbose or env_flag("DG_PRINT_HIPCC_COMMAND")
    resource_usage = env_flag("DG_RESOURCE_USAGE")
    os.makedirs(BUILD_DIR, exist_ok=True)

    def compile_one(src: str):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        return obj, compile_source(src, obj, verbose, resource_usage)

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    if resource_usage:
        for src, (_, text) in zip(SOURCES, results):
            for line in resource_remarks(text):
                print(f"[{src}] {line}", file=sys.stderr)
    objs = [obj for obj, _ in results]
    tmp = LIB + ".tmp%d" % os.getpid()
    run_tool([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
