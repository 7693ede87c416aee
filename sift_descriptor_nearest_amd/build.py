"""Build the HIP library ``libserac.so`` for gfx950 with hipcc."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "serac.hip")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libserac.so")
PROBE_SRC = os.path.join(HERE, "csrc", "probe.hip")
PROBE_LIB = os.path.join(HERE, "libserac_probe.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    # keep the compiler from forming packed-FP32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # run LLVM's machine-code verifier after every backend pass, so that a
    # register-allocation inconsistency fails the build instead of producing
    # a kernel that computes wrong results
    "-mllvm", "-verify-machineinstrs",
    # pass the first 16 dwords of scalar kernel arguments in SGPRs at wave
    # launch (kernels whose first loads depend on them take them first)
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
    # an inline-assembly statement that clobbers a register the compiler
    # reserves (M0, EXEC, VCC, ...) is a build error, not a warning
    "-Werror=inline-asm",
]


def _hipcc(src: str, out: str, extra: tuple = ()) -> str:
    hipcc = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", INCLUDE, src, "-o", tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(out: str = LIB, extra: tuple = ()) -> str:
    """Compile the matcher library (always); returns its path."""
    return _hipcc(SRC, out, extra)


def build_probe(out: str = PROBE_LIB) -> str:
    """Compile the benchmark's measurement kernels (always); returns the path."""
    return _hipcc(PROBE_SRC, out)


if __name__ == "__main__":
    print(build())
    print(build_probe())
