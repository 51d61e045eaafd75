"""Build libzero_shard.so (the HIP library behind include/zero_shard.h) in-tree.

    python sharded_optimizer_step_shard_amd/build.py

(run as a script: importing the package needs the library already built).

compiles csrc/zero_kernels.hip, csrc/zero_probes.hip, csrc/zero_chunks.cpp and
csrc/zero_api.cpp for gfx950 with hipcc.
Flags that matter for the results:
  -ffp-contract=off  no fused multiply-add: the double arithmetic of the step
                     must be the separately rounded operations it is defined as.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                     keep the compiler from emitting packed fp32 instructions.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzero_shard.so")
ARCH = os.environ.get("ZERO_SHARD_ARCH", "gfx950")

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-fno-fast-math",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(verbose: bool = True, out: str = LIB, extra=()) -> str:
    srcs = [os.path.join(CSRC, f)
            for f in ("zero_kernels.hip", "zero_probes.hip", "zero_chunks.cpp", "zero_api.cpp")]
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-o", out, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


def build_c_example(verbose: bool = True) -> str:
    """The plain C consumer of the ABI used by the tests (gcc, no hipcc, no
    Python): tests/c_abi/step_c."""
    src = os.path.join(ROOT, "tests", "c_abi", "step_c.c")
    out = os.path.join(ROOT, "tests", "c_abi", "step_c")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           "-I", INCLUDE, "-o", out, src, "-L", PKG, "-lzero_shard", f"-L{rocm}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../sharded_optimizer_step_shard_amd", f"-Wl,-rpath,{rocm}/lib"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build_c_example(verbose=True)
    sys.exit(0)
