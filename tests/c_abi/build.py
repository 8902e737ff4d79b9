"""Build the plain-C test program that uses the library through its header.

gcc compiles it as C11 against include/moe_dispatch.h and the HIP runtime's C
header, links libmoe_dispatch.so (found next to the program through an
$ORIGIN-relative rpath) and compiles the CPU oracle's C source in.  Test
infrastructure: the product never runs this program.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PROGRAM = os.path.join(HERE, "c_abi_smoke")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    pkg = os.path.join(ROOT, "combine_moe_dispatch_amd")
    tmp = PROGRAM + ".tmp"
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-fno-fast-math", "-ffp-contract=off",
           "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "oracle"), "-I", os.path.join(ROCM, "include"),
           os.path.join(HERE, "c_abi_smoke.c"), os.path.join(ROOT, "oracle", "moe_oracle.c"),
           "-o", tmp, "-L", pkg, "-lmoe_dispatch", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-lm", "-Wl,-rpath,$ORIGIN/../../combine_moe_dispatch_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    subprocess.run(cmd, check=True)
    os.replace(tmp, PROGRAM)
    return PROGRAM


if __name__ == "__main__":
    print(build())
