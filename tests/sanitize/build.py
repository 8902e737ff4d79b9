"""Host-sanitizer builds: AddressSanitizer and UndefinedBehaviorSanitizer on
CPU code only (the device code of the library is compiled exactly as in the
normal build).  Test infrastructure; the product never loads these.

Builds, under _build/sanitize/:
  tree/             a copy of the package, oracle, tests and header in which
                    the package's libmoe_dispatch.so and libmoe_ceiling.so and
                    oracle/libmoe_oracle.so are the instrumented builds;
  reject_paths      the C ABI's argument checks called from plain C;
  libplanted.so     a deliberate heap overflow, to show the run reports one.
All are built with clang from the ROCm toolchain so that one sanitizer
runtime (clang's, preloaded into the process) serves every library.
"""
from __future__ import annotations

import concurrent.futures
import glob
import hashlib
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
OUT = os.path.join(ROOT, "_build", "sanitize")
TREE = os.path.join(OUT, "tree")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
SAN_C = ["-fsanitize=address,undefined", "-shared-libsan", "-fno-omit-frame-pointer", "-g", "-O1"]
# host-only instrumentation for hipcc: each sanitizer flag behind -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-shared-libsan", "-Xarch_host", "-fno-omit-frame-pointer"]


def runtime() -> str:
    """clang's AddressSanitizer runtime (to preload into the test process)."""
    found = sorted(glob.glob(os.path.join(ROCM, "llvm", "lib", "clang", "*", "lib", "linux",
                                          "libclang_rt.asan-x86_64.so")))
    if not found:
        raise FileNotFoundError("clang's AddressSanitizer runtime is not installed")
    return found[-1]


def _sources_hash(paths) -> str:
    h = hashlib.sha256()
    for p in sorted(paths):
        h.update(p.encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()


def _library(out_so: str) -> None:
    from combine_moe_dispatch_amd import build as b
    objdir = os.path.join(OUT, "obj")
    os.makedirs(objdir, exist_ok=True)

    def one(src):
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmd = [HIPCC, *[f for f in b.FLAGS if f != "-O3"], "-O1", "-g", *HOST_SAN, "-c",
               os.path.join(b.CSRC, src), "-o", obj]
        subprocess.run(cmd, check=True, capture_output=True)
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=8) as ex:
        objs = list(ex.map(one, b.SOURCES + [b.CEILING_SOURCE]))
    # the library, and the benchmark's streaming-floor library beside it
    for so, part in ((out_so, objs[:-1]), (os.path.join(os.path.dirname(out_so),
                                                       "libmoe_ceiling.so"), objs[-1:])):
        subprocess.run([HIPCC, f"--offload-arch={b.ARCH}", "-shared", "-fPIC", *HOST_SAN,
                        "-o", so, *part], check=True, capture_output=True)


def build() -> str:
    """Build everything (again only when a source changed); returns the tree."""
    srcs = (glob.glob(os.path.join(ROOT, "combine_moe_dispatch_amd", "csrc", "*")) +
            glob.glob(os.path.join(ROOT, "oracle", "*.[ch]")) +
            glob.glob(os.path.join(ROOT, "include", "*.h")) + glob.glob(os.path.join(HERE, "*.c")))
    stamp = os.path.join(OUT, "sources.sha256")
    digest = _sources_hash(srcs)
    fresh = os.path.exists(stamp) and open(stamp).read() == digest
    # the tree's Python files and tests are always refreshed
    if os.path.exists(TREE):
        keep = {}
        for rel in ("combine_moe_dispatch_amd/libmoe_dispatch.so",
                    "combine_moe_dispatch_amd/libmoe_ceiling.so", "oracle/libmoe_oracle.so"):
            p = os.path.join(TREE, rel)
            if fresh and os.path.exists(p):
                keep[rel] = open(p, "rb").read()
        shutil.rmtree(TREE)
    else:
        keep = {}
    os.makedirs(TREE)
    ign = shutil.ignore_patterns("__pycache__", "*.so", "*.o", ".pytest_cache")
    for d in ("combine_moe_dispatch_amd", "oracle", "tests", "include"):
        shutil.copytree(os.path.join(ROOT, d), os.path.join(TREE, d), ignore=ign)
    shutil.copy(os.path.join(ROOT, "bench.py"), TREE)
    # the plain-C GPU test program is not run here; a copy keeps the tree's
    # conftest from building one against the instrumented library
    smoke = os.path.join(ROOT, "tests", "c_abi", "c_abi_smoke")
    if os.path.exists(smoke):
        shutil.copy(smoke, os.path.join(TREE, "tests", "c_abi", "c_abi_smoke"))
    lib = os.path.join(TREE, "combine_moe_dispatch_amd", "libmoe_dispatch.so")
    ora = os.path.join(TREE, "oracle", "libmoe_oracle.so")
    if len(keep) == 3:
        for rel, data in keep.items():
            open(os.path.join(TREE, rel), "wb").write(data)
    else:
        _library(lib)
        subprocess.run([CLANG, "-std=c11", *SAN_C, "-fPIC", "-shared", "-fno-fast-math",
                        "-ffp-contract=off", "-Wall", os.path.join(ROOT, "oracle", "moe_oracle.c"),
                        "-o", ora, "-lm"], check=True)
    pkg = os.path.dirname(lib)
    subprocess.run([CLANG, "-std=c11", *SAN_C, "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(HERE, "reject_paths.c"), "-o", os.path.join(OUT, "reject_paths"),
                    "-L", pkg, "-lmoe_dispatch", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath," + pkg, "-Wl,-rpath," + os.path.join(ROCM, "lib")], check=True)
    subprocess.run([CLANG, "-std=c11", *SAN_C, "-fPIC", "-shared",
                    os.path.join(HERE, "planted_overflow.c"),
                    "-o", os.path.join(OUT, "libplanted.so")], check=True)
    open(stamp, "w").write(digest)
    return TREE


if __name__ == "__main__":
    print(build())
