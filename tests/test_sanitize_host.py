"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle and the library's host code (argument checks, launch set-up) are
rebuilt with clang's sanitizers (tests/sanitize/build.py; device code
unchanged), the sanitizer runtime is preloaded, and then: a planted heap
overflow must be reported (the run can see errors); the instrumented
libraries must be the ones loaded; the C ABI's argument-rejection paths are
called from plain C; and the whole CPU test suite runs against the
instrumented builds.  Any sanitizer report fails the run.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.sanitize

HERE = os.path.dirname(os.path.abspath(__file__))


def _builder():
    spec = importlib.util.spec_from_file_location("sanitize_build",
                                                  os.path.join(HERE, "sanitize", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.fixture(scope="module")
def san():
    b = _builder()
    try:
        rt = b.runtime()
    except FileNotFoundError as e:
        pytest.skip(str(e))
    tree = b.build()
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    return b, tree, env


def test_planted_overflow_is_reported(san):
    b, tree, env = san
    lib = os.path.join(b.OUT, "libplanted.so")
    r = subprocess.run([sys.executable, "-c", f"import ctypes; ctypes.CDLL({lib!r})."
                        "planted_read_past_end(8)"], env=env, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_instrumented_libraries_are_the_ones_loaded(san):
    b, tree, env = san
    code = ("import oracle, combine_moe_dispatch_amd.api as api; oracle._load(); "
            "print(open('/proc/self/maps').read())")
    r = subprocess.run([sys.executable, "-c", code], cwd=tree, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    maps = r.stdout
    assert "libclang_rt.asan" in maps
    assert os.path.join(tree, "combine_moe_dispatch_amd", "libmoe_dispatch.so") in maps
    assert os.path.join(tree, "oracle", "libmoe_oracle.so") in maps


def test_c_abi_rejection_paths(san):
    b, tree, env = san
    r = subprocess.run([os.path.join(b.OUT, "reject_paths")], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, (r.stdout, r.stderr[-2000:])
    assert "reject_paths: ok" in r.stdout


def test_cpu_suite_under_sanitizers(san):
    b, tree, env = san
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu and not sanitize", "tests"], cwd=tree, env=env,
                       capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
