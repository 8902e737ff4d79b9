import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "sanitize: rebuilds host code with AddressSanitizer and "
                            "UndefinedBehaviorSanitizer and runs the CPU tests against it")
    # Load what is built; build only when nothing is (hipcc cross-compiles on
    # a CPU-only host too).
    lib = os.path.join(ROOT, "combine_moe_dispatch_amd", "libmoe_dispatch.so")
    if not os.path.exists(lib):
        from combine_moe_dispatch_amd import build as _b
        _b.build()
    if not os.path.exists(os.path.join(ROOT, "oracle", "libmoe_oracle.so")):
        import oracle
        oracle.build()
    if not os.path.exists(os.path.join(ROOT, "tests", "c_abi", "c_abi_smoke")):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "c_abi_build", os.path.join(ROOT, "tests", "c_abi", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
