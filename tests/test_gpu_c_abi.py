"""The library used from plain C: a C11 program built against
include/moe_dispatch.h alone routes, dispatches and combines on the GPU and
checks the results against the C oracle (see tests/c_abi/c_abi_smoke.c)."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_c_program_through_the_header():
    print("[case] c_abi_smoke", flush=True)
    prog = os.path.join(HERE, "c_abi", "c_abi_smoke")
    r = subprocess.run([prog], capture_output=True, text=True, timeout=100)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "c_abi_smoke: ok" in r.stdout
