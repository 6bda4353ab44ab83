"""The C ABI called from C++ alone, with no Python binding and no torch.

tests/c_abi_check.cpp (compiled by the repository's build step into
``_build/c_abi_check``) allocates device memory with hipMalloc, calls
blockattn_fwd and blockattn_bwd on seeded bf16 inputs and compares them with
the fp64 oracle at the bf16 tolerances; it also checks the status codes of
calls the library must reject.
"""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_abi_from_cpp():
    exe = os.path.join(ROOT, "_build", "c_abi_check")
    assert os.path.exists(exe), "the build step compiles tests/c_abi_check.cpp into _build/c_abi_check"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=180)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
    assert "PASSED (0 failures)" in r.stdout
