"""The C ABI from plain C, with no Python or torch in the process:
tests/c/abi_smoke.c runs a gather-scatter and a gather on a HIP stream and
compares every byte with the oracle; an argument error returns its status."""
import importlib.util
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c")
EXE = os.path.join(HERE, "abi_smoke")


def test_c_program_matches_oracle():
    if not os.path.exists(EXE):                 # built by build(); build it if missing
        spec = importlib.util.spec_from_file_location("abi_smoke_build",
                                                      os.path.join(HERE, "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    p = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert p.returncode == 0, p.stdout + p.stderr
    assert "abi_smoke ok" in p.stdout, p.stdout
