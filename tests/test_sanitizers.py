"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only,
nothing launches a kernel): the oracle, built with gcc's sanitizers, runs
every pin; the library's host side -- argument validation, dispatch and both
precondition checkers -- built with clang's sanitizers on the host pass only,
runs the host ABI and checker tests.  Each runs in a child process with its
sanitizer runtime preloaded; any report fails the test."""
import glob
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")

ORACLE_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
oracle._lib = oracle.bind({lib!r})
from tests import oracle_pins
for check in oracle_pins.ALL_CHECKS:
    check()
print("oracle pins clean", len(oracle_pins.ALL_CHECKS))
"""

LIB_CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import scatter_kvx_gather_amd as kvx
kvx._LIB_PATH = {lib!r}
kvx._lib = None
import pytest
sys.exit(pytest.main(["-q", "-x", "-p", "no:cacheprovider",
                      "-k", "not workload_tables",       # full-size tables: minutes under ASan
                      "tests/test_abi_host.py", "tests/test_check_disjoint.py"]))
"""


def run_child(code, preload):
    env = dict(ENV, LD_PRELOAD=preload)
    p = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=600, env=env, cwd=ROOT)
    out = p.stdout + p.stderr
    assert p.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    return out


def test_oracle_under_asan_ubsan():
    libasan = subprocess.run(["gcc", "-print-file-name=libasan.so"], capture_output=True,
                             text=True, check=True).stdout.strip()
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "liboracle_asan.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-pthread",
                        "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                        os.path.join(ROOT, "oracle", "kvx_oracle.c"), "-o", lib], check=True)
        out = run_child(ORACLE_CHILD.format(root=ROOT, lib=lib), libasan)
    assert "oracle pins clean" in out


def test_library_host_code_under_asan_ubsan():
    rts = glob.glob(os.path.join(ROCM, "lib", "llvm", "lib", "clang", "*", "lib", "linux",
                                 "libclang_rt.asan-x86_64.so"))
    if not rts:
        pytest.skip("clang's shared ASan runtime is not installed")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer"]
    with tempfile.TemporaryDirectory() as tmp:
        lib = os.path.join(tmp, "libkvx_asan.so")
        subprocess.run([os.path.join(ROCM, "bin", "hipcc"), "--offload-arch=gfx950", "-O1", "-g",
                        "-std=c++17", "-fPIC", "-shared", "-Xclang", "-target-feature",
                        "-Xclang", "-packed-fp32-ops", *san,
                        "-I", os.path.join(ROOT, "include"),
                        "-I", os.path.join(ROOT, "scatter_kvx_gather_amd", "csrc"),
                        os.path.join(ROOT, "scatter_kvx_gather_amd", "csrc", "kvx.hip"),
                        "-o", lib], check=True, capture_output=True)
        out = run_child(LIB_CHILD.format(root=ROOT, lib=lib), rts[0])
    assert "passed" in out
