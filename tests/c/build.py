"""Build the plain-C ABI smoke program tests/c/abi_smoke (gcc, host code
only) against libkvx.so and the oracle library, with run paths relative to
the binary so the tree can move."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "abi_smoke.c")
EXE = os.path.join(HERE, "abi_smoke")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC,
           "-L", os.path.join(ROOT, "scatter_kvx_gather_amd"), "-lkvx",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../scatter_kvx_gather_amd:$ORIGIN/../../oracle:"
           + os.path.join(ROCM, "lib"),
           "-o", EXE + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
