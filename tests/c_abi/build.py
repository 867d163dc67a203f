"""Build tests/c_abi/lce_c_check: a plain-C caller of liblce.so (test infrastructure).

    python tests/c_abi/build.py

Compiled with gcc (C11) against include/lce.h and the HIP runtime; it finds
liblce.so through an rpath relative to itself, so the tree can move.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "lce_c_check.c")
OUT = os.path.join(HERE, "lce_c_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
           "-o", OUT + ".tmp", "-L", os.path.join(ROOT, "vocab_projection_amd"), "-llce",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm",
           "-Wl,-rpath,$ORIGIN/../../vocab_projection_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
