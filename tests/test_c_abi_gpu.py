"""The library through its C ABI alone: tests/c_abi/lce_c_check (plain C, hipMalloc
buffers, the null stream, no Python in the process), built by the build step.

It checks the closed forms at W = 0 (lse = ln V, loss = ln V, d_hidden = 0,
d_weight from softmax minus one-hot at uniform probabilities) and that the
strip-level calls in reverse strip order agree with the whole passes.
"""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu
BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "lce_c_check")


def test_c_program_through_the_abi():
    assert os.path.exists(BIN), "tests/c_abi/lce_c_check is not built (python tests/c_abi/build.py)"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c-abi check: ok" in r.stdout
