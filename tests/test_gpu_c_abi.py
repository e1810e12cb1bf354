"""The C ABI from plain C on the GPU: tests/c_abi/abi_forward creates a handle,
runs one forward on a stream of its own and checks it against the fp64 oracle
(dispatch bit for bit, outputs within the layer's tolerance) with no Python in
its process; bf16 and block-FP8, a shared expert of another width, ids -1."""
import os
import subprocess

import pytest

from gpu_util import say

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "abi_forward")


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_c_program_runs_the_layer(dtype):
    assert os.path.exists(BIN), "tests/c_abi/abi_forward is not built (the build step builds it)"
    r = subprocess.run([BIN, dtype], capture_output=True, text=True, timeout=120)
    say(r.stdout.strip(), r.stderr.strip()[-2000:])
    assert r.returncode == 0, r.stdout + r.stderr
    assert "PASS" in r.stdout and "dispatch exact" in r.stdout
