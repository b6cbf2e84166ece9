"""The library through its C ABI alone: tests/c_abi/check_c_abi.c (plain C,
hipMalloc'd buffers, a stream of its own, no Python or torch) runs softmax
forward (fp32 and bf16, from a [2, 3] tensor whose second row starts off
a 16-byte boundary to the split-k shape), the backward and LayerNorm, compares every output with the CPU oracle
under the same bounds as the Python parity tests, and checks the error
statuses of bad arguments.  The binary is built by the package build."""
import os
import subprocess

import pytest

from gpu_util import have_gpu

BINARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "check_c_abi")


@pytest.mark.gpu
@pytest.mark.skipif(not have_gpu(), reason="needs an MI355X GPU")
def test_c_abi_against_oracle():
    assert os.path.isfile(BINARY) and os.access(BINARY, os.X_OK), \
        "tests/c_abi/check_c_abi missing: run __graft_entry__.build()"
    print(f"running {BINARY}", flush=True)
    r = subprocess.run([BINARY], capture_output=True, text=True, timeout=110)
    print(r.stdout)
    print(r.stderr)
    assert r.returncode == 0, f"check_c_abi exited {r.returncode}:\n{r.stdout}\n{r.stderr}"
    assert "passed: 0 failure(s)" in r.stdout
