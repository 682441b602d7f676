"""The C ABI from a plain C program: tests/native/c_caller (built by
__graft_entry__.build()) runs the fused step, the reduction and Adam from the
reduced gradient through libzero.so with hipMalloc'd buffers -- no Python and
no PyTorch in that process -- and checks every result bit against the oracle's
C functions."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "native", "c_caller")


@pytest.mark.gpu
def test_plain_c_caller(gpu):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is not built; run __graft_entry__.build()")
    print("[c caller] psi=100003 n_d=4 owner=2, 3 steps", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c_caller ok" in r.stdout
