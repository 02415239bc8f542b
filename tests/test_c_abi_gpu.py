"""The C ABI used from plain C (tests/c_abi/afq_c_example.c): a C program
with no Python or torch allocates with hipMalloc, calls the four entry
points and checks the outputs against the C oracle linked into it.  It is
built by __graft_entry__.build() and run here as a child process."""
import os
import subprocess

import pytest

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "afq_c_example")


@pytest.mark.gpu
def test_c_program_against_oracle():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build() first")
    print(f"[c-abi] running {EXE}", flush=True)
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=120)
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c example ok" in r.stdout
