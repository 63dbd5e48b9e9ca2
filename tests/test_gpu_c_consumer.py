"""The ABI from plain C: tests/c_abi_consumer.c (built by build() into
tests/_build/) includes only include/libvjp.h and the HIP runtime's C API,
calls an entry point of every op family on device buffers, and checks the
results against closed forms (see its header).  It runs as a child process."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROG = os.path.join(ROOT, "tests", "_build", "c_abi_consumer")

pytestmark = pytest.mark.gpu


def test_c_consumer_runs(gpu_lib):
    assert os.path.exists(PROG), "tests/_build/c_abi_consumer missing: run __graft_entry__.build()"
    print(f"\n[c consumer] {PROG}", flush=True)
    r = subprocess.run([PROG], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
