"""The C ABI from a plain host program (tests/c_abi/vl_c_check.cpp: HIP
runtime + include/vl.h + libvl.so, no Python in the loop), run as a child
process: every call on inputs with a closed-form result.  The program is
built by __graft_entry__.build().  Needs an MI355X."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROG = os.path.join(ROOT, "tests", "c_abi", "vl_c_check")


def test_c_program_closed_forms():
    assert os.path.exists(PROG), f"{PROG} is missing: run __graft_entry__.build()"
    r = subprocess.run([PROG], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
