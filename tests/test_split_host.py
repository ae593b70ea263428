"""Host logic of the split-row kernels (CPU): their launch shapes stay in
bounds and their mailbox handshake, run by real threads under random
delays, hands every member each partner's record of the same row and leaves
the mailbox empty; compiled from the library's own header and run; see
tests/host/split_check.cpp."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_split_shapes_and_handshake(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / "split_check"
    subprocess.run([hipcc, "-O1", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                    f"-I{ROOT}/vocab_softmax_loss_amd/csrc",
                    os.path.join(HERE, "host", "split_check.cpp"), "-o", str(exe), "-pthread"],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")
