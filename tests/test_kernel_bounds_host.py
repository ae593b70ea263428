"""Host checks (CPU) of the index arithmetic of the top-k and fused row
kernels, compiled from the header their launchers use and run before the
kernels run on a GPU:

- tests/host/topk_check.cpp replays one wave's pass over a row with the
  kernel's filter, capacity and compaction rules (topk_cap,
  topk_sel_limit): every candidate-buffer write, every compaction read and
  in-place rewrite, every histogram bin stays in bounds, and the final
  selection equals a brute-force top-k, on normal, ascending (a compaction
  on every sub-tile), descending, all-tied, few-valued, Zipf-like, signed
  zero and outlier rows, float32, bf16 and element paths, k from 1 to 2048.
- tests/host/rows_check.cpp walks the row kernels' launch table and LDS
  layout (row_shape, row_lds) for V up to 2^19: staged shapes hold the
  row, the LDS regions are disjoint and within the block's share, and every
  teacher id's bitmap bit and 16-byte vector bits stay inside the bitmap.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def build_and_run(tmp_path, name):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    exe = tmp_path / name
    subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--offload-arch=gfx950",
                    f"-I{ROOT}/vocab_softmax_loss_amd/csrc",
                    os.path.join(HERE, "host", name + ".cpp"), "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok"), r.stdout
    return r.stdout


def test_topk_buffer_bounds(tmp_path):
    build_and_run(tmp_path, "topk_check")


def test_row_kernel_plans(tmp_path):
    build_and_run(tmp_path, "rows_check")
