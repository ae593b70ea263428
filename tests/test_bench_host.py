"""bench.py's host logic on the CPU: it refuses more than one GPU, its
algorithmic byte counts follow the per-row formulas, the counter file is
used only while the kernel sources match its hash, and counter CSVs are
averaged per kernel and counter.  No GPU and no kernel launch."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_per_kernel():
    b = bench.algorithmic_bytes()
    row = 32000 * 4
    # top-k: every row read once, k ids and k probs written
    assert b["topk"] == 4096 * row + 4096 * 64 * 8 == 526_385_152
    # KL: every row read and written, ids and probs read, loss written
    assert b["kl"] == 4096 * 2 * row + 4096 * 64 * 8 + 4096 * 4 == 1_050_689_536
    # CE: 8 x 384 rows in the loss read and written, 8 x 128 prompt rows
    # written only; labels read, loss written
    assert b["ce"] == 3072 * 2 * row + 1024 * row + 4096 * 8 == 917_536_768
    # slice accumulate: two [4096][1024] float32 read, one written
    assert b["acc"] == 3 * 4096 * 1024 * 4 == 50_331_648


def _traffic_file(tmp_path, sha, kl_bytes):
    p = tmp_path / "traffic.md"
    p.write_text(f"# counters\n\n```\nkernel_sources_sha256: {sha}\n"
                 f"traffic_bytes.kl: {kl_bytes}\n```\n")
    return str(p)


def test_traffic_used_only_for_matching_sources(tmp_path, monkeypatch):
    sha = bench.kernel_sources_sha256()
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _traffic_file(tmp_path, sha, 123456789))
    assert bench.measured_traffic("kl") == 123456789
    assert bench.measured_traffic("ce") is None  # no line for it
    other = ("0" if sha[0] != "0" else "1") + sha[1:]
    monkeypatch.setattr(bench, "TRAFFIC_FILE", _traffic_file(tmp_path, other, 123456789))
    assert bench.measured_traffic("kl") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("kl") is None


def test_kernel_sources_hash_changes_with_a_source(tmp_path, monkeypatch):
    csrc = tmp_path / "vocab_softmax_loss_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES:
        (csrc / f).write_text("// " + f + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h1 = bench.kernel_sources_sha256()
    (csrc / bench.KERNEL_SOURCES[0]).write_text("// changed\n")
    assert bench.kernel_sources_sha256() != h1


def test_pmc_summary_averages_per_kernel_and_counter(tmp_path, capsys):
    p = tmp_path / "run_counter_collection.csv"
    p.write_text("Kernel_Name,Counter_Name,Counter_Value\n"
                 "k1,FETCH_SIZE,10\nk1,FETCH_SIZE,30\nk2,FETCH_SIZE,5\nk1,WRITE_SIZE,7\n")
    bench.pmc_summary([str(p)])
    lines = sorted(capsys.readouterr().out.strip().splitlines())
    assert lines == ["FETCH_SIZE\t1\t5.0\tk2", "FETCH_SIZE\t2\t20.0\tk1",
                     "WRITE_SIZE\t1\t7.0\tk1"]


@pytest.mark.parametrize("ms,nbytes", [(0.5, 10 ** 9), (2.0, None)])
def test_kernel_table_rates(ms, nbytes):
    t = bench.kernel_table({"x": ms}, {"x": nbytes}, 4096)["x"]
    assert t["rows/s"] == round(4096 / (ms * 1e-3), 1)
    if nbytes is None:
        assert "GB/s" not in t
    else:
        assert t["GB/s"] == round(nbytes / (ms * 1e-3) / 1e9, 1)
        assert t["frac"] == round(t["GB/s"] / bench.HBM_PEAK_GBS, 4)


def test_workload_cpu_baseline_times_the_oracle_on_all_threads_and_one():
    """The per-configuration CPU baseline runs the given oracle stages on
    every OpenMP thread and then on one, restores the thread count, and
    reports rows/s for each with the samples it timed."""
    import numpy as np
    import oracle

    x = np.random.default_rng(7).normal(size=(64, 256)).astype(np.float32)
    lab = np.arange(64, dtype=np.uint32) % 256
    seen = []

    def run(n):
        seen.append((n, oracle.threads()))
        oracle.ce(x[:n], lab[:n])

    before = oracle.threads()
    c = bench.workload_cpu_baseline(run, 64, 64, 16, "CE")
    assert oracle.threads() == before
    assert seen[0] == (2, before) and seen[1] == (64, before) and seen[2] == (16, 1)
    assert c["kind"] == "oracle" and c["unit"] == "rows/s" and c["cores"] == before
    assert c["value"] > 0 and c["single_core"]["value"] > 0 and c["single_core"]["cores"] == 1
    assert "first 64 of the 64 rows (CE)" in c["sample"] and c["cpu_model"]
