"""CPU checks of the measurement plumbing in bench.py: the one-GPU guard, the HBM-counter
summary (each counter scaled by what it reads for a plain copy of known size) and the gate
that reports `traffic` only for the kernel source and workload the counters were taken on."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for kernel, counter, value in rows:
            w.writerow({"Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_pmc_summary_scales_by_the_copy_probe_and_gates_on_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    k = "dsa::indexer_mfma_kernel<true, false, false>(args)"
    other = "dsa::indexer_mfma_kernel<true, false, true>(args)"
    # the kernel: FETCH 100, 102, 101 KiB per dispatch (median 101), WRITE 10; another
    # instantiation in the same file must be ignored
    _counter_csv(tmp_path / "f.csv", [(k, "FETCH_SIZE", 100), (k, "FETCH_SIZE", 102),
                                      (k, "FETCH_SIZE", 101), (other, "FETCH_SIZE", 9999)])
    _counter_csv(tmp_path / "w.csv", [(k, "WRITE_SIZE", 10), (other, "WRITE_SIZE", 9999)])
    # a 4 MiB copy that FETCH_SIZE counts as half its bytes and WRITE_SIZE as all of them
    _counter_csv(tmp_path / "cf.csv", [("copy_kernel", "FETCH_SIZE", 2048)])
    _counter_csv(tmp_path / "cw.csv", [("copy_kernel", "WRITE_SIZE", 4096)])
    bench.summarize_pmc("indexer_mfma_kernel<true, false, false>", str(tmp_path / "f.csv"),
                        str(tmp_path / "w.csv"), str(tmp_path / "cf.csv"),
                        str(tmp_path / "cw.csv"), 4, 4, "cmd")
    d = json.load(open(tmp_path / "indexer_mfma_kernel_pmc.json"))
    assert d["fetch_scale"] == pytest.approx(2.0) and d["write_scale"] == pytest.approx(1.0)
    assert d["hbm_read_bytes_per_launch"] == pytest.approx(101 * 2.0 * 1024)
    assert d["hbm_write_bytes_per_launch"] == pytest.approx(10 * 1.0 * 1024)
    assert d["dispatches"] == [3, 1]
    total = (101 * 2.0 + 10) * 1024
    assert bench.pmc_traffic("indexer_mfma_kernel", 4) == pytest.approx(total)
    assert bench.pmc_traffic("indexer_mfma_kernel", 2) is None        # another workload
    monkeypatch.setattr(bench, "source_hash", lambda kernel: "0" * 16)
    assert bench.pmc_traffic("indexer_mfma_kernel", 4) is None        # the kernel changed


def test_committed_counter_profile_matches_the_kernel_source():
    """The HBM counters under profiles/ were taken on the indexer as it is in the tree (after a
    change to the kernel or the device header, they must be taken again)."""
    assert bench.pmc_traffic("indexer_mfma_kernel", 4) is not None


def test_implementation_bytes_are_reported_beside_the_algorithmic_ones():
    """Score rows are written once and read once (4 bytes a score); split partials likewise."""
    import types
    wl = types.SimpleNamespace()
    d = bench.implementation_bytes(wl, [10, 20], 1000)
    assert d == {"logits_write_and_read": 2 * 4 * 30, "split_partials_write_and_read": 2000}
