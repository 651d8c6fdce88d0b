"""Host logic of bench.py that runs without a GPU: the counter digest that
turns two rocprofv3 --pmc CSVs into the per-launch HBM traffic of the main
kernel, and the --gpus guard."""
import csv
import json
import subprocess
import sys
from pathlib import Path

import bench

FIELDS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Counter_Name", "Counter_Value"]


def write_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (name, grid, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Grid_Size": grid, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


def test_digest_calibrates_on_the_first_copy(tmp_path, monkeypatch):
    """The calibration copy is the run's first device copy; a later, larger
    copy (inputs cloned while building the workload) must not be taken for it."""
    calib_kib = bench.CALIB_BYTES // 1024
    kernel = "void sa::gqa_forward_kernel<false, false, true>(...)"
    # FETCH_SIZE reads half the copied bytes, WRITE_SIZE all of them
    fetch = [("__amd_rocclr_copyBuffer", 131072, calib_kib / 2),
             ("__amd_rocclr_copyBuffer", 131072, 4 * calib_kib / 2),   # a 1 GiB clone
             (kernel, 2048, 1000.0), (kernel, 2048, 1002.0)]
    write = [("__amd_rocclr_copyBuffer", 131072, calib_kib),
             ("__amd_rocclr_copyBuffer", 131072, 4 * calib_kib),
             (kernel, 2048, 10.0), (kernel, 2048, 10.0)]
    f, w = tmp_path / "f.csv", tmp_path / "w.csv"
    write_csv(f, "FETCH_SIZE", fetch)
    write_csv(w, "WRITE_SIZE", write)
    monkeypatch.setattr(bench, "PROFILES", tmp_path / "profiles")

    class Args:
        digest = (str(f), str(w))
        workload = "capacity_decode"

    bench.digest(Args)
    out = json.loads((tmp_path / "profiles" / "gqa_forward_kernel_capacity_decode_counters.json").read_text())
    assert out["calibration"]["fetch_scale"] == 0.5 and out["calibration"]["write_scale"] == 1.0
    assert out["fetch_bytes_per_launch"] == 1001.0 * 1024 / 0.5
    assert out["write_bytes_per_launch"] == 10.0 * 1024
    assert out["dispatches"] == 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(Path(bench.__file__)), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
