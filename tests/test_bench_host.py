"""Host logic of bench.py, on the CPU: the HBM-traffic conversion of the
rocprofv3 counter CSVs (calibrated on the copy kernel), the kernel-source
hash that voids stale traffic figures, the workload keys, and the refusal
of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write_counters(path, counter, kernel_vals, copy_vals):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        d = 0
        for v in copy_vals:
            d += 1
            w.writerow(dict(Dispatch_Id=d, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name=counter,
                            Counter_Value=v))
        for v in kernel_vals:
            d += 1
            w.writerow(dict(Dispatch_Id=d, Kernel_Name="void fa::fa_prefill_bf16_kernel<128, false, 0, false>(x)",
                            Counter_Name=counter, Counter_Value=v))
            w.writerow(dict(Dispatch_Id=d, Kernel_Name="void other_kernel()", Counter_Name=counter,
                            Counter_Value=1e9))


def test_traffic_from_counters_scales_by_the_copy(tmp_path, monkeypatch):
    """HBM bytes = mean kernel FETCH_SIZE x (copy bytes / copy FETCH_SIZE)
    + mean kernel WRITE_SIZE x (copy bytes / copy WRITE_SIZE); other kernels
    are ignored; the entry lands in <root>/profiles/traffic.json with the
    current source hash."""
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_sha", lambda kind: "sha-" + kind)
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counters(fcsv, "FETCH_SIZE", [1000.0, 3000.0], [131072.0])
    _write_counters(wcsv, "WRITE_SIZE", [500.0, 500.0], [262144.0])
    e = bench.traffic_from_counters(str(fcsv), str(wcsv), "config2", "prefill")
    sf = bench.COPY_BYTES / 131072.0
    sw = bench.COPY_BYTES / 262144.0
    assert e["hbm_bytes_per_launch"] == round(2000.0 * sf + 500.0 * sw)
    assert e["dispatches"] == [2, 2] and e["kernel_sha"] == "sha-prefill"
    tab = json.loads((tmp_path / "profiles" / "traffic.json").read_text())
    assert tab["config2"]["hbm_bytes_per_launch"] == e["hbm_bytes_per_launch"]
    # the bench line takes it while the hash matches, and not once it moves on
    assert bench.measured_traffic("config2", "prefill") == e["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_sha", lambda kind: "changed")
    assert bench.measured_traffic("config2", "prefill") is None


def test_traffic_needs_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counters(fcsv, "FETCH_SIZE", [1000.0], [])
    _write_counters(wcsv, "WRITE_SIZE", [500.0], [262144.0])
    with pytest.raises(SystemExit):
        bench.traffic_from_counters(str(fcsv), str(wcsv), "config2", "prefill")


def test_kernel_sha_covers_each_kernels_sources():
    """Each kind hashes its own sources: the bf16 and FP8 prefill kernels
    are separate kinds, so a change to one does not void the other's
    traffic figure; every listed source exists."""
    for kind, files in bench.KERNEL_SOURCES.items():
        for f in files:
            assert os.path.exists(os.path.join(ROOT, f)), f
        assert len(bench.kernel_sha(kind)) == 16
    assert "attention_fa_fwd_03_amd/csrc/fa_prefill.hip" not in bench.KERNEL_SOURCES["prefill"]
    assert "attention_fa_fwd_03_amd/csrc/fa_prefill_bf16.hip" not in bench.KERNEL_SOURCES["prefill_fp8"]
    assert set(bench.DOMINANT) == set(bench.KERNEL_SOURCES)


def test_workload_keys():
    assert bench._key(2) == "config2"
    assert bench._key(5, "window") == "config5_window"
    assert bench._key(3, layout="vec", q_dtype="fp8", dv=192) == "config3_vec_q8_dv192"
    assert bench._key(4, page_size=16) == "config4_ps16"
    assert bench._key(6, page_size=64, layout="vec") == "config6_ps64_vec"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
