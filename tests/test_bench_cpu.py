"""Host logic of bench.py on the CPU: the one-GPU contract, the counter-summary arithmetic
(per-launch HBM bytes scaled by the calibration copy) and the source-digest guard that
keeps a stale summary out of the bench line."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stdout + res.stderr


def _write_counters(path, counter, values):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "out_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, vals in values.items():
            for v in vals:
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_PATH", str(out))
    copy_kib = bench.COPY_BYTES / 1024.0
    # the calibration copy reads 2x and writes 1x its bytes in these synthetic counters
    fetch = {"neg_kernel": [2 * copy_kib, 2 * copy_kib]}
    write = {"neg_kernel": [copy_kib]}
    for key, (sub, _) in bench.COUNTER_KERNELS.items():
        name = sub + ", 8>(...)"
        fetch[name] = [1000.0, 3000.0]          # mean 2000 KiB -> 1000 KiB scaled
        write[name] = [500.0]
    _write_counters(str(tmp_path / "fetch"), "FETCH_SIZE", fetch)
    _write_counters(str(tmp_path / "write"), "WRITE_SIZE", write)
    assert bench.traffic_summary(str(tmp_path / "fetch"), str(tmp_path / "write")) == 0
    data = json.loads(out.read_text())
    assert data["calibration"]["fetch_factor"] == pytest.approx(0.5)
    assert data["calibration"]["write_factor"] == pytest.approx(1.0)
    for key, ent in data["kernels"].items():
        assert ent["fetch_bytes"] == 1000 * 1024
        assert ent["write_bytes"] == 500 * 1024
        assert ent["hbm_bytes_per_launch"] == 1500 * 1024
        assert ent["source_digest"] == bench._source_digest(bench.COUNTER_KERNELS[key][1])
    assert any("FETCH_SIZE" in c for c in data["commands"])


def test_traffic_is_withheld_for_other_sources(tmp_path, monkeypatch):
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_PATH", str(out))
    out.write_text(json.dumps({"kernels": {"gemm_i8_residues": {
        "source_digest": "0123456789abcdef", "hbm_bytes_per_launch": 42}}}))
    assert bench._traffic("gemm_i8_residues", "0123456789abcdef") == 42
    assert bench._traffic("gemm_i8_residues", "fedcba9876543210") is None
    assert bench._traffic("crt", "0123456789abcdef") is None
    monkeypatch.setattr(bench, "TRAFFIC_PATH", str(tmp_path / "missing.json"))
    assert bench._traffic("gemm_i8_residues", "0123456789abcdef") is None


def _fake_extras(products_ms):
    runs = [{"nrhs": n, "native_fp64": {"ms": 3.0}, "on_the_fly_cached_exps": {"ms": 2.0},
             "stored_planes": {"ms": 2.5}} for n in (1, 8, 32)]
    return {"gemv_32768": {"runs": runs},
            "square_4096": {"step_r16_max": {"ms": 1.2, "products_ms": products_ms},
                            "deconstruct_rows": {"ms": 0.1}, "deconstruct_cols": {"ms": 0.12}}}


def test_calibrated_time_model_reduces_to_the_datasheet_model():
    """With measured ceilings equal to the datasheet rates (and an unbounded copy rate)
    the calibrated model equals the datasheet one; with slower products and streams every
    calibrated time is at least the datasheet one."""
    peak_ms = 16 * 2.0 * bench.SQ ** 3 / (bench.PEAK_INT8_TOPS * 1e12) * 1e3
    fast = bench.tme_model(_fake_extras(peak_ms),
                           {"hbm_read_gbs": bench.PEAK_HBM_GBS, "hbm_copy_gbs": 1e12})
    assert fast is not None
    for case in fast["cases"]:
        if "model_calibrated_ms" in case:
            assert case["model_calibrated_ms"] == pytest.approx(case["model_ms"], abs=2e-3)
    slow = bench.tme_model(_fake_extras(2 * peak_ms),
                           {"hbm_read_gbs": 6000.0, "hbm_copy_gbs": 5000.0})
    cal = [c for c in slow["cases"] if "model_calibrated_ms" in c]
    assert len(cal) == 5   # four GEMV paths and the DGEMM step
    for case in cal:
        assert case["model_calibrated_ms"] >= case["model_ms"] - 1e-9
